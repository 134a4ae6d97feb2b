"""MI355X-native jagged generalized dot-product attention (forward).

The compute path is libjagged_attn.so (hand-written gfx950 HIP kernels behind
a C ABI, include/jagged_attn.h).  This package holds its ctypes binding, a
torch-tensor front end that only marshals arguments, the seeded input
generator and the host-side work accounting.
"""
from ._lib import (JA_SELF, JA_CROSS, JA_PMA, JA_SLIDING, JA_SOFTMAX, JA_GELU_TANH, JA_F32, JA_BF16,  # noqa: F401
                   JA_MXFP8_E4M3, JA_OK, JA_EINVAL, JA_EUNSUPPORTED, JA_EWORKSPACE, JA_EHIP,
                   JA_EOFFSETS, JaIo, JaggedAttnError, jagged_attn_fwd, jagged_attn_workspace_size,
                   jagged_attn_check, jagged_attn_version, strerror)
from .api import forward, backward, mx_quantize, Workspace  # noqa: F401
