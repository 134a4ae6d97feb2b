"""ctypes binding of libjagged_attn.so (the C ABI in include/jagged_attn.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  There is no fallback: if the shared library is missing, loading
raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libjagged_attn.so")

JA_SELF, JA_CROSS, JA_PMA, JA_SLIDING = 0, 1, 2, 3
JA_SOFTMAX, JA_GELU_TANH, JA_GELU_POLY = 0, 1, 2
JA_F32, JA_BF16, JA_MXFP8_E4M3 = 0, 1, 2
JA_OK, JA_EINVAL, JA_EUNSUPPORTED, JA_EWORKSPACE, JA_EHIP, JA_EOFFSETS = 0, -1, -2, -3, -4, -5

VARIANTS = {"self": JA_SELF, "cross": JA_CROSS, "pma": JA_PMA, "sliding": JA_SLIDING}
ACTS = {"softmax": JA_SOFTMAX, "gelu_tanh": JA_GELU_TANH, "gelu_poly": JA_GELU_POLY}
DTYPES = {"f32": JA_F32, "bf16": JA_BF16, "mxfp8": JA_MXFP8_E4M3}

# Every function the header declares (checked by the CPU tests).
EXPORTS = ("jagged_attn_fwd", "jagged_attn_fwd_noalloc", "jagged_attn_workspace_size", "jagged_attn_check",
           "jagged_attn_strerror", "jagged_attn_version", "jagged_attn_mx_quantize",
           "jagged_attn_bwd", "jagged_attn_bwd_workspace_size")


class JaIo(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("total_q", ctypes.c_int32),
        ("total_kv", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("ev_start", ctypes.c_void_p),
        ("ev_stop", ctypes.c_void_p),
        ("max_workgroups", ctypes.c_int32),
        ("status", ctypes.c_void_p),
        ("softmax_stats", ctypes.c_void_p),
        ("fp8_pv", ctypes.c_int32),
        ("lse", ctypes.c_void_p),
        ("fwd_out", ctypes.c_void_p),
    ]


class JaggedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_LIB = None


def load() -> ctypes.CDLL:
    """Load the in-tree library once; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m recsys_jagged_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.jagged_attn_fwd.restype = ctypes.c_int
        lib.jagged_attn_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
            ctypes.c_void_p, ctypes.POINTER(JaIo)]
        lib.jagged_attn_fwd_noalloc.restype = ctypes.c_int
        lib.jagged_attn_fwd_noalloc.argtypes = lib.jagged_attn_fwd.argtypes
        lib.jagged_attn_workspace_size.restype = ctypes.c_size_t
        lib.jagged_attn_workspace_size.argtypes = [ctypes.c_int] * 7 + [ctypes.c_int32] * 2
        lib.jagged_attn_check.restype = ctypes.c_int
        lib.jagged_attn_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.jagged_attn_strerror.restype = ctypes.c_char_p
        lib.jagged_attn_strerror.argtypes = [ctypes.c_int]
        lib.jagged_attn_version.restype = ctypes.c_int
        lib.jagged_attn_version.argtypes = []
        lib.jagged_attn_bwd.restype = ctypes.c_int
        lib.jagged_attn_bwd.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 3 + [
            ctypes.POINTER(JaIo)]
        lib.jagged_attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.jagged_attn_bwd_workspace_size.argtypes = [ctypes.c_int] * 7 + [ctypes.c_int32] * 2
        lib.jagged_attn_mx_quantize.restype = ctypes.c_int
        lib.jagged_attn_mx_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _LIB = lib
    return _LIB


def strerror(status: int) -> str:
    return load().jagged_attn_strerror(int(status)).decode()


def jagged_attn_version() -> int:
    return load().jagged_attn_version()


def jagged_attn_workspace_size(B, H, D, variant, act, window, dtype, total_q, total_kv) -> int:
    return int(load().jagged_attn_workspace_size(B, H, D, variant, act, window, dtype, total_q, total_kv))


def jagged_attn_fwd(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window, out, io: JaIo) -> int:
    """Raw call: pointers are ints (device addresses), returns the status code."""
    return int(load().jagged_attn_fwd(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window,
                                      out, ctypes.byref(io)))


def jagged_attn_fwd_noalloc(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window, out, io: JaIo) -> int:
    """Raw call of the no-allocation forward (io.workspace must be 0)."""
    return int(load().jagged_attn_fwd_noalloc(q, k, v, q_offsets, kv_offsets, B, H, D, variant, act, window,
                                              out, ctypes.byref(io)))


def jagged_attn_check(workspace, stream) -> int:
    return int(load().jagged_attn_check(workspace, stream))


def jagged_attn_bwd_workspace_size(B, H, D, variant, act, window, dtype, total_q, total_kv) -> int:
    return int(load().jagged_attn_bwd_workspace_size(B, H, D, variant, act, window, dtype, total_q, total_kv))


def jagged_attn_bwd(q, k, v, dout, q_offsets, kv_offsets, B, H, D, variant, act, window, dq, dk, dv,
                    io: JaIo) -> int:
    return int(load().jagged_attn_bwd(q, k, v, dout, q_offsets, kv_offsets, B, H, D, variant, act, window,
                                      dq, dk, dv, ctypes.byref(io)))


def jagged_attn_mx_quantize(x, dtype, rows, D, codes, scales, stream) -> int:
    return int(load().jagged_attn_mx_quantize(x, dtype, rows, D, codes, scales, stream))
