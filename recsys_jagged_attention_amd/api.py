"""torch-tensor front end of the C ABI (argument marshalling only).

``forward(q, k, v, q_offsets, kv_offsets, ...)`` checks dtypes/devices/shapes,
passes ``data_ptr()`` values and the current HIP stream to
``jagged_attn_fwd`` and returns ``out``.  PyTorch provides device memory and
streams; all attention arithmetic runs in libjagged_attn's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_IN_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": torch.uint8}


class Workspace:
    """A reusable device workspace (grown on demand, never shrunk)."""

    def __init__(self, device=None):
        self.device = torch.device(device if device is not None else "cuda")
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            q_offsets: torch.Tensor, kv_offsets: torch.Tensor,
            variant: str = "self", act: str = "softmax", window: int = 0,
            dtype: str = "bf16", scales=None, out: Optional[torch.Tensor] = None,
            workspace: Optional[Workspace] = None, rms_eps: float = 1e-6,
            stream: Optional[torch.cuda.Stream] = None, check: Optional[bool] = None,
            events=None, max_workgroups: int = 0, status: Optional[torch.Tensor] = None,
            softmax_stats: Optional[torch.Tensor] = None, fp8_pv: bool = False,
            lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Jagged GDPA forward.  q [Nq,H,D], k/v [Nk,H,D] on one GPU; offsets int32 [B+1].

    dtype "f32"/"bf16": q/k/v of that dtype; "mxfp8": uint8 e4m3 codes with
    ``scales=(q_scale, k_scale, v_scale)`` uint8 [rows,H,D/32].  Output is
    float32 for "f32", else bfloat16.

    The call is asynchronous on ``stream`` (default: the current stream).
    Offsets are validated on the device; the output is unspecified unless that
    status is JA_OK.  With ``check=True`` the call synchronises and raises on
    a device-side status (e.g. bad offsets).  ``check`` defaults to True when
    no ``workspace`` is passed (the status lives in the temporary workspace,
    which is released on return) and to False otherwise; a caller that keeps
    its workspace can check later with ``jagged_attn_check``, or pass
    ``status`` (a 1-element int32 CUDA tensor the device writes the status
    word into).  ``events=(start, stop)`` are raw hipEvent_t handles the
    attention kernel's dispatch writes its start and end into.
    ``max_workgroups`` caps the attention kernel's grid (0: every resident
    slot); results do not depend on it.  ``softmax_stats`` (3 int64 on the
    device, diagnostics) receives the tile-stream softmax's counts: tiles,
    first-tile max passes, later rescales.  ``fp8_pv`` asks for O += P V on
    the fp8 MFMA too (MXFP8 self-attention at D = 128, P and V requantised
    along the keys); this version does not provide it and raises
    JaggedAttnError with JA_EUNSUPPORTED.  ``lse`` (a contiguous float32
    [Nq, H] CUDA tensor, softmax only) receives each query row's natural
    log-sum-exp of its scaled scores, -inf for rows without keys (MXFP8 calls
    other than PMA and D = 128 self-attention with windows of at most four
    blocks raise JA_EUNSUPPORTED)."""
    if dtype not in _IN_DTYPES:
        raise ValueError(f"dtype must be one of {list(_IN_DTYPES)}")
    want = _IN_DTYPES[dtype]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != want or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D {want} CUDA tensor")
    for name, t in (("q_offsets", q_offsets), ("kv_offsets", kv_offsets)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{name} must be a contiguous 1-D int32 CUDA tensor")
    Nq, H, D = q.shape
    Nk = k.shape[0]
    if k.shape != (Nk, H, D) or v.shape != k.shape:
        raise ValueError("k and v must be [Nk, H, D] with q's H and D")
    B = q_offsets.numel() - 1
    if kv_offsets.numel() != B + 1:
        raise ValueError("q_offsets and kv_offsets must both have B+1 entries")
    out_dtype = torch.float32 if dtype == "f32" else torch.bfloat16
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if check is None:
        check = workspace is None
    v_id, a_id, d_id = _lib.VARIANTS[variant], _lib.ACTS[act], _lib.DTYPES[dtype]
    nbytes = _lib.jagged_attn_workspace_size(B, H, D, v_id, a_id, window, d_id, Nq, Nk)
    if nbytes == 0:
        # invalid or unsupported arguments: let the library report which
        nbytes = 256
    # Temporaries are allocated on the launch stream: the caching allocator
    # then reuses their blocks only for work ordered after these kernels.
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((Nq, H, D), dtype=out_dtype, device=q.device)
        ws = (workspace or Workspace(q.device)).get(nbytes)
    if out.shape != (Nq, H, D) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    if status is not None and (status.dtype != torch.int32 or not status.is_cuda or status.numel() < 1):
        raise ValueError("status must be an int32 CUDA tensor")
    io = _lib.JaIo()
    io.dtype = d_id
    if dtype == "mxfp8":
        if scales is None or len(scales) != 3:
            raise ValueError("mxfp8 needs scales=(q_scale, k_scale, v_scale)")
        for name, s, rows in zip("qkv", scales, (Nq, Nk, Nk)):
            if s.dtype != torch.uint8 or not s.is_cuda or s.shape != (rows, H, D // 32) or not s.is_contiguous():
                raise ValueError(f"{name}_scale must be a contiguous uint8 [rows,H,D/32] CUDA tensor")
        io.q_scale, io.k_scale, io.v_scale = (s.data_ptr() for s in scales)
    io.workspace = ws.data_ptr()
    io.workspace_bytes = ws.numel()
    io.stream = st.cuda_stream
    io.total_q = Nq
    io.total_kv = Nk
    io.rms_eps = rms_eps
    io.max_workgroups = max_workgroups
    io.fp8_pv = 1 if fp8_pv else 0
    if status is not None:
        io.status = status.data_ptr()
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or lse.shape != (Nq, H) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [Nq, H] CUDA tensor")
        io.lse = lse.data_ptr()
    if softmax_stats is not None:
        if softmax_stats.dtype != torch.int64 or not softmax_stats.is_cuda or softmax_stats.numel() < 3:
            raise ValueError("softmax_stats must be an int64 CUDA tensor of 3 elements")
        io.softmax_stats = softmax_stats.data_ptr()
    if events is not None:
        io.ev_start, io.ev_stop = events   # raw hipEvent_t handles (ints)
    rc = _lib.jagged_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_offsets.data_ptr(),
                              kv_offsets.data_ptr(), B, H, D, v_id, a_id, window, out.data_ptr(), io)
    if rc != _lib.JA_OK:
        raise _lib.JaggedAttnError(rc, "jagged_attn_fwd")
    if check:
        rc = _lib.jagged_attn_check(ws.data_ptr(), st.cuda_stream)
        if rc != _lib.JA_OK:
            raise _lib.JaggedAttnError(rc, "jagged_attn_check")
    return out


def mx_quantize(x: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
    """MX-encode x [..., D] (float32 or bfloat16 CUDA tensor, D a multiple of
    32) on the device: returns (codes uint8 [..., D], scales uint8 [..., D/32]),
    the MXFP8 input format of ``forward``."""
    if x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 or bfloat16 CUDA tensor")
    D = x.shape[-1]
    if D % 32 or D == 0:
        raise ValueError("the last dimension must be a positive multiple of 32")
    rows = x.numel() // D
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.stream(st):
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        scales = torch.empty(tuple(x.shape[:-1]) + (D // 32,), dtype=torch.uint8, device=x.device)
    dtype = _lib.JA_F32 if x.dtype == torch.float32 else _lib.JA_BF16
    status = _lib.jagged_attn_mx_quantize(x.data_ptr(), dtype, rows, D, codes.data_ptr(), scales.data_ptr(),
                                          st.cuda_stream)
    if status != _lib.JA_OK:
        raise _lib.JaggedAttnError(status, "jagged_attn_mx_quantize")
    return codes, scales


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
             q_offsets: torch.Tensor, kv_offsets: torch.Tensor,
             variant: str = "self", act: str = "softmax", window: int = 0, dtype: str = "bf16",
             workspace: Optional[Workspace] = None, rms_eps: float = 1e-6,
             stream: Optional[torch.cuda.Stream] = None, check: Optional[bool] = None, events=None,
             out=None, lse: Optional[torch.Tensor] = None, fwd_out: Optional[torch.Tensor] = None):
    """Gradients of the forward (act "softmax" or "gelu_tanh"): returns float32
    (dq, dk, dv) shaped like q, k, v.  q/k/v/dout are "f32" or "bf16" tensors
    laid out as for ``forward``; ``stream`` and ``check`` as for ``forward``.
    ``out=(dq, dk, dv)`` gives the (contiguous float32) outputs; every element
    of them is written.  Softmax only: ``lse`` (the forward's float32 [Nq, H]
    log-sum-exp) and ``fwd_out`` (its output) together let the backward skip
    recomputing the row statistics."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("backward takes f32 or bf16 inputs")
    want = _IN_DTYPES[dtype]
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if t.dtype != want or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D {want} CUDA tensor")
    Nq, H, D = q.shape
    Nk = k.shape[0]
    if dout.shape != q.shape or k.shape != (Nk, H, D) or v.shape != k.shape:
        raise ValueError("dout must match q, and k, v must be [Nk, H, D]")
    B = q_offsets.numel() - 1
    v_id, a_id, d_id = _lib.VARIANTS[variant], _lib.ACTS[act], _lib.DTYPES[dtype]
    nbytes = _lib.jagged_attn_bwd_workspace_size(B, H, D, v_id, a_id, window, d_id, Nq, Nk) or 256
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if check is None:
        check = workspace is None
    with torch.cuda.stream(st):  # (temporaries on the launch stream, as in forward)
        ws = (workspace or Workspace(q.device)).get(nbytes)
        if out is None:
            dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
            dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
            dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
        else:
            dq, dk, dv = out
            for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
                if t.dtype != torch.float32 or t.shape != ref.shape or not t.is_contiguous() or not t.is_cuda:
                    raise ValueError(f"{name} must be a contiguous float32 CUDA tensor shaped like its input")
    io = _lib.JaIo()
    io.dtype = d_id
    io.workspace = ws.data_ptr()
    io.workspace_bytes = ws.numel()
    io.stream = st.cuda_stream
    io.total_q = Nq
    io.total_kv = Nk
    io.rms_eps = rms_eps
    if events is not None:
        io.ev_start, io.ev_stop = events
    if lse is not None or fwd_out is not None:
        if lse is None or fwd_out is None:
            raise ValueError("lse and fwd_out go together")
        if lse.dtype != torch.float32 or not lse.is_cuda or lse.shape != (Nq, H) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [Nq, H] CUDA tensor")
        if fwd_out.dtype != want or not fwd_out.is_cuda or fwd_out.shape != q.shape or not fwd_out.is_contiguous():
            raise ValueError(f"fwd_out must be a contiguous {want} CUDA tensor shaped like q")
        io.lse = lse.data_ptr()
        io.fwd_out = fwd_out.data_ptr()
    rc = _lib.jagged_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), q_offsets.data_ptr(),
                              kv_offsets.data_ptr(), B, H, D, v_id, a_id, window, dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), io)
    if rc != _lib.JA_OK:
        raise _lib.JaggedAttnError(rc, "jagged_attn_bwd")
    if check:
        rc = _lib.jagged_attn_check(ws.data_ptr(), st.cuda_stream)
        if rc != _lib.JA_OK:
            raise _lib.JaggedAttnError(rc, "jagged_attn_check")
    return dq, dk, dv
