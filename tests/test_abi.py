"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (these paths return before any HIP call, so no GPU is
needed)."""
import ctypes
import os
import re

import pytest

from recsys_jagged_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "jagged_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jagged_attn_\w+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert _lib.jagged_attn_version() == 101


def test_strerror_covers_all_codes():
    for code in (0, -1, -2, -3, -4, -5):
        assert _lib.strerror(code) != "unknown status"
    assert _lib.strerror(-99) == "unknown status"


def ws(*a):
    return _lib.jagged_attn_workspace_size(*a)


def test_workspace_size_rejects_bad_arguments():
    ok = ws(4, 2, 32, _lib.JA_SELF, _lib.JA_SOFTMAX, 0, _lib.JA_F32, 100, 100)
    assert ok > 0
    assert ws(0, 2, 32, 0, 0, 0, 0, 100, 100) == 0                 # B < 1
    assert ws(4, 2, 48, 0, 0, 0, 0, 100, 100) == 0                 # unsupported D
    assert ws(4, 2, 32, 0, 0, 100, 0, 100, 100) == 0               # window not a multiple of 64
    assert ws(4, 2, 32, 1, 0, 64, 0, 100, 100) == 0                # window on cross
    assert ws(4, 2, 32, 0, 1, 64, 0, 100, 100) == 0                # windowed GELU
    assert ws(4, 2, 32, 0, 0, 0, 0, 100, 99) == 0                  # self with different totals
    assert ws(4, 2, 32, 4, 0, 0, 0, 100, 100) == 0                 # bad variant
    sl = _lib.JA_SLIDING
    assert ws(4, 2, 32, sl, 0, 100, _lib.JA_BF16, 100, 100) > 0     # sliding window, any W >= 1
    assert ws(4, 2, 32, sl, 0, 1, _lib.JA_F32, 100, 100) > 0
    assert ws(4, 2, 32, sl, 0, 0, _lib.JA_BF16, 100, 100) == 0      # sliding needs W >= 1
    assert ws(4, 2, 32, sl, 1, 64, _lib.JA_BF16, 100, 100) == 0     # sliding GELU
    assert ws(4, 2, 32, sl, 0, 64, _lib.JA_MXFP8_E4M3, 100, 100) == 0  # sliding MXFP8
    assert ws(4, 2, 32, sl, 0, 64, _lib.JA_BF16, 100, 99) == 0      # sliding needs self offsets
    assert ws(4, 2, 32, 0, 0, 0, 7, 100, 100) == 0                 # bad dtype


def test_workspace_grows_with_key_split_partials():
    small = ws(512, 8, 64, _lib.JA_PMA, _lib.JA_SOFTMAX, 0, _lib.JA_BF16, 512 * 32, 1000)
    big = ws(512, 8, 64, _lib.JA_PMA, _lib.JA_SOFTMAX, 0, _lib.JA_BF16, 512 * 32, 2_000_000)
    assert big > small > 0


def call(B=2, H=1, D=32, variant=0, act=0, window=0, dtype=0, tq=10, tk=10, ws_bytes=1 << 20,
         ptr=4096, io=True, scales=False, fp8_pv=0, lse=None):
    j = _lib.JaIo()
    j.dtype = dtype
    j.fp8_pv = fp8_pv
    j.lse = lse
    j.total_q, j.total_kv = tq, tk
    j.workspace = 1 << 20
    j.workspace_bytes = ws_bytes
    if scales:
        j.q_scale = j.k_scale = j.v_scale = 4096
    lib = _lib.load()
    return lib.jagged_attn_fwd(ptr, ptr, ptr, ptr, ptr, B, H, D, variant, act, window, ptr,
                               ctypes.byref(j) if io else None)


def test_fwd_host_validation():
    assert call(io=False) == _lib.JA_EINVAL
    assert call(B=0) == _lib.JA_EINVAL
    assert call(D=96) == _lib.JA_EUNSUPPORTED
    assert call(window=32) == _lib.JA_EUNSUPPORTED
    assert call(variant=_lib.JA_CROSS, window=64) == _lib.JA_EINVAL
    assert call(act=_lib.JA_GELU_TANH, window=64) == _lib.JA_EUNSUPPORTED
    assert call(tq=10, tk=11) == _lib.JA_EINVAL
    assert call(variant=_lib.JA_SLIDING) == _lib.JA_EINVAL            # window 0
    assert call(variant=_lib.JA_SLIDING, window=5, act=_lib.JA_GELU_TANH) == _lib.JA_EUNSUPPORTED
    assert call(ptr=0) == _lib.JA_EINVAL
    assert call(dtype=_lib.JA_MXFP8_E4M3) == _lib.JA_EINVAL          # scales missing
    assert call(ws_bytes=16) == _lib.JA_EWORKSPACE
    assert call(ptr=4100) == _lib.JA_EINVAL                            # misaligned
    assert call(dtype=_lib.JA_MXFP8_E4M3, scales=True, ws_bytes=16) == _lib.JA_EWORKSPACE
    assert call(fp8_pv=1) == _lib.JA_EUNSUPPORTED                      # fp8 P V: switched off
    assert call(fp8_pv=1, dtype=_lib.JA_MXFP8_E4M3, scales=True, D=128) == _lib.JA_EUNSUPPORTED
    # the log-sum-exp output: softmax only, 4-byte aligned
    assert call(lse=4096, variant=_lib.JA_CROSS, act=_lib.JA_GELU_TANH, tk=7) == _lib.JA_EINVAL
    assert call(lse=4096, variant=_lib.JA_PMA, act=_lib.JA_GELU_TANH, dtype=_lib.JA_BF16, tk=70) == _lib.JA_EINVAL
    assert call(lse=4098) == _lib.JA_EINVAL
    assert call(lse=4098, variant=_lib.JA_PMA, dtype=_lib.JA_BF16, tk=70) == _lib.JA_EINVAL
    assert call(lse=4096, dtype=_lib.JA_MXFP8_E4M3, scales=True, D=64) == _lib.JA_EUNSUPPORTED
    assert call(lse=4096, dtype=_lib.JA_MXFP8_E4M3, scales=True, D=128, window=320) == _lib.JA_EUNSUPPORTED


def test_bwd_host_validation():
    lib = _lib.load()
    ok = _lib.jagged_attn_bwd_workspace_size(4, 2, 32, _lib.JA_SELF, _lib.JA_SOFTMAX, 0, _lib.JA_BF16, 100, 100)
    assert ok > 0
    soft = _lib.jagged_attn_bwd_workspace_size(4, 2, 32, _lib.JA_CROSS, _lib.JA_SOFTMAX, 0, _lib.JA_BF16, 100, 50)
    gelu = _lib.jagged_attn_bwd_workspace_size(4, 2, 32, _lib.JA_CROSS, _lib.JA_GELU_TANH, 0, _lib.JA_BF16, 100, 50)
    assert gelu >= soft + 4 * 2 * (100 + 50)  # + the RMS factors of every query and key row
    assert _lib.jagged_attn_bwd_workspace_size(4, 2, 32, _lib.JA_CROSS, _lib.JA_GELU_POLY, 0, _lib.JA_BF16,
                                               100, 50) == 0
    assert _lib.jagged_attn_bwd_workspace_size(4, 2, 32, _lib.JA_SELF, _lib.JA_GELU_TANH, 64, _lib.JA_BF16,
                                               100, 100) == 0
    assert _lib.jagged_attn_bwd_workspace_size(4, 2, 32, _lib.JA_SELF, _lib.JA_SOFTMAX, 0, _lib.JA_MXFP8_E4M3,
                                               100, 100) == 0

    def call(act=_lib.JA_SOFTMAX, dtype=_lib.JA_BF16, ptr=4096, ws_bytes=1 << 24, lse=None, fwd_out=None):
        j = _lib.JaIo()
        j.dtype = dtype
        j.lse, j.fwd_out = lse, fwd_out
        j.total_q = j.total_kv = 10
        j.workspace = 1 << 20
        j.workspace_bytes = ws_bytes
        return lib.jagged_attn_bwd(ptr, ptr, ptr, ptr, ptr, ptr, 2, 1, 32, _lib.JA_SELF, act, 0,
                                   ptr, ptr, ptr, ctypes.byref(j))

    assert call(act=_lib.JA_GELU_POLY) == _lib.JA_EUNSUPPORTED
    assert call(dtype=_lib.JA_MXFP8_E4M3) == _lib.JA_EUNSUPPORTED
    assert call(ptr=0) == _lib.JA_EINVAL
    assert call(ptr=4100) == _lib.JA_EINVAL
    assert call(ws_bytes=16) == _lib.JA_EWORKSPACE
    # the forward's log-sum-exp and output: both or neither, softmax, aligned
    assert call(lse=4096) == _lib.JA_EINVAL
    assert call(fwd_out=4096) == _lib.JA_EINVAL
    assert call(act=_lib.JA_GELU_TANH, lse=4096, fwd_out=4096) == _lib.JA_EINVAL
    assert call(lse=4098, fwd_out=4096) == _lib.JA_EINVAL
    assert call(lse=4096, fwd_out=4104) == _lib.JA_EINVAL


def test_mx_quantize_host_validation():
    q = lambda x=4096, dt=_lib.JA_BF16, rows=4, D=64, c=4096, s=4096: _lib.jagged_attn_mx_quantize(
        x, dt, rows, D, c, s, None)
    assert q(x=0) == _lib.JA_EINVAL
    assert q(c=0) == _lib.JA_EINVAL
    assert q(s=0) == _lib.JA_EINVAL
    assert q(dt=_lib.JA_MXFP8_E4M3) == _lib.JA_EINVAL
    assert q(D=48) == _lib.JA_EINVAL
    assert q(D=0) == _lib.JA_EINVAL
    assert q(rows=-1) == _lib.JA_EINVAL
    assert q(x=4100) == _lib.JA_EINVAL
    assert q(rows=0, x=0, c=0, s=0) == _lib.JA_OK  # no rows: nothing to do (empty tensors)
    assert q(rows=1 << 40) == _lib.JA_EINVAL


def test_check_rejects_null_workspace():
    assert _lib.jagged_attn_check(None, None) == _lib.JA_EINVAL


def test_noalloc_host_validation():
    """The no-allocation forward rejects a caller workspace and batches whose
    workspace exceeds its 64 MiB scratch, before any HIP call."""
    lib = _lib.load()
    j = _lib.JaIo()
    j.dtype = _lib.JA_BF16
    j.total_q = j.total_kv = 1 << 24
    big = lib.jagged_attn_fwd_noalloc(4096, 4096, 4096, 4096, 4096, 4096, 64, 64, _lib.JA_PMA, _lib.JA_SOFTMAX, 0,
                                      4096, ctypes.byref(j))
    assert big == _lib.JA_EWORKSPACE
    j.total_q = j.total_kv = 10
    j.workspace, j.workspace_bytes = 1 << 20, 1 << 20
    assert lib.jagged_attn_fwd_noalloc(4096, 4096, 4096, 4096, 4096, 2, 1, 32, 0, 0, 0, 4096,
                                       ctypes.byref(j)) == _lib.JA_EINVAL
    j.workspace, j.workspace_bytes = None, 0
    assert lib.jagged_attn_fwd_noalloc(4096, 4096, 4096, 4096, 4096, 0, 1, 32, 0, 0, 0, 4096,
                                       ctypes.byref(j)) == _lib.JA_EINVAL       # B < 1
    assert lib.jagged_attn_fwd_noalloc(4096, 4096, 4096, 4096, 4096, 2, 1, 48, 0, 0, 0, 4096,
                                       ctypes.byref(j)) == _lib.JA_EUNSUPPORTED  # D
    assert lib.jagged_attn_fwd_noalloc(4096, 4096, 4096, 4096, 4096, 2, 1, 32, 0, 0, 0, 4096,
                                       None) == _lib.JA_EINVAL


def test_ja_io_layout_matches_the_header(tmp_path):
    """The ctypes mirror of ja_io (_lib.JaIo) has the header's field order,
    offsets and size: a C program built from include/jagged_attn.h prints
    offsetof of every field and sizeof(ja_io)."""
    import subprocess
    names = [f[0] for f in _lib.JaIo._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{n} %zu\\n", offsetof(ja_io, {n}));' for n in names)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "jagged_attn.h"\n'
                   f'int main(void) {{\n{body}\n  printf("sizeof %zu\\n", sizeof(ja_io));\n  return 0;\n}}\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = dict(line.split() for line in out if line.strip())
    for n in names:
        assert int(got[n]) == getattr(_lib.JaIo, n).offset, n
    assert int(got["sizeof"]) == ctypes.sizeof(_lib.JaIo)
