"""ctypes binding of libfa_std.so: the standard (materializing) attention
forward that FlashAttention is compared against. Argument marshalling only:
the GEMMs run in rocBLAS and the softmax in this package's HIP kernel, behind
the C ABI in include/fa_std.h. When libfa_std.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

from ._binding import FA_OK, FAError, _ptr, _stream

_PKG = os.path.dirname(os.path.abspath(__file__))
STD_LIB_PATH = os.path.join(_PKG, "libfa_std.so")
STD_EXPORTS = ("fa_std_workspace_bytes", "fa_std_fwd", "fa_std_scores", "fa_std_softmax",
               "fa_std_output")
_lib = None


def load_std():
    """Load libfa_std.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(STD_LIB_PATH):
        raise RuntimeError(f"{STD_LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(STD_LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_std_workspace_bytes.argtypes = [i, i, i]
    lib.fa_std_workspace_bytes.restype = sz
    lib.fa_std_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
    lib.fa_std_scores.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp]
    lib.fa_std_softmax.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.fa_std_output.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    for name in STD_EXPORTS[1:]:
        getattr(lib, name).restype = i
    _lib = lib
    return lib


def fa_std_workspace_bytes(B, H, N) -> int:
    return int(load_std().fa_std_workspace_bytes(int(B), int(H), int(N)))


def fa_std_fwd(q, k, v, o, lse, ws, ws_bytes, B, H, N, d, scale, causal, stream=None) -> int:
    return int(load_std().fa_std_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws),
                                     int(ws_bytes), int(B), int(H), int(N), int(d), float(scale),
                                     int(bool(causal)), _stream(stream, (q, k, v, o, lse))))


def fa_std_scores(q, k, s, gemm_ws, B, H, N, d, scale, stream=None) -> int:
    return int(load_std().fa_std_scores(_ptr(q), _ptr(k), _ptr(s), _ptr(gemm_ws), int(B), int(H),
                                        int(N), int(d), float(scale), _stream(stream, (q, k, s))))


def fa_std_softmax(s, p, lse, B, H, N, causal, stream=None) -> int:
    return int(load_std().fa_std_softmax(_ptr(s), _ptr(p), _ptr(lse), int(B), int(H), int(N),
                                         int(bool(causal)), _stream(stream, (s, p, lse))))


def fa_std_output(p, v, o, gemm_ws, B, H, N, d, stream=None) -> int:
    return int(load_std().fa_std_output(_ptr(p), _ptr(v), _ptr(o), _ptr(gemm_ws), int(B), int(H),
                                        int(N), int(d), _stream(stream, (p, v, o))))


def standard_attention(q, k, v, causal=False, scale=None, ws=None, stream=None):
    """Allocate o, lse (and the workspace, unless given as a uint8 CUDA tensor)
    with torch and run the three materializing steps. q, k, v: contiguous bf16
    [B, H, N, d] CUDA tensors. Returns (o, lse); raises FAError on a status."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if any(t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must be contiguous bf16 GPU tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_std_workspace_bytes(B, H, N)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_std_fwd(q, k, v, o, lse, ws, ws.numel(), B, H, N, d, scale, causal, stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse
