"""ctypes binding of libfa.so: argument marshalling only.

Every step of the forward pass runs in the HIP kernels behind the C ABI in
include/fa.h. This module passes device pointers, sizes and the stream
handle through, and there is no other implementation to fall back to: when
libfa.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
_lib = None

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_UNSUPPORTED_HEAD_DIM",
    4: "FA_ERR_BAD_SCALE", 5: "FA_ERR_MISALIGNED", 6: "FA_ERR_ALIASING", 7: "FA_ERR_LAUNCH",
    8: "FA_ERR_TOO_LARGE", 9: "FA_ERR_WORKSPACE", 10: "FA_ERR_LIBRARY",
    11: "FA_ERR_SCRATCH_LIMIT",
}
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_bwd", "fa_bwd_noalloc",
           "fa_bwd_noalloc_max_rows", "fa_decode_paged", "fa_decode_workspace_bytes",
           "fa_status_string", "fa_tile_rows", "fa_tile_cols", "fa_fwd_grid")


class FAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {fa_status_string(status)}")


def load():
    """Load libfa.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("fa_fwd", "fa_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        fn.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, f, f, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_max_rows.argtypes = []
    lib.fa_bwd_noalloc_max_rows.restype = ctypes.c_longlong
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_decode_paged.argtypes = [vp] * 8 + [ctypes.c_size_t] + [i] * 7 + [f, vp]
    lib.fa_decode_paged.restype = i
    lib.fa_bwd.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_tile_rows.restype = i
    lib.fa_tile_cols.restype = i
    lib.fa_fwd_grid.argtypes = [i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.fa_fwd_grid.restype = ctypes.c_longlong
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(stream, tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if hasattr(t, "is_cuda") and t.is_cuda:
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None) -> int:
    """C fa_fwd: bf16 q, k, v, o [B,H,N,d] and fp32 lse [B,H,N] device tensors
    (or raw device addresses). stream: a torch stream, a raw hipStream_t int,
    or None for the current torch stream of the tensors' device. Returns the
    fa_status code."""
    return int(load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                             int(N), int(d), float(scale), int(bool(causal)),
                             _stream(stream, (q, k, v, o, lse))))


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None) -> int:
    """C fa_fwd_f32: as fa_fwd with fp32 q, k, v and o."""
    return int(load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                                 int(H), int(N), int(d), float(scale), int(bool(causal)),
                                 _stream(stream, (q, k, v, o, lse))))


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, q_scale, k_scale, v_scale, causal,
               stream=None) -> int:
    """C fa_fwd_fp8: uint8 E4M3 codes q, k, v [B,H,N,d] with per-tensor scales,
    bf16 o, fp32 lse. Returns the fa_status code."""
    return int(load().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                 int(N), int(d), float(scale), float(q_scale), float(k_scale),
                                 float(v_scale), int(bool(causal)),
                                 _stream(stream, (q, k, v, o, lse))))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, d, scale, causal, stream=None) -> int:
    """C fa_bwd: bf16 q, k, v, o, dout, dq, dk, dv [B,H,N,d], fp32 lse and workspace
    ws [B,H,N] device tensors (or raw device addresses). Returns the fa_status code."""
    return int(load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), int(B), int(H), int(N),
                             int(d), float(scale), int(bool(causal)),
                             _stream(stream, (q, k, v, o, lse, dout))))


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                   stream=None) -> int:
    """C fa_bwd_noalloc: fa_bwd without the workspace argument (the library's
    static device scratch holds D; B*H*N <= fa_bwd_noalloc_max_rows()).
    Returns the fa_status code."""
    return int(load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                     _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H), int(N),
                                     int(d), float(scale), int(bool(causal)),
                                     _stream(stream, (q, k, v, o, lse, dout))))


def fa_bwd_noalloc_max_rows() -> int:
    return int(load().fa_bwd_noalloc_max_rows())


def fa_decode_workspace_bytes(B, H, d, page_size, max_pages) -> int:
    return int(load().fa_decode_workspace_bytes(int(B), int(H), int(d), int(page_size),
                                                int(max_pages)))


def fa_decode_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse, ws, ws_bytes, B, H, H_kv,
                    d, num_pages, page_size, max_pages, scale, stream=None) -> int:
    """C fa_decode_paged (see include/fa.h). Returns the fa_status code."""
    return int(load().fa_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), _ptr(o),
        _ptr(lse), _ptr(ws), int(ws_bytes), int(B), int(H), int(H_kv), int(d), int(num_pages),
        int(page_size), int(max_pages), float(scale),
        _stream(stream, (q, k_cache, v_cache, o, lse))))


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_tile_rows() -> int:
    return int(load().fa_tile_rows())


def fa_tile_cols() -> int:
    return int(load().fa_tile_cols())


def fa_fwd_grid(B: int, H: int, N: int, causal: bool):
    """fa_fwd's launch shape: (workgroups, query rows per block, paired).
    Raises FAError for invalid sizes."""
    rows, paired = ctypes.c_int(0), ctypes.c_int(0)
    g = int(load().fa_fwd_grid(int(B), int(H), int(N), int(bool(causal)),
                               ctypes.byref(rows), ctypes.byref(paired)))
    if g < 0:
        raise FAError(-g)
    return g, rows.value, bool(paired.value)


def _need(t, name, shape, dtype, device):
    """Raise ValueError unless tensor t has exactly this shape, dtype and
    device and is contiguous: the C ABI receives raw pointers only and cannot
    see the extent of a buffer, so a wrong one would be written or read past
    its end."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_outputs(q, out, lse):
    """The forward's o must match q (shape, dtype, device, contiguous) and lse
    must be contiguous fp32 [B, H, N] on q's device; ValueError otherwise."""
    import torch
    B, H, N, _ = q.shape
    _need(out, "out", q.shape, q.dtype, q.device)
    _need(lse, "lse", (B, H, N), torch.float32, q.device)


def attention(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """Allocate o and lse with torch (when not given) and run the forward pass.

    q, k, v: contiguous [B, H, N, d] CUDA tensors, all bf16 or all fp32.
    scale defaults to 1/sqrt(d). Returns (o, lse); raises FAError on a status.
    """
    import torch
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bf16 or all fp32")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if not (k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    check_outputs(q, out, lse)
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    st = fn(q, k, v, out, lse, B, H, N, d, scale, causal, stream)
    if st != FA_OK:
        raise FAError(st)
    return out, lse


def attention_backward(q, k, v, o, lse, dout, causal=False, scale=None, stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run the backward pass.

    q, k, v, o, dout: contiguous bf16 [B, H, N, d] CUDA tensors (o and lse from
    the forward pass with the same q, k, v, causal and scale). Returns
    (dq, dk, dv); raises FAError on a status.
    """
    import torch
    ts = (q, k, v, o, dout)
    if any(t.shape != q.shape for t in ts) or q.dim() != 4:
        raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape")
    if any(t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() for t in ts):
        raise ValueError("q, k, v, o, dout must be contiguous bf16 GPU tensors")
    B, H, N, d = q.shape
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    if any(t.device != q.device for t in ts):
        raise ValueError("q, k, v, o, dout must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, d, scale, causal, stream)
    if st != FA_OK:
        raise FAError(st)
    return dq, dk, dv


def attention_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal=False, scale=None, stream=None):
    """Allocate o (bf16) and lse with torch and run the FP8 forward pass.

    q8, k8, v8: contiguous uint8 [B, H, N, 128] CUDA tensors of E4M3 codes;
    *_scale: the per-tensor scales. Returns (o, lse); raises FAError on a status.
    """
    import torch
    ts = (q8, k8, v8)
    if q8.dim() != 4 or any(t.shape != q8.shape for t in ts):
        raise ValueError("q8, k8, v8 must share one [B, H, N, d] shape")
    if any(t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() for t in ts):
        raise ValueError("q8, k8, v8 must be contiguous uint8 GPU tensors")
    if any(t.device != q8.device for t in ts):
        raise ValueError("q8, k8, v8 must be on one device")
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    st = fa_fwd_fp8(q8, k8, v8, o, lse, B, H, N, d, scale, q_scale, k_scale, v_scale, causal,
                    stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse


def decode_paged(q, k_cache, v_cache, page_table, seq_lens, scale=None, ws=None, stream=None):
    """Allocate o, lse (and the workspace unless given) with torch and run one
    decode step over the paged KV cache. q: bf16 [B, H, d]; caches: bf16
    [num_pages, H_kv, page_size, d]; page_table: int32 [B, max_pages];
    seq_lens: int32 [B]; all contiguous CUDA tensors. Returns (o, lse)."""
    import torch
    B, H, d = q.shape
    num_pages, H_kv, page_size, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or page_table.dim() != 2 or \
            page_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("inconsistent decode shapes")
    for t, dt in ((q, torch.bfloat16), (k_cache, torch.bfloat16), (v_cache, torch.bfloat16),
                  (page_table, torch.int32), (seq_lens, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("decode inputs must be contiguous CUDA tensors of the stated dtypes")
        if t.device != q.device:
            raise ValueError("decode inputs must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    max_pages = page_table.shape[1]
    need = fa_decode_workspace_bytes(B, H, d, page_size, max_pages)
    if ws is None:
        ws = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=q.device)
    elif not isinstance(ws, torch.Tensor) or ws.device != q.device or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous tensor on q's device")
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = fa_decode_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse, ws,
                         ws.numel() * ws.element_size(), B, H, H_kv, d, num_pages, page_size,
                         max_pages, scale, stream)
    if st != FA_OK:
        raise FAError(st)
    return o, lse
