"""Attention oracle, forward and backward (fp64, CPU): TEST INFRASTRUCTURE, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It loads ``liboracle.so``, built from
``oracle.c`` with gcc (OpenMP, no fast-math); it shares no code with the HIP
path and the HIP path never imports it.

Every function takes and returns float64 numpy arrays. Inputs handed to the
GPU in bf16 or fp32 are upcast exactly to float64 before they get here.

Parity status of each function (what pins it, in ``tests/test_oracle_pins.py``):

* ``softmax_row``: the worked examples printed on the pages, closed forms.
* ``online_row_two_scale`` / ``online_row_single_max``: the worked examples
  (final outputs and block states), brute force against ``softmax_row`` for
  every block size on tiny rows.
* ``attention_fwd`` / ``attention_rows``: closed forms (N = 1, Q = 0, causal
  row 0), invariances (key/value permutation, value scaling, per-row score
  shift), rows of P summing to 1, and torch's CPU float64 scaled dot-product
  attention and logsumexp on random inputs.
* ``attention_bwd_sampled``: the full ``attention_bwd`` on small inputs and
  torch's CPU float64 autograd (it evaluates D as dO . O instead of
  sum_j P_ij dP_ij, and P from lse instead of a stored row).
* ``decode_e4m3``: torch's float8_e4m3fn -> float64 conversion of all 254
  non-NaN codes, and the format's closed forms (1.0 = 0x38, 448 = 0x7E, the
  smallest subnormal 2^-9 = 0x01, signs).
* ``attention_fwd_fp8``: ``decode_e4m3`` followed by ``attention_fwd`` (no
  arithmetic of its own).
* ``decode_paged``: ``attention_rows`` on the same rows stored contiguously
  (the last row of each sequence attending to all earlier ones), torch's
  float64 SDPA on the gathered rows, invariance under a permutation of the
  physical pages (with the table permuted alike), and query-head groups
  sharing one KV head equal to repeating that head.
* ``attention_bwd``: central finite differences of the forward oracle's loss
  sum(dO * O) on tiny inputs, torch's CPU float64 autograd of
  scaled_dot_product_attention, the identities D = rowsum(dO * O) and
  sum over keys of dK = 0, and the closed forms for N = 1 and scale 0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_long)


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_softmax_row.argtypes = [_dp, _dp, ctypes.c_long, ctypes.c_long, _dp, _dp]
    for name in ("oracle_online_row_two_scale", "oracle_online_row_single_max"):
        getattr(lib, name).argtypes = [_dp, _dp, ctypes.c_long, ctypes.c_long,
                                       ctypes.c_long, _dp, _dp, _dp]
    lib.oracle_attention_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp,
                                         ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                         ctypes.c_long, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_rows.argtypes = [_dp, _dp, _dp, ctypes.c_long, ctypes.c_long,
                                          ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                          ctypes.c_int, _lp, ctypes.c_long, _dp, _dp]
    lib.oracle_attention_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                         ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                         ctypes.c_long, ctypes.c_double, ctypes.c_int]
    lib.oracle_attention_bwd_sampled.argtypes = [
        _dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
        ctypes.c_double, ctypes.c_int, _lp, ctypes.c_long, _lp, ctypes.c_long, _lp,
        ctypes.c_long, _dp, _dp, _dp]
    _ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_decode_paged.argtypes = [_dp, _dp, _dp, _ip, _ip] + [ctypes.c_long] * 7 + [
        ctypes.c_double, _dp, _dp]
    lib.oracle_decode_paged.restype = ctypes.c_int
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_double, _dp]
    lib.oracle_decode_e4m3.restype = ctypes.c_int
    for name in ("oracle_softmax_row", "oracle_online_row_two_scale",
                 "oracle_online_row_single_max", "oracle_attention_fwd",
                 "oracle_attention_rows", "oracle_attention_bwd",
                 "oracle_attention_bwd_sampled"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor: exact upcast on the CPU
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def _row_args(s, v):
    s = _f64(s).reshape(-1)
    v = _f64(v)
    if v.ndim == 1:
        v = v.reshape(-1, 1)
    if v.shape[0] != s.shape[0]:
        raise ValueError("scores and values disagree in length")
    return s, np.ascontiguousarray(v)


def softmax_row(s, v):
    """Direct softmax-weighted sum of one row; returns (out[dv], lse)."""
    s, v = _row_args(s, v)
    out = np.empty(v.shape[1])
    lse = ctypes.c_double()
    _check(_load().oracle_softmax_row(_ptr(s), _ptr(v), s.size, v.shape[1], _ptr(out),
                                      ctypes.byref(lse)), "softmax_row")
    return out, lse.value


def _online(name, s, v, block):
    s, v = _row_args(s, v)
    out = np.empty(v.shape[1])
    m = ctypes.c_double()
    l_ = ctypes.c_double()
    _check(getattr(_load(), name)(_ptr(s), _ptr(v), s.size, v.shape[1], int(block),
                                  _ptr(out), ctypes.byref(m), ctypes.byref(l_)), name)
    return out, m.value, l_.value


def online_row_two_scale(s, v, block):
    """Block-local online softmax (two correction factors); (out, m, l)."""
    return _online("oracle_online_row_two_scale", s, v, block)


def online_row_single_max(s, v, block):
    """Single running-max online softmax; (out, m, l)."""
    return _online("oracle_online_row_single_max", s, v, block)


def attention_fwd(q, k, v, scale, causal, return_p=False):
    """Standard attention on [B, H, N, d] inputs, S and P materialized.

    Returns (o [B,H,N,d], lse [B,H,N]) or, with return_p, also P [B,H,N,N].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape) or q.ndim != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    p = np.empty((B, H, N, N)) if return_p else None
    _check(_load().oracle_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        _ptr(p) if p is not None else None,
                                        B, H, N, d, float(scale), int(bool(causal))),
           "attention_fwd")
    return (o, lse, p) if return_p else (o, lse)


def attention_rows(q, k, v, scale, causal, rows):
    """Standard attention for selected rows.

    rows: int array [B*H, R] (or [R], the same rows for every head).
    Returns (o_rows [B*H, R, d], lse_rows [B*H, R]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape) or q.ndim != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    r = np.asarray(rows.numpy() if hasattr(rows, "numpy") else rows, dtype=np.int64)
    if r.ndim == 1:
        r = np.broadcast_to(r, (B * H, r.size))
    r = np.ascontiguousarray(r, dtype=np.int64)
    if r.shape[0] != B * H:
        raise ValueError("rows must have one row list per head")
    R = r.shape[1]
    o = np.empty((B * H, R, d))
    lse = np.empty((B * H, R))
    _check(_load().oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d,
                                         float(scale), int(bool(causal)),
                                         r.ctypes.data_as(_lp), R, _ptr(o), _ptr(lse)),
           "attention_rows")
    return o, lse


def attention_bwd(q, k, v, dout, scale, causal, return_delta=False):
    """Backward pass of standard attention on [B, H, N, d] inputs.

    Returns (dq, dk, dv), each [B, H, N, d], and with return_delta also
    D [B, H, N] (D_i = sum_j P_ij dP_ij).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape) or q.ndim != 4:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    delta = np.empty((B, H, N))
    _check(_load().oracle_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(delta), B, H, N, d,
                                        float(scale), int(bool(causal))),
           "attention_bwd")
    return (dq, dk, dv, delta) if return_delta else (dq, dk, dv)


def _idx(a, rows: int, what: str) -> np.ndarray:
    a = np.asarray(a.numpy() if hasattr(a, "numpy") else a, dtype=np.int64)
    if a.ndim == 1:
        a = np.broadcast_to(a, (rows, a.size))
    if a.ndim != 2 or a.shape[0] != rows:
        raise ValueError(f"{what} must have one index list per sampled head")
    return np.ascontiguousarray(a, dtype=np.int64)


def attention_bwd_sampled(q, k, v, dout, scale, causal, heads, qrows, krows):
    """Backward pass on selected heads (flat b*H + h), query rows and key rows.

    heads: [Hs]; qrows: [Hs, R] (or [R]); krows: [Hs, C] (or [C]).
    Returns (dq_rows [Hs,R,d], dk_rows [Hs,C,d], dv_rows [Hs,C,d]).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape) or q.ndim != 4:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int64).reshape(-1))
    qr = _idx(qrows, hs.size, "qrows")
    kr = _idx(krows, hs.size, "krows")
    R, C = qr.shape[1], kr.shape[1]
    dq = np.empty((hs.size, R, d))
    dk = np.empty((hs.size, C, d))
    dv = np.empty((hs.size, C, d))
    _check(_load().oracle_attention_bwd_sampled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, float(scale), int(bool(causal)),
        hs.ctypes.data_as(_lp), hs.size, qr.ctypes.data_as(_lp), R, kr.ctypes.data_as(_lp), C,
        _ptr(dq), _ptr(dk), _ptr(dv)), "attention_bwd_sampled")
    return dq, dk, dv


def decode_e4m3(x, scale=1.0) -> np.ndarray:
    """Exact fp64 values of FP8 E4M3 codes (uint8 array or torch uint8 /
    float8_e4m3fn tensor), times ``scale``; same shape."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu()
        if x.dtype != torch.uint8:
            x = x.view(torch.uint8)
        x = x.numpy()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.uint8))
    out = np.empty(a.shape, dtype=np.float64)
    _check(_load().oracle_decode_e4m3(a.ctypes.data_as(ctypes.c_void_p), a.size, float(scale),
                                      _ptr(out)), "decode_e4m3")
    return out


def attention_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal):
    """Standard attention on the decoded 8-bit inputs: Q = q_scale * decode(q8),
    likewise K and V, then ``attention_fwd``. Returns (o, lse)."""
    return attention_fwd(decode_e4m3(q8, q_scale), decode_e4m3(k8, k_scale),
                         decode_e4m3(v8, v_scale), scale, causal)


def attention_rows_fp8(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal, rows):
    """``attention_rows`` on the decoded 8-bit inputs."""
    return attention_rows(decode_e4m3(q8, q_scale), decode_e4m3(k8, k_scale),
                          decode_e4m3(v8, v_scale), scale, causal, rows)


def decode_paged(q, k_cache, v_cache, page_table, seq_lens, scale):
    """Decode-step attention over a paged KV cache.

    q: [B, H, d]; k_cache, v_cache: [num_pages, H_kv, page_size, d];
    page_table: int [B, max_pages]; seq_lens: int [B]. Query head h reads KV
    head h // (H // H_kv). Returns (o [B, H, d], lse [B, H]).
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    pt = page_table.numpy() if hasattr(page_table, "numpy") else page_table
    sl = seq_lens.numpy() if hasattr(seq_lens, "numpy") else seq_lens
    pt = np.ascontiguousarray(np.asarray(pt, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(sl, dtype=np.int32))
    B, H, d = q.shape
    num_pages, H_kv, page_size, d2 = kc.shape
    if d2 != d or vc.shape != kc.shape or pt.shape[0] != B or sl.shape != (B,):
        raise ValueError("inconsistent decode shapes")
    o = np.empty((B, H, d))
    lse = np.empty((B, H))
    ip = ctypes.POINTER(ctypes.c_int)
    _check(_load().oracle_decode_paged(_ptr(q), _ptr(kc), _ptr(vc), pt.ctypes.data_as(ip),
                                       sl.ctypes.data_as(ip), B, H, H_kv, d, num_pages,
                                       page_size, pt.shape[1], float(scale), _ptr(o), _ptr(lse)),
           "decode_paged")
    return o, lse
