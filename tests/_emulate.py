"""fp32 CPU emulation of the HIP kernels' rounding points: TEST
INFRASTRUCTURE, used only to derive the tolerances of the GPU parity tests.

The GPU parity bounds for the backward pass (and the other derived bounds)
are not given by the pages; they come from modelling where the kernels round.
This module writes that model out in numpy: the same operands rounded to
bf16 at the same points, products and sums in fp32, the same base-2 softmax
with the same reference-max slack. The model is compared with the fp64
oracle exactly as the GPU result is, and the bound is set above what the
model reaches on the same inputs. It shares no code with the HIP path (it
reads no kernel source and calls no library) and carries none of the
oracle's arithmetic: the oracle is the definition, this is a model of the
GPU's deviation from it.

Arrays are one head at a time: q, k, v, dout are float32 [N, d] holding the
exact bf16 values the GPU receives.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned
    as float32. Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(F32)


def fma32(a, b, c) -> np.ndarray:
    """fp32 fused multiply-add: a*b + c rounded once (via float64, where the
    product of two fp32 values is exact)."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(F32)


def kernel_c(scale: float) -> np.float32:
    """scale * log2(e) as the host hands it to the kernels (double product,
    then float)."""
    return F32(float(scale) * LOG2E)


def scores(q, k, causal) -> np.ndarray:
    """S = q k^T in fp32 (the kernels accumulate exact bf16 products in fp32),
    masked entries -inf."""
    s = np.asarray(q, F32) @ np.asarray(k, F32).T
    if causal:
        n = s.shape[0]
        s[np.triu_indices(n, 1)] = -np.inf
    return s


def flash_fwd(q, k, v, scale, causal, tile=64, slack=3.0):
    """The bf16 forward kernel's arithmetic: key tiles of `tile` in ascending
    order; per row a reference max (base 2) that moves only when a tile's
    max passes it by more than `slack`; p = exp2(fma(s, c, -m)) in fp32; the
    row sum adds the fp32 p; P rounded to bf16 for P V (fp32 accumulation);
    the output rescaled by exp2(m_old - m_new) when the reference moves;
    O = acc * (1 / l) rounded to bf16; lse = (m + log2 l) * ln 2.
    Returns (o float32 [N, d] holding bf16 values, lse float32 [N])."""
    N, d = q.shape
    c = kernel_c(scale)
    S = scores(q, k, causal)
    m = np.full(N, -np.inf, F32)
    l = np.zeros(N, F32)
    acc = np.zeros((N, d), F32)
    for t0 in range(0, N, tile):
        s = S[:, t0:t0 + tile]
        raw = s.max(axis=1)
        mt = np.where(raw > -np.inf, raw * c, -np.inf).astype(F32)
        grow = mt > m + F32(slack)
        m_new = np.where(grow, mt, m).astype(F32)
        with np.errstate(invalid="ignore"):
            alpha = np.exp2(np.where(np.isfinite(m), m - m_new, -np.inf)).astype(F32)
        m = m_new
        p = np.exp2(fma32(s, c, -m[:, None])).astype(F32)
        l = (l * alpha + p.sum(axis=1, dtype=F32)).astype(F32)
        acc = (acc * alpha[:, None]).astype(F32)
        acc = (acc + bf16(p) @ np.asarray(v[t0:t0 + tile], F32)).astype(F32)
    inv = (F32(1.0) / l).astype(F32)
    o = bf16(acc * inv[:, None])
    lse = ((m + np.log2(l).astype(F32)) * F32(LN2)).astype(F32)
    return o, lse


def flash_bwd(q, k, v, o, lse, dout, scale, causal):
    """The backward kernels' arithmetic, given the forward's bf16 o and fp32
    lse: D = sum_t dO*O in fp32; P = exp2(fma(s, c, -lse*log2e)) in fp32;
    dV = bf16(P)^T dO; dP = dO V^T in fp32; dS = P (dP - D) in fp32, rounded
    to bf16 for its products: the dQ kernel forms it from the fp32 P, the
    dK/dV kernel from the bf16 P its partner wave hands over (a second
    rounding); dQ = scale dS K and dK = scale dS^T Q; gradients stored as
    bf16. Returns (dq, dk, dv), float32 [N, d] holding bf16 values."""
    c = kernel_c(scale)
    o = np.asarray(o, F32)
    do = np.asarray(dout, F32)
    D = (do * o).sum(axis=1, dtype=F32)
    lse2 = (np.asarray(lse, F32) * F32(LOG2E)).astype(F32)
    P = np.exp2(fma32(scores(q, k, causal), c, -lse2[:, None])).astype(F32)
    Pb = bf16(P)
    dv = bf16(Pb.T @ do)
    dP = (do @ np.asarray(v, F32).T - D[:, None]).astype(F32)
    dq = bf16((bf16(P * dP) @ np.asarray(k, F32)) * F32(scale))
    del P
    dk = bf16((bf16(Pb * dP).T @ np.asarray(q, F32)) * F32(scale))
    return dq, dk, dv


def e4m3(x) -> np.ndarray:
    """Round non-negative float32 values to the nearest OCP FP8 E4M3 value
    (ties to even): 3 mantissa bits in the normal range [2^-6, 448],
    multiples of 2^-9 below it. Values above 448 are not expected."""
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32)
    normal = (u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))) & np.uint32(0xFFF00000)
    sub = (np.round(x.astype(np.float64) * 512.0) / 512.0).astype(F32)
    return np.where(x >= F32(2.0 ** -6), normal.view(F32), sub).astype(F32)


def flash_fwd_fp8(q, k, v, scale, causal, tile=128, slack=3.0, pscale=48.0):
    """The FP8 forward kernel's arithmetic on decoded inputs (q, k, v already
    q_scale * code etc., as float32): key tiles of `tile`; scores in fp32
    (exact products of 8-bit values, fp32 sums); per row a reference max
    (base 2) moved only when a tile's max passes it by more than `slack`;
    w = exp2(fma(s, c, -(m - log2 pscale))) = pscale * p in fp32, summed in
    fp32; P for the product with V rounded to E4M3 as w; the output rescaled
    when the reference moves; O = acc / l rounded to bf16 (the codes' v scale
    is in v already); lse = (m + log2(l / pscale)) * ln 2."""
    N, d = q.shape
    c = kernel_c(scale)
    S = scores(q, k, causal)
    lg = F32(np.log2(pscale))
    m = np.full(N, -np.inf, F32)
    l = np.zeros(N, F32)
    acc = np.zeros((N, d), F32)
    for t0 in range(0, N, tile):
        s = S[:, t0:t0 + tile]
        raw = s.max(axis=1)
        mt = np.where(raw > -np.inf, raw * c, -np.inf).astype(F32)
        grow = mt > m + F32(slack)
        m_new = np.where(grow, mt, m).astype(F32)
        with np.errstate(invalid="ignore"):
            alpha = np.exp2(np.where(np.isfinite(m), m - m_new, -np.inf)).astype(F32)
        m = m_new
        w = np.exp2(fma32(s, c, -(m - lg)[:, None])).astype(F32)
        l = (l * alpha + w.sum(axis=1, dtype=F32)).astype(F32)
        acc = (acc * alpha[:, None]).astype(F32)
        acc = (acc + e4m3(w) @ np.asarray(v[t0:t0 + tile], F32)).astype(F32)
    o = bf16(acc * (F32(1.0) / l)[:, None])
    lse = ((m + np.log2(l / F32(pscale)).astype(F32)) * F32(LN2)).astype(F32)
    return o, lse
