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


def standard_rows(q, k, v, scale, causal, rows=None):
    """The standard (materializing) path's rounding points for one head:
    S = scale * (Q K^T) with fp32 accumulation of the exact bf16 products,
    the row softmax in fp32 (max, p = exp2(s log2e - m log2e), sum, times
    1/sum), P rounded to bf16, O = P V with fp32 accumulation, O rounded to
    bf16; lse = m + log2(sum) ln 2. rows: query rows to model (default all).
    Returns (o [R, d], lse [R]) float64."""
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    s = (q[rows].astype(F32) @ k.astype(F32).T).astype(F32) * F32(scale)
    if causal:
        s = np.where(np.arange(n)[None, :] <= rows[:, None], s, F32(-np.inf))
    m = s.max(axis=1, keepdims=True)
    mc = (m * F32(LOG2E)).astype(F32)
    p = np.exp2(fma32(s, np.full_like(s, LOG2E), -np.broadcast_to(mc, s.shape)))
    p = np.where(np.isneginf(s), F32(0), p).astype(F32)
    l = p.sum(axis=1, dtype=F32, keepdims=True)
    pb = bf16(p * (F32(1) / l))
    o = bf16((pb @ v.astype(F32)).astype(F32))
    lse = m[:, 0].astype(np.float64) + np.log2(l[:, 0].astype(np.float64)) * LN2
    return o.astype(np.float64), lse


def decode_row(q, k, v, c_log2, unroll):
    """The decode kernels' rounding points for one (sequence, query head):
    q [d], k, v [L, d] float32 holding bf16 values; c_log2 = float32(scale *
    log2 e). Keys go in runs of 512; in a run, group g (of 16) takes key
    16 b + g of each 16-key block b, `unroll` blocks at a time: the batch's
    max moves the group's reference, l and acc are rescaled once, then each
    key adds p = exp2(s - m) (fp32 dot products: each of 16 lanes sums its
    d/16 slice with fmas, then a butterfly over the 16 lanes). The 16 group
    states merge in pairs (g, g^1), then (g, g^2), then the four resulting
    states in order; the runs merge in order; O = acc * (1/l) rounded to
    bf16, lse = (m + log2 l) ln 2. Returns (o [d] float64, lse float)."""
    L, d = k.shape
    E = d // 16
    # fp32 dot products in the kernel's order
    qs = q.reshape(16, E).astype(F32)
    ks = k.reshape(L, 16, E).astype(F32)
    part = np.zeros((L, 16), dtype=F32)
    for e in range(E):
        part = fma32(np.broadcast_to(qs[:, e], (L, 16)), ks[:, :, e], part)
    for off in (8, 4, 2, 1):
        part = (part + part[:, np.arange(16) ^ off]).astype(F32)
    s_all = (part[:, 0] * F32(c_log2)).astype(F32)

    def merge(a, b):
        m1, l1, a1 = a
        m2, l2, a2 = b
        mn = max(m1, m2)
        if mn == -np.inf:
            return a
        f1 = np.exp2(F32(m1 - mn)).astype(F32)
        f2 = np.exp2(F32(m2 - mn)).astype(F32)
        return (mn, F32(F32(l1 * f1) + F32(l2 * f2)),
                (a1 * f1 + a2 * f2).astype(F32))

    runs = []
    for r0 in range(0, L, 512):
        r1 = min(L, r0 + 512)
        groups = []
        for g in range(16):
            m, l, acc = -np.inf, F32(0), np.zeros(d, dtype=F32)
            keys = list(range(r0 + g, r1, 16))
            for b0 in range(0, (r1 - r0 + 15) // 16, unroll):
                batch = [r0 + 16 * b + g for b in range(b0, b0 + unroll) if r0 + 16 * b + g < r1]
                if not batch:
                    continue
                mx = max(float(s_all[j]) for j in batch)
                mn = max(m, mx)
                alpha = np.exp2(F32(m - mn)).astype(F32) if m != -np.inf else F32(0)
                m = mn
                l = F32(l * alpha)
                acc = (acc * alpha).astype(F32)
                for j in batch:
                    p = np.exp2(F32(s_all[j] - F32(mn))).astype(F32)
                    l = F32(l + p)
                    acc = fma32(np.full(d, p, dtype=F32), v[j].astype(F32), acc)
            del keys
            groups.append((F32(m) if m != -np.inf else -np.inf, l, acc))
        for off in (1, 2):
            groups = [merge(groups[g], groups[g ^ off]) for g in range(16)]
        st = groups[0]
        for w in (4, 8, 12):
            st = merge(st, groups[w])
        runs.append(st)
    st = runs[0]
    for r in runs[1:]:
        st = merge(st, r)
    m, l, acc = st
    o = bf16((acc * (F32(1) / l)).astype(F32))
    return o.astype(np.float64), (float(m) + float(np.log2(np.float64(l)))) * LN2
