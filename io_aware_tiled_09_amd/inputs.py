"""Seeded synthetic attention inputs.

This module only draws random numbers, shapes them like the workloads the
FlashAttention pages talk about, and casts them to the storage dtype. It holds
none of the attention arithmetic, so both the HIP path and the CPU oracle can
take their inputs from here without sharing any computation.

Workloads (stand-ins for the pages' examples; no dataset or weights exist here):

* ``single_head``   one head, N=256, d=64, fp32 storage, non-causal.
* ``bert512``       BERT-shaped self-attention, B=4, H=12, N=512, d=64.
                    [FlashAttention: The GPU Memory Hack That Changed Everything,
                    "The Numbers: Speed and Memory", BERT (seq 512) row]
* ``gpt2_1k``       GPT-2-shaped causal attention, B=8, H=12, N=1024, d=64.
                    [same page and table, GPT-2 (seq 1K) row]
* ``gpt2_1k_spiky`` the same with 1% of the key rows multiplied by 20, so the
                    running maximum of the online softmax moves often.
* ``longdoc8k``     long-document causal attention, B=2, H=32, N=8192, d=128.
                    [Flash Attention Optimization (aicomputerinstitute.com),
                    opening section: 8,000-30,000-token documents]
* ``longctx32k``    very long context, B=1, H=32, N=32768, d=128, entries
                    N(0, 0.5^2) times one U[0.5, 2] factor per head.

All draws come from ``torch.Generator('cpu').manual_seed(seed)`` in the order
Q, K, V, then the variant's extra draws, in fp32; bf16 storage is the
round-to-nearest-even cast of those fp32 values. The tensors returned are the
exact values both the GPU and the oracle consume.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_qkv_fp8", "make_dout", "make_scores",
           "sample_rows", "useful_flops", "backward_flops", "DecodeWorkload", "DECODE_WORKLOADS",
           "make_decode", "decode_kv_bytes"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str  # "bf16" or "fp32" (storage dtype of q, k, v and o)
    seed: int
    std: float = 1.0
    spike_frac: float = 0.0  # fraction of K rows (over flattened b, h, j) scaled
    spike_factor: float = 1.0
    head_scale: tuple | None = None  # (lo, hi): one U[lo, hi] factor per head
    oracle_rows: int | None = None  # rows per head the oracle checks; None = all
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head", 1, 1, 256, 64, False, "fp32", 1000,
                 note="single head, fp32 storage"),
        Workload("bert512", 4, 12, 512, 64, False, "bf16", 1001,
                 note="BERT-shaped self-attention"),
        Workload("gpt2_1k", 8, 12, 1024, 64, True, "bf16", 1002,
                 note="GPT-2-shaped causal attention"),
        Workload("gpt2_1k_spiky", 8, 12, 1024, 64, True, "bf16", 1003,
                 spike_frac=0.01, spike_factor=20.0,
                 note="GPT-2 shape, 1% of K rows x20"),
        Workload("longdoc8k", 2, 32, 8192, 128, True, "bf16", 1004,
                 note="long-document causal attention"),
        Workload("longctx32k", 1, 32, 32768, 128, True, "bf16", 1005,
                 std=0.5, head_scale=(0.5, 2.0), oracle_rows=256,
                 note="very long context, per-head scale"),
    ]
}


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)  # round to nearest even
    if dtype == "fp32":
        return x.contiguous()
    raise ValueError(f"unknown storage dtype {dtype!r}")


def make_qkv(w: Workload | str | None = None, *, B=None, H=None, N=None, d=None,
             dtype=None, seed=None, std=None):
    """Return contiguous CPU tensors ``(q, k, v)`` of shape [B, H, N, d].

    Either name a workload (its fields may be overridden by keyword) or give
    the shape, dtype and seed directly. Entries are i.i.d. N(0, std^2) fp32
    draws, then the workload's variant draws, then the storage cast.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w is None:
        w = Workload("custom", B, H, N, d, False, dtype or "bf16",
                     0 if seed is None else seed, std=1.0 if std is None else std)
    else:
        over = {k_: v_ for k_, v_ in dict(B=B, H=H, N=N, d=d, dtype=dtype,
                                           seed=seed, std=std).items()
                if v_ is not None}
        if over:
            w = Workload(**{**w.__dict__, **over})
    g = torch.Generator(device="cpu").manual_seed(int(w.seed))
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.std != 1.0:
        q.mul_(w.std)
        k.mul_(w.std)
        v.mul_(w.std)
    if w.spike_frac > 0.0:
        rows = w.B * w.H * w.N
        count = int(round(w.spike_frac * rows))
        idx = torch.randperm(rows, generator=g)[:count]
        k.view(rows, w.d)[idx] *= w.spike_factor
    if w.head_scale is not None:
        lo, hi = w.head_scale
        c = torch.rand(w.H, generator=g, dtype=torch.float32) * (hi - lo) + lo
        c = c.view(1, w.H, 1, 1)
        q.mul_(c)
        k.mul_(c)
        v.mul_(c)
    return _cast(q, w.dtype), _cast(k, w.dtype), _cast(v, w.dtype)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor FP8 E4M3 quantization of an fp32 tensor: scale = amax / 448
    (448 is the format's largest finite value), codes = round-to-nearest-even
    of x / scale (torch's float8_e4m3fn cast). Returns (uint8 codes, scale)."""
    amax = float(x.abs().max())
    scale = amax / 448.0 if amax > 0 else 1.0
    codes = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, scale


def make_qkv_fp8(w: Workload | str | None = None, **kw):
    """The workload's fp32 draws (as ``make_qkv`` with dtype "fp32"), each
    quantized per tensor to FP8 E4M3. Returns ((q8, k8, v8) uint8 CPU tensors,
    (q_scale, k_scale, v_scale) floats)."""
    q, k, v = make_qkv(w, dtype="fp32", **kw)
    (q8, qs), (k8, ks), (v8, vs) = (quantize_e4m3(t) for t in (q, k, v))
    return (q8, k8, v8), (qs, ks, vs)


def make_dout(w: Workload | str | None = None, *, B=None, H=None, N=None, d=None,
              dtype=None, seed=None):
    """Upstream gradient dO for the backward pass: a contiguous CPU tensor of
    shape [B, H, N, d] with i.i.d. N(0, 1) fp32 entries cast to the storage
    dtype, drawn from its own generator seeded with ``seed + 500009`` so that
    it is independent of the workload's Q, K and V draws."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w is not None:
        B, H, N, d = (w.B if B is None else B, w.H if H is None else H,
                      w.N if N is None else N, w.d if d is None else d)
        dtype = dtype or w.dtype
        seed = w.seed if seed is None else seed
    g = torch.Generator(device="cpu").manual_seed(int(seed or 0) + 500009)
    x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    return _cast(x, dtype or "bf16")


def make_scores(B: int, H: int, N: int, seed: int, std: float = 3.0) -> torch.Tensor:
    """Score matrices for testing a row softmax on its own: contiguous fp32
    [B, H, N, N], i.i.d. N(0, std^2) from torch.Generator('cpu') seeded with
    ``seed``."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn((B, H, N, N), generator=g, dtype=torch.float32) * std


def sample_rows(N: int, count: int, seed: int, heads: int = 1) -> torch.Tensor:
    """Seeded, sorted sample of ``count`` distinct query rows per head.

    Rows 0 and N-1 are always in the sample; the rest are drawn without
    replacement. Returns int64 [heads, min(count, N)].
    """
    count = min(count, N)
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = torch.empty((heads, count), dtype=torch.int64)
    for h in range(heads):
        if count == N:
            out[h] = torch.arange(N)
            continue
        fixed = [0, N - 1] if N > 1 else [0]
        inner = torch.randperm(N - 2, generator=g)[: count - len(fixed)] + 1 \
            if N > 2 else torch.empty(0, dtype=torch.int64)
        rows = torch.cat([torch.tensor(fixed, dtype=torch.int64), inner])
        out[h] = torch.sort(rows).values
    return out


def useful_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Useful FLOPs of one forward call: 2*N*N*d for QK^T plus 2*N*N*d for PV
    per head, halved when causal (only keys j <= i count)."""
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def backward_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Useful FLOPs of one backward call: the five N x N x d products
    S = Q K^T (recomputed), dP = dO V^T, dV = P^T dO, dQ = dS K and
    dK = dS^T Q, 2*N*N*d each per head, halved when causal; i.e. 2.5 times
    the forward's useful FLOPs."""
    f = 10.0 * B * H * N * N * d
    return f / 2.0 if causal else f



# ---------------------------------------------------------------- decode over a paged KV cache
@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step of B concurrent sequences: one new query token each,
    attending to its L_b cached tokens stored in pages of ``page_size`` rows.

    Lengths are drawn uniformly from [min_len, max_len_draw]; the page table
    has room for ``max_context`` tokens per sequence. Physical pages are
    handed out in a seeded random order (a fragmented pool), with
    ``spare_pages`` extra pages that no sequence uses."""
    name: str
    B: int
    H: int
    H_kv: int
    d: int
    page_size: int
    max_context: int
    min_len: int
    max_len_draw: int
    seed: int
    spare_pages: int = 64
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_pages(self) -> int:
        return (self.max_context + self.page_size - 1) // self.page_size


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        # 50 users served at once, memory sized for an 8K context, about 30%
        # of it in use on average (mean length ~2460 of 8192).
        # [FlashAttention: The GPU Memory Hack That Changed Everything,
        #  "What's Next?": 50 concurrent users, pre-allocated max-context
        #  memory mostly unused; PagedAttention's pages and page tables]
        DecodeWorkload("decode50", 50, 32, 32, 128, 16, 8192, 64, 4864, 2001,
                       note="50 sequences, MHA, 16-token pages"),
        DecodeWorkload("decode50_gqa", 50, 32, 8, 128, 16, 8192, 64, 4864, 2002,
                       note="the same with 4 query heads per KV head"),
        DecodeWorkload("decode_small", 3, 4, 2, 128, 16, 1024, 1, 700, 2003,
                       note="small case for the oracle in seconds"),
    ]
}


def make_decode(w: DecodeWorkload | str, fill_unused=float("nan"), **over):
    """Seeded inputs of one decode step. Returns a dict with q [B, H, d] bf16,
    k_cache, v_cache [num_pages, H_kv, page_size, d] bf16, page_table int32
    [B, max_pages] (-1 past each sequence's last page) and seq_lens int32 [B].

    Draw order from torch.Generator('cpu').manual_seed(seed): the lengths,
    the permutation of physical pages, then q, k_cache, v_cache as N(0, 1)
    fp32 cast to bf16. Cache rows that no sequence owns (spare pages and the
    rows after each sequence's last token) are set to ``fill_unused`` (NaN by
    default, so that reading them would show)."""
    if isinstance(w, str):
        w = DECODE_WORKLOADS[w]
    if over:
        w = DecodeWorkload(**{**w.__dict__, **over})
    g = torch.Generator(device="cpu").manual_seed(int(w.seed))
    lens = torch.randint(w.min_len, w.max_len_draw + 1, (w.B,), generator=g, dtype=torch.int64)
    lens = torch.clamp(lens, max=w.max_context)
    pages_per = (lens + w.page_size - 1) // w.page_size
    used = int(pages_per.sum())
    num_pages = used + w.spare_pages
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((w.B, w.max_pages), -1, dtype=torch.int32)
    at = 0
    for b in range(w.B):
        n = int(pages_per[b])
        table[b, :n] = perm[at:at + n].to(torch.int32)
        at += n
    q = torch.randn((w.B, w.H, w.d), generator=g, dtype=torch.float32)
    kc = torch.randn((num_pages, w.H_kv, w.page_size, w.d), generator=g, dtype=torch.float32)
    vc = torch.randn((num_pages, w.H_kv, w.page_size, w.d), generator=g, dtype=torch.float32)
    owned = torch.zeros((num_pages, w.page_size), dtype=torch.bool)
    for b in range(w.B):
        L = int(lens[b])
        for t in range(int(pages_per[b])):
            rows = min(w.page_size, L - t * w.page_size)
            owned[int(table[b, t]), :rows] = True
    mask = (~owned)[:, None, :, None].expand_as(kc)
    kc[mask] = fill_unused
    vc[mask] = fill_unused
    return dict(q=q.to(torch.bfloat16), k_cache=kc.to(torch.bfloat16),
                v_cache=vc.to(torch.bfloat16), page_table=table,
                seq_lens=lens.to(torch.int32), workload=w)


def decode_kv_bytes(w: DecodeWorkload, seq_lens) -> int:
    """Algorithmic bytes of one decode step: every cached K and V row of every
    sequence read once (bf16), q read and o written once (bf16), lse (fp32)."""
    tokens = int(torch.as_tensor(seq_lens).sum())
    return tokens * w.H_kv * w.d * 2 * 2 + w.B * w.H * (w.d * 2 * 2 + 4)
