"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64
backward oracle. The GPU's own forward supplies O and lse, as in training;
dO is a seeded N(0, 1) draw. Bounds are in tests/_parity.py."""
import math

import pytest
import torch

import io_aware_tiled_09_amd as fa
from io_aware_tiled_09_amd.inputs import WORKLOADS, make_dout, make_qkv, sample_rows

import oracle

from _parity import (GRAD_LONG_MAX_REL, GRAD_SPIKY_MAX_REL, GRAD_SPIKY_MEAN_REL, assert_grads_close,
                     check_bwd_full, check_bwd_sampled, run_gpu_bwd, say)

pytestmark = pytest.mark.gpu

TINY_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", TINY_N)
def test_bwd_tiny_shapes(N, d, causal):
    say(f"bwd tiny N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B=1, H=2, N=N, d=d, seed=N * 13 + d)
    do = make_dout(B=1, H=2, N=N, d=d, seed=N * 13 + d)
    check_bwd_full(q, k, v, do, causal, 1.0 / math.sqrt(d), f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_ragged_multi_block(d, causal):
    say(f"bwd ragged B=2 H=3 N=333 d={d} causal={causal}")
    q, k, v = make_qkv(B=2, H=3, N=333, d=d, seed=31 + d)
    do = make_dout(B=2, H=3, N=333, d=d, seed=31 + d)
    check_bwd_full(q, k, v, do, causal, 1.0 / math.sqrt(d), "N=333")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(2, 64, 2100), (16, 64, 200), (16, 64, 100)])
def test_bwd_phased_dq(B, H, N, d, causal):
    # Grids of at least 1024 query blocks of 256 rows run dQ in the phased
    # kernel: N = 2100 ends in a 52-row query block and a 52-key tile, cleared
    # in the phase loop; N = 200 has four key tiles, the partial one cleared at
    # the first phase that may; N = 100 has two, cleared in the prologue.
    # Every row of three heads against the oracle.
    heads = [0, (B * H) // 2 + 1, B * H - 1]
    say(f"bwd phased dQ B={B} H={H} N={N} d={d} causal={causal}, heads {heads}")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=N + d + causal)
    do = make_dout(B=B, H=H, N=N, d=d, seed=N + d + causal)
    check_bwd_full(q, k, v, do, causal, 1.0 / math.sqrt(d), f"phased N={N} d={d} causal={causal}",
                   heads=heads)


def _bwd_random_shapes(seed=20261203):
    # Eight small shapes (B, H 1-3, N 1-2000), then four whose grids of
    # 256-row query blocks reach four rounds of the CUs, so that dQ runs in
    # the phased kernel (B = 4, H 24-40, N from the smallest such length to
    # 700 past it, at most 3000).
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(8):
        out.append((rng.randint(1, 3), rng.randint(1, 3), rng.randint(1, 2000),
                    rng.choice([64, 128]), rng.choice([False, True])))
    for _ in range(4):
        B, H = 4, rng.randint(24, 40)
        nqb = -(-1024 // (B * H))
        N = rng.randint((nqb - 1) * 256 + 1, min(nqb * 256 + 700, 3000))
        N = max(N, (nqb - 1) * 256 + 1)
        out.append((B, H, N, rng.choice([64, 128]), rng.choice([False, True])))
    return out


@pytest.mark.parametrize("B,H,N,d,causal", _bwd_random_shapes())
def test_bwd_random_shapes(B, H, N, d, causal):
    # Seeded shapes with ragged last query blocks and key tiles; every row of
    # the first and last head against the oracle.
    phased = B * H * -(-N // 256) >= 1024
    heads = [0, B * H - 1] if B * H > 1 else [0]
    say(f"bwd random B={B} H={H} N={N} d={d} causal={causal} "
        f"({'phased' if phased else '128-query'} dQ), heads {heads}")
    seed = B * 1000 + H * 100 + N + d
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=seed)
    do = make_dout(B=B, H=H, N=N, d=d, seed=seed)
    check_bwd_full(q, k, v, do, causal, 1.0 / math.sqrt(d), f"random N={N} d={d}", heads=heads)


@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_bwd_explicit_scale(scale):
    say(f"bwd scale={scale} B=1 H=3 N=300 d=64 causal")
    q, k, v = make_qkv(B=1, H=3, N=300, d=64, seed=41)
    do = make_dout(B=1, H=3, N=300, d=64, seed=41)
    check_bwd_full(q, k, v, do, True, scale, f"scale={scale}")


@pytest.mark.parametrize("name", ["bert512", "gpt2_1k", "gpt2_1k_spiky"])
def test_bwd_workload_heads(name):
    w = WORKLOADS[name]
    heads = [0, (w.B * w.H) // 2 + 1, w.B * w.H - 1]
    say(f"bwd workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}, heads {heads}")
    q, k, v = make_qkv(w)
    bounds = {}
    if w.spike_frac > 0:
        bounds = dict(max_rel=GRAD_SPIKY_MAX_REL, mean_rel=GRAD_SPIKY_MEAN_REL)
    check_bwd_full(q, k, v, make_dout(w), w.causal, w.scale, name, heads=heads, **bounds)


def test_bwd_longdoc8k_sampled():
    w = WORKLOADS["longdoc8k"]
    heads = [0, 37, w.B * w.H - 1]
    fixed = torch.tensor([0, 63, 64, 127, 128, 255, 256, w.N // 2, w.N - 129, w.N - 2,
                          w.N - 1], dtype=torch.int64)
    qrows = torch.cat([sample_rows(w.N, 24, seed=w.seed + 91, heads=len(heads)),
                       fixed.expand(len(heads), -1)], dim=1)
    krows = torch.cat([sample_rows(w.N, 24, seed=w.seed + 92, heads=len(heads)),
                       fixed.expand(len(heads), -1)], dim=1)
    say(f"bwd workload longdoc8k: B={w.B} H={w.H} N={w.N} d={w.d} causal, heads {heads}, "
        f"{qrows.shape[1]} query rows and {krows.shape[1]} key rows each")
    q, k, v = make_qkv(w)
    check_bwd_sampled(q, k, v, make_dout(w), w.causal, w.scale, heads, qrows, krows,
                      "longdoc8k", max_rel=GRAD_LONG_MAX_REL)


def test_bwd_longdoc8k_full_heads():
    # Every row of dQ, dK and dV in 8 of the 64 heads of the long-document
    # workload (both batches, first, last and interior heads), from one
    # fa_bwd call over the whole workload, against the materializing backward
    # oracle, head by head (each head's own rms in the bound).
    w = WORKLOADS["longdoc8k"]
    heads = [0, 5, 13, 31, 32, 42, 50, 63]
    say(f"bwd workload longdoc8k: every row of heads {heads}")
    q, k, v = make_qkv(w)
    do = make_dout(w)
    got = run_gpu_bwd(q, k, v, do, w.causal, w.scale)
    B, H, N, d = q.shape
    for bh in heads:
        sel = lambda x: x.reshape(B * H, N, d)[bh].reshape(1, 1, N, d)
        ref = oracle.attention_bwd(sel(q), sel(k), sel(v), sel(do), w.scale, w.causal)
        assert_grads_close([sel(g).numpy() for g in got], ref, f"longdoc8k head {bh}",
                           max_rel=GRAD_LONG_MAX_REL)


def test_bwd_deterministic_bitwise():
    say("bwd determinism B=2 H=4 N=1000 d=128 causal")
    q, k, v = make_qkv(B=2, H=4, N=1000, d=128, seed=7)
    do = make_dout(B=2, H=4, N=1000, d=128, seed=7)
    a = run_gpu_bwd(q, k, v, do, True, 1.0 / math.sqrt(128))
    b = run_gpu_bwd(q, k, v, do, True, 1.0 / math.sqrt(128))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_leaves_inputs_untouched():
    say("bwd inputs untouched B=1 H=2 N=200 d=64")
    q, k, v = (t.cuda() for t in make_qkv(B=1, H=2, N=200, d=64, seed=8))
    do = make_dout(B=1, H=2, N=200, d=64, seed=8).cuda()
    o, lse = fa.attention(q, k, v, causal=False)
    before = [t.clone() for t in (q, k, v, o, lse, do)]
    fa.attention_backward(q, k, v, o, lse, do, causal=False)
    torch.cuda.synchronize()
    for x, y in zip(before, (q, k, v, o, lse, do)):
        assert torch.equal(x, y)
