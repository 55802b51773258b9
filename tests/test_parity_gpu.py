"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Inputs are the seeded generators' tensors; the oracle receives the exact
values the GPU receives (bf16 or fp32, upcast to fp64). Bounds are in
tests/_parity.py.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_tiled_09_amd as fa
import oracle
from io_aware_tiled_09_amd.inputs import WORKLOADS, make_qkv, sample_rows

from _parity import (LSE_REL, O_MAX_ABS, O_MEAN_ABS, assert_close, check_full, check_rows,
                     run_gpu, say)

pytestmark = pytest.mark.gpu


TINY_N = [1, 2, 3, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", TINY_N)
def test_tiny_shapes(N, d, causal):
    say(f"tiny N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B=1, H=2, N=N, d=d, seed=N * 7 + d)
    check_full(q, k, v, causal, 1.0 / math.sqrt(d), f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_multi_tile(d, causal):
    say(f"ragged B=2 H=3 N=333 d={d} causal={causal}")
    q, k, v = make_qkv(B=2, H=3, N=333, d=d, seed=11 + d)
    check_full(q, k, v, causal, 1.0 / math.sqrt(d), "N=333")


def _grid(B, H, N, causal):
    """fa_fwd's launch shape (workgroups, rows per block, paired)."""
    return fa.fa_fwd_grid(B, H, N, causal)


def _boundary_rows(N, *extra):
    """Rows at block and tile edges (0, 63, 64, 127, 128, 255, 256, ...) and
    the last rows, within [0, N)."""
    rows = {0, 1, N - 2, N - 1, *extra}
    for b in range(0, N + 256, 128):
        rows.update({b - 1, b, b + 63, b + 64})
    return sorted(r for r in rows if 0 <= r < N)


@pytest.mark.parametrize("B,H,N,d", [(1, 128, 700, 64), (1, 128, 700, 128), (2, 64, 1300, 128),
                                     (1, 128, 2100, 64), (3, 64, 513, 128)])
def test_paired_query_blocks(B, H, N, d):
    # Causal grids with N <= 8192 that fill the CUs run one workgroup per pair
    # of 256-row query blocks (nqb-1-p, p); odd block counts leave the middle
    # block alone and ragged N puts the partial block in a pair. Many heads,
    # so that the paired grid has at least 256 workgroups; rows sampled per
    # head, every block and tile edge included.
    grid, rows_per_block, paired = _grid(B, H, N, True)
    assert rows_per_block == 256 and paired and grid >= 256
    say(f"paired blocks B={B} H={H} N={N} d={d} causal ({grid} workgroups)")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=N + d + B)
    edge = torch.tensor(_boundary_rows(N), dtype=torch.int64)
    rows = torch.cat([sample_rows(N, 12, seed=N + d, heads=B * H), edge.expand(B * H, -1)], 1)
    check_rows(q, k, v, True, 1.0 / math.sqrt(d), rows, f"paired N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 40, 2000), (3, 9, 1300), (1, 33, 2300)])
def test_balanced_causal_groups(B, H, N, d):
    # Small causal grids whose key-split grid would take several rounds run
    # groups of query blocks with equal work: {nqb-1}, {nqb-2-p, p} and, for
    # even nqb, the middle blocks of two heads (27 heads: one alone; nqb = 9:
    # none). Every output against the oracle.
    grid, rows_per_block, paired = _grid(B, H, N, True)
    nqb = (N + 255) // 256
    per = 1 + (nqb - 1) // 2
    assert rows_per_block == 256 and paired
    assert grid == B * H * per + ((B * H + 1) // 2 if nqb % 2 == 0 else 0)
    say(f"balanced groups B={B} H={H} N={N} d={d} causal ({grid} workgroups)")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=N + d + H)
    check_full(q, k, v, True, 1.0 / math.sqrt(d), f"balanced N={N} d={d}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [129, 200, 257, 333, 700, 1000, 2100])
def test_key_split_blocks(N, d, causal):
    # Grids too small for the CUs run 128-row blocks whose two wave groups take
    # alternate key tiles and merge their (max, sum, output) states: every
    # output against the oracle, ragged tails and odd tile counts included.
    grid, rows_per_block, paired = _grid(1, 2, N, causal)
    assert rows_per_block == 128 and not paired
    say(f"key split B=1 H=2 N={N} d={d} causal={causal} ({grid} workgroups)")
    q, k, v = make_qkv(B=1, H=2, N=N, d=d, seed=N * 3 + d + causal)
    check_full(q, k, v, causal, 1.0 / math.sqrt(d), f"key split N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_key_split_wide(d, causal):
    # The largest key-split grids (256 workgroups) with long rows: B=2 H=16
    # N=1000 (8 blocks of 128 per head).
    B, H, N = 2, 16, 1000
    grid, rows_per_block, _ = _grid(B, H, N, causal)
    assert rows_per_block == 128 and grid == 256
    say(f"key split wide B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=1000 + d + causal)
    check_full(q, k, v, causal, 1.0 / math.sqrt(d), f"key split wide d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_unpaired_causal_ragged(d):
    # Past N = 8192 a causal grid of more than 512 query blocks runs one block
    # per workgroup; N = 8300 leaves a ragged last block of 108 rows.
    B, H, N = 1, 16, 8300
    assert _grid(B, H, N, True) == (16 * 33, 256, False)
    say(f"unpaired causal B={B} H={H} N={N} d={d}")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=8300 + d)
    rows = sample_rows(N, 24, seed=91 + d, heads=B * H)
    fixed = torch.tensor([0, 255, 256, 4095, 8191, 8192, 8255, 8256, N - 2, N - 1],
                         dtype=torch.int64)
    check_rows(q, k, v, True, 1.0 / math.sqrt(d), torch.cat([rows, fixed.expand(B * H, -1)], 1),
               f"unpaired N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H", [16, 4])
def test_long_ragged(H, d):
    # N = 8000 <= 8192, causal. H = 16: the paired kernel over 32 query blocks
    # (16 pairs) per head, the last block ragged (64 rows) and paired with
    # block 0. H = 4: 252 key-split workgroups of 128 rows (63 per head), the
    # last one ragged.
    B, N = 1, 8000
    grid, rows_per_block, paired = _grid(B, H, N, True)
    assert (rows_per_block, paired) == ((256, True) if H == 16 else (128, False))
    say(f"long ragged B={B} H={H} N={N} d={d} ({grid} workgroups of {rows_per_block} rows)")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=8000 + d + H)
    rows = sample_rows(N, 32, seed=57 + d, heads=B * H)
    fixed = torch.tensor([0, 1, 127, 128, 255, 256, 3967, 3968, 4031, 7935, 7936, 7937, N - 2,
                          N - 1], dtype=torch.int64)
    check_rows(q, k, v, True, 1.0 / math.sqrt(d), torch.cat([rows, fixed.expand(B * H, -1)], 1),
               f"long ragged H={H} N={N} d={d}")


def _random_shapes(n=12, seed=4242):
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        out.append((rng.randint(1, 3), rng.randint(1, 3), rng.randint(1, 2600),
                    rng.choice([64, 128]), rng.choice([False, True])))
    return out


@pytest.mark.parametrize("B,H,N,d,causal", _random_shapes())
def test_random_shapes(B, H, N, d, causal):
    # Seeded shapes: query-block counts odd and even, ragged tails, paired and
    # unpaired grids.
    say(f"random B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=B * 1000 + H * 100 + N + d)
    check_full(q, k, v, causal, 1.0 / math.sqrt(d), f"random N={N} d={d}")


# Shapes drawn from a seeded generator (B 1-4, H 1-40, N 1-3000, d 64/128,
# causal 60%) and kept ten per launch mode of fa_fwd: one 256-row block per
# workgroup, 128-row key-split blocks, paired causal blocks and balanced
# causal groups.
_MODE_SHAPES = [
    (2, 29, 1826, 128, False, "one"), (3, 7, 2584, 64, False, "one"),
    (3, 33, 515, 128, False, "one"), (1, 35, 1613, 128, False, "one"),
    (4, 8, 2678, 128, False, "one"), (3, 38, 2090, 64, False, "one"),
    (3, 32, 2806, 128, False, "one"), (3, 7, 1584, 64, False, "one"),
    (4, 3, 46, 128, True, "one"), (3, 34, 116, 64, True, "one"),
    (3, 35, 164, 128, False, "key_split"), (3, 8, 468, 128, False, "key_split"),
    (1, 1, 2635, 128, True, "key_split"), (1, 25, 730, 128, False, "key_split"),
    (3, 13, 388, 64, False, "key_split"), (1, 1, 1931, 128, True, "key_split"),
    (3, 1, 691, 128, False, "key_split"), (1, 40, 219, 128, False, "key_split"),
    (2, 9, 1330, 128, True, "key_split"), (2, 6, 1891, 64, False, "key_split"),
    (1, 29, 1051, 128, True, "paired"), (4, 26, 1823, 128, True, "paired"),
    (3, 20, 1747, 128, True, "paired"), (2, 11, 1754, 128, True, "paired"),
    (3, 31, 1587, 64, True, "paired"), (2, 31, 1657, 64, True, "paired"),
    (4, 31, 1436, 128, True, "paired"), (2, 36, 1691, 128, True, "paired"),
    (3, 37, 1435, 64, True, "paired"), (4, 31, 2579, 64, True, "paired"),
    (1, 23, 2498, 64, True, "balanced"), (3, 32, 387, 64, True, "balanced"),
    (1, 18, 2003, 128, True, "balanced"), (2, 7, 2469, 128, True, "balanced"),
    (4, 20, 788, 64, True, "balanced"), (3, 14, 1867, 128, True, "balanced"),
    (4, 10, 942, 128, True, "balanced"), (2, 10, 2928, 64, True, "balanced"),
    (1, 24, 2900, 128, True, "balanced"), (1, 23, 2404, 64, True, "balanced"),
]


def _launch_mode(B, H, N, causal):
    grid, rows_per_block, paired = _grid(B, H, N, causal)
    nqb = (N + 255) // 256
    if rows_per_block == 128:
        return "key_split"
    if paired and grid != B * H * ((nqb + 1) // 2):
        return "balanced"
    return "paired" if paired else "one"


@pytest.mark.parametrize("B,H,N,d,causal,mode", _MODE_SHAPES)
def test_random_launch_modes(B, H, N, d, causal, mode):
    # The launch mode the shape is filed under is the one fa_fwd picks; then
    # sampled rows of every head, every block and tile edge included, against
    # the oracle.
    assert _launch_mode(B, H, N, causal) == mode
    say(f"launch mode {mode}: B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=7 * N + 11 * H + B + d + causal)
    edge = torch.tensor(_boundary_rows(N), dtype=torch.int64)
    rows = torch.cat([sample_rows(N, 8, seed=N + H, heads=B * H), edge.expand(B * H, -1)], 1)
    check_rows(q, k, v, causal, 1.0 / math.sqrt(d), rows, f"{mode} N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_storage_path(d):
    say(f"fp32 storage B=2 H=2 N=300 d={d}")
    for causal in (False, True):
        q, k, v = make_qkv(B=2, H=2, N=300, d=d, dtype="fp32", seed=21 + d)
        check_full(q, k, v, causal, 1.0 / math.sqrt(d), f"fp32 causal={causal}")


@pytest.mark.parametrize("name", ["single_head", "bert512", "gpt2_1k", "gpt2_1k_spiky"])
def test_workload_full(name):
    w = WORKLOADS[name]
    say(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} {w.dtype}")
    q, k, v = make_qkv(w)
    check_full(q, k, v, w.causal, w.scale, name)


def _rows_for(w, count):
    rows = sample_rows(w.N, count, seed=w.seed + 77, heads=w.B * w.H)
    fixed = torch.tensor([31, 32, 63, 64, 127, 128, 129, w.N // 2, w.N - 2, w.N - 1],
                         dtype=torch.int64)
    return torch.cat([rows, fixed.expand(w.B * w.H, -1)], dim=1)


def test_workload_full_longdoc8k():
    # Every output of the long-document workload (B=2, H=32, N=8192, d=128,
    # causal): the GPU result of one fa_fwd call, in the launch configuration
    # bench.py times, against the materializing oracle run head by head (one
    # head's S and P, 2 x 512 MiB, at a time). The bound applies to the whole
    # output: max and mean over all 64 x 8192 x 128 values, lse over all rows.
    w = WORKLOADS["longdoc8k"]
    say(f"workload longdoc8k, every row: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = make_qkv(w)
    o_gpu, lse_gpu = run_gpu(q, k, v, w.causal, w.scale)
    B, H, N, d = q.shape
    o_max, o_sum, l_max, worst = 0.0, 0.0, 0.0, None
    for bh in range(B * H):
        b, h = divmod(bh, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, lse_ref = oracle.attention_fwd(q[sl], k[sl], v[sl], w.scale, w.causal)
        dlt = np.abs(o_gpu[sl].numpy() - o_ref)
        assert np.isfinite(dlt).all(), f"non-finite GPU output in head {bh}"
        lrel = np.abs(lse_gpu[sl].numpy() - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
        if dlt.max() > o_max:
            o_max = float(dlt.max())
            worst = (b, h) + np.unravel_index(int(dlt.argmax()), dlt.shape)[2:]
        o_sum += float(dlt.sum())
        l_max = max(l_max, float(lrel.max()))
        if bh % 16 == 15:
            say(f"  heads 0..{bh}: max|dO|={o_max:.3e} lse rel={l_max:.3e}")
    o_mean = o_sum / (B * H * N * d)
    say(f"  longdoc8k, all rows: max|dO|={o_max:.3e} mean|dO|={o_mean:.3e} lse rel={l_max:.3e} "
        f"worst O at {worst}")
    assert o_max <= O_MAX_ABS and o_mean <= O_MEAN_ABS and l_max <= LSE_REL


@pytest.mark.parametrize("name,count", [("longdoc8k", 48), ("longctx32k", 256)])
def test_workload_sampled_rows(name, count):
    w = WORKLOADS[name]
    count = w.oracle_rows or count
    say(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}, "
        f"{count}+10 rows per head")
    q, k, v = make_qkv(w)
    check_rows(q, k, v, w.causal, w.scale, _rows_for(w, count), name)


def test_deterministic_bitwise():
    say("determinism B=2 H=4 N=1000 d=128 causal")
    q, k, v = (t.cuda() for t in make_qkv(B=2, H=4, N=1000, d=128, seed=5))
    o1, l1 = fa.attention(q, k, v, causal=True)
    o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_no_writes_outside_outputs(dtype):
    say(f"canaries {dtype}")
    B, H, N, d = 1, 3, 77, 64
    q, k, v = (t.cuda() for t in make_qkv(B=B, H=H, N=N, d=d, seed=9,
                                          dtype="bf16" if dtype == torch.bfloat16 else "fp32"))
    pad = 4096
    n = B * H * N * d
    obuf = torch.full((pad + n + pad,), 7.0, dtype=dtype, device="cuda")
    lbuf = torch.full((pad + B * H * N + pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    fa.attention(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7.0).all() and (obuf[pad + n:] == 7.0).all()
    assert (lbuf[:pad] == 7.0).all() and (lbuf[pad + B * H * N:] == 7.0).all()
    o_ref, lse_ref = oracle.attention_fwd(q.cpu(), k.cpu(), v.cpu(), 1 / 8, True)
    assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, "canary")


def test_side_stream():
    say("non-default stream")
    q, k, v = (t.cuda() for t in make_qkv(B=1, H=4, N=700, d=128, seed=3))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, causal=True)
    s.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q.cpu(), k.cpu(), v.cpu(), 1 / math.sqrt(128), True)
    assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, "stream")


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_gives_means(causal):
    say(f"scale 0 causal={causal}")
    B, H, N, d = 1, 2, 190, 64
    q, k, v = make_qkv(B=B, H=H, N=N, d=d, seed=4)
    o, lse = run_gpu(q, k, v, causal, 0.0)
    vv = v.double()
    if causal:
        ref = torch.cumsum(vv, dim=2) / torch.arange(1, N + 1, dtype=torch.float64).view(1, 1, N, 1)
        lref = torch.log(torch.arange(1, N + 1, dtype=torch.float64)).expand(B, H, N)
    else:
        ref = vv.mean(dim=2, keepdim=True).expand_as(vv)
        lref = torch.full((B, H, N), math.log(N), dtype=torch.float64)
    assert_close(o.numpy(), lse.numpy(), ref.numpy(), lref.numpy(), "scale=0")


def test_large_logits_d128():
    say("large logits: q, k x8 at d=128")
    q, k, v = make_qkv(B=1, H=2, N=520, d=128, seed=8)
    q = (q.float() * 8).to(torch.bfloat16)
    k = (k.float() * 8).to(torch.bfloat16)
    check_full(q, k, v, True, 1 / math.sqrt(128), "x8 logits")


def test_gpu_argument_errors():
    say("argument errors on device tensors")
    q, k, v = (t.cuda() for t in make_qkv(B=1, H=1, N=64, d=64, seed=1))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 64), device="cuda")
    flat = torch.empty(64 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    mis = flat[1:1 + 64 * 64].view(1, 1, 64, 64)
    assert fa.fa_fwd(mis, k, v, o, lse, 1, 1, 64, 64, 0.125, 0) == 5
    assert fa.fa_fwd(q, k, v, q, lse, 1, 1, 64, 64, 0.125, 0) == 6
    with pytest.raises(fa.FAError):
        fa.attention(q[..., :32].contiguous(), k[..., :32].contiguous(), v[..., :32].contiguous())
    # buffers of the wrong extent are refused before any launch
    with pytest.raises(ValueError):
        fa.attention(q, k, v, out=torch.empty((1, 1, 32, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.attention(q, k, v, lse=torch.empty((1, 1, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.attention_backward(q, k, v, o, torch.empty((1, 1, 32), device="cuda"), q)
    torch.cuda.synchronize()


def test_empty_sequence():
    say("empty N=0")
    q = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.attention(q, q, q, causal=True)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 64) and lse.shape == (2, 3, 0)
