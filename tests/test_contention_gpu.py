"""Race check of the kernels' load waits and barriers under memory contention.

Every kernel here streams tiles into LDS with asynchronous loads and relies
on wait counts and workgroup barriers to read a tile only after it landed
and to refill a ring slot only after every wave is done with it. A wait
that is one load too short, or a barrier that publishes too early, can still
give right answers when loads return quickly. This test stretches the load
latency instead: each entry point first runs alone, then several times while
a second stream (default priority, like every stream here) keeps HBM busy
with 1 GiB device copies; every result must be bitwise equal to the lone
run (the kernels are deterministic). Outputs are filled with NaN (or zeros)
before each run, so a skipped write shows as well. HIP events on both
streams record whether the two streams' work overlapped in time; the test
requires that it did in at least one run, so that it is not passing on
serialized work."""
import math

import pytest
import torch

import io_aware_tiled_09_amd as fa
from io_aware_tiled_09_amd.inputs import make_decode, make_dout, make_qkv, make_qkv_fp8

from _parity import say

pytestmark = pytest.mark.gpu

_HOG_FLOATS = 256 << 20  # 1 GiB per copy


@pytest.fixture(scope="module")
def hog():
    # Both streams made once, one after the other: torch hands out pooled
    # streams in turn and the runtime spreads them over its hardware queues,
    # so two consecutive streams do not share a queue (a stream made anew
    # for every test would, now and then, land on the copies' queue and be
    # serialized behind them).
    src = torch.ones(_HOG_FLOATS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copies, calls = torch.cuda.Stream(), torch.cuda.Stream()
    yield copies, calls, src, dst
    torch.cuda.synchronize()
    del src, dst


def _check_under_contention(hog, run, outs, label, reps=4):
    """run(stream) enqueues the call(s) on `stream`; outs: the tensors they
    write."""
    hs, main, src, dst = hog
    torch.cuda.synchronize()
    with torch.cuda.stream(main):
        run(main)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    overlapped = 0
    for rep in range(reps):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(hs)
        with torch.cuda.stream(hs):
            for _ in range(2 + rep):
                dst.copy_(src)
        ev[1].record(hs)
        ev[2].record(main)
        with torch.cuda.stream(main):
            run(main)
        ev[3].record(main)
        torch.cuda.synchronize()
        # the call started before the copies ended and ended after they started
        if ev[2].elapsed_time(ev[1]) > 0 and ev[0].elapsed_time(ev[3]) > 0:
            overlapped += 1
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (label, rep, i)
    say(f"  {label}: {reps} runs beside HBM copies bitwise equal to the lone run "
        f"({overlapped} overlapped in time)")
    assert overlapped >= 1, f"{label}: the copies never overlapped the call"


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 16, 8192, 128, True), (1, 16, 4096, 64, False),
                                            (4, 12, 1000, 64, True)])
def test_forward_under_contention(hog, B, H, N, d, causal):
    say(f"contention: fa_fwd B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = (t.cuda() for t in make_qkv(B=B, H=H, N=N, d=d, seed=31))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    sc = 1.0 / math.sqrt(d)

    def run(stream):
        assert fa.fa_fwd(q, k, v, o, lse, B, H, N, d, sc, int(causal), stream) == 0

    _check_under_contention(hog, run, [o, lse], "fa_fwd")


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 16, 8192, 128, True), (2, 32, 4096, 128, True),
                                            (2, 8, 1500, 64, False)])
def test_backward_under_contention(hog, B, H, N, d, causal):
    # (2, 32, 4096) runs the phased dQ kernel, the others the 128-query one
    say(f"contention: fa_bwd B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = (t.cuda() for t in make_qkv(B=B, H=H, N=N, d=d, seed=32))
    do = make_dout(B=B, H=H, N=N, d=d, seed=32).cuda()
    sc = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    assert fa.fa_fwd(q, k, v, o, lse, B, H, N, d, sc, int(causal)) == 0
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def run(stream):
        assert fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, B, H, N, d, sc, int(causal),
                         stream) == 0

    _check_under_contention(hog, run, [dq, dk, dv], "fa_bwd")


@pytest.mark.parametrize("B,H,N,causal", [(2, 16, 8192, True), (1, 8, 3000, False)])
def test_fp8_under_contention(hog, B, H, N, causal):
    say(f"contention: fa_fwd_fp8 B={B} H={H} N={N} d=128 causal={causal}")
    (q8, k8, v8), (qs, ks, vs) = make_qkv_fp8(B=B, H=H, N=N, d=128, seed=33)
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    o = torch.empty((B, H, N, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def run(stream):
        assert fa.fa_fwd_fp8(q8, k8, v8, o, lse, B, H, N, 128, 128 ** -0.5, qs, ks, vs,
                             int(causal), stream) == 0

    _check_under_contention(hog, run, [o, lse], "fa_fwd_fp8")


def test_decode_under_contention(hog):
    say("contention: fa_decode_paged, decode50")
    x = make_decode("decode50", seed=34)
    w = x["workload"]
    g = {kk: x[kk].cuda() for kk in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    need = fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.page_size, w.max_pages)
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")

    def run(stream):
        assert fa.fa_decode_paged(g["q"], g["k_cache"], g["v_cache"], g["page_table"],
                                  g["seq_lens"], o, lse, ws, need, w.B, w.H, w.H_kv, w.d,
                                  g["k_cache"].shape[0], w.page_size, w.max_pages, w.scale,
                                  stream) == 0

    _check_under_contention(hog, run, [o, lse], "fa_decode_paged")
