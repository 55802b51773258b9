"""The library's entry points inside a captured HIP graph (torch.cuda.CUDAGraph
on ROCm): each launches plain kernels on the caller's stream and allocates
nothing, so a step can be captured once and replayed. Every replay is
checked bitwise against the eager result, with eager work and
synchronizations between the replays."""
import math

import pytest
import torch

import io_aware_tiled_09_amd as fa
from io_aware_tiled_09_amd.inputs import make_decode, make_dout, make_qkv, make_qkv_fp8

from _parity import say

pytestmark = pytest.mark.gpu


def _replay_and_compare(run, outs, label):
    """run(stream) enqueues the call(s) on `stream`; outs: tensors it writes."""
    torch.cuda.synchronize()
    eager_stream = torch.cuda.Stream()
    with torch.cuda.stream(eager_stream):
        run(eager_stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            run(cap)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), (label, rep)
        # eager work between replays
        _ = (outs[0].float() * 2).sum().item()
    say(f"  {label}: 3 replays bitwise equal to the eager call")


def test_graph_forward_and_backward():
    say("graph: fa_fwd + fa_bwd, B=1 H=4 N=700 d=128 causal")
    q, k, v = (t.cuda() for t in make_qkv(B=1, H=4, N=700, d=128, seed=21))
    do = make_dout(B=1, H=4, N=700, d=128, seed=21).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 700), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((1, 4, 700), dtype=torch.float32, device="cuda")
    sc = 1.0 / math.sqrt(128)

    def run(stream):
        assert fa.fa_fwd(q, k, v, o, lse, 1, 4, 700, 128, sc, 1, stream) == 0
        assert fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, 1, 4, 700, 128, sc, 1, stream) == 0

    _replay_and_compare(run, [o, lse, dq, dk, dv], "fwd+bwd")


def test_graph_fp8_and_decode():
    say("graph: fa_fwd_fp8 and fa_decode_paged")
    (q8, k8, v8), (qs, ks, vs) = make_qkv_fp8(B=1, H=2, N=500, d=128, seed=22)
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    o8 = torch.empty((1, 2, 500, 128), dtype=torch.bfloat16, device="cuda")
    l8 = torch.empty((1, 2, 500), dtype=torch.float32, device="cuda")
    x = make_decode("decode_small", seed=23)
    w = x["workload"]
    g = {kk: x[kk].cuda() for kk in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    need = fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.page_size, w.max_pages)
    dws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    od = torch.empty_like(g["q"])
    ld = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")

    def run(stream):
        assert fa.fa_fwd_fp8(q8, k8, v8, o8, l8, 1, 2, 500, 128, 0.1, qs, ks, vs, 1, stream) == 0
        assert fa.fa_decode_paged(g["q"], g["k_cache"], g["v_cache"], g["page_table"],
                                  g["seq_lens"], od, ld, dws, need, w.B, w.H, w.H_kv, w.d,
                                  g["k_cache"].shape[0], w.page_size, w.max_pages, w.scale,
                                  stream) == 0

    _replay_and_compare(run, [o8, l8, od, ld], "fp8+decode")
