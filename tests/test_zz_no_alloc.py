"""The allocation-free backward entry point (fa_bwd_noalloc, through the C
ABI) against fa_bwd with a caller-provided workspace: the same kernels, with
D held in the library's static device scratch instead of the workspace.

Two calls in a row, the second on a smaller input, each bitwise equal to
fa_bwd on the same inputs (the kernels are deterministic), and within the
backward bound of the oracle."""
import math

import pytest
import torch

import io_aware_tiled_09_amd as fa
import oracle
from io_aware_tiled_09_amd.inputs import make_dout, make_qkv

from _parity import assert_grads_close, say

pytestmark = pytest.mark.gpu


def _grads(entry, q, k, v, o, lse, do, causal, scale):
    B, H, N, d = q.shape
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    if entry == "noalloc":
        st = fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, scale, causal)
    else:
        ws = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        st = fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, B, H, N, d, scale, causal)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return dq, dk, dv


def test_bwd_noalloc_matches_fa_bwd_twice():
    for (B, H, N, d, causal, seed) in [(2, 3, 700, 128, True, 71), (1, 2, 300, 64, False, 72)]:
        say(f"fa_bwd_noalloc B={B} H={H} N={N} d={d} causal={causal}")
        qc, kc, vc = make_qkv(B=B, H=H, N=N, d=d, seed=seed)
        doc = make_dout(B=B, H=H, N=N, d=d, seed=seed)
        q, k, v, do = (t.cuda() for t in (qc, kc, vc, doc))
        scale = 1.0 / math.sqrt(d)
        o, lse = fa.attention(q, k, v, causal=causal, scale=scale)
        got = _grads("noalloc", q, k, v, o, lse, do, causal, scale)
        ref = _grads("ws", q, k, v, o, lse, do, causal, scale)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name} differs from fa_bwd"
        refs = oracle.attention_bwd(qc, kc, vc, doc, scale, causal)
        assert_grads_close([g.double().cpu().numpy() for g in got], refs, "noalloc")
