"""The seeded input generators (CPU only)."""
import dataclasses

import torch

from io_aware_tiled_09_amd.inputs import WORKLOADS, Workload, make_qkv, sample_rows, useful_flops


def test_deterministic_and_shaped():
    a = make_qkv("bert512", N=64)
    b = make_qkv("bert512", N=64)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (4, 12, 64, 64) and x.is_contiguous()
        assert torch.equal(x, y)
    q32, _, _ = make_qkv("single_head")
    assert q32.dtype == torch.float32 and q32.shape == (1, 1, 256, 64)


def test_bf16_is_the_rounded_fp32_draw():
    q16, k16, v16 = make_qkv("gpt2_1k", B=1, H=2, N=40)
    q32, k32, v32 = make_qkv("gpt2_1k", B=1, H=2, N=40, dtype="fp32")
    for lo, hi in ((q16, q32), (k16, k32), (v16, v32)):
        assert torch.equal(lo, hi.to(torch.bfloat16))


def test_spiky_keys():
    w = WORKLOADS["gpt2_1k_spiky"]
    plain = dataclasses.replace(w, spike_frac=0.0, dtype="fp32")
    spiky = dataclasses.replace(w, dtype="fp32")
    q0, k0, v0 = make_qkv(plain)
    q1, k1, v1 = make_qkv(spiky)
    assert torch.equal(q0, q1) and torch.equal(v0, v1)
    rows = k0.reshape(-1, w.d)
    rows1 = k1.reshape(-1, w.d)
    changed = (rows1 != rows).any(dim=1)
    assert int(changed.sum()) == round(0.01 * w.B * w.H * w.N) == 983
    assert torch.equal(rows1[changed], rows[changed] * 20.0)


def test_per_head_scale():
    w = dataclasses.replace(WORKLOADS["longctx32k"], N=64, dtype="fp32")
    base = dataclasses.replace(w, std=1.0, head_scale=None)
    q, k, v = make_qkv(w)
    q0, k0, v0 = make_qkv(base)
    ratio = q / q0
    c = ratio[0, :, 0, 0]
    assert ((c >= 0.25) & (c <= 1.0)).all()  # 0.5 std times a factor in [0.5, 2]
    torch.testing.assert_close(ratio, c.view(1, -1, 1, 1).expand_as(ratio), rtol=1e-5, atol=0)
    torch.testing.assert_close(k / k0, ratio, rtol=1e-5, atol=0)


def test_sample_rows():
    r = sample_rows(1000, 16, seed=3, heads=4)
    assert r.shape == (4, 16)
    for row in r:
        assert row[0] == 0 and row[-1] == 999
        assert len(set(row.tolist())) == 16
        assert torch.equal(row, torch.sort(row).values)
    assert torch.equal(r, sample_rows(1000, 16, seed=3, heads=4))
    assert torch.equal(sample_rows(5, 16, seed=1), torch.arange(5).view(1, 5))


def test_useful_flops():
    assert useful_flops(2, 32, 8192, 128, True) == 4.0 * 2 * 32 * 8192 ** 2 * 128 / 2
    assert useful_flops(1, 1, 10, 4, False) == 1600.0
    assert isinstance(WORKLOADS["longdoc8k"], Workload)


def test_make_dout_is_seeded_and_independent_of_qkv():
    from io_aware_tiled_09_amd.inputs import make_dout, make_qkv
    a = make_dout("gpt2_1k", B=1, H=2, N=64)
    b = make_dout("gpt2_1k", B=1, H=2, N=64)
    assert a.dtype == torch.bfloat16 and a.shape == (1, 2, 64, 64) and a.is_contiguous()
    assert torch.equal(a, b)
    q, k, v = make_qkv("gpt2_1k", B=1, H=2, N=64)
    assert not any(torch.equal(a, t) for t in (q, k, v))
    c = make_dout(B=1, H=1, N=3, d=64, seed=1, dtype="fp32")
    assert c.dtype == torch.float32 and not torch.equal(c, make_dout(B=1, H=1, N=3, d=64, seed=2,
                                                                      dtype="fp32"))


def test_backward_flops_is_two_and_a_half_forwards():
    from io_aware_tiled_09_amd.inputs import backward_flops, useful_flops
    for causal in (False, True):
        assert backward_flops(2, 32, 8192, 128, causal) == 2.5 * useful_flops(2, 32, 8192, 128,
                                                                               causal)
