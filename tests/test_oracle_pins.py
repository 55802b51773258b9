"""Pins for the fp64 oracle (CPU only).

The oracle is pinned to things other than itself: the numbers the pages print
for their worked examples (fixtures in tests/golden/), closed forms,
invariances, brute force of the tiled recurrences against the direct
definition, and torch's own CPU float64 attention and logsumexp. Each group
is chosen so that a plausible slip in the oracle (a dropped correction
factor, a wrong sign, a transposed operand, a wrong mask index, a missing
normalization) fails at least one test here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked examples


def test_worked_example_direct_softmax():
    g = _golden("worked_example_online_softmax.json")
    out, lse = oracle.softmax_row(g["scores"], g["values"])
    pr = g["printed"]
    assert abs(out[0] - pr["output_traced_code"]) < 1e-11
    assert abs(out[0] - pr["output_4dp"]) < 5e-5
    # lse = max + ln(sum of exps relative to the max); the page prints the exps
    exps = np.array(pr["direct_exps"])
    assert abs(lse - (5.0 + math.log(exps.sum()))) < 2e-5


def test_worked_example_weights_via_full_attention():
    """Scores [1,3,2,5] made by d=1 queries of 1 against keys [1,3,2,5]."""
    g = _golden("worked_example_online_softmax.json")
    s = np.array(g["scores"])
    n = s.size
    q = np.ones((1, 1, n, 1))
    k = s.reshape(1, 1, n, 1)
    v = np.array(g["values"]).reshape(1, 1, n, 1)
    o, lse, p = oracle.attention_fwd(q, k, v, 1.0, False, return_p=True)
    pr = g["printed"]
    for i in range(n):
        np.testing.assert_allclose(p[0, 0, i], pr["direct_weights"], atol=5e-6)
        # exps relative to the global max = weights * sum
        np.testing.assert_allclose(p[0, 0, i] * math.exp(lse[0, 0, i] - 5.0),
                                   pr["direct_exps"], atol=5e-6)
        assert abs(o[0, 0, i, 0] - pr["output_traced_code"]) < 1e-11


@pytest.mark.parametrize("fn", [oracle.online_row_two_scale, oracle.online_row_single_max])
def test_worked_example_online(fn):
    g = _golden("worked_example_online_softmax.json")
    s, v, bs = g["scores"], g["values"], g["block_size"]
    pr = g["printed"]
    out, m, l_ = fn(s, v, bs)
    assert abs(out[0] - pr["output_traced_code"]) < 1e-11
    assert m == 5.0
    assert abs(out[0] * l_ - pr["final_acc"]) < 1e-4
    # running state after block 1 = the recurrence over the first block alone
    out1, m1, l1 = fn(s[:2], v[:2], bs)
    assert m1 == pr["block1_m"]
    assert abs(l1 - pr["block1_l"]) < 5e-6
    assert abs(out1[0] * l1 - pr["block1_acc"]) < 2e-4  # page multiplies 5-digit exps by values up to 40
    # block 2's local statistics: the recurrence over block 2 alone
    out2, m2, l2 = fn(s[2:], v[2:], bs)
    assert abs(l2 - pr["block2_local_l"]) < 5e-6
    assert abs(out2[0] * l2 - pr["block2_local_acc"]) < 2e-4
    # merge factors exp(m_old - m_new) and exp(m_block - m_new)
    assert abs(math.exp(m1 - m) - pr["merge_scale_old"]) < 5e-6
    assert math.exp(m2 - m) == pr["merge_scale_new"]


@pytest.mark.parametrize("fn", [oracle.online_row_two_scale, oracle.online_row_single_max])
def test_active_recall_no_rescale_branch(fn):
    g = _golden("active_recall_q1.json")
    s, v, bs = g["scores"], g["values"], g["block_size"]
    pr = g["printed"]
    out, m, l_ = fn(s, v, bs)
    assert abs(out[0] - pr["output"]) < 5e-4
    assert abs(out[0] * l_ - pr["final_acc"]) < 2e-4
    out1, m1, l1 = fn(s[:2], v[:2], bs)
    # the second block does not move the running max: no rescale of block 1
    assert m1 == pr["block1_m"] and m == pr["block1_m"]
    assert abs(l1 - pr["block1_l"]) < 1e-4
    assert abs(out1[0] * l1 - pr["block1_acc"]) < 2e-4  # the page rounds exps to 4 digits
    out2, m2, l2 = fn(s[2:], v[2:], bs)
    assert abs(out2[0] * l2 - pr["block2_local_acc"]) < 2e-4
    assert abs(math.exp(m2 - m) - pr["merge_scale_new"]) < 5e-5
    # and the direct definition agrees with the page's answer too
    d_out, _ = oracle.softmax_row(s, v)
    assert abs(d_out[0] - pr["output"]) < 5e-4


# ---------------------------------------------------------------- brute force


def _row_cases():
    rng = np.random.default_rng(7)
    for n in range(1, 17):
        yield rng.normal(0, 3, n), rng.normal(0, 1, (n, 3))
        yield np.sort(rng.normal(0, 5, n)), rng.normal(0, 1, (n, 3))  # max rises each block
        yield -np.sort(-rng.normal(0, 5, n)), rng.normal(0, 1, (n, 3))  # max never rises
        s = rng.normal(0, 1, n)
        s[rng.integers(0, n)] += 40.0  # one spike
        yield s, rng.normal(0, 1, (n, 3))


def test_recurrences_match_direct_for_every_block_size():
    for s, v in _row_cases():
        ref, ref_lse = oracle.softmax_row(s, v)
        n = s.size
        for bs in range(1, n + 1):
            for fn in (oracle.online_row_two_scale, oracle.online_row_single_max):
                out, m, l_ = fn(s, v, bs)
                np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
                assert m == s.max()
                assert abs(m + math.log(l_) - ref_lse) <= 1e-12 * max(1.0, abs(ref_lse))


def test_direct_softmax_closed_forms():
    # equal scores: plain mean of the values; lse = s + ln n
    v = np.arange(12.0).reshape(4, 3)
    out, lse = oracle.softmax_row([0.7] * 4, v)
    np.testing.assert_allclose(out, v.mean(axis=0), rtol=1e-15)
    assert abs(lse - (0.7 + math.log(4))) < 1e-15
    # two keys: logistic weights
    a, b = 0.3, -1.1
    out, lse = oracle.softmax_row([a, b], [[1.0], [0.0]])
    assert abs(out[0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
    assert abs(lse - math.log(math.exp(a) + math.exp(b))) < 1e-15
    # masked keys (-inf) get zero weight
    out, lse = oracle.softmax_row([1.0, -math.inf, 1.0], [[2.0], [1e300], [4.0]])
    assert out[0] == 3.0 and abs(lse - (1.0 + math.log(2.0))) < 1e-15
    # huge spread: no overflow, the spike takes all the weight
    out, lse = oracle.softmax_row([1000.0, 0.0], [[5.0], [7.0]])
    assert out[0] == 5.0 and lse == 1000.0


# ---------------------------------------------------------------- full attention


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(0, scale, shape)


@pytest.mark.parametrize("causal", [False, True])
def test_n_equals_one(causal):
    q, k, v = _rand((2, 3, 1, 8), 1), _rand((2, 3, 1, 8), 2), _rand((2, 3, 1, 8), 3)
    o, lse = oracle.attention_fwd(q, k, v, 0.25, causal)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse[..., 0], 0.25 * (q * k).sum(-1)[..., 0], rtol=1e-15)


def test_zero_queries_give_means():
    B, H, N, d = 1, 2, 9, 5
    q = np.zeros((B, H, N, d))
    k, v = _rand((B, H, N, d), 4), _rand((B, H, N, d), 5)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(N), rtol=1e-15)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1).reshape(1, 1, N, 1)
    np.testing.assert_allclose(o, prefix, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), rtol=1e-15)


def test_causal_first_row_and_mask():
    B, H, N, d = 2, 2, 11, 7
    q, k, v = _rand((B, H, N, d), 6), _rand((B, H, N, d), 7), _rand((B, H, N, d), 8)
    o, lse, p = oracle.attention_fwd(q, k, v, 0.4, True, return_p=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.4 * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=1e-14)
    upper = np.triu(np.ones((N, N), dtype=bool), 1)
    assert (p[:, :, upper] == 0.0).all()
    assert (p[:, :, ~upper] > 0.0).all()
    # row i only depends on keys/values 0..i: changing the last key changes no earlier row
    k2, v2 = k.copy(), v.copy()
    k2[:, :, -1] += 3.0
    v2[:, :, -1] -= 2.0
    o2, lse2 = oracle.attention_fwd(q, k2, v2, 0.4, True)
    np.testing.assert_array_equal(o2[:, :, :-1], o[:, :, :-1])
    np.testing.assert_array_equal(lse2[:, :, :-1], lse[:, :, :-1])
    assert not np.allclose(o2[:, :, -1], o[:, :, -1])


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k, v = _rand((1, 3, 33, 16), 9, 2.0), _rand((1, 3, 33, 16), 10, 2.0), _rand((1, 3, 33, 16), 11)
    o, lse, p = oracle.attention_fwd(q, k, v, 0.25, causal, return_p=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (p >= 0).all()
    np.testing.assert_allclose(o, p @ v, rtol=1e-12, atol=1e-13)


def test_permuting_keys_and_values_together():
    B, H, N, d = 1, 2, 20, 8
    q, k, v = _rand((B, H, N, d), 12), _rand((B, H, N, d), 13), _rand((B, H, N, d), 14)
    perm = np.random.default_rng(15).permutation(N)
    o, lse = oracle.attention_fwd(q, k, v, 0.35, False)
    o2, lse2 = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.35, False)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # permuting only the values does change the answer
    o3, _ = oracle.attention_fwd(q, k, v[:, :, perm], 0.35, False)
    assert not np.allclose(o3, o)


@pytest.mark.parametrize("causal", [False, True])
def test_value_scaling_and_score_shift(causal):
    B, H, N, d = 2, 1, 15, 6
    q, k, v = _rand((B, H, N, d), 16), _rand((B, H, N, d), 17), _rand((B, H, N, d), 18)
    o, lse = oracle.attention_fwd(q, k, v, 0.5, causal)
    o2, _ = oracle.attention_fwd(q, k, -2.5 * v, 0.5, causal)
    np.testing.assert_allclose(o2, -2.5 * o, rtol=1e-12, atol=1e-14)
    # adding one vector u to every key shifts row i's scores by scale*q_i.u:
    # P and O unchanged, lse shifted by that amount
    u = _rand((d,), 19)
    o3, lse3 = oracle.attention_fwd(q, k + u, v, 0.5, causal)
    np.testing.assert_allclose(o3, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse3, lse + 0.5 * (q @ u), rtol=1e-12, atol=1e-12)


def _torch_reference(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    s = (tq @ tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), -math.inf)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,spread", [((2, 3, 37, 16), 1.0), ((1, 2, 64, 64), 1.0),
                                          ((1, 1, 50, 8), 12.0)])
def test_matches_torch_float64_sdpa(causal, shape, spread):
    q, k, v = _rand(shape, 20, spread), _rand(shape, 21, spread), _rand(shape, 22)
    scale = 1.0 / math.sqrt(shape[-1])
    o, lse = oracle.attention_fwd(q, k, v, scale, causal)
    ro, rlse = _torch_reference(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_match_full(causal):
    B, H, N, d = 2, 2, 41, 12
    q, k, v = _rand((B, H, N, d), 23), _rand((B, H, N, d), 24), _rand((B, H, N, d), 25)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, causal)
    rows = np.array([[0, 5, 40], [1, 2, 3], [40, 39, 0], [7, 7, 20]])
    o_r, lse_r = oracle.attention_rows(q, k, v, 0.3, causal, rows)
    for bh in range(B * H):
        b, h = divmod(bh, H)
        np.testing.assert_array_equal(o_r[bh], o[b, h, rows[bh]])
        np.testing.assert_array_equal(lse_r[bh], lse[b, h, rows[bh]])


def test_rejects_bad_rows():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, q, 1.0, False, np.array([[4]]))
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, q, 1.0, False, np.array([[-1]]))


def test_empty_is_a_no_op():
    z = np.zeros((0, 2, 5, 4))
    o, lse = oracle.attention_fwd(z, z, z, 1.0, True)
    assert o.shape == (0, 2, 5, 4) and lse.shape == (0, 2, 5)


# ---------------------------------------------------------------- backward pass
# The backward oracle is pinned to the forward oracle through finite
# differences (no shared formula), to torch's float64 autograd, and to
# identities that a dropped term, a wrong sign or a transposed operand breaks.


def _bwd_inputs(seed, B=1, H=2, N=6, d=4):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_finite_differences(causal):
    """dL/dx for L = sum(dO * O) by central differences of the forward oracle."""
    q, k, v, do = _bwd_inputs(3, B=1, H=1, N=5, d=3)
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_fwd(q_, k_, v_, scale, causal)
        return float((o * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.125, 0.5, 2.0])
def test_bwd_matches_torch_autograd(causal, scale):
    q, k, v, do = _bwd_inputs(4, B=2, H=2, N=9, d=8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    o.backward(torch.tensor(do))
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_delta_is_rowsum_do_o(causal):
    """D_i = sum_j P_ij dP_ij equals sum_t dO_it O_it (O from the forward)."""
    q, k, v, do = _bwd_inputs(5, N=11, d=6)
    _, _, _, delta = oracle.attention_bwd(q, k, v, do, 0.4, causal, return_delta=True)
    o, _ = oracle.attention_fwd(q, k, v, 0.4, causal)
    np.testing.assert_allclose(delta, (do * o).sum(-1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dk_sums_to_zero_over_keys(causal):
    """Each row of dS sums to 0 (softmax Jacobian), so sum_j dK_j = 0."""
    q, k, v, do = _bwd_inputs(6, N=10, d=5)
    _, dk, dv = oracle.attention_bwd(q, k, v, do, 0.6, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # and dV collects every row's weight once: sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_bwd_closed_forms():
    # N = 1: P = 1, so dS = 0 and dV = dO
    q, k, v, do = _bwd_inputs(7, N=1, d=4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, True)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, do, atol=0)
    # scale 0: uniform weights, dQ = dK = 0, dV_j = sum over the rows that see
    # key j of dO_i / (number of keys row i sees)
    q, k, v, do = _bwd_inputs(8, N=7, d=3)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.0, causal)
        assert np.all(dq == 0) and np.all(dk == 0)
        N = q.shape[2]
        expect = np.zeros_like(dv)
        for i in range(N):
            n_vis = i + 1 if causal else N
            for j in range(n_vis):
                expect[:, :, j] += do[:, :, i] / n_vis
        np.testing.assert_allclose(dv, expect, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sampled_matches_torch_autograd_and_full(causal):
    """The sampled backward (D from dO . O, P from lse) against torch's float64
    autograd and the materializing backward, on every head or a subset."""
    q, k, v, do = _bwd_inputs(9, B=2, H=3, N=37, d=8)
    scale = 0.35
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    o.backward(torch.tensor(do))
    full = oracle.attention_bwd(q, k, v, do, scale, causal)
    heads = np.array([0, 4, 5])
    qrows = np.array([[0, 1, 36], [5, 17, 36], [2, 3, 30]])
    krows = np.array([[0, 20, 36], [0, 1, 2], [36, 35, 9]])
    dq, dk, dv = oracle.attention_bwd_sampled(q, k, v, do, scale, causal, heads, qrows, krows)
    tg = [t.grad.numpy().reshape(6, 37, 8) for t in (tq, tk, tv)]
    fg = [g.reshape(6, 37, 8) for g in full]
    for x, h in enumerate(heads):
        for ref in (tg, fg):
            np.testing.assert_allclose(dq[x], ref[0][h, qrows[x]], atol=1e-12, rtol=1e-10)
            np.testing.assert_allclose(dk[x], ref[1][h, krows[x]], atol=1e-12, rtol=1e-10)
            np.testing.assert_allclose(dv[x], ref[2][h, krows[x]], atol=1e-12, rtol=1e-10)
    with pytest.raises(ValueError):
        oracle.attention_bwd_sampled(q, k, v, do, scale, causal, [6], [0], [0])
    with pytest.raises(ValueError):
        oracle.attention_bwd_sampled(q, k, v, do, scale, causal, [0], [37], [0])


# ---------------------------------------------------------------- FP8 E4M3 decoding
def test_decode_e4m3_matches_torch_for_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.decode_e4m3(codes), ref)
    np.testing.assert_array_equal(oracle.decode_e4m3(codes, 0.5), ref * 0.5)


def test_decode_e4m3_closed_forms():
    got = oracle.decode_e4m3(np.array([0x38, 0x7E, 0x01, 0x08, 0x00, 0x80, 0xB8, 0x39, 0x07],
                                      dtype=np.uint8))
    assert list(got) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 0.0, -0.0, -1.0, 1.125,
                         7 * 2.0 ** -9]
    with pytest.raises(ValueError):
        oracle.decode_e4m3(np.array([0x7F], dtype=np.uint8))


def test_attention_fwd_fp8_is_attention_of_decoded_inputs():
    rng = np.random.default_rng(11)
    codes = [rng.integers(0, 0x7E, size=(1, 2, 9, 4)).astype(np.uint8) |
             (rng.integers(0, 2, size=(1, 2, 9, 4)).astype(np.uint8) << 7) for _ in range(3)]
    o, lse = oracle.attention_fwd_fp8(*codes, 0.01, 0.02, 0.5, 0.7, True)
    deq = [torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64) * s
           for c, s in zip(codes, (0.01, 0.02, 0.5))]
    ref = torch.nn.functional.scaled_dot_product_attention(*deq, is_causal=True, scale=0.7)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=1e-10)


# ---------------------------------------------------------------- decode over a paged KV cache
def _decode_case(seed=3, B=3, H=4, H_kv=2, d=8, ps=4, max_pages=6):
    from io_aware_tiled_09_amd.inputs import make_decode
    return make_decode("decode_small", fill_unused=0.0, seed=seed, B=B, H=H, H_kv=H_kv, d=d,
                       page_size=ps, max_context=ps * max_pages, min_len=1,
                       max_len_draw=ps * max_pages, spare_pages=5)


def _gather(c, table, L, ps):
    rows = [c[int(table[t // ps]), :, t % ps, :] for t in range(L)]
    return torch.stack(rows, dim=1).double()  # [H_kv, L, d]


def test_decode_paged_matches_torch_sdpa_on_gathered_rows():
    x = _decode_case()
    q, kc, vc, pt, sl = x["q"], x["k_cache"], x["v_cache"], x["page_table"], x["seq_lens"]
    w = x["workload"]
    o, lse = oracle.decode_paged(q, kc, vc, pt, sl, 0.35)
    for b in range(w.B):
        L = int(sl[b])
        K = _gather(kc, pt[b], L, w.page_size).repeat_interleave(w.H // w.H_kv, dim=0)
        V = _gather(vc, pt[b], L, w.page_size).repeat_interleave(w.H // w.H_kv, dim=0)
        qb = q[b].double()[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, K, V, scale=0.35)[:, 0]
        np.testing.assert_allclose(o[b], ref.numpy(), atol=1e-12, rtol=1e-10)
        lref = torch.logsumexp(0.35 * (qb @ K.transpose(-1, -2))[:, 0], dim=-1)
        np.testing.assert_allclose(lse[b], lref.numpy(), atol=1e-12, rtol=1e-12)


def test_decode_paged_page_permutation_invariance():
    x = _decode_case(seed=4)
    o, lse = oracle.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["page_table"],
                                 x["seq_lens"], 0.5)
    n = x["k_cache"].shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9))
    inv = torch.argsort(perm)
    pt = x["page_table"].clone()
    pt[pt >= 0] = inv[pt[pt >= 0].long()].to(torch.int32)
    o2, lse2 = oracle.decode_paged(x["q"], x["k_cache"][perm], x["v_cache"][perm], pt,
                                   x["seq_lens"], 0.5)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_paged_gqa_equals_repeated_kv_heads():
    x = _decode_case(seed=5, H=4, H_kv=2)
    o, lse = oracle.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["page_table"],
                                 x["seq_lens"], 0.3)
    rep = lambda c: c.repeat_interleave(2, dim=1)  # noqa: E731
    o2, lse2 = oracle.decode_paged(x["q"], rep(x["k_cache"]), rep(x["v_cache"]),
                                   x["page_table"], x["seq_lens"], 0.3)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_paged_closed_forms_and_errors():
    x = _decode_case(seed=6)
    sl = torch.ones_like(x["seq_lens"])
    o, lse = oracle.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["page_table"], sl, 0.7)
    w = x["workload"]
    for b in range(w.B):
        p0 = int(x["page_table"][b, 0])
        for h in range(w.H):
            k0 = x["k_cache"][p0, h // (w.H // w.H_kv), 0].double().numpy()
            v0 = x["v_cache"][p0, h // (w.H // w.H_kv), 0].double().numpy()
            np.testing.assert_allclose(o[b, h], v0, atol=1e-15)
            np.testing.assert_allclose(lse[b, h], 0.7 * x["q"][b, h].double().numpy() @ k0,
                                       atol=1e-12)
    bad = x["page_table"].clone()
    bad[0, 0] = x["k_cache"].shape[0]
    with pytest.raises(ValueError):
        oracle.decode_paged(x["q"], x["k_cache"], x["v_cache"], bad, x["seq_lens"], 0.7)
    with pytest.raises(ValueError):
        oracle.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["page_table"],
                            torch.zeros_like(x["seq_lens"]), 0.7)
