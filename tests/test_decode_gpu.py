"""GPU parity of decode-step attention over a paged KV cache (fa_decode_paged
through the C ABI) against the fp64 oracle (oracle.decode_paged).

Bound, per element, from the kernel's arithmetic: bf16 inputs, exact
products summed in fp32, an fp32 online softmax and fp32 accumulation of the
weighted V rows (the partial states of 16-key groups and 512-key runs merged
with the two-correction-factor merge), O rounded to bf16:
    |O_gpu - O| <= 2^-8 |O| + 2^-12 A + 1e-6,  A_t = sum_j P_j |V_jt|
(2^-8: the bf16 rounding of O; 2^-12 A: fp32 summation over up to 8K terms,
with A from the oracle run on |V|); lse within 1e-5 relative (fp32). An
fp32 model of the kernels' exact order of operations (tests/_emulate.py:
decode_row) reaches 0.631 to 0.879 of the bound on the sixteen small cases
below, the GPU's figures to the digit (tests/test_bounds.py:
test_decode_bound_model). Cache rows no sequence owns are NaN, so any read of
them would show."""
import math

import numpy as np
import pytest
import torch

import io_aware_tiled_09_amd as fa
import oracle
from io_aware_tiled_09_amd.inputs import make_decode

from _parity import say

pytestmark = pytest.mark.gpu


def run_decode(x, scale):
    g = {k: x[k].to("cuda:0") for k in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    o, lse = fa.decode_paged(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                             scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(x, scale, label):
    o, lse = run_decode(x, scale)
    args = (x["q"], x["k_cache"], x["v_cache"], x["page_table"], x["seq_lens"], scale)
    o_ref, lse_ref = oracle.decode_paged(*args)
    vabs = torch.nan_to_num(x["v_cache"].float(), nan=0.0).abs()
    kz = torch.nan_to_num(x["k_cache"].float(), nan=0.0)
    a_ref, _ = oracle.decode_paged(x["q"], kz, vabs, x["page_table"], x["seq_lens"], scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    d = np.abs(o - o_ref)
    bound = 2.0 ** -8 * np.abs(o_ref) + 2.0 ** -12 * a_ref + 1e-6
    lrel = float((np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max())
    say(f"  {label}: max|dO|={d.max():.3e} mean|dO|={d.mean():.3e} max |dO|/bound="
        f"{(d / bound).max():.3f} lse rel={lrel:.3e}")
    assert (d <= bound).all(), np.unravel_index(int((d / bound).argmax()), d.shape)
    assert lrel <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (4, 2), (8, 2), (8, 1)])
@pytest.mark.parametrize("page_size", [16, 64])
def test_decode_small(d, H, H_kv, page_size):
    say(f"decode small d={d} H={H} H_kv={H_kv} page_size={page_size}")
    x = make_decode("decode_small", d=d, H=H, H_kv=H_kv, page_size=page_size,
                    seed=100 + d + 10 * H + H_kv + page_size)
    check(x, 1.0 / math.sqrt(d), f"d={d} H={H}/{H_kv} ps={page_size}")


def test_decode_split_boundaries():
    """Lengths around the 16-key row blocks, the unrolled steps (64 and 128
    keys) and the 512-key runs."""
    say("decode split boundaries")
    lens = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1023, 1024]
    x = make_decode("decode_small", B=len(lens), H=4, H_kv=4, seed=7, max_context=1024)
    w = x["workload"]
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    # re-own rows: the generator marked rows past its own lengths NaN; rebuild
    # the caches as finite everywhere the new lengths can reach
    x["k_cache"] = torch.nan_to_num(x["k_cache"].float(), nan=0.25).to(torch.bfloat16)
    x["v_cache"] = torch.nan_to_num(x["v_cache"].float(), nan=-0.5).to(torch.bfloat16)
    need = [(L + w.page_size - 1) // w.page_size for L in lens]
    pool = torch.randperm(x["k_cache"].shape[0], generator=torch.Generator().manual_seed(3))
    if sum(need) > pool.numel():
        pytest.skip("pool too small for the chosen lengths")
    table = torch.full((len(lens), w.max_pages), -1, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = pool[at:at + n].to(torch.int32)
        at += n
    x["page_table"] = table
    check(x, 0.2, "split boundaries")


@pytest.mark.parametrize("name", ["decode50", "decode50_gqa"])
def test_decode_workloads(name):
    say(f"decode workload {name}")
    x = make_decode(name)
    check(x, x["workload"].scale, name)


def test_decode_empty_and_unmapped_sequences():
    say("decode: seq_len 0 and a sequence whose pages are all unmapped")
    x = make_decode("decode_small", B=3, seed=11)
    x["seq_lens"] = torch.tensor([0, 40, 5], dtype=torch.int32)
    x["page_table"][1, :] = -1
    x["page_table"][2, 0] = 1 << 30
    o, lse = run_decode(x, 0.1)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_decode_deterministic_bitwise():
    say("decode determinism")
    x = make_decode("decode_small", seed=12)
    a = run_decode(x, 0.1)
    b = run_decode(x, 0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
