"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on
the same inputs, compare within the stated bound.

Bound (floating point): on O, max |GPU - oracle| <= 2e-2 and mean
|GPU - oracle| <= 2e-3; on lse, |GPU - oracle| / max(|oracle|, 1) <= 1e-3.
"""
import sys

import numpy as np
import torch

import io_aware_tiled_09_amd as fa
import oracle

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_REL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, causal, scale):
    """Copy CPU inputs to cuda:0, run the library, return CPU (o fp64, lse fp64)."""
    dq, dk, dv = (t.to("cuda:0") for t in (q, k, v))
    o, lse = fa.attention(dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.double().cpu(), lse.double().cpu()


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    d = np.abs(o_gpu - o_ref)
    lrel = np.abs(lse_gpu - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    assert np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all(), "non-finite GPU output"
    return dict(o_max=float(d.max()), o_mean=float(d.mean()), lse_rel=float(lrel.max()),
                o_worst=np.unravel_index(int(d.argmax()), d.shape))


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, label=""):
    e = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    say(f"  {label}: max|dO|={e['o_max']:.3e} mean|dO|={e['o_mean']:.3e} "
        f"lse rel={e['lse_rel']:.3e} worst O at {e['o_worst']}")
    assert e["o_max"] <= O_MAX_ABS, e
    assert e["o_mean"] <= O_MEAN_ABS, e
    assert e["lse_rel"] <= LSE_REL, e
    return e


def check_full(q, k, v, causal, scale, label=""):
    """Whole-output parity against the materializing oracle."""
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, causal)
    o_gpu, lse_gpu = run_gpu(q, k, v, causal, scale)
    return assert_close(o_gpu.numpy(), lse_gpu.numpy(), o_ref, lse_ref, label)


def check_rows(q, k, v, causal, scale, rows, label=""):
    """Parity on sampled query rows (rows: int64 [B*H, R])."""
    o_gpu, lse_gpu = run_gpu(q, k, v, causal, scale)
    B, H, N, d = q.shape
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, causal, rows)
    r = torch.as_tensor(rows)
    og = o_gpu.reshape(B * H, N, d)
    lg = lse_gpu.reshape(B * H, N)
    idx = r.unsqueeze(-1).expand(-1, -1, d)
    og_s = torch.gather(og, 1, idx).numpy()
    lg_s = torch.gather(lg, 1, r).numpy()
    return assert_close(og_s, lg_s, o_ref, lse_ref, label)
