#!/usr/bin/env python3
"""Benchmark of the FlashAttention forward (default) or backward pass on one MI355X.

One step = one forward call (every step of the hot path runs inside the one
kernel launch) over the long-document causal workload: B=2, H=32, N=8192,
d=128, bf16, scale 1/sqrt(128), seeded synthetic N(0,1) inputs already
resident in HBM. Prints one JSON line on stdout; progress goes to stderr.

Timing: the same-box GEMM reference (bf16 fwd/bwd passes; it also takes the
board through the clock dip that follows idle), W untimed warm-up calls,
then K calls bracketed by synchronizations,
with HIP events recorded around every launch on the stream the kernel is
launched on (torch's current stream, which the binding passes to fa_fwd).
`value` is useful TFLOP/s over the K calls (4*B*H*N^2*d, halved for causal).
The CPU baseline times the fp64 oracle on a bounded sample (whole heads of
the same workload) on this host's cores.

With --pass std one step is the standard, materializing forward
(libfa_std.so: S = scale QK^T to HBM by rocBLAS, the row softmax kernel,
O = PV by rocBLAS) on the same workload; `value` counts the same useful
FLOPs as the flash forward, and the roofline object is the softmax kernel's
(HBM-bound: visible fp32 scores read, bf16 P written).

With --pass fp8 one step is one FP8 forward call (fa_fwd_fp8) on the same
workload's draws quantized per tensor to E4M3; `value` counts the same useful
FLOPs and the roofline peak is the FP8 MFMA rate (5.0 PFLOP/s dense).

With --pass bwd one step is one backward call (fa_bwd: the D, dK/dV and dQ
kernels) on the same workload with a seeded N(0,1) dO, O and lse from one
forward call made before timing; `value` is useful backward TFLOP/s
(2.5 times the forward's FLOPs: S recomputed, dP, dV, dQ, dK).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILES = {"fwd": os.path.join(ROOT, "profiles", "hbm_traffic_longdoc8k.json"),
                 "bwd": os.path.join(ROOT, "profiles", "hbm_traffic_longdoc8k_bwd.json"),
                 "std": os.path.join(ROOT, "profiles", "hbm_traffic_longdoc8k_std.json"),
                 "fp8": os.path.join(ROOT, "profiles", "hbm_traffic_longdoc8k_fp8.json"),
                 "decode": os.path.join(ROOT, "profiles", "hbm_traffic_decode50.json")}
# Sources each pass's kernels are compiled from (the traffic summary is valid
# only for the exact sources it was taken on).
PASS_SOURCES = {"fwd": ("fa_common.h", "fa_lds.h", "fa_fwd_bf16.hip"),
                "bwd": ("fa_common.h", "fa_lds.h", "fa_bwd_bf16.hip"),
                "std": ("fa_common.h", "fa_std.hip"),
                "fp8": ("fa_common.h", "fa_lds.h", "fa_fwd_fp8.hip"),
                "decode": ("fa_common.h", "fa_decode.hip")}
# Kernel names (substrings) rocprofv3 reports for each pass.
PASS_KERNELS = {"fwd": ("fa_fwd_bf16_kernel",),
                "bwd": ("fa_bwd_delta_kernel", "fa_bwd_dkdv_kernel", "fa_bwd_dq_phased_kernel"),
                "std": ("fa_std_softmax",),
                "fp8": ("fa_fwd_fp8_kernel",),
                "decode": ("fa_decode_split_kernel", "fa_decode_merge_kernel")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest(pass_: str = "fwd") -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "io_aware_tiled_09_amd", "csrc")
    for name in PASS_SOURCES[pass_]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(digest: str, pass_: str = "fwd", workload: str = ""):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it
    was taken on this exact kernel source and workload; else None."""
    try:
        with open(TRAFFIC_FILES[pass_]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != digest:
        return None
    if workload and t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def _counter_means(path, counter):
    """Mean counter value per kernel name, over the dispatches with that
    kernel's largest grid (so that the 1 GiB calibration copy is not averaged
    with small runtime copies of the same blit kernel)."""
    import csv
    by_kernel = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                by_kernel.setdefault(r["Kernel_Name"], []).append(
                    (int(r.get("Grid_Size") or 0), float(r["Counter_Value"])))
    out = {}
    for k_, v_ in by_kernel.items():
        g = max(x[0] for x in v_)
        vals = [x[1] for x in v_ if x[0] == g]
        out[k_] = sum(vals) / len(vals)
    return out


def ingest_counters(fetch_csv, write_csv, copy_mib, command, pass_="fwd"):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch) of `command` into HBM bytes per attention call (the sum over the
    pass's kernels), each counter scaled by what it reads for the plain device
    copy of copy_mib MiB that the same command runs (its true traffic is
    copy_mib MiB read + written)."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")

    def pick(table, needle):
        hits = [v_ for k_, v_ in table.items() if needle in k_]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {needle!r}, found {len(hits)}")
        return hits[0]

    copy = "copyBuffer"
    true_kib = copy_mib * 1024.0
    f_fetch = true_kib / pick(fetch, copy)
    f_write = true_kib / pick(write, copy)
    per_kernel = {}
    for name in PASS_KERNELS[pass_]:
        fk, wk = pick(fetch, name), pick(write, name)
        per_kernel[name] = {"fetch_kib_raw": fk, "write_kib_raw": wk,
                            "hbm_bytes": round((fk * f_fetch + wk * f_write) * 1024.0)}
    fetch_kib = sum(x["fetch_kib_raw"] for x in per_kernel.values())
    write_kib = sum(x["write_kib_raw"] for x in per_kernel.values())
    traffic = (fetch_kib * f_fetch + write_kib * f_write) * 1024.0
    out = {
        "kernel_source_digest": kernel_source_digest(pass_),
        "workload": "decode50" if pass_ == "decode" else "longdoc8k",
        "pass": pass_,
        "hbm_bytes_per_launch": round(traffic),
        "fetch_kib_raw": fetch_kib,
        "write_kib_raw": write_kib,
        "per_kernel": per_kernel,
        "copy_kib_true": true_kib,
        "fetch_scale": f_fetch,
        "write_scale": f_write,
        "command": command,
    }
    with open(TRAFFIC_FILES[pass_], "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def gemm_reference(torch, stream, n=8192, iters=20, warmup=30):
    """Same-box reference for the MFMA rate: torch's bf16 GEMM (hipBLASLt) at
    n^3, timed with HIP events on the bench stream. The 2.5 PFLOP/s datasheet
    peak assumes a 2.4 GHz engine clock that dense MFMA work does not hold on
    these boards; this number says what a vendor GEMM reaches on the same
    GPU in the same run. It runs before the pass's warm-up calls: the engine
    clock dips and recovers over the first few tens of milliseconds of dense
    MFMA work after a pause (forward launches 6-25 after an idle GPU run ~8%
    slower than launches 40-60), and its 50 GEMMs (~40 ms) take the board
    through that dip, so the timed calls see the clock the step holds under
    sustained load whatever --warmup is. The GEMM gets 30 warm-up calls
    itself. The caller adds kernel_over_reference."""
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            c = a @ b
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            c = a @ b
        e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    log(f"reference bf16 GEMM {n}^3: {ms:.4f} ms -> {tflops:.1f} TFLOP/s")
    return {"what": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), same GPU and run, "
                    "timed before the pass's warm-up calls",
            "tflops": round(tflops, 1), "ms": round(ms, 4)}


def parse_engine_clock(text):
    """Engine clock in MHz from the text of a `pp_dpm_sclk` file (one line
    per clock level, the current one marked with '*'), or None."""
    import re
    for line in text.splitlines():
        if "*" in line:
            m = re.search(r"(\d+)\s*Mhz", line, re.I)
            if m:
                return int(m.group(1))
    return None


def gpu_sysfs_dir(torch):
    """sysfs directory of the GPU that torch calls cuda:0 (its PCI device
    directory, which holds the kernel driver's pp_dpm_sclk and hwmon files),
    or the only DRM card's device directory when the address is not there,
    else None."""
    import glob
    import os
    try:
        pr = torch.cuda.get_device_properties(0)
        addr = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        path = f"/sys/bus/pci/devices/{addr}"
        if os.path.exists(os.path.join(path, "pp_dpm_sclk")):
            return path
    except (AttributeError, RuntimeError):
        pass
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return os.path.dirname(paths[0]) if len(paths) == 1 else None


def _read_microwatts(dev_dir, name):
    """A hwmon power file of the device in W (the files hold microwatts), or
    None."""
    import glob
    if dev_dir is None:
        return None
    for path in sorted(glob.glob(f"{dev_dir}/hwmon/hwmon*/{name}")):
        try:
            with open(path) as f:
                return int(f.read().strip()) / 1e6
        except (OSError, ValueError):
            continue
    return None


def engine_clock_sample(dev_dir):
    """(engine clock MHz, board power W) of the GPU under `dev_dir`, read from
    the kernel driver's sysfs files (pp_dpm_sclk; hwmon power1_average, else
    power1_input): plain file reads, with no subprocess, so nothing is
    started from this process, which has initialised the GPU. None for what
    cannot be read."""
    if dev_dir is None:
        return None, None
    try:
        with open(f"{dev_dir}/pp_dpm_sclk") as f:
            mhz = parse_engine_clock(f.read())
    except OSError:
        mhz = None
    watts = _read_microwatts(dev_dir, "power1_average")
    if watts is None:
        watts = _read_microwatts(dev_dir, "power1_input")
    return mhz, watts


def power_cap_watts(dev_dir):
    """The board's power cap in W (hwmon power1_cap), or None."""
    return _read_microwatts(dev_dir, "power1_cap")


def sustained_run(torch, stream, call, seconds, ms_hint):
    """Run `call` back to back on `stream` for about `seconds`, keeping the
    queue full, while a thread samples the engine clock every ~0.5 s. Returns
    the mean ms per call over the second half of the run (HIP events) and the
    median clock and board power of the samples taken in that half, with the
    board's power cap."""
    import statistics
    import threading
    chunk = max(1, int(0.1 / max(ms_hint * 1e-3, 1e-6)))  # ~0.1 s of work per chunk
    nchunks = max(6, int(seconds / 0.1))
    samples, stop = [], threading.Event()
    half = threading.Event()
    dev_dir = gpu_sysfs_dir(torch)

    def sampler():
        while not stop.is_set():
            clk, pw = engine_clock_sample(dev_dir)
            if half.is_set():
                samples.append((clk, pw))
            stop.wait(0.5)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    evs = []
    with torch.cuda.stream(stream):
        for c in range(nchunks):
            for _ in range(chunk):
                call()
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            evs.append(ev)
            if c >= 3:
                evs[c - 3].synchronize()  # at most ~0.3 s of work queued ahead
            if c == nchunks // 2:
                half.set()
    evs[-1].synchronize()
    stop.set()
    th.join()
    mid = nchunks // 2
    ms = evs[mid].elapsed_time(evs[-1]) / ((nchunks - 1 - mid) * chunk)
    clks = [c for c, _ in samples if c is not None]
    pws = [p for _, p in samples if p is not None]
    return {"seconds": round(seconds, 1), "calls_timed": (nchunks - 1 - mid) * chunk,
            "ms_per_call": round(ms, 5),
            "sclk_mhz": statistics.median(clks) if clks else None,
            "power_w": statistics.median(pws) if pws else None,
            "power_cap_w": power_cap_watts(dev_dir), "clock_samples": len(clks)}


def sustained_reference(torch, stream, step, seconds, ms_hint, flops, peak, gemm):
    """--sustained: the pass's step back to back for `seconds` (timed over the
    second half, engine clock sampled), then torch's 8192^3 bf16 GEMM the same
    way when `gemm`. The datasheet peaks assume 2.4 GHz; `peak_at_clock`
    scales the peak to the clock the step actually ran at."""
    log(f"sustained run: {seconds:.1f} s of back-to-back calls, engine clock sampled ...")
    r = sustained_run(torch, stream, step, seconds, ms_hint)
    r["tflops"] = round(flops / (r["ms_per_call"] * 1e-3) / 1e12, 1)
    if r["sclk_mhz"]:
        r["peak_at_clock"] = round(peak * r["sclk_mhz"] / 2400.0, 1)
        r["frac_at_clock"] = round(r["tflops"] / r["peak_at_clock"], 4)
    log(f"sustained: {r['ms_per_call']:.4f} ms per call, {r['tflops']} TFLOP/s, "
        f"engine clock {r['sclk_mhz']} MHz, power {r['power_w']} W")
    if gemm:
        n = 8192
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        out = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        rg = sustained_run(torch, stream, lambda: torch.matmul(a, b, out=out), seconds, 1.0)
        rg["tflops"] = round(2.0 * n ** 3 / (rg["ms_per_call"] * 1e-3) / 1e12, 1)
        rg["what"] = f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)"
        log(f"sustained GEMM: {rg['tflops']} TFLOP/s, engine clock {rg['sclk_mhz']} MHz, "
            f"power {rg['power_w']} W")
        r["gemm"] = rg
        del a, b, out
    return r


def hbm_reference(torch, stream, achieved_gbs, mib=1024, iters=10):
    """Same-box reference for the HBM rate: torch's device copy of `mib` MiB
    (bytes read + written), timed with HIP events on the bench stream after
    the timed region."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            dst.copy_(src)
        e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / iters
    gbs = 2.0 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    log(f"reference device copy {mib} MiB: {ms:.4f} ms -> {gbs:.0f} GB/s")
    return {"what": f"torch device copy of {mib} MiB (read + write), same GPU and run",
            "gbs": round(gbs, 1), "ms": round(ms, 4),
            "kernel_over_reference": round(achieved_gbs / gbs, 4)}


def cpu_baseline(w, q, k, v, budget_s: float, fp8=None):
    """Time the oracle over whole heads of the workload until about budget_s.
    fp8: ((q8, k8, v8), (q_scale, k_scale, v_scale)) to time the oracle on the
    decoded 8-bit inputs instead."""
    import oracle
    B, H, N, d = q.shape
    heads, elapsed = 0, 0.0
    t_start = time.perf_counter()
    while heads < B * H and elapsed < budget_s:
        b, h = divmod(heads, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        if fp8 is None:
            oracle.attention_fwd(q[sl], k[sl], v[sl], w.scale, w.causal)
        else:
            (q8, k8, v8), sc = fp8
            oracle.attention_fwd_fp8(q8[sl], k8[sl], v8[sl], *sc, w.scale, w.causal)
        elapsed += time.perf_counter() - t0
        heads += 1
        log(f"  oracle head {heads}: {elapsed:.1f} s")
    from io_aware_tiled_09_amd.inputs import useful_flops
    flops = useful_flops(1, heads, N, d, w.causal)
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{heads} of {B * H} heads (all {N} query rows each) of {w.name}"
                  f"{' (decoded FP8 inputs)' if fp8 is not None else ''}, "
                  f"fp64 with S and P materialized; useful FLOPs of the sample / "
                  f"{elapsed:.1f} s wall (incl. the fp64 upcast: {time.perf_counter() - t_start:.1f} s)",
    }


def cpu_baseline_bwd(w, q, k, v, do, budget_s: float):
    """Time the backward oracle over whole heads of the workload until about budget_s."""
    import oracle
    B, H, N, d = q.shape
    heads, elapsed = 0, 0.0
    while heads < B * H and elapsed < budget_s:
        b, h = divmod(heads, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        oracle.attention_bwd(q[sl], k[sl], v[sl], do[sl], w.scale, w.causal)
        elapsed += time.perf_counter() - t0
        heads += 1
        log(f"  backward oracle head {heads}: {elapsed:.1f} s")
    from io_aware_tiled_09_amd.inputs import backward_flops
    flops = backward_flops(1, heads, N, d, w.causal)
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{heads} of {B * H} heads (all {N} rows each) of {w.name}, fp64 backward "
                  f"with P and dS materialized; useful backward FLOPs of the sample / "
                  f"{elapsed:.1f} s wall",
    }


def bench_decode(args):
    """One step = one fa_decode_paged call (split + merge kernels) over the
    paged KV cache of a decode workload; value = algorithmic HBM bytes (every
    cached K and V row read once, q, o, lse) / time, in GB/s."""
    import torch
    import io_aware_tiled_09_amd as fa
    from io_aware_tiled_09_amd.inputs import DECODE_WORKLOADS, decode_kv_bytes, make_decode

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    fa.load()
    name = args.workload if args.workload in DECODE_WORKLOADS else "decode50"
    x = make_decode(name)
    w = x["workload"]
    dev = torch.device("cuda:0")
    g = {k: x[k].to(dev) for k in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    log(f"decode workload {name}: B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} page_size={w.page_size} "
        f"pages={g['k_cache'].shape[0]} mean len={float(x['seq_lens'].float().mean()):.0f}")
    need = fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.page_size, w.max_pages)
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    num_pages = g["k_cache"].shape[0]

    def step():
        st = fa.fa_decode_paged(g["q"], g["k_cache"], g["v_cache"], g["page_table"],
                                g["seq_lens"], o, lse, ws, need, w.B, w.H, w.H_kv, w.d,
                                num_pages, w.page_size, w.max_pages, w.scale, stream)
        if st != 0:
            raise fa.FAError(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    avg_ms = sum(per) / K
    span_ms = starts[0].elapsed_time(ends[-1]) / K
    nbytes = decode_kv_bytes(w, x["seq_lens"])
    value = nbytes / (span_ms * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    log(f"avg call {avg_ms:.4f} ms, span/step {span_ms:.4f} ms, {nbytes / 1e9:.3f} GB -> "
        f"{value:.0f} GB/s")
    if args.copy_kernel_mib > 0:
        n = args.copy_kernel_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy kernel: {args.copy_kernel_mib} MiB read + written, 3 times")
    digest = kernel_source_digest("decode")
    result = {
        "metric": "decode-step attention over a paged KV cache, GB/s of cache read (bf16, 1 MI355X)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(span_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "d": w.d,
                   "page_size": w.page_size, "max_context": w.max_context,
                   "tokens": int(x["seq_lens"].sum()), "seed": w.seed,
                   "algorithmic_bytes": nbytes, "pass": "decode"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(digest, "decode", name),
                     "avg_launch_ms": round(avg_ms, 5),
                     "kernels": list(PASS_KERNELS["decode"]), "kernel_source_digest": digest},
        "cpu_baseline": None,
    }
    if args.gemm_ref:
        result["hbm_reference"] = hbm_reference(torch, torch.cuda.current_stream(), achieved)
    if args.cpu_budget > 0:
        import oracle
        t0 = time.perf_counter()
        oracle.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["page_table"], x["seq_lens"],
                            w.scale)
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": nbytes / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole step ({w.B} sequences, {int(x['seq_lens'].sum())} tokens) "
                      f"in fp64, {el:.1f} s wall including the fp64 upcast of the cache"}
    print(json.dumps(result), flush=True)
    return 0


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_time(w, q, k, v, budget_s: float):
    """Wall time of the oracle on the whole workload: timed head by head until
    budget_s, then extrapolated by useful FLOPs. longctx32k (whose parity test
    samples rows) is timed on 256 sampled query rows per head the same way.
    Returns (seconds for the whole config, description)."""
    import oracle
    from io_aware_tiled_09_amd.inputs import sample_rows, useful_flops
    B, H, N, d = q.shape
    total = useful_flops(B, H, N, d, w.causal)
    done_flops, elapsed, heads = 0.0, 0.0, 0
    rows_mode = w.name == "longctx32k"
    while heads < B * H and (heads == 0 or elapsed < budget_s):
        b, h = divmod(heads, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        if rows_mode:
            r = sample_rows(N, 256, seed=77 + heads)
            oracle.attention_rows(q[sl], k[sl], v[sl], w.scale, w.causal, r)
            vis = (r + 1).double() if w.causal else torch_full(r, N)
            done_flops += float(4.0 * d * vis.sum())
        else:
            oracle.attention_fwd(q[sl], k[sl], v[sl], w.scale, w.causal)
            done_flops += useful_flops(1, 1, N, d, w.causal)
        elapsed += time.perf_counter() - t0
        heads += 1
    whole = elapsed * total / done_flops
    what = (f"{heads} of {B * H} heads" + (" x 256 sampled rows" if rows_mode else "")
            + f" in {elapsed:.2f} s" + ("" if done_flops >= total else ", extrapolated by FLOPs"))
    return whole, what


def torch_full(r, N):
    import torch
    return torch.full(r.shape, float(N), dtype=torch.float64)


def bench_table(args):
    """Every configuration of the forward: GPU time per call and TFLOP/s, the
    launch shape, and the oracle's wall time for the same config."""
    import torch
    import io_aware_tiled_09_amd as fa
    import oracle
    from io_aware_tiled_09_amd.inputs import WORKLOADS, make_qkv, useful_flops
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    fa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cpu = cpu_model()
    threads = oracle.num_threads()
    rows = []
    for name in ("single_head", "bert512", "gpt2_1k", "gpt2_1k_spiky", "longdoc8k", "longctx32k"):
        w = WORKLOADS[name]
        q, k, v = make_qkv(w)
        dq, dk, dv = (t.to(dev) for t in (q, k, v))
        o = torch.empty_like(dq)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32

        def step(on=None):
            st = fn(dq, dk, dv, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal, on or stream)
            if st != 0:
                raise fa.FAError(st)
        for _ in range(args.warmup):
            step()
        K = args.steps
        flops = useful_flops(w.B, w.H, w.N, w.d, w.causal)

        def median_of_5(run):
            reps = []
            for _ in range(5):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                run()
                e1.record(stream)
                e1.synchronize()
                reps.append(e0.elapsed_time(e1) / K)
            return sorted(reps)[2]

        # (1) K calls back to back between two events: the host enqueues as
        # fast as it can, and for kernels of a few microseconds the GPU may
        # wait on it between calls.
        stream_ms = median_of_5(lambda: [step() for _ in range(K)])
        # (2) the same K calls captured once in a HIP graph and replayed: the
        # device time per call without host launch gaps.
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for _ in range(K):
                    step(cap)
        torch.cuda.synchronize()
        graph_ms = median_of_5(g.replay)
        del g
        best_ms = min(stream_ms, graph_ms)
        if w.dtype == "bf16":
            grid, rows_per_block, paired = fa.fa_fwd_grid(w.B, w.H, w.N, w.causal)
            shape = f"{grid} WGs x {rows_per_block} rows" + (", paired" if paired else "")
            peak = PEAK_BF16_TFLOPS
        else:
            grid = w.B * w.H * ((w.N + 127) // 128)
            shape = f"{grid} WGs x 128 rows (fp32 kernel: 3 bf16 MFMAs per product)"
            peak = round(PEAK_BF16_TFLOPS / 3, 1)
        ora_s, ora_what = oracle_time(w, q, k, v, args.cpu_budget if args.cpu_budget > 0 else 15.0)
        row = {"workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
               "dtype": w.dtype, "launch": shape,
               "us_stream": round(stream_ms * 1e3, 2), "us_graph": round(graph_ms * 1e3, 2),
               "tflops": round(flops / (best_ms * 1e-3) / 1e12, 1),
               "pct_of_peak": round(100.0 * flops / (best_ms * 1e-3) / 1e12 / peak, 2),
               "peak": peak, "oracle_s": round(ora_s, 3), "oracle_timed": ora_what,
               "oracle_over_gpu": round(ora_s / (best_ms * 1e-3), 0)}
        log(f"{name}: {row['us_stream']} us/call in a stream, {row['us_graph']} us in a graph, "
            f"{row['tflops']} TFLOP/s ({shape}); oracle {ora_s:.2f} s ({ora_what})")
        print(json.dumps(row), flush=True)
        rows.append(row)
        del dq, dk, dv, o, lse
    print("| config | shape | launch | us / call, stream | us / call, graph | TFLOP/s | "
          "% of peak | oracle wall | oracle / GPU |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['workload']} | B{r['B']} H{r['H']} N{r['N']} d{r['d']} "
              f"{'causal' if r['causal'] else 'full'} {r['dtype']} | {r['launch']} | "
              f"{r['us_stream']} | {r['us_graph']} | {r['tflops']} | {r['pct_of_peak']} | "
              f"{r['oracle_s']} s ({r['oracle_timed']}) | {int(r['oracle_over_gpu'])}x |")
    print(f"\nOracle: {threads} threads on {cpu} (model name from /proc/cpuinfo); TFLOP/s "
          f"and % of peak from the faster of the two timings; useful FLOPs = 4 N^2 d B H "
          f"(halved when causal).")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)  # the engine clock settles over the first ~20 launches
    ap.add_argument("--workload", default="longdoc8k")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd", "std", "fp8", "decode"),
                    default="fwd",
                    help="fwd: one step = one forward call (the default line); bwd: one "
                         "step = one backward call (fa_bwd) given O and lse; std: one step = "
                         "the standard materializing forward (S and P through HBM); fp8: one "
                         "step = one FP8 (E4M3) forward call (fa_fwd_fp8); decode: one step = "
                         "one decode step over a paged KV cache (fa_decode_paged, --workload "
                         "decode50 by default)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--gemm-ref", type=int, default=1,
                    help="time a same-box reference on the same stream: torch's bf16 GEMM "
                         "(8192^3, hipBLASLt) before the warm-up calls of the fwd/bwd passes "
                         "(MFMA rate the chip sustains; it also takes the board through the "
                         "clock dip after idle), torch's 1 GiB device copy after the timed "
                         "region of the std and decode passes (HBM rate); 0 = skip")
    ap.add_argument("--sustained", type=float, default=3.0,
                    help="after the timed region, run the step back to back for this many "
                         "seconds with the engine clock sampled from sysfs (and, for the "
                         "bf16 passes, torch's 8192^3 GEMM the same way): the rate and the "
                         "clock under sustained load, beside the K timed calls; 0 = skip")
    ap.add_argument("--copy-kernel-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB 3 times "
                         "(reference kernel for HBM counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: write the HBM traffic summary from two rocprofv3 "
                         "counter CSVs of a run made with --copy-kernel-mib")
    ap.add_argument("--profile-command", default="",
                    help="with --ingest-counters: the command line the counters came from")
    ap.add_argument("--table", action="store_true",
                    help="every forward configuration (single_head .. longctx32k): GPU time "
                         "per call, TFLOP/s, launch shape and the oracle's wall time for the "
                         "same config (--cpu-budget seconds per config, then extrapolated), "
                         "one JSON line each and a markdown table")
    args = ap.parse_args(argv)
    if args.ingest_counters:
        return ingest_counters(*args.ingest_counters, args.copy_kernel_mib or 1024,
                               args.profile_command, args.pass_)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this attention forward has no "
              "multi-GPU path (each (batch, head) is independent; see the sharding "
              "notes in the design document).", file=sys.stderr)
        return 2

    if args.pass_ == "decode":
        return bench_decode(args)
    if args.table:
        return bench_table(args)

    import torch
    import io_aware_tiled_09_amd as fa
    from io_aware_tiled_09_amd.inputs import (WORKLOADS, backward_flops, make_dout, make_qkv,
                                              useful_flops)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    fa.load()  # fail loudly if the HIP library is not built
    w = WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} {w.dtype}")
    q, k, v = make_qkv(w)
    dev = torch.device("cuda:0")
    dq, dk, dv = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32
    bwd = args.pass_ == "bwd"
    if bwd and w.dtype != "bf16":
        print("the backward pass takes bf16 storage only", file=sys.stderr)
        return 2

    def fwd_step():
        st = fn(dq, dk, dv, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal, stream)
        if st != 0:
            raise fa.FAError(st)

    fp8 = args.pass_ == "fp8"
    stdp = args.pass_ == "std"
    std_sm = None  # (start, end) event pairs around the softmax launches
    if fp8:
        from io_aware_tiled_09_amd.inputs import make_qkv_fp8
        if w.d != 128:
            print("the FP8 forward takes d = 128 only", file=sys.stderr)
            return 2
        (q8, k8, v8), (qs, ks, vs) = make_qkv_fp8(w)
        g8 = [t.to(dev) for t in (q8, k8, v8)]
        del dq, dk, dv

        def step():
            st = fa.fa_fwd_fp8(*g8, o, lse, w.B, w.H, w.N, w.d, w.scale, qs, ks, vs, w.causal,
                               stream)
            if st != 0:
                raise fa.FAError(st)
    elif stdp:
        from io_aware_tiled_09_amd import standard as stdlib
        need = stdlib.fa_std_workspace_bytes(w.B, w.H, w.N)
        ws8 = torch.empty(need, dtype=torch.uint8, device=dev)
        nn = w.B * w.H * w.N * w.N
        s_buf = ws8[: nn * 4].view(torch.float32)
        p_off = (nn * 4 + 255) // 256 * 256
        p_buf = ws8[p_off: p_off + nn * 2].view(torch.bfloat16)
        g_off = p_off + (nn * 2 + 255) // 256 * 256
        gws = ws8[g_off:]
        std_sm = []

        def step(sm_events=None):
            st = stdlib.fa_std_scores(dq, dk, s_buf, gws, w.B, w.H, w.N, w.d, w.scale, stream)
            if st == 0:
                if sm_events is not None:
                    sm_events[0].record(stream)
                st = stdlib.fa_std_softmax(s_buf, p_buf, lse, w.B, w.H, w.N, w.causal, stream)
                if sm_events is not None:
                    sm_events[1].record(stream)
            if st == 0:
                st = stdlib.fa_std_output(p_buf, dv, o, gws, w.B, w.H, w.N, w.d, stream)
            if st != 0:
                raise fa.FAError(st)
    elif bwd:
        do_cpu = make_dout(w)
        ddo = do_cpu.to(dev)
        gq, gk, gv = torch.empty_like(dq), torch.empty_like(dq), torch.empty_like(dq)
        ws = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        fwd_step()  # O and lse for the backward

        def step():
            st = fa.fa_bwd(dq, dk, dv, o, lse, ddo, gq, gk, gv, ws, w.B, w.H, w.N, w.d,
                           w.scale, w.causal, stream)
            if st != 0:
                raise fa.FAError(st)
    else:
        step = fwd_step

    gemm_ref = None
    if args.gemm_ref and not (fp8 or stdp):
        gemm_ref = gemm_reference(torch, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        if stdp:
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            std_sm.append(ev)
            step(ev)
        else:
            step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    span_ms = starts[0].elapsed_time(ends[-1])
    avg_launch_ms = sum(per_launch_ms) / K
    med_launch_ms = sorted(per_launch_ms)[K // 2]
    flops = (backward_flops if bwd else useful_flops)(w.B, w.H, w.N, w.d, w.causal)
    ms_per_step = max(span_ms, 1e-9) / K
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    if stdp:
        # Dominant kernel: the softmax over the stored scores, HBM-bound.
        # Algorithmic bytes per launch: the visible scores read once (fp32),
        # all of P written once (bf16), lse written (fp32).
        sm_ms = sum(a.elapsed_time(b) for a, b in std_sm) / K
        vis = w.N * (w.N + 1) // 2 if w.causal else w.N * w.N
        sm_bytes = w.B * w.H * (vis * 4 + w.N * w.N * 2 + w.N * 4)
        sm_gbs = sm_bytes / (sm_ms * 1e-3) / 1e9
        log(f"softmax launch {sm_ms:.4f} ms, {sm_bytes / 1e9:.3f} GB -> {sm_gbs:.0f} GB/s")
    log(f"avg launch {avg_launch_ms:.4f} ms, median {med_launch_ms:.4f} ms, span/step "
        f"{ms_per_step:.4f} ms, wall/step {wall / K * 1e3:.4f} ms -> {value:.1f} TFLOP/s")

    if args.copy_kernel_mib > 0:
        n = args.copy_kernel_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy kernel: {args.copy_kernel_mib} MiB read + written, 3 times")

    digest = kernel_source_digest(args.pass_)
    traffic = measured_traffic(digest, args.pass_, w.name)
    metric = "attention fwd TFLOP/s (bf16, 1 MI355X) at N=8K d=128 causal; % of MFMA peak"
    if w.name != "longdoc8k":
        metric = (f"attention fwd TFLOP/s (1 MI355X) on {w.name} (B={w.B} H={w.H} N={w.N} "
                  f"d={w.d} causal={w.causal}); % of MFMA peak")
    if bwd:
        metric = ("attention bwd TFLOP/s (bf16, 1 MI355X) at N=8K d=128 causal; % of MFMA peak "
                  "(useful FLOPs = 2.5x forward)")
    if fp8:
        metric = ("attention fwd TFLOP/s with FP8 (E4M3) Q, K, V (1 MI355X) at N=8K d=128 causal; "
                  "% of the FP8 MFMA peak")
    if stdp:
        metric = ("standard (materializing) attention fwd TFLOP/s (bf16, 1 MI355X) at N=8K "
                  "d=128 causal; useful FLOPs as the flash forward")
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "useful_flop_per_call": flops, "pass": args.pass_},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(avg_launch_ms, 5),
            "kernels": list(PASS_KERNELS[args.pass_]),
            "kernel_source_digest": digest,
        },
        "cpu_baseline": None,
    }
    if fp8:
        result["dtype"] = "fp8_e4m3"
        result["pct_of_peak"] = round(100.0 * value / PEAK_FP8_TFLOPS, 2)
        result["roofline"]["peak"] = PEAK_FP8_TFLOPS
        result["roofline"]["frac"] = round(achieved / PEAK_FP8_TFLOPS, 4)
        result["roofline"]["kernels"] = list(PASS_KERNELS["fp8"])
    if stdp:
        result["roofline"] = {
            "bound": "hbm",
            "achieved": round(sm_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(sm_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(sm_ms, 5),
            "kernels": list(PASS_KERNELS["std"]),
            "algorithmic_bytes": sm_bytes,
            "kernel_source_digest": digest,
            "call_ms": round(avg_launch_ms, 5),
        }
    if args.gemm_ref and not (fp8 or stdp):
        gemm_ref["kernel_over_reference"] = round(achieved / gemm_ref["tflops"], 4)
        result["mfma_reference"] = gemm_ref
    if args.gemm_ref and stdp:
        result["hbm_reference"] = hbm_reference(torch, stream, sm_gbs)
    if args.sustained > 0:
        result["sustained"] = sustained_reference(
            torch, stream, step, args.sustained, ms_per_step, flops,
            PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS, not (fp8 or stdp))
    if args.cpu_budget > 0:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = (cpu_baseline_bwd(w, q, k, v, do_cpu, args.cpu_budget) if bwd
                                  else cpu_baseline(w, q, k, v, args.cpu_budget,
                                                    ((q8, k8, v8), (qs, ks, vs)) if fp8 else None))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
