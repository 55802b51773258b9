"""Compile the gfx950 HIP libraries in-tree with hipcc: ``libfa.so`` (the
FlashAttention forward and backward) and ``libfa_std.so`` (the standard,
materializing attention baseline, which links rocBLAS)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfa.so")
STD_LIB = os.path.join(PKG, "libfa_std.so")
STD_SOURCES = [os.path.join(PKG, "csrc", "fa_std.hip")]
SOURCES = [os.path.join(PKG, "csrc", "fa_fwd_bf16.hip"),
           os.path.join(PKG, "csrc", "fa_bwd_bf16.hip"),
           os.path.join(PKG, "csrc", "fa_fwd_f32.hip"),
           os.path.join(PKG, "csrc", "fa_fwd_fp8.hip"),
           os.path.join(PKG, "csrc", "fa_decode.hip"),
           os.path.join(PKG, "csrc", "fa_scratch.hip"),
           os.path.join(PKG, "csrc", "fa_plan.cpp"),
           os.path.join(PKG, "csrc", "fa_api.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, sources=None, libs=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # no packed-fp32 VALU forms anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-o", out, *(sources or SOURCES), *libs]


def _compile(out, sources, libs=(), verbose=False):
    tmp = out + ".tmp"
    cmd = command(tmp, sources, libs)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Always recompiles both libraries; writes them atomically next to this file."""
    _compile(LIB, SOURCES, verbose=verbose)
    _compile(STD_LIB, STD_SOURCES, ("-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"),
             verbose=verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
