"""The committed profile summaries match the kernel sources they describe (CPU only).

`bench.py` fills `roofline.traffic` from `profiles/hbm_traffic_*.json` only when
that file's kernel-source digest equals the digest of the sources as they are
now; these tests catch a kernel edit that was not followed by new counters and
a new summary.
"""
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

# pass -> the summary that reports its kernel trace and HBM traffic
SUMMARIES = {
    "fwd": ["hbm_traffic_longdoc8k.md", "fa_fwd_bf16_longdoc8k_kernel_trace.md"],
    "bwd": ["fa_bwd_bf16_longdoc8k.md"],
    "std": ["fa_std_longdoc8k.md"],
    "fp8": ["fa_fwd_fp8_longdoc8k.md"],
    "decode": ["fa_decode_paged_decode50.md"],
}


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("pass_", sorted(SUMMARIES))
def test_traffic_counters_match_current_sources(bench, pass_):
    path = bench.TRAFFIC_FILES[pass_]
    with open(path) as f:
        rec = json.load(f)
    assert rec["pass"] == pass_
    assert rec["kernel_source_digest"] == bench.kernel_source_digest(pass_), (
        f"{os.path.basename(path)} was taken on other kernel sources: re-take FETCH_SIZE/WRITE_SIZE")
    assert rec["hbm_bytes_per_launch"] > 0
    assert rec["command"], "the counters' command line is recorded"


@pytest.mark.parametrize("pass_", sorted(SUMMARIES))
def test_summaries_name_the_current_digest(bench, pass_):
    digest = bench.kernel_source_digest(pass_)
    for name in SUMMARIES[pass_]:
        with open(os.path.join(PROFILES, name)) as f:
            text = f.read()
        assert digest in text, f"{name} does not describe the current sources ({digest})"
        assert "rocprofv3" in text, f"{name} gives the command that produced it"


def test_profiles_hold_text_only():
    for name in os.listdir(PROFILES):
        assert os.path.splitext(name)[1] in (".md", ".txt", ".json"), name
        assert os.path.getsize(os.path.join(PROFILES, name)) < 64 * 1024, name


@pytest.mark.parametrize("pass_", sorted(SUMMARIES))
def test_traffic_is_reported_only_for_its_workload(bench, pass_):
    # roofline.traffic comes from a counter run on one workload; another
    # workload (or another kernel source) reports null instead.
    with open(bench.TRAFFIC_FILES[pass_]) as f:
        rec = json.load(f)
    digest = bench.kernel_source_digest(pass_)
    assert bench.measured_traffic(digest, pass_, rec["workload"]) == rec["hbm_bytes_per_launch"]
    assert bench.measured_traffic(digest, pass_, rec["workload"] + "_other") is None
    assert bench.measured_traffic("0" * 16, pass_, rec["workload"]) is None


def test_bench_refuses_more_than_one_gpu(bench, capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_engine_clock_parser(bench):
    # `bench.py --sustained` reads the engine clock from the kernel driver's
    # pp_dpm_sclk file: one line per clock level, '*' on the current one.
    assert bench.parse_engine_clock("0: 500Mhz\n1: 1633Mhz *\n2: 2400Mhz\n") == 1633
    assert bench.parse_engine_clock("S: 130Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 130
    assert bench.parse_engine_clock("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.engine_clock_sample(None) == (None, None)
    assert bench.engine_clock_sample("/nonexistent") == (None, None)


def test_engine_clock_sample_reads_sysfs_layout(bench, tmp_path):
    # the driver's layout: pp_dpm_sclk in the device directory, power in
    # microwatts under hwmon/hwmonN
    (tmp_path / "pp_dpm_sclk").write_text("S: 1708Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    hw = tmp_path / "hwmon" / "hwmon3"
    hw.mkdir(parents=True)
    (hw / "power1_input").write_text("1012500000\n")
    (hw / "power1_cap").write_text("1400000000\n")
    assert bench.engine_clock_sample(str(tmp_path)) == (1708, 1012.5)
    assert bench.power_cap_watts(str(tmp_path)) == 1400.0
    (hw / "power1_average").write_text("998000000\n")
    assert bench.engine_clock_sample(str(tmp_path)) == (1708, 998.0)
