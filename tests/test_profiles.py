"""The measurement records under profiles/ match the sources they describe.

bench.py reports a workload's HBM traffic only while the roofline kernel's
sources hash as they did when the FETCH_SIZE / WRITE_SIZE counters were
taken; these checks fail (on the CPU) as soon as a kernel source changes
without its records being re-taken, instead of the benchmark line silently
carrying `traffic: null`.
"""

import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


BENCH = _bench()
WORKLOADS = sorted(BENCH.TRAFFIC_KERNELS)
# MFMA-bound workloads whose instruction counters are recorded as well
COUNTER_WORKLOADS = ["dense_causal_prefill_d128", "dense_causal_prefill_d256", "ragged_paged_prefill_80k",
                     "mla_decode_80k_bf16", "mla_decode_80k_fp8_q", "fp8_mla_prefill_8k"]


@pytest.mark.parametrize("workload", WORKLOADS)
def test_traffic_record_matches_sources(workload):
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    assert os.path.exists(path), f"{path} missing"
    with open(path) as f:
        rec = json.load(f)
    kernel, sources = BENCH.TRAFFIC_KERNELS[workload]
    assert rec["source_hash"] == BENCH.kernel_source_hash(sources), (
        f"{workload}: the counters were taken on other sources of {sources}; re-take FETCH_SIZE / WRITE_SIZE")
    assert kernel.split("<")[0] in rec["kernel"]
    assert rec["bytes_per_launch"] > 0 and rec["dispatches"][0] > 0 and rec["dispatches"][1] > 0
    cal = rec["copy_calibration"]
    assert 1.5 < cal["fetch_scale"] < 2.5 and 0.5 < cal["write_scale"] < 1.5
    # every command it was made with runs committed files only
    for cmd in rec["commands"]:
        assert "bench.py" in cmd and "_work" not in cmd


@pytest.mark.parametrize("workload", WORKLOADS)
def test_kernel_trace_names_the_roofline_kernel(workload):
    path = os.path.join(PROFILES, f"kernel_trace_{workload}.md")
    assert os.path.exists(path), f"{path} missing"
    with open(path) as f:
        text = f.read()
    kernel = BENCH.TRAFFIC_KERNELS[workload][0]
    assert kernel.split("<")[0] in text
    assert f"bench.py --only {workload}" in text and "_work" not in text


@pytest.mark.parametrize("workload", COUNTER_WORKLOADS)
def test_counter_summary_present(workload):
    path = os.path.join(PROFILES, f"counters_{workload}.md")
    assert os.path.exists(path), f"{path} missing"
    with open(path) as f:
        text = f.read()
    assert "MfmaUtil" in text and f"bench.py --only {workload}" in text and "_work" not in text
