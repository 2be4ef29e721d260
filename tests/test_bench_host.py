"""Host-side pieces of bench.py, on the CPU: the algorithmic FLOP count against a brute-force
count of kept entries, the readers of the committed counter summaries (values only for the
workload and kernel sources they were taken on), and the refusal of more than one GPU."""

import importlib.util
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,d", [(1, 64), (5, 64), (37, 128)])
def test_alg_flops_counts_kept_entries(bench, causal, N, d):
    kept = sum(1 for i in range(N) for j in range(N) if (j <= i or not causal))
    fwd, bwd = bench.alg_flops(2, 3, N, d, causal)
    # forward: two score contractions, backward: two recomputed scores and two gradient
    # contractions, each 2 d flops per kept entry
    assert fwd == 2 * 3 * 2 * (2 * d * kept)
    assert bwd == 2 * fwd


def test_executed_backward_flops_match_the_counted_mfmas(bench):
    # SQ_INSTS_MFMA of one backward dispatch at 32 heads x 32K (the committed counter run):
    # 8.056e8 wave-level MFMAs of 32x32x16 (32768 flops each)
    ex = bench.executed_bwd_flops(1, 32, 32768, 128)
    assert abs(ex / 32768 - 8.056e8) / 8.056e8 < 1e-3
    _, alg = bench.alg_flops(1, 32, 32768, 128, True)
    assert 1.49 < ex / alg < 1.51  # full-row ownership: 6 units executed for 4 algorithmic


def _recorded_digest(path, key):
    with open(os.path.join(ROOT, path)) as f:
        m = re.search(key + r".*source_sha256=([0-9a-f]+)", f.read())
    assert m, path
    return m.group(1)


def test_profile_readers_follow_the_recorded_sources(bench, monkeypatch):
    dig_t = _recorded_digest(bench.TRAFFIC_PROFILE, "traffic:")
    dig_c = _recorded_digest(bench.COUNTER_PROFILE, "counters:")
    assert dig_t == dig_c  # both summaries come from one set of kernel sources
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: dig_t)
    t = bench.measured_traffic("llama2_32k")
    assert isinstance(t, int) and t > 0
    c = bench.measured_counters("llama2_32k")
    for k in ("bwd_mfma_busy", "bwd_coexec", "fwd_mfma_busy", "fwd_coexec"):
        assert 0.0 < c[k] < 1.0
    assert 1.9 < c["fwd_trans_per_elem"] < 2.1 and 3.9 < c["bwd_trans_per_elem"] < 4.1
    assert bench.measured_traffic("llama2_4k") is None  # another workload
    assert bench.measured_counters("llama2_4k") is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)  # other sources
    assert bench.measured_traffic("llama2_32k") is None
    assert bench.measured_counters("llama2_32k") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line
