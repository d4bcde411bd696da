"""The committed measurements in profiles/ (CPU): every bench line's figures
follow from its own fields (tokens/s from the step time, the roofline's
achieved rate from its algorithmic work and launch time, the fraction from the
peak), its algorithmic bytes are those of bench.py's work model, and its
traffic is the one stored by the counter runs taken on the same kernel
sources, rebuilt from the raw counter readings and the copy calibration; each
kernel-trace summary agrees with its bench line."""
import glob
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from afd_inputs import CONFIGS  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
LINES = sorted(glob.glob(os.path.join(PROFILES, "bench_*.json")))


def _load(path):
    with open(path) as f:
        return json.load(f)


def _close(a, b, rel):
    return abs(a - b) <= rel * abs(b)


def test_every_benchmarked_workload_has_a_line():
    names = {os.path.basename(p)[len("bench_"):-len(".json")] for p in LINES}
    assert bench.DEFAULT_WORKLOAD in names
    assert names <= set(CONFIGS)
    assert len(names) >= 5


@pytest.mark.parametrize("path", LINES, ids=os.path.basename)
def test_bench_line_is_consistent(path):
    d = _load(path)
    name = os.path.basename(path)[len("bench_"):-len(".json")]
    s = CONFIGS[name]
    assert d["metric"] == bench.METRIC and d["unit"] == "tokens/s"
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True
    assert d["config"]["workload"] == name and d["config"]["T"] == s.T
    assert d["config"]["mode"] == s.mode
    # tokens per second from the step time: one step is the whole batch
    assert _close(d["value"], s.T / (d["ms_per_step"] * 1e-3), 1e-4)
    f = d["forward"]
    assert _close(f["hbm_gbs"], f["bytes"] / (d["ms_per_step"] * 1e-3) / 1e9, 1e-3)
    r = d["roofline"]
    assert _close(r["frac"], r["achieved"] / r["peak"], 1e-3)
    if r["bound"] == "hbm":
        assert r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
        assert _close(r["achieved"],
                      r["algorithmic_bytes_per_launch"] / (r["avg_launch_ms"] * 1e-3) / 1e9,
                      1e-3)
        # every expert is touched at these sizes (thousands of selections
        # over at most 256 experts), so the work model needs no routing
        m = bench.work_model(s, [1] * s.E)
        assert m["touched_experts"] == f["touched_experts"] == s.E
        launch = m["ffn_bytes"] if "stream_ffn_kernel" in r["kernel"] else m["gate_up_bytes"]
        assert r["algorithmic_bytes_per_launch"] == int(launch)
    else:
        assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
        assert r["peak"] == bench.MFMA_PEAK_TFLOPS[s.mode]
        assert _close(r["achieved"],
                      r["algorithmic_flops_per_launch"] / (r["avg_launch_ms"] * 1e-3) / 1e12,
                      1e-3)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "tokens/s"
    assert c["value"] > 0 and c["cores"] >= 1 and c["sample"]


@pytest.mark.parametrize("path", LINES, ids=os.path.basename)
def test_bench_traffic_matches_counter_runs(path):
    d = _load(path)
    name = os.path.basename(path)[len("bench_"):-len(".json")]
    r = d["roofline"]
    kind = "ffn" if "stream_ffn_kernel" in r["kernel"] else "gate_up"
    t = _load(os.path.join(PROFILES, f"traffic_{kind}_{name}.json"))
    assert t["workload"] == name
    if r["traffic"] is None:
        assert t["kernel_source_hash"] != d["kernel_source_hash"]
        return
    # reported only when both were taken on the same kernel sources
    assert t["kernel_source_hash"] == d["kernel_source_hash"]
    assert r["traffic"] == t["hbm_bytes_per_launch"]
    rebuilt = 1024 * (t["fetch_kib_per_launch_raw"] * t["fetch_scale"]
                      + t["write_kib_per_launch_raw"] * t["write_scale"])
    assert _close(t["hbm_bytes_per_launch"], rebuilt, 1e-6)
    if "algorithmic_bytes_per_launch" in t:
        assert t["algorithmic_bytes_per_launch"] == r["algorithmic_bytes_per_launch"]


def test_traffic_files_name_their_commands():
    for p in glob.glob(os.path.join(PROFILES, "traffic_*.json")):
        t = _load(p)
        cmds = t["commands"]
        assert any("--pmc FETCH_SIZE" in c for c in cmds), p
        assert any("--pmc WRITE_SIZE" in c for c in cmds), p
        assert any("--copy-calibration" in c for c in cmds), p
        assert all("bench.py" in c for c in cmds), p


TRACES = sorted(glob.glob(os.path.join(PROFILES, "kernels_*.md")))


@pytest.mark.parametrize("path", TRACES, ids=os.path.basename)
def test_trace_agrees_with_bench_line(path):
    """Each kernel-trace summary was taken with its bench line's command on
    the same box; the trace's average of the dominant launch over the same
    dispatches matches the line's HIP-event average (0.5%), except the decode
    h4096 single launch, which runs up to about 5% slower under the profiler
    (its summary shows this with the profiled run's own step time)."""
    import re
    name = os.path.basename(path)[len("kernels_"):-len(".md")]
    text = open(path).read()
    d = _load(os.path.join(PROFILES, f"bench_{name}.json"))
    m = re.search(r"The trace's average of `[^`]+` over the \d+ dispatches of [^.]* is ([0-9.]+) us", text)
    assert m, "no trace average in the summary"
    traced_us = float(m.group(1))
    events_us = d["roofline"]["avg_launch_ms"] * 1e3
    tol = 0.06 if name == "decode_h4096_e64" else 0.005
    assert abs(traced_us - events_us) <= tol * events_us, (traced_us, events_us)
    # the summary quotes the committed line, and its command is the line's own
    assert f"{d['ms_per_step']} ms per step" in text
    cmd = next(ln for ln in text.splitlines() if ln.strip().startswith("rocprofv3"))
    if "--steps" in cmd:
        assert f"--steps {d['steps']} --warmup {d['warmup']}" in cmd
