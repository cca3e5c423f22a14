"""Host logic of bench.py (no GPU): the roofline's byte counts and the rule
that counter-measured traffic is reported only for the kernel sources the
counters were taken on."""

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

S = 256 << 20                     # bytes per rank at 8 x 2^26 float32


def test_algorithmic_bytes_and_busbw():
    assert bench.algorithmic_bytes("allreduce", 8, S) == 2 * 8 * S
    assert bench.algorithmic_bytes("reduce_scatter", 8, S) == 9 * S
    assert bench.busbw_factor("allreduce", 8) == pytest.approx(1.75)
    assert bench.busbw_factor("reduce_scatter", 8) == pytest.approx(0.875)
    assert bench.busbw_factor("allreduce", 1) == 0.0


# bytes each form names per call at the headline (8 ranks, S = 256 MiB), in units of S
NAMED = {"staged": 16, "fused": 16, "phases": 17, "double_binary_tree": 16,
         "double_binary_tree_steps": bench.dbt_steps_bytes_factor(8)}


@pytest.mark.parametrize("form", sorted(bench.COUNTERS_FILES))
def test_committed_counter_summaries_parse(form):
    """Each committed summary holds a traffic line for one call of its form at
    the headline, between the algorithmic minimum (2N*S) and 10% above the
    bytes the form names."""
    path = bench.COUNTERS_FILES[form]
    if not os.path.exists(path):
        pytest.skip(f"no counter summary for {form}")
    text = open(path).read()
    line = [ln for ln in text.splitlines() if ln.startswith("traffic_json: ")]
    assert len(line) == 1
    d = json.loads(line[0][len("traffic_json: "):])
    assert 2 * 8 * S <= d["bytes_per_call"] <= 1.1 * NAMED[form] * S
    assert d["fetch_bytes"] + d["write_bytes"] == d["bytes_per_call"]
    if d["kernel_source_sha256_16"] == bench.kernel_source_hash(form):
        assert bench.measured_traffic(form) == d["bytes_per_call"]
    else:
        assert bench.measured_traffic(form) is None


def test_traffic_withheld_for_other_sources(tmp_path, monkeypatch):
    good = {"kernel_source_sha256_16": bench.kernel_source_hash(), "bytes_per_call": 123}
    stale = dict(good, kernel_source_sha256_16="0" * 16)
    for name, d in (("good", good), ("stale", stale)):
        (tmp_path / f"{name}.md").write_text(f"# summary\n\ntraffic_json: {json.dumps(d)}\n")
    (tmp_path / "none.md").write_text("# summary without a traffic line\n")
    monkeypatch.setattr(bench, "COUNTERS_FILES", {f: str(tmp_path / f"{f}.md") for f in ("good", "stale", "none")})
    assert bench.measured_traffic("good") == 123
    assert bench.measured_traffic("stale") is None
    assert bench.measured_traffic("none") is None
    assert bench.measured_traffic("unknown") is None


def test_more_than_one_gpu_is_refused():
    """bench.py --gpus N with N above 1 exits with a message, before touching a GPU."""
    import subprocess

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_every_step_algorithm_names_its_kernels():
    """bench.py --algo accepts the library's AllReduce algorithms, and names the
    kernels of each in its line (staged and auto are named from the plan)."""
    from ring_allreduce_reduction_virtual_amd import _lib

    for algo in bench.STEP_ALGOS:
        assert algo in _lib.ALGOS, algo
        if algo not in ("auto", "staged"):
            assert bench.STEP_KERNELS[algo].format(launches=6)
    assert set(bench.STEP_KERNELS) | {"auto", "staged"} == set(bench.STEP_ALGOS)
