"""bench.py end to end on the GPU at the small workload: one JSON line with every field
of the benchmark record (throughput, roofline of the whole step, per-launch times, the oracle's
CPU baseline), produced through the C ABI."""
import json

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def test_bench_record_fields(capsys):
    import bench

    # 40 steps: one replay of the 36-step graph and a remainder graph of 4
    rc = bench.main(["--workload", "tiny_4k", "--steps", "40", "--warmup", "2", "--stage-steps", "4",
                     "--cpu-budget", "0.3", "--no-plan-exec", "--pipeline-reps", "2"])
    assert rc == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1, lines          # stdout carries the record alone
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "layer_pipelined"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["unit"] == "steps/s" and r["higher_is_better"] is True
    assert r["config"]["workload"] == "tiny_4k" and r["config"]["graph_steps"] == 36
    assert r["steps"] == 40 and r["step_ms"]["n"] == 300
    assert r["value"] > 0 and r["ms_per_step"] > 0
    assert abs(r["value"] - 1.0 / r["ms_per_step"] * 1e3) <= 0.01 * r["value"] + 0.01
    roof = r["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["scope"] == "whole step" and roof["bytes_per_step"] > 0
    assert abs(roof["achieved"] - roof["bytes_per_step"] / (r["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * roof["achieved"] + 0.2
    dom = r["dominant_kernel"]
    assert dom["avg_launch_us"] > 0 and dom["kernel"] in roof["kernels"]
    assert set(r["launches"]) == {"launch1", "launch2"}
    assert r["launches"]["launch1"]["bytes_per_launch"] > 0
    cpu = r["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert r["checks"].get("graph_matches_eager", True) is True
    assert r["checks"]["handoff_status_zero"] is True
    # the serial step at this shape (cap 0) takes the overlapped launch 1 and the merge
    assert r["serial_form"] == "overlapped launch 1, touched splits redone, merge"
