"""bench.py end to end on the GPU on the tiny fp32 workload: one JSON line on
stdout with every field of its contract (metric, throughput, timing, the
roofline object of the dominant call and the oracle's CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny_f32",
                        "--steps", "3", "--warmup", "1", "--no-gemm-ref"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in out, k
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["unit"] == "TFLOP/s" and out["dtype"] == "f32" and out["vs_baseline"] is None
    assert out["config"]["workload"] == "tiny_f32"
    roof = out["roofline"]
    assert set(roof) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert roof["bound"] == "alu" and roof["peak"] == 157.3   # fp32 vector kernels
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    # the headline recomputes from the step time and the algorithmic flop count
    assert abs(out["value_without_recompute"] - out["value"] * 12 / 14) < 0.02
