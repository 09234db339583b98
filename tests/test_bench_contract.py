"""The bench.py contract: one JSON line with the headline metric, the roofline
of the dominant kernel and the per-kernel breakdown; --gpus above 1 is refused
with a message (this benchmark measures one GPU)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-extra", "--no-cpu-baseline"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    out = json.loads(lines[0])
    assert out["metric"].startswith("attention fwd/bwd TFLOP/s")
    assert out["unit"] == "TFLOP/s" and out["value"] > 0 and out["higher_is_better"] is True
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["ms_per_step"] > 0 and out["scaling"] == "weak" and out["vs_baseline"] is None
    assert out["dtype"] == "bf16" and out["data"] == "synthetic"
    assert "B=1 Hq=32 Hkv=8 S=2048 D=128" in out["config"]["workload"]
    # value is the counted fwd+bwd flops (2.5x the forward for the backward) per step time
    fwd_flops = 4.0 * 32 * 128 * (2048 * 2049 // 2)
    assert abs(out["value"] - 3.5 * fwd_flops / (out["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * out["value"]
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["kernel"] in out["kernels"]
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    for n in ("fwd", "bwd_dq", "bwd_dkdv", "bwd_group_sum"):
        assert out["kernels"][n]["ms"] > 0
    assert set(out["inputs_sha256"]) == {"q", "k", "v", "do"}
    assert all(len(h) == 64 for h in out["inputs_sha256"].values())
    assert "cpu_baseline" not in out
