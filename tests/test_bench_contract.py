"""The bench's command-line contract: one GPU only, and one JSON line with the fields
the measurement needs (tokens/s, the dominant kernel's roofline, the oracle's rate)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr and p.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.stderr.write("[gpu] bench.py --steps 8 --warmup 2 --instances 2 --cpu-seconds 1\n")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "8", "--warmup", "2",
                        "--instances", "2", "--cpu-seconds", "1", "--event-every", "1"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2 and d["value"] > 0
    assert d["config"]["workload"] == "decode_7b" and d["unit"] == "tokens/s"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] < r["peak"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["copy_gbps"] > 0 and r["frac_of_copy"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["unit"] == "tokens/s"
    assert c["single_thread"]["cores"] == 1 and c["single_thread"]["value"] > 0
    assert d["workspace_status"] == "clean"
    k = d["kernels"][r["kernel"]]
    assert k["p10_us"] <= k["p50_us"] <= k["p90_us"] and k["pct_launches"] >= 8
    f = d["fetch"]
    assert f["h2d_copy_engine_gbps"] > 0 and f["kernel_gbps"] > 0 and 0 < f["kernel_ms"] <= f["ms"]
    assert d["device"]["compute_units"] > 0
    pf = d["prefill"]
    assert pf["workload"] == "prefill_sgmv" and pf["value"] > 0 and pf["workspace_status"] == "clean"
    # the four projections in one slora_apply_multi per step
    pr = pf["roofline"]["multi_fused"]
    assert pr["unit"] == "GB/s" and 0 < pr["frac"] < 1 and 0 < pr["mfma_frac"] < 1
    assert set(pf["kernels"]) == {"multi_fused"}
