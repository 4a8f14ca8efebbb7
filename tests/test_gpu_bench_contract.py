"""bench.py's JSON line on the GPU: every field of the reporting contract is
present and consistent (a short run: 3 timed steps, the CPU oracle leg on)."""
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
    print("case bench.py --steps 3 --warmup 1 --no-per-call", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--warmup-seconds", "0.2", "--no-per-call"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    assert d["metric"] == "selective-scan fwd HBM GB/s and % of peak, Mamba-1.4B shape, 1\u00d7MI355X"
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["dtype"] == "bf16" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"].startswith("m1p4b")
    assert (d["config"]["batch"], d["config"]["dim"], d["config"]["dstate"],
            d["config"]["seqlen"]) == (8, 4096, 16, 2048)
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-3)
    assert roof["achieved"] == pytest.approx(
        roof["bytes_per_launch"] / (d["kernel_avg_us_hip_events"] * 1e-6) / 1e9, rel=1e-3)
    assert "traffic" in roof
    ssd = d["ssd"]
    assert ssd["ms_per_call"] > 0 and ssd["mfma"]["peak"] == 2500.0
    assert ssd["mfma"]["frac"] == pytest.approx(ssd["mfma"]["achieved"] / 2500.0, rel=1e-3)
    assert "traffic" in ssd
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["unit"] == d["unit"]
