"""Every bench.py mode runs end to end on the small dense workload and
prints one JSON document (the default line with its roofline, the
compensation sweep, the W4A16 and FP8 comparisons)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mode", [[], ["--rac-sweep"], ["--w4a16"], ["--fp8"], ["--ceilings"]])
def test_bench_mode_prints_json(dev, mode):
    print(f"bench.py {' '.join(mode)} --config 1", flush=True)
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", "1", "--steps", "4",
           "--warmup", "1", "--no-cpu-baseline", "--no-decode", *mode]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    if not mode:
        assert d["config"]["workload"] == "dense_64x512x512"
        assert d["roofline"]["bound"] == "mfma" and d["value"] > 0
        assert set(d["step_ms_events"]) == {"p10", "p50", "p90"}
        assert d["ceilings"]["mfma_f16_tflops"] > 0 and d["ceilings"]["hbm_read_GBps"] > 0
        assert d["ceilings"]["mfma_f16_nvfp4_operands_tflops"] > 0
        assert d["roofline"]["frac_of_f16_rate_on_these_operands"] > 0
        assert "gemm1" in d["rac_overhead"] and "gates" in d
    else:
        assert d["mode"] in ("rac_sweep", "w4a16", "fp8", "ceilings")
