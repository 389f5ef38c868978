"""bench.py end to end on small workloads: one JSON line with the contract's
fields, every in-run check held, the oracle baseline and the roofline object
present.  The Wan line itself is the benchmark run; these keep its code path
exercised by the GPU tests."""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import HAVE_GPU

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, "bench.py", *args], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("mode,extra", [("uos", []), ("ocp", ["--no-pnq"])])
def test_bench_tiny_line(mode, extra):
    d = run_bench("--workload", "tiny", "--steps", "3", "--warmup", "1", "--mode", mode, *extra)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["valid"] is True and all(d["checks"].values()), d["checks"]
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["roofline"]["bound"] == "mfma" and 0 < d["roofline"]["frac"] < 1
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["cores"] >= 1
    assert d["config"]["mode"] == mode and d["config"]["pnq"] is (not extra)

