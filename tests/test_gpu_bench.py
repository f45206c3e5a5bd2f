"""bench.py end to end on the GPU at a small size, with and without dropout.

The timed step is a HIP graph of several back-to-back steps, checked
bitwise against the same steps run eagerly from the same RNG state before
any timing; with dropout each captured step draws its own offset, so this
covers the check's handling of the RNG state as well as the JSON contract.
"""

import json
import os
import subprocess
import sys

import pytest

from tests._util import gpu_available, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("shape", ["2,3,256,256,64,1", "2,3,256,256,64,1,0.1",
                                   "1,2,200,300,128,0"])
def test_bench_line_at_a_small_shape(shape):
    say(f"bench.py --shape {shape}")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--shape", shape,
                        "--steps", "6", "--warmup", "1", "--no-cpu-baseline", "--no-cold"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 6 and d["warmup"] == 1
    assert d["steps_per_graph"] == 6
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["roofline"]["achieved"] > 0 and 0 < d["roofline"]["frac"] < 1
    assert d["cpu_baseline"] is None
