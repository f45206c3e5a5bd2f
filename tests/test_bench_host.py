"""Host-side checks of bench.py's contract (no GPU needed)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--gpus", "--workload", "--shape", "--bias", "--keep-bits",
                "--no-cold", "--no-cpu-baseline", "--copy-bytes"):
        assert opt in r.stdout


def test_algorithmic_work_counts():
    # FLOPs: 4*B*H*Sq*Sk*E, halved when causal; backward 2.5x (five products).
    sys.path.insert(0, ROOT)
    import workloads

    w = workloads.WORKLOADS["b2_h12_s1024_d64_causal"]
    assert w.fwd_flops() == 4 * 2 * 12 * 1024 * 1024 * 64 // 2
    assert w.bwd_flops() == w.fwd_flops() * 5 // 2
    x = workloads.WORKLOADS["b1_h32_q4096_k8192_d128_cross"]
    assert x.fwd_flops() == 4 * 1 * 32 * 4096 * 8192 * 128
    json.dumps({"fwd": w.fwd_flops()})
