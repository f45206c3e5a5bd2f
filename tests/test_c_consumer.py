"""The C ABI used from C: tests/c_abi_consumer.c, built with gcc -std=c99.

The host test needs no GPU: it runs the argument checks, sizes, RNG state and
the launch-failure hook through the header alone.  The GPU test has the C
program run the forward and backward on seeded inputs written by this test,
and compares what it wrote with the oracle at the same bars as the other
parity tests.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_grads, assert_lse, assert_out, gpu_available, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.dirname(sdpa.LIB_PATH)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    if not os.path.exists(sdpa.LIB_PATH):
        pytest.fail("libsdpa14.so is not built")
    exe = str(tmp_path_factory.mktemp("c_abi") / "c_abi_consumer")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", f"-I{ROCM}/include", os.path.join(ROOT, "tests", "c_abi_consumer.c"),
           "-o", exe, f"-L{LIB_DIR}", "-lsdpa14", f"-Wl,-rpath,{LIB_DIR}", f"-L{ROCM}/lib",
           "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_on_the_host(consumer):
    r = subprocess.run([consumer, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks: 0 failed" in r.stdout


def _bf16_bytes(t: torch.Tensor) -> bytes:
    return t.contiguous().view(torch.int16).numpy().tobytes()


def _read_bf16(path, shape):
    raw = np.fromfile(path, dtype=np.int16).reshape(shape)
    return torch.from_numpy(raw).view(torch.bfloat16).double().numpy()


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
@pytest.mark.parametrize("B,H,Sq,Sk,E,causal", [(1, 2, 128, 128, 64, True),
                                                 (2, 2, 200, 333, 128, False),
                                                 (1, 3, 257, 257, 40, True)])
def test_c_program_on_the_gpu(consumer, tmp_path, B, H, Sq, Sk, E, causal):
    say(f"C consumer on the GPU: B{B} H{H} Sq{Sq} Sk{Sk} E{E} causal={causal}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 81, 1.0, "BHSE")
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        (tmp_path / f"{name}.bin").write_bytes(_bf16_bytes(t))
    r = subprocess.run([consumer, "gpu", str(tmp_path), str(B), str(H), str(Sq), str(Sk), str(E),
                        str(int(causal))], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = _read_bf16(tmp_path / "out.bin", (B, H, Sq, E))
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(B, H, Sq).astype(np.float64)
    dq = _read_bf16(tmp_path / "dq.bin", (B, H, Sq, E))
    dk = _read_bf16(tmp_path / "dk.bin", (B, H, Sk, E))
    dv = _read_bf16(tmp_path / "dv.bin", (B, H, Sk, E))
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, 0.0, causal)
    ref_dq, ref_dk, ref_dv = sdpa_ref.bwd(do, q, k, v, 0.0, causal)
    assert_out(out, ref_out)
    assert_lse(lse, ref_lse)
    assert_grads([("dq", dq, ref_dq), ("dk", dk, ref_dk), ("dv", dv, ref_dv)])
