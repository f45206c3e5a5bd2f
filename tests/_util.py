"""Shared helpers for the GPU parity tests: device transfer and error metrics.

Tolerances (the targets of the method's parity statement):
  out   max |gpu - oracle| <= 1e-2, plus the rounding of the bf16 output: an
        element also passes when its error is within 1e-2 + half a bf16 ulp of
        the oracle value (a bf16 number cannot be closer than half an ulp to an
        arbitrary real; for |O| >= 4 that is already 2^-6 > 1e-2)
  lse   max |gpu - oracle| <= 1e-3
  grads ||g - g_ref||_F / max(||g_ref||_F, 1e-3 * sqrt(n)) <= 2e-2 per tensor; the
        floor (an RMS of 1e-3) only matters where the exact gradient vanishes,
        e.g. dQ = dK = 0 with a single key, where a relative error is undefined
  mask  bit-exact on every visible element
"""

import math
import sys

import numpy as np
import torch

import workloads

OUT_TOL = 1e-2
LSE_TOL = 1e-3
GRAD_TOL = 2e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_dev(t: torch.Tensor, layout: str) -> torch.Tensor:
    return workloads.to_layout(t.to("cuda"), layout)


def host64(t) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def out_errors(gpu: np.ndarray, ref: np.ndarray):
    """(strict max abs error, number of elements failing the bf16-aware bar)."""
    err = np.abs(gpu - ref)
    bad = err > OUT_TOL + bf16_half_ulp(ref)
    return float(err.max()), int(bad.sum())


def rel_fro(gpu: np.ndarray, ref: np.ndarray) -> float:
    floor = 1e-3 * math.sqrt(ref.size)
    return float(np.linalg.norm((gpu - ref).ravel()) / max(np.linalg.norm(ref.ravel()), floor))


def assert_out(gpu, ref, what="out"):
    strict, nbad = out_errors(gpu, ref)
    say(f"  {what}: max abs err {strict:.3e} (bf16-aware failures: {nbad})")
    assert nbad == 0, f"{what}: {nbad} elements beyond 1e-2 + half bf16 ulp (max {strict})"


def assert_lse(gpu, ref):
    err = float(np.abs(gpu - ref).max())
    say(f"  lse: max abs err {err:.3e}")
    assert err <= LSE_TOL


def assert_grads(pairs):
    for name, g, r in pairs:
        e = rel_fro(g, r)
        say(f"  {name}: rel Frobenius err {e:.3e}")
        assert e <= GRAD_TOL, (name, e)


def fwd_flops(B, H, Sq, Sk, E, causal):
    f = 4.0 * B * H * Sq * Sk * E
    return f / 2 if causal else f


def heads_subset(B, H, n, seed=0):
    rng = np.random.default_rng(seed)
    all_heads = [(b, h) for b in range(B) for h in range(H)]
    idx = sorted(rng.choice(len(all_heads), size=min(n, len(all_heads)), replace=False))
    return [all_heads[i] for i in idx]


def ceil_div(a, b):
    return -(-a // b)

