"""Shared helpers for the GPU parity tests: device transfer and error metrics.

Tolerances (the targets of the method's parity statement):
  out   |gpu - oracle| <= 1e-2 on every element, compared with the unrounded
        fp64 oracle.  The one exemption is an element the output format itself
        cannot bring within 1e-2: its rounding floor |round(ref) - ref| (round
        to nearest in the output's own format, bf16 or fp16) plus the kernel's
        pre-rounding budget 2^-8 |ref| (probabilities enter the P.V product as
        16-bit values) exceeds 1e-2.  Such an element must then be one of the
        two representable neighbours of ref.  For bf16 this only happens at
        |ref| >= 2 (half an ulp is 2^-6 > 1e-2 from |ref| = 4 on); for fp16
        never below |ref| = 2.56, where an ulp is already below 1e-2.  Every
        check prints the strict maximum, the largest floor and the number of
        exempt elements.
  lse   max |gpu - oracle| <= 1e-3
  grads ||g - g_ref||_F / max(||g_ref||_F, 1e-3 * sqrt(n)) <= 2e-2 per tensor; the
        floor (an RMS of 1e-3) only matters where the exact gradient vanishes,
        e.g. dQ = dK = 0 with a single key, where a relative error is undefined
  mask  bit-exact on every visible element
"""

import math
import os
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


def neighbours(x: np.ndarray, dtype=torch.bfloat16):
    """The two values of the 16-bit format bracketing each float64 x (equal when
    x is representable), computed exactly in float64."""
    mant, emin = (8, -126) if dtype == torch.bfloat16 else (11, -14)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.exp2(np.maximum(e, emin) - (mant - 1))
    lo = np.floor(x / ulp) * ulp
    hi = np.where(lo == x, lo, lo + ulp)
    return lo, hi


def out_report(gpu: np.ndarray, ref: np.ndarray, dtype=torch.bfloat16) -> dict:
    """Strict and exempt error figures of one output comparison (see the module note)."""
    err = np.abs(gpu - ref)
    lo, hi = neighbours(ref, dtype)
    floor = np.minimum(ref - lo, hi - ref)
    over = err > OUT_TOL
    eligible = floor + np.ldexp(np.abs(ref), -8) > OUT_TOL
    neighbour = (gpu == lo) | (gpu == hi)
    exempt = over & eligible & neighbour
    return {
        "strict_max": float(err.max()) if err.size else 0.0,
        "floor_max": float(floor.max()) if floor.size else 0.0,
        "n_floor_over": int((floor > OUT_TOL).sum()),
        "n_over": int(over.sum()),
        "n_exempt": int(exempt.sum()),
        "n_fail": int((over & ~exempt).sum()),
        "n": int(err.size),
        "dtype": str(dtype).split(".")[-1],
    }


REPORT = []  # every out comparison of the session, for the parity report


def rel_fro(gpu: np.ndarray, ref: np.ndarray) -> float:
    floor = 1e-3 * math.sqrt(ref.size)
    return float(np.linalg.norm((gpu - ref).ravel()) / max(np.linalg.norm(ref.ravel()), floor))


def assert_out(gpu, ref, what="out", dtype=torch.bfloat16):
    r = out_report(gpu, ref, dtype)
    r["what"] = what
    r["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    REPORT.append(r)
    say(f"  {what}: max abs err {r['strict_max']:.3e}, rounding floor max {r['floor_max']:.3e}, "
        f"exempt {r['n_exempt']} of {r['n']} ({r['dtype']})")
    assert r["n_fail"] == 0, f"{what}: {r['n_fail']} elements beyond 1e-2 and not exempt ({r})"


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

