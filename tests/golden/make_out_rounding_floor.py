"""Writes out_rounding_floor.txt: how close a 16-bit output can get to the oracle.

For every named workload the oracle's forward output O_ref (fp64) is rounded
to bf16, the output format, and the script records the largest rounding floor
|round(O_ref) - O_ref|, the number of elements whose floor alone exceeds the
1e-2 bar on out, and the number the parity tests may exempt (floor plus the
pre-rounding budget 2^-8 |O_ref| above 1e-2).  Only the oracle and the input
generators are used.

    python tests/golden/make_out_rounding_floor.py
"""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import sdpa_ref  # noqa: E402
from tests._util import OUT_TOL, neighbours  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "out_rounding_floor.txt")


def floor_stats(w):
    q, k, v, _ = workloads.make_inputs(w, device="cpu")
    fmax, n_floor, n_elig, amax = 0.0, 0, 0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            o, _ = sdpa_ref.fwd(q, k, v, w.dropout_p, w.causal, None, w.rng_seed, w.rng_offset,
                                heads=[(b, h)])
            o = o[b, h]
            lo, hi = neighbours(o, torch.bfloat16)
            fl = np.minimum(o - lo, hi - o)
            fmax = max(fmax, float(fl.max()))
            amax = max(amax, float(np.abs(o).max()))
            n_floor += int((fl > OUT_TOL).sum())
            n_elig += int((fl + np.ldexp(np.abs(o), -8) > OUT_TOL).sum())
    return fmax, n_floor, n_elig, amax


def main():
    lines = ["# workload  elements  max|O_ref|  max_floor  n_floor_over_1e-2  n_exemptible"]
    for name, w in workloads.WORKLOADS.items():
        fmax, n_floor, n_elig, amax = floor_stats(w)
        n = w.B * w.H * w.Sq * w.E
        lines.append(f"{name} {n} {amax:.6f} {fmax:.6e} {n_floor} {n_elig}")
        print(lines[-1], flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
