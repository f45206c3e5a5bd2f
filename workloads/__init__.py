"""Seeded synthetic inputs for the fused SDPA path.

This module holds no attention arithmetic: it only draws inputs.  Both the HIP
library's callers and the CPU oracle's callers take their inputs from here, so
the two sides see bit-identical bf16 values.

Recipe (the same for every workload):

* ``torch.Generator('cpu').manual_seed(gen_seed)``;
* draw float32 ``randn`` in logical [B, H, S, E] order: Q, K, V, dO;
* K is multiplied by ``k_scale`` in float32 (3 for the wide-score workload);
* each tensor is rounded once to bfloat16 (round to nearest even);
* BSHE layout (memory [b, s, h, e], logical [b, h, s, e]) is materialised as
  ``x.transpose(1, 2).contiguous().transpose(1, 2)``, so its logical values
  equal the BHSE draw.

The shapes are those of the nvFuser PR "DID loop split for SDPA"
(``test_sdpa_loop_split``: b=2, h=12, s=1024, e=768 so head dim 64, bf16,
BHSE and BSHE stride orders, causal), plus a tiny case, a wide-score BSHE case,
a ragged dropout case with more than 64 keys (the regression of the PyTorch PR
"REDO of dropout support for mem eff") and a long cross-attention case with
head dim 128.
"""

from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    E: int
    layout: str  # "BHSE" or "BSHE"
    causal: bool
    dropout_p: float
    gen_seed: int
    k_scale: float = 1.0
    rng_seed: int = 0  # Philox seed set before the forward (dropout only)
    rng_offset: int = 0

    @property
    def scale(self) -> float:
        return self.E ** -0.5

    def fwd_flops(self) -> float:
        """Counted forward FLOPs: 4*B*H*Sq*Sk*E, halved when causal."""
        f = 4.0 * self.B * self.H * self.Sq * self.Sk * self.E
        return f * 0.5 if self.causal else f

    def bwd_flops(self) -> float:
        """Counted backward FLOPs: 2.5 x forward (five products of the same size)."""
        return 2.5 * self.fwd_flops()


WORKLOADS = {
    "tiny_causal": Workload("tiny_causal", 1, 2, 128, 128, 64, "BHSE", True, 0.0, 1),
    "b2_h12_s1024_d64_causal": Workload("b2_h12_s1024_d64_causal", 2, 12, 1024, 1024, 64,
                                        "BHSE", True, 0.0, 2),
    "tiny_bshe_wide_scores": Workload("tiny_bshe_wide_scores", 1, 2, 128, 128, 64, "BSHE",
                                      False, 0.0, 3, k_scale=3.0),
    "b4_h16_s1000_dropout_causal": Workload("b4_h16_s1000_dropout_causal", 4, 16, 1000, 1000,
                                            64, "BHSE", True, 0.1, 4, rng_seed=1234,
                                            rng_offset=0),
    "b1_h32_q4096_k8192_d128_cross": Workload("b1_h32_q4096_k8192_d128_cross", 1, 32, 4096,
                                              8192, 128, "BHSE", False, 0.0, 5),
}

# Numbered in the order the workloads are listed (1..5).
BY_INDEX = {i + 1: w for i, w in enumerate(WORKLOADS.values())}


def to_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    """Give a logical [B, H, S, E] tensor the requested memory layout."""
    if layout == "BHSE":
        return x.contiguous()
    if layout == "BSHE":
        return x.transpose(1, 2).contiguous().transpose(1, 2)
    raise ValueError(f"unknown layout {layout!r}")


def draw(B: int, H: int, Sq: int, Sk: int, E: int, gen_seed: int, k_scale: float = 1.0,
         layout: str = "BHSE", device="cpu"):
    """Seeded bf16 (q, k, v, dout) with the recipe above."""
    g = torch.Generator("cpu").manual_seed(gen_seed)
    q = torch.randn((B, H, Sq, E), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Sk, E), generator=g, dtype=torch.float32)
    if k_scale != 1.0:
        k = k * k_scale
    v = torch.randn((B, H, Sk, E), generator=g, dtype=torch.float32)
    dout = torch.randn((B, H, Sq, E), generator=g, dtype=torch.float32)
    out = []
    for x in (q, k, v, dout):
        x = to_layout(x.to(torch.bfloat16), layout)
        if device != "cpu":
            x = to_layout(x.to(device), layout)
        out.append(x)
    return tuple(out)


def make_inputs(w: Workload, device="cpu"):
    """Inputs of a named workload: (q, k, v, dout), bf16, in its layout."""
    return draw(w.B, w.H, w.Sq, w.Sk, w.E, w.gen_seed, w.k_scale, w.layout, device)
