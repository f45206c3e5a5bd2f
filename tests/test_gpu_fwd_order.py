"""The causal split forward with and without its dispatch table.

When the whole grid of the split launch is resident, a host-built table says
which tile each workgroup takes, so that long and short tiles share a compute
unit (per XCD when B*H is a multiple of 8, one entry per workgroup otherwise).
Placement must not change a value: every tile runs the same code on the same
rows wherever it lands.  Each case runs the launch twice from the same RNG
state, with the table and with ``SDPA14_FWD_ORDER=1`` (the default order), and
asks for bitwise equal O and LSE; the outputs start as NaN, so every element
must be written.  The cases cover both table forms, tiles paired and alone,
dropout, an additive bias, fp16, BSHE, a padded head dim and ragged lengths.
Values themselves are held to the oracle by the parity tests.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from tests._util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, H, Sq, Sk, E, layout, p, bias, dtype)
    (2, 12, 1024, 1024, 64, "BHSE", 0.0, False, torch.bfloat16),  # per XCD, paired
    (2, 12, 1024, 1024, 64, "BSHE", 0.1, True, torch.bfloat16),   # per XCD, dropout + bias
    (1, 8, 700, 900, 40, "BSHE", 0.0, False, torch.float16),      # per XCD, every tile alone
    (1, 12, 1536, 1536, 64, "BHSE", 0.0, False, torch.bfloat16),  # one entry per workgroup
    (2, 10, 1000, 1000, 64, "BHSE", 0.2, True, torch.float16),    # the same, dropout + bias
    (2, 16, 832, 832, 64, "BHSE", 0.1, False, torch.bfloat16),    # 512 workgroups: every slot
    (1, 20, 1280, 1280, 64, "BSHE", 0.0, False, torch.bfloat16),  # 500 of 512, one per workgroup
]


def _forward(q, k, v, p, bias, rng):
    B, H, Sq, _ = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    sdpa.sdpa_set_rng_state(*rng)
    sdpa.sdpa_fwd_ext(q, k, v, p, True, bias=bias, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,p,with_bias,dtype", CASES)
def test_dispatch_table_changes_no_value(monkeypatch, B, H, Sq, Sk, E, layout, p, with_bias,
                                         dtype):
    say(f"split forward orders: B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} p={p} "
        f"bias={with_bias} {str(dtype).split('.')[-1]}")
    monkeypatch.setenv("SDPA14_FWD_SHAPE", "4")
    q, k, v, _ = (t.to(dtype) for t in
                  workloads.draw(B, H, Sq, Sk, E, 90, 1.0, layout, device="cuda"))
    bias = None
    if with_bias:
        g = torch.Generator("cpu").manual_seed(91)
        pad = (Sk + 7) // 8 * 8
        bias = (torch.randn((Sq, pad), generator=g) * 2).to(dtype).to("cuda")[..., :Sk]
    rng = (93, 1 << 12)
    out_t, lse_t = _forward(q, k, v, p, bias, rng)
    monkeypatch.setenv("SDPA14_FWD_ORDER", "1")
    out_d, lse_d = _forward(q, k, v, p, bias, rng)
    assert not torch.isnan(out_t).any().item() and not torch.isnan(out_d).any().item()
    assert torch.isfinite(lse_t).all().item() and torch.isfinite(lse_d).all().item()
    assert torch.equal(out_t, out_d), "the dispatch table changed the output"
    assert torch.equal(lse_t, lse_d), "the dispatch table changed the LSE"
