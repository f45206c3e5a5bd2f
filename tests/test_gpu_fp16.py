"""GPU parity of the fp16 (IEEE half) path against the fp64 oracle.

The same kernels run with half operands (v_mfma_f32_32x32x16_f16) and half
conversions of P, dS and the outputs; everything else (fp32 softmax, Philox
mask, tiling) is shared with bf16.  Inputs are the seeded bf16 draws converted
to half, which is exact for these values, so the oracle sees the same numbers.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_grads, assert_lse, assert_out, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,p,with_bias", [
    (1, 2, 128, 128, 64, "BHSE", True, 0.0, False),
    (2, 3, 200, 200, 64, "BSHE", True, 0.2, False),
    (1, 2, 130, 248, 128, "BHSE", False, 0.0, True),
    (2, 12, 1024, 1024, 64, "BHSE", True, 0.0, False),
])
def test_fp16_parity(B, H, Sq, Sk, E, layout, causal, p, with_bias):
    say(f"fp16 B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} p={p} bias={with_bias}")
    q, k, v, do = (t.to(torch.float16) for t in
                   workloads.draw(B, H, Sq, Sk, E, 22, 1.0, layout, device="cuda"))
    if layout == "BSHE":
        q, k, v, do = (workloads.to_layout(t, "BSHE") for t in (q, k, v, do))
        assert q.stride(2) == H * E
    bias = None
    if with_bias:
        g = torch.Generator("cpu").manual_seed(23)
        bias = (torch.randn((1, H, Sq, Sk), generator=g) * 2).to(torch.float16).to("cuda")
    seed, off = 99, 12
    sdpa.sdpa_set_rng_state(seed, off)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    dq, dk, dv = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, bias=bias)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16 and dq.dtype == torch.float16
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off, bias=bias)
    ref_dq, ref_dk, ref_dv = sdpa_ref.bwd(do, q, k, v, p, causal, seed, off, None, bias=bias)
    assert_out(host64(out), ref_out, dtype=out.dtype)
    assert_lse(lse.cpu().double().numpy(), ref_lse)
    assert_grads([("dq", host64(dq), ref_dq), ("dk", host64(dk), ref_dk), ("dv", host64(dv), ref_dv)])
