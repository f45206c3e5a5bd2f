"""GPU parity of every forward workgroup shape against the fp64 oracle.

The forward picks its workgroup shape from the problem size: four query
sub-tiles; two sub-tiles with the keys split in two; one sub-tile with the keys
split in four; or (causal, head dim 64) a split launch whose last rows per head
take 32-row, four-share workgroups with 32-key tiles and the rest two by two.
``SDPA14_FWD_SHAPE`` (1-4) forces one.  Each shape has its own merge of key
shares, stage count and dropout-group indexing, so each is checked here on
ragged sizes, both layouts, dropout, an additive bias and fp16.  Head dim 128
has no four-share shape and the split launch is causal with head dim 64;
otherwise asking for them runs the two-by-two shape, which the test also
checks.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_lse, assert_out, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, H, Sq, Sk, E, layout, causal, p, bias, dtype)
    (1, 2, 200, 200, 64, "BHSE", True, 0.2, None, torch.bfloat16),
    (2, 2, 130, 333, 128, "BSHE", False, 0.0, None, torch.bfloat16),
    (1, 3, 257, 129, 64, "BHSE", True, 0.0, "1hqk", torch.bfloat16),
    (2, 1, 96, 300, 64, "BSHE", False, 0.1, "qk", torch.bfloat16),
    (1, 2, 200, 264, 64, "BHSE", True, 0.1, "qk", torch.float16),
    # Both kinds of the split launch (384 rows two by two, 316 in 32-row tiles).
    (1, 2, 700, 700, 64, "BHSE", True, 0.1, "qk", torch.bfloat16),
    (2, 1, 640, 640, 64, "BSHE", True, 0.0, None, torch.float16),
    # Causal with Sq != Sk (top-left: row i sees keys 0..i), both directions.
    (1, 2, 600, 300, 64, "BHSE", True, 0.1, None, torch.bfloat16),
    (1, 2, 520, 900, 64, "BSHE", True, 0.0, "qk", torch.bfloat16),
]


@pytest.mark.parametrize("shape", [1, 2, 3, 4])
@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,p,bias_kind,dtype", CASES)
def test_forward_shape_parity(monkeypatch, shape, B, H, Sq, Sk, E, layout, causal, p, bias_kind,
                              dtype):
    say(f"forward shape {shape}: B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} p={p} "
        f"bias={bias_kind} {str(dtype).split('.')[-1]}")
    monkeypatch.setenv("SDPA14_FWD_SHAPE", str(shape))
    q, k, v, _ = (t.to(dtype) for t in
                  workloads.draw(B, H, Sq, Sk, E, 40 + shape, 1.0, "BHSE", device="cuda"))
    if layout == "BSHE":
        q, k, v = (workloads.to_layout(t, "BSHE") for t in (q, k, v))
    bias = None
    if bias_kind is not None:
        g = torch.Generator("cpu").manual_seed(41)
        lead = (1, H) if bias_kind == "1hqk" else ()
        pad = (Sk + 7) // 8 * 8  # rows of a multiple of 8 elements, as the library requires
        bias = (torch.randn(lead + (Sq, pad), generator=g) * 2).to(dtype).to("cuda")[..., :Sk]
    seed, off = 77, 4096
    sdpa.sdpa_set_rng_state(seed, off)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    torch.cuda.synchronize()
    assert (s, o) == (seed, off)
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off, bias=bias)
    assert_out(host64(out), ref_out, dtype=out.dtype)
    assert_lse(lse.cpu().double().numpy(), ref_lse)
