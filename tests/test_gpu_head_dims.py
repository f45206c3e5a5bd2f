"""Head dims other than 64 and 128, forward and backward, against the oracle.

A head dim E (a multiple of 8, at most 128) runs in the head-dim-64 kernels
when E <= 64 and in the head-dim-128 kernels otherwise; the missing columns
read as zeros and are never stored.  nvFuser issue 2278 notes that Flash
Attention does not cover every input case; here the same kernels take them.
Cases cover causal masking with dropout, BSHE strides, an additive bias, fp16,
ragged lengths and every forward workgroup shape.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_grads, assert_lse, assert_out, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, H, Sq, Sk, E, layout, causal, p, bias, dtype)
    (2, 3, 300, 300, 32, "BHSE", True, 0.2, False, torch.bfloat16),
    (1, 4, 257, 190, 32, "BSHE", False, 0.0, False, torch.bfloat16),
    (2, 2, 200, 333, 8, "BHSE", True, 0.1, False, torch.bfloat16),
    (1, 3, 130, 130, 40, "BSHE", True, 0.0, True, torch.bfloat16),
    (2, 2, 144, 200, 48, "BHSE", False, 0.15, False, torch.float16),
    (1, 2, 260, 260, 96, "BSHE", True, 0.1, False, torch.bfloat16),
    (2, 2, 129, 300, 120, "BHSE", False, 0.0, True, torch.bfloat16),
    (1, 1, 1, 1, 32, "BHSE", True, 0.0, False, torch.bfloat16),
]


def _run(B, H, Sq, Sk, E, layout, causal, p, with_bias, dtype, seed):
    q, k, v, do = (t.to(dtype) for t in
                   workloads.draw(B, H, Sq, Sk, E, seed, 1.0, "BHSE", device="cuda"))
    if layout == "BSHE":
        q, k, v, do = (workloads.to_layout(t, "BSHE") for t in (q, k, v, do))
        assert q.stride(2) == H * E
    bias = None
    if with_bias:
        pad = (Sk + 7) // 8 * 8
        g = torch.Generator("cpu").manual_seed(seed + 1)
        bias = (torch.randn((1, H, Sq, pad), generator=g) * 2).to(dtype).to("cuda")[..., :Sk]
    rng = (seed * 31, seed * 7)
    sdpa.sdpa_set_rng_state(*rng)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    grads = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, bias=bias)
    torch.cuda.synchronize()
    assert (s, o) == rng
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, causal, None, *rng, bias=bias)
    ref_g = sdpa_ref.bwd(do, q, k, v, p, causal, *rng, None, bias=bias)
    assert_out(host64(out), ref_out, dtype=out.dtype)
    assert_lse(lse.cpu().double().numpy(), ref_lse)
    assert_grads([(n, host64(a), r) for n, a, r in zip(("dq", "dk", "dv"), grads, ref_g)])
    return out, grads


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,p,with_bias,dtype", CASES)
def test_head_dim_parity(B, H, Sq, Sk, E, layout, causal, p, with_bias, dtype):
    say(f"head dim {E}: B{B} H{H} Sq{Sq} Sk{Sk} {layout} causal={causal} p={p} bias={with_bias} "
        f"{str(dtype).split('.')[-1]}")
    _run(B, H, Sq, Sk, E, layout, causal, p, with_bias, dtype, 50 + E)


@pytest.mark.parametrize("shape", [1, 2, 3, 4])
def test_head_dim_32_every_forward_shape(monkeypatch, shape):
    say(f"head dim 32 through forward shape {shape}")
    monkeypatch.setenv("SDPA14_FWD_SHAPE", str(shape))
    _run(1, 2, 600, 600, 32, "BHSE", True, 0.1, False, torch.bfloat16, 90 + shape)


def test_head_dim_32_at_the_benchmarked_sizes():
    say("head dim 32 at b2 h12 s1024 causal")
    _run(2, 12, 1024, 1024, 32, "BHSE", True, 0.0, False, torch.bfloat16, 99)


def test_padded_columns_are_left_untouched():
    # Outputs live in a larger buffer whose extra columns hold a sentinel: the
    # kernels must write the head dim's columns and nothing past them.
    B, H, S, E = 1, 2, 96, 40
    q, k, v, do = workloads.draw(B, H, S, S, E, 98, 1.0, "BHSE", device="cuda")
    big = torch.full((B, H, S, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[..., :E]
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    sdpa.sdpa_fwd(q, k, v, 0.0, True, None, out=out, lse=lse)
    gbig = [torch.full((B, H, S, 64), 5.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    sdpa.sdpa_bwd(do, q, k, v, out, lse, 0.0, True, 0, 0, None, *(t[..., :E] for t in gbig))
    torch.cuda.synchronize()
    assert (big[..., E:] == 7.0).all()
    for t in gbig:
        assert (t[..., E:] == 5.0).all()
    ref_out, _ = sdpa_ref.fwd(q, k, v, 0.0, True)
    assert_out(host64(out), ref_out)
