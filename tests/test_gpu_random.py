"""Seeded random configurations, forward and backward, against the oracle.

Each case draws its shape and options from a fixed seed: batch and heads,
query and key lengths from 1 to 400 (so most tiles are ragged), every head
dim the kernels take (multiples of 8 up to 128), BHSE or BSHE strides, causal
or not, dropout, an additive bias of several broadcast shapes, bf16 or fp16,
an explicit softmax scale, outputs given as padded views (whose spare
columns must stay untouched), and the forward workgroup shape and backward
launch form forced through SDPA14_FWD_SHAPE / SDPA14_BWD_ROLES.  The bars are
the same as for the fixed parity cases.
"""

import os
import random

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_grads, assert_lse, assert_out, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N_CASES = 64


def _case(i):
    r = random.Random(9000 + i)
    c = {
        "B": r.choice([1, 2]),
        "H": r.choice([1, 2, 3, 4]),
        "Sq": r.choice([1, 31, 64, 65, 127, 200, 257, r.randint(1, 400), r.randint(1, 400)]),
        "Sk": r.choice([1, 3, 32, 63, 64, 129, 256, r.randint(1, 400), r.randint(1, 400)]),
        "E": 8 * r.randint(1, 16),
        "layout": r.choice(["BHSE", "BSHE"]),
        "causal": r.random() < 0.5,
        "p": r.choice([0.0, 0.0, 0.1, 0.25]),
        "bias": r.choice([None, None, "bhqk", "qk", "1hqk"]),
        "dtype": r.choice([torch.bfloat16, torch.bfloat16, torch.float16]),
        "scale": r.choice([None, None, round(r.uniform(0.03, 0.4), 4)]),
        "fwd_shape": r.choice([0, 0, 1, 2, 3, 4]),
        "bwd_roles": r.choice([0, 0, 1, 2]),
        "seed": 500 + i,
        "pad_out": r.random() < 0.5,
    }
    return c


def _bias(tag, B, H, Sq, Sk, seed, dtype):
    if tag is None:
        return None
    shape = {"bhqk": (B, H, Sq), "qk": (Sq,), "1hqk": (1, H, Sq)}[tag]
    pad = (Sk + 7) // 8 * 8
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape + (pad,), generator=g) * 1.5).to(dtype).to("cuda")[..., :Sk]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i, monkeypatch):
    c = _case(i)
    say(f"random case {i}: {c}")
    B, H, Sq, Sk, E = c["B"], c["H"], c["Sq"], c["Sk"], c["E"]
    monkeypatch.setenv("SDPA14_FWD_SHAPE", str(c["fwd_shape"]))
    monkeypatch.setenv("SDPA14_BWD_ROLES", str(c["bwd_roles"]))
    q, k, v, do = (t.to(c["dtype"]) for t in
                   workloads.draw(B, H, Sq, Sk, E, c["seed"], 1.0, "BHSE", device="cuda"))
    if c["layout"] == "BSHE":
        q, k, v, do = (workloads.to_layout(t, "BSHE") for t in (q, k, v, do))
    bias = _bias(c["bias"], B, H, Sq, Sk, c["seed"] + 1, c["dtype"])
    rng = (c["seed"] * 13 + 1, c["seed"] * 5)
    sdpa.sdpa_set_rng_state(*rng)
    p, causal, scale = c["p"], c["causal"], c["scale"]
    pads = []
    if c["pad_out"]:
        # Outputs as NaN-filled views with 8 spare columns per row: the spare
        # columns must stay NaN.
        def padded(S):
            buf = torch.full((B, H, S, E + 8), float("nan"), dtype=c["dtype"], device="cuda")
            pads.append(buf)
            return buf[..., :E]
        out, dq, dk, dv = padded(Sq), padded(Sq), padded(Sk), padded(Sk)
        out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, scale, out=out, bias=bias)
        sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, scale, dq, dk, dv, bias=bias)
    else:
        out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, scale, bias=bias)
        dq, dk, dv = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, scale, bias=bias)
    torch.cuda.synchronize()
    for buf in pads:
        assert torch.isnan(buf[..., E:]).all().item(), "a kernel wrote into a row's spare columns"
    assert (s, o) == rng
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, causal, scale, *rng, bias=bias)
    ref_dq, ref_dk, ref_dv = sdpa_ref.bwd(do, q, k, v, p, causal, *rng, scale, bias=bias)
    assert_out(host64(out), ref_out, dtype=out.dtype)
    assert_lse(lse.cpu().double().numpy(), ref_lse)
    if not (Sk == 1 or (causal and Sq == 1)):
        assert_grads([("dq", host64(dq), ref_dq), ("dk", host64(dk), ref_dk),
                      ("dv", host64(dv), ref_dv)])
        return
    # Every row sees one key (Sk = 1, or a causal single row): P = 1 there, so
    # dS = P * (dP - D) and with it dq and dk vanish exactly, and a relative
    # error is undefined.  The kernels take D
    # from the stored 16-bit output (D = rowsum(dO * O)), so what they return
    # is dq_i = scale * (dP_i - D_i) * k_0 with |dP_i - D_i| at most
    # sum_e |dO_ie| * |O_ie - O_exact_ie| (plus fp32 rounding); with dropout O
    # is v_0 / (1 - p), which the output format rounds.  Both gradients are
    # held to that bound element by element; dv does not vanish and takes the
    # usual bar.
    assert_grads([("dv", host64(dv), ref_dv)])
    sc = scale if scale is not None else E ** -0.5
    dO64, q64, k64 = host64(do), host64(q), host64(k)
    o_err = abs(host64(out) - ref_out)
    dd = (abs(dO64) * o_err).sum(-1) + 1e-5 * (abs(dO64) * abs(ref_out)).sum(-1)  # [B, H, Sq]
    bound_dq = sc * dd[..., None] * abs(k64[:, :, :1, :]) * 1.01 + 1e-6
    bound_dk = sc * (dd[..., None] * abs(q64)).sum(2, keepdims=True) * 1.01 + 1e-6
    got_dq, got_dk = host64(dq), host64(dk)
    say(f"  one key: max |dq| {abs(got_dq).max():.3e} (bound {bound_dq.max():.3e}), "
        f"max |dk| {abs(got_dk).max():.3e} (bound {bound_dk.max():.3e})")
    assert (abs(got_dq - ref_dq) <= bound_dq).all()
    assert (abs(got_dk - ref_dk) <= bound_dk).all()
