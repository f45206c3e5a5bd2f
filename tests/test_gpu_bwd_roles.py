"""The backward main pass as one launch or as two (dK/dV blocks, then dQ blocks).

Large problems without dropout or a bias run the two workgroup roles as two
launches, the dQ one with a two-stage ring; SDPA14_BWD_ROLES forces either
form.  Both compute the same sums in the same order, so their gradients must
be bitwise equal, and the two-launch form is held to the oracle on shapes
that span ragged tiles, causal Sq > Sk and Sq < Sk, BSHE strides, fp16 and
padded head dims.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_grads, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = [
    # (B, H, Sq, Sk, E, layout, causal, dtype)
    (2, 3, 257, 200, 64, "BSHE", True, torch.bfloat16),
    (1, 2, 190, 700, 64, "BHSE", False, torch.bfloat16),
    (2, 2, 130, 300, 128, "BHSE", True, torch.bfloat16),
    (1, 3, 300, 129, 128, "BSHE", True, torch.float16),
    (2, 2, 200, 200, 40, "BHSE", True, torch.bfloat16),
    (1, 2, 96, 333, 96, "BHSE", False, torch.bfloat16),
]


def _bwd(monkeypatch, roles, do, q, k, v, out, lse, causal):
    monkeypatch.setenv("SDPA14_BWD_ROLES", str(roles))
    g = sdpa.sdpa_bwd(do, q, k, v, out, lse, 0.0, causal, 0, 0)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,dtype", CASES)
def test_one_and_two_launches_agree_and_match_the_oracle(monkeypatch, B, H, Sq, Sk, E, layout,
                                                          causal, dtype):
    say(f"backward roles: B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} {dtype}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 90, 1.0, layout, device="cuda")
    q, k, v, do = (t.to(dtype) for t in (q, k, v, do))
    out, lse, _, _ = sdpa.sdpa_fwd(q, k, v, 0.0, causal)
    one = _bwd(monkeypatch, 1, do, q, k, v, out, lse, causal)
    two = _bwd(monkeypatch, 2, do, q, k, v, out, lse, causal)
    for name, a, b in zip(("dq", "dk", "dv"), one, two):
        assert torch.equal(a, b), f"{name} differs between one and two launches"
    ref = sdpa_ref.bwd(do, q, k, v, 0.0, causal)
    assert_grads([(n, host64(g), r) for n, g, r in zip(("dq", "dk", "dv"), two, ref)])


def test_dropout_and_bias_keep_one_launch(monkeypatch):
    # Two launches are not taken with dropout or a bias; forcing them changes nothing.
    B, H, S, E = 1, 2, 160, 128
    q, k, v, do = workloads.draw(B, H, S, S, E, 91, 1.0, "BHSE", device="cuda")
    bias = torch.randn((S, S), generator=torch.Generator("cpu").manual_seed(92)).to(
        torch.bfloat16).to("cuda")
    sdpa.sdpa_set_rng_state(5, 0)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, 0.2, True, bias=bias)
    res = []
    for roles in (1, 2):
        monkeypatch.setenv("SDPA14_BWD_ROLES", str(roles))
        res.append(sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, 0.2, True, s, o, bias=bias))
        torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_two_launches_chosen_for_a_large_problem(monkeypatch):
    # 8 x 16 x 2048^2 causal: 4096 blocks per role, past the point where the
    # library takes two launches by itself.  One head of each of the eight
    # XCD head groups is checked against the oracle, and the whole gradient
    # against the one-launch form.
    monkeypatch.delenv("SDPA14_BWD_ROLES", raising=False)
    B, H, S, E = 8, 16, 2048, 64
    q, k, v, do = workloads.draw(B, H, S, S, E, 93, 1.0, "BHSE", device="cuda")
    out, lse, _, _ = sdpa.sdpa_fwd(q, k, v, 0.0, True)
    auto = sdpa.sdpa_bwd(do, q, k, v, out, lse, 0.0, True, 0, 0)
    one = _bwd(monkeypatch, 1, do, q, k, v, out, lse, True)
    for a, b in zip(auto, one):
        assert torch.equal(a, b)
    heads = [((16 * g + 5) // H, (16 * g + 5) % H) for g in range(8)]
    qc, kc, vc, dc = (t.cpu() for t in (q, k, v, do))
    ref = sdpa_ref.bwd(dc, qc, kc, vc, 0.0, True, heads=heads)
    sel = (tuple(b for b, _ in heads), tuple(h for _, h in heads))
    assert_grads([(n, host64(g)[sel], r[sel]) for n, g, r in zip(("dq", "dk", "dv"), auto, ref)])


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,dtype", CASES[:4])
@pytest.mark.parametrize("p", [0.0, 0.1])
def test_the_computed_order_gives_the_same_gradients(monkeypatch, B, H, Sq, Sk, E, layout,
                                                     causal, dtype, p):
    # Problems of more than 1024 key plus query blocks per head deal their
    # blocks in an order computed from the block index (alternating roles, or
    # one role per launch) instead of the host-built table; SDPA14_BWD_ORDER=1
    # takes that path at any size.  A block is computed the same way whichever
    # workgroup takes it, so the gradients are bitwise those of the table order.
    say(f"backward order: B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} {dtype} p={p}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 93, 1.0, layout, device="cuda")
    q, k, v, do = (t.to(dtype) for t in (q, k, v, do))
    sdpa.sdpa_set_rng_state(5, 64)
    out, lse, s, o = sdpa.sdpa_fwd(q, k, v, p, causal)
    for roles in (1, 2):
        monkeypatch.setenv("SDPA14_BWD_ROLES", str(roles))
        monkeypatch.delenv("SDPA14_BWD_ORDER", raising=False)
        table = sdpa.sdpa_bwd(do, q, k, v, out, lse, p, causal, s, o)
        monkeypatch.setenv("SDPA14_BWD_ORDER", "1")
        computed = sdpa.sdpa_bwd(do, q, k, v, out, lse, p, causal, s, o)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), table, computed):
            assert torch.equal(a, b), f"{name} differs between the two orders ({roles} launch(es))"
    monkeypatch.delenv("SDPA14_BWD_ORDER", raising=False)
    monkeypatch.delenv("SDPA14_BWD_ROLES", raising=False)
    ref = sdpa_ref.bwd(do, q, k, v, p, causal, s, o)
    assert_grads([(n, host64(g), r) for n, g, r in zip(("dq", "dk", "dv"), computed, ref)])
