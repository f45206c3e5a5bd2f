"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself:

* closed forms -- the causal first row, zero queries (uniform attention), one key;
* invariants -- softmax rows sum to one, sum_j dK_j = 0, sum_j dV_j = sum_i dO_i;
* an independent formula -- log-sum-exp without max subtraction;
* brute force -- central finite differences of L = sum(dO * O), with dropout;
* a library routine -- PyTorch's own CPU float64 attention and autograd.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import philox_ref, sdpa_ref


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _case(B, H, Sq, Sk, E, seed=0, kscale=1.0):
    q = _rand((B, H, Sq, E), seed)
    k = _rand((B, H, Sk, E), seed + 1, kscale)
    v = _rand((B, H, Sk, E), seed + 2)
    do = _rand((B, H, Sq, E), seed + 3)
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k, v, _ = _case(1, 1, 37, 53, 16, seed=1, kscale=3.0)
    s = sdpa_ref.resolve_scale(None, 16)
    valid = sdpa_ref.valid_mask(37, 53, causal)
    _, _, P = sdpa_ref.head_forward(q[0, 0], k[0, 0], v[0, 0], s, valid, np.ones((37, 53)))
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert (P[~valid] == 0).all()


def test_default_scale():
    assert sdpa_ref.resolve_scale(None, 64) == 0.125
    assert sdpa_ref.resolve_scale(float("nan"), 128) == 1 / math.sqrt(128)
    assert sdpa_ref.resolve_scale(0.3, 64) == 0.3


@pytest.mark.parametrize("p", [0.0, 0.25])
def test_causal_first_row(p):
    # Row 0 attends to key 0 only: O_0 = v_0 * M_00 and LSE_0 = s * q_0 . k_0.
    B, H, Sq, Sk, E = 2, 3, 9, 11, 8
    q, k, v, _ = _case(B, H, Sq, Sk, E, seed=2)
    seed, off = 1234, 77
    out, lse = sdpa_ref.fwd(q, k, v, p, True, None, seed, off)
    s = 1 / math.sqrt(E)
    keep = philox_ref.keep_mask(seed, off, p, B, H, Sq, Sk) if p > 0 else np.ones((B, H, Sq, Sk))
    for b in range(B):
        for h in range(H):
            m = keep[b, h, 0, 0] / (1 - p) if p > 0 else 1.0
            assert np.allclose(out[b, h, 0], v[b, h, 0] * m, atol=1e-14)
            assert math.isclose(lse[b, h, 0], s * float(q[b, h, 0] @ k[b, h, 0]), abs_tol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_equals_direct_log_sum_exp(causal):
    B, H, Sq, Sk, E = 1, 2, 33, 40, 64
    q, k, v, _ = _case(B, H, Sq, Sk, E, seed=3, kscale=3.0)
    _, lse = sdpa_ref.fwd(q, k, v, 0.0, causal)
    s = 1 / math.sqrt(E)
    for h in range(H):
        S = s * q[0, h] @ k[0, h].T
        for i in range(Sq):
            n = i + 1 if causal else Sk
            direct = math.log(sum(math.exp(S[i, j]) for j in range(n)))
            assert math.isclose(lse[0, h, i], direct, rel_tol=0, abs_tol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_zero_queries_give_uniform_attention(causal, p):
    # Q = 0 makes every valid score 0: P is uniform over the n_i valid keys, so
    # O_i = (1/n_i) sum_{valid j} M_ij v_j and LSE_i = ln(n_i).
    B, H, Sq, Sk, E = 2, 2, 13, 10, 8
    _, k, v, _ = _case(B, H, Sq, Sk, E, seed=4)
    q = np.zeros((B, H, Sq, E))
    seed, off = 42, 5
    out, lse = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off)
    keep = philox_ref.keep_mask(seed, off, p, B, H, Sq, Sk)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                n = min(i + 1, Sk) if causal else Sk
                w = keep[b, h, i, :n] / (1 - p) if p > 0 else np.ones(n)
                expect = (w[:, None] * v[b, h, :n]).sum(axis=0) / n
                assert np.allclose(out[b, h, i], expect, atol=1e-13)
                assert math.isclose(lse[b, h, i], math.log(n), abs_tol=1e-13)


def test_single_key():
    # Sk = 1: every row copies v_0; dQ = dK = 0; dV = sum_i dO_i.
    B, H, Sq, E = 1, 2, 7, 8
    q, k, v, do = _case(B, H, Sq, 1, E, seed=5)
    for causal in (False, True):
        out, _ = sdpa_ref.fwd(q, k, v, 0.0, causal)
        assert np.allclose(out, np.broadcast_to(v, out.shape), atol=1e-14)
        dq, dk, dv = sdpa_ref.bwd(do, q, k, v, 0.0, causal)
        assert np.allclose(dq, 0, atol=1e-13) and np.allclose(dk, 0, atol=1e-13)
        assert np.allclose(dv[:, :, 0], do.sum(axis=2), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    B, H, Sq, Sk, E = 1, 2, 24, 31, 16
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=6)
    out, _ = sdpa_ref.fwd(q, k, v, 0.0, causal)
    dq, dk, dv = sdpa_ref.bwd(do, q, k, v, 0.0, causal)
    # Rows of dS sum to zero, so sum_j dK_j = s * sum_i (sum_j dS_ij) q_i = 0.
    assert np.allclose(dk.sum(axis=2), 0, atol=1e-12)
    # With p = 0 the columns of P^T sum to one over each row i.
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # D = sum_j P dP equals rowsum(dO * O).
    s = 1 / math.sqrt(E)
    valid = sdpa_ref.valid_mask(Sq, Sk, causal)
    for h in range(H):
        *_, D = sdpa_ref.head_backward(do[0, h], q[0, h], k[0, h], v[0, h], s, valid,
                                       np.ones((Sq, Sk)))
        assert np.allclose(D, (do[0, h] * out[0, h]).sum(axis=1), atol=1e-12)


@pytest.mark.parametrize("Sq", [1, 3, 5])
@pytest.mark.parametrize("Sk", [1, 4, 7])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_finite_differences(Sq, Sk, causal, p):
    B, H, E = 1, 2, 4
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=10 + Sq * 7 + Sk)
    seed, off = 2024, 3

    def loss(qq, kk, vv):
        out, _ = sdpa_ref.fwd(qq, kk, vv, p, causal, None, seed, off)
        return float((do * out).sum())

    dq, dk, dv = sdpa_ref.bwd(do, q, k, v, p, causal, seed, off)
    step = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                       - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * step)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-30)
        assert err <= 1e-6 or np.abs(fd - g).max() < 1e-8, (name, err)


def _torch_attention(q, k, v, do, causal, scale):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale)
    out.backward(torch.tensor(do, dtype=torch.float64))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("shape,causal,kscale", [
    ((1, 2, 128, 128, 64), True, 1.0),     # tiny causal workload's shape
    ((1, 2, 128, 128, 64), False, 3.0),    # wide-score workload's shape
    ((1, 2, 64, 128, 128), False, 1.0),    # reduced long cross-attention, head dim 128
    ((1, 1, 48, 80, 32), True, 1.0),       # causal with Sq < Sk (top-left)
    ((2, 1, 80, 48, 32), True, 1.0),       # causal with Sq > Sk (top-left)
])
def test_against_torch_cpu_float64(shape, causal, kscale):
    B, H, Sq, Sk, E = shape
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=20, kscale=kscale)
    s = 1 / math.sqrt(E)
    out, _ = sdpa_ref.fwd(q, k, v, 0.0, causal)
    dq, dk, dv = sdpa_ref.bwd(do, q, k, v, 0.0, causal)
    t_out, t_dq, t_dk, t_dv = _torch_attention(q, k, v, do, causal, s)
    for a, b in ((out, t_out), (dq, t_dq), (dk, t_dk), (dv, t_dv)):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11)


def test_workload_inputs_feed_the_oracle():
    # The bf16 workload tensors are widened exactly; BSHE holds the BHSE values.
    w = workloads.WORKLOADS["tiny_bshe_wide_scores"]
    q, k, v, do = workloads.make_inputs(w)
    assert q.dtype == torch.bfloat16 and q.stride()[-1] == 1
    assert q.stride(2) == w.H * w.E  # memory [b, s, h, e]
    q2, k2, v2, do2 = workloads.draw(w.B, w.H, w.Sq, w.Sk, w.E, w.gen_seed, w.k_scale, "BHSE")
    for a, b in ((q, q2), (k, k2), (v, v2), (do, do2)):
        assert torch.equal(a, b)
    out_a, lse_a = sdpa_ref.fwd(q, k, v, 0.0, w.causal)
    out_b, lse_b = sdpa_ref.fwd(q2, k2, v2, 0.0, w.causal)
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_rows_and_heads_subsets_match_full():
    B, H, Sq, Sk, E = 2, 2, 21, 19, 8
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=30)
    for p, causal in ((0.0, True), (0.2, True), (0.2, False)):
        out, lse = sdpa_ref.fwd(q, k, v, p, causal, None, 9, 11)
        rows = [0, 5, 20]
        o_r, l_r = sdpa_ref.fwd_rows(q, k, v, 1, 0, rows, p, causal, None, 9, 11)
        assert np.array_equal(o_r, out[1, 0, rows]) and np.array_equal(l_r, lse[1, 0, rows])
        out_h, _ = sdpa_ref.fwd(q, k, v, p, causal, None, 9, 11, heads=[(1, 1)])
        assert np.array_equal(out_h[1, 1], out[1, 1]) and np.isnan(out_h[0, 0]).all()


# ---- additive bias ----------------------------------------------------------

def test_bias_constant_along_keys_shifts_only_the_lse():
    # softmax is invariant to adding c_i to every score of row i: O and the
    # gradients stay, LSE_i moves by c_i.
    B, H, Sq, Sk, E = 1, 2, 9, 13, 8
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=40)
    c = _rand((B, H, Sq, 1), 41, 3.0)
    for causal in (False, True):
        o0, l0 = sdpa_ref.fwd(q, k, v, 0.0, causal)
        o1, l1 = sdpa_ref.fwd(q, k, v, 0.0, causal, bias=np.broadcast_to(c, (B, H, Sq, Sk)))
        assert np.allclose(o1, o0, rtol=1e-12, atol=1e-13)
        assert np.allclose(l1, l0 + c[..., 0], rtol=1e-12, atol=1e-12)
        g0 = sdpa_ref.bwd(do, q, k, v, 0.0, causal)
        g1 = sdpa_ref.bwd(do, q, k, v, 0.0, causal, bias=np.broadcast_to(c, (B, H, Sq, Sk)))
        for a, b in zip(g0, g1):
            assert np.allclose(a, b, rtol=1e-11, atol=1e-12)


def test_causal_mask_as_a_minus_infinity_bias():
    # Non-causal attention with -inf above the diagonal is causal attention.
    B, H, Sq, Sk, E = 2, 1, 11, 11, 8
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=42)
    bias = np.where(np.arange(Sk)[None, :] > np.arange(Sq)[:, None], -np.inf, 0.0)
    o_b, l_b = sdpa_ref.fwd(q, k, v, 0.0, False, bias=bias)
    o_c, l_c = sdpa_ref.fwd(q, k, v, 0.0, True)
    assert np.allclose(o_b, o_c, rtol=1e-13, atol=1e-14) and np.allclose(l_b, l_c)
    for a, b in zip(sdpa_ref.bwd(do, q, k, v, 0.0, False, bias=bias),
                    sdpa_ref.bwd(do, q, k, v, 0.0, True)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("shape,bshape,causal", [
    ((1, 2, 48, 64, 32), (1, 2, 48, 64), False),
    ((2, 2, 40, 40, 16), (1, 2, 40, 40), True),
    ((1, 3, 32, 56, 16), (32, 56), True),
])
def test_bias_against_torch_cpu_float64(shape, bshape, causal):
    # PyTorch's float attn_mask is an additive term on the scaled scores.
    B, H, Sq, Sk, E = shape
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=44)
    bias = _rand(bshape, 45, 2.0)
    s = 1 / math.sqrt(E)
    out, _ = sdpa_ref.fwd(q, k, v, 0.0, causal, bias=bias)
    dq, dk, dv = sdpa_ref.bwd(do, q, k, v, 0.0, causal, bias=bias)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = torch.tensor(np.broadcast_to(bias, (B, H, Sq, Sk)), dtype=torch.float64)
    if causal:
        tri = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        mask = mask.masked_fill(~tri, -math.inf)
    t_out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s)
    t_out.backward(torch.tensor(do, dtype=torch.float64))
    for a, b in ((out, t_out.detach().numpy()), (dq, tq.grad.numpy()), (dk, tk.grad.numpy()),
                 (dv, tv.grad.numpy())):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11)


def test_bias_finite_differences_with_dropout():
    B, H, Sq, Sk, E = 1, 1, 4, 6, 4
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=46)
    bias = _rand((Sq, Sk), 47, 1.5)
    p, seed, off = 0.3, 7, 5

    def loss(qq, kk, vv):
        out, _ = sdpa_ref.fwd(qq, kk, vv, p, True, None, seed, off, bias=bias)
        return float((do * out).sum())

    grads = sdpa_ref.bwd(do, q, k, v, p, True, seed, off, bias=bias)
    step = 1e-6
    for i, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xs = [q, k, v]
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            xs_p, xs_m = list(xs), list(xs)
            xs_p[i], xs_m[i] = xp, xm
            fd[idx] = (loss(*xs_p) - loss(*xs_m)) / (2 * step)
        g = grads[i]
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-30)
        assert err <= 1e-6 or np.abs(fd - g).max() < 1e-8, (i, err)


# ---- bias gradient (step 9 of the oracle) ----------------------------------------


@pytest.mark.parametrize("Sq,Sk", [(3, 4), (5, 7), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_dbias_finite_differences(Sq, Sk, causal, p):
    # Central differences of sum(dO * O) in every bias entry of a full
    # [B, H, Sq, Sk] bias; entries a row cannot see must get exactly zero.
    B, H, E = 1, 2, 4
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=60 + Sq * 5 + Sk)
    bias = _rand((B, H, Sq, Sk), 61 + Sq, 1.5)
    seed, off = 99, 11

    def loss(bb):
        out, _ = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off, bias=bb)
        return float((do * out).sum())

    *_, db = sdpa_ref.bwd(do, q, k, v, p, causal, seed, off, bias=bias, want_dbias=True)
    step = 1e-6
    fd = np.zeros_like(bias)
    for idx in np.ndindex(bias.shape):
        bp, bm = bias.copy(), bias.copy()
        bp[idx] += step
        bm[idx] -= step
        fd[idx] = (loss(bp) - loss(bm)) / (2 * step)
    err = np.linalg.norm(fd - db) / max(np.linalg.norm(db), 1e-30)
    assert err <= 1e-6 or np.abs(fd - db).max() < 1e-8, err
    hidden = ~sdpa_ref.valid_mask(Sq, Sk, causal)
    assert (db[:, :, hidden] == 0).all()


@pytest.mark.parametrize("shape,bshape,causal", [
    ((1, 2, 48, 64, 32), (1, 2, 48, 64), False),
    ((2, 2, 40, 40, 16), (1, 2, 40, 40), True),
    ((2, 3, 32, 56, 16), (32, 56), True),
])
def test_dbias_against_torch_attn_mask_grad(shape, bshape, causal):
    # PyTorch's float attn_mask with requires_grad: its gradient is the bias
    # gradient summed over the dimensions the mask broadcasts.
    B, H, Sq, Sk, E = shape
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=62)
    bias = _rand(bshape, 63, 2.0)
    s = 1 / math.sqrt(E)
    *_, db = sdpa_ref.bwd(do, q, k, v, 0.0, causal, bias=bias, want_dbias=True)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    tb = torch.tensor(bias, dtype=torch.float64, requires_grad=True)
    mask = tb.expand(B, H, Sq, Sk)
    if causal:
        tri = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        mask = mask.masked_fill(~tri, -math.inf)
    t_out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s)
    t_out.backward(torch.tensor(do, dtype=torch.float64))
    summed = db.reshape((B, H, Sq, Sk))
    lead = len(summed.shape) - len(bshape)
    summed = summed.sum(axis=tuple(range(lead)))
    for ax, n in enumerate(bshape):
        if n == 1:
            summed = summed.sum(axis=ax, keepdims=True)
    assert np.allclose(summed, tb.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_dbias_rows_sum_to_zero_with_dropout():
    # sum_j dS_ij = sum_j P_ij dP_ij - D_i sum_j P_ij = D_i - D_i = 0 on every row.
    B, H, Sq, Sk, E = 2, 2, 37, 53, 16
    q, k, v, do = _case(B, H, Sq, Sk, E, seed=64)
    bias = _rand((B, H, Sq, Sk), 65, 1.0)
    *_, db = sdpa_ref.bwd(do, q, k, v, 0.25, True, 3, 8, bias=bias, want_dbias=True)
    assert np.abs(db.sum(axis=3)).max() < 1e-12 * np.abs(db).max() * Sk


# ---- non-finite inputs --------------------------------------------------------
# The definition fixes what a NaN or an infinity does: only the outputs whose
# defining sums contain it are NaN.  A query row enters only its own row of S;
# a key row enters column j of S, which a causal row i < j never reads.


@pytest.mark.parametrize("bad", [math.nan, math.inf, -math.inf])
def test_non_finite_query_row_poisons_only_its_row(bad):
    q, k, v, _ = workloads.draw(1, 2, 40, 40, 8, 37, 1.0, "BHSE")
    o_ref, l_ref = sdpa_ref.fwd(q, k, v, 0.0, True)
    q2 = q.clone()
    q2[0, 1, 17, 3] = bad
    o, l = sdpa_ref.fwd(q2, k, v, 0.0, True)
    assert np.isnan(o[0, 1, 17]).all() and not np.isfinite(l[0, 1, 17])
    keep = np.ones(40, dtype=bool)
    keep[17] = False
    assert np.array_equal(o[0, 1, keep], o_ref[0, 1, keep])
    assert np.array_equal(l[0, 1, keep], l_ref[0, 1, keep])
    assert np.array_equal(o[0, 0], o_ref[0, 0]) and np.array_equal(l[0, 0], l_ref[0, 0])


def test_nan_key_row_poisons_the_rows_that_see_it():
    q, k, v, _ = workloads.draw(1, 1, 40, 40, 8, 38, 1.0, "BHSE")
    o_ref, l_ref = sdpa_ref.fwd(q, k, v, 0.0, True)
    k2 = k.clone()
    k2[0, 0, 25, 0] = math.nan
    o, l = sdpa_ref.fwd(q, k2, v, 0.0, True)
    assert np.isnan(o[0, 0, 25:]).all() and np.isnan(l[0, 0, 25:]).all()
    assert np.array_equal(o[0, 0, :25], o_ref[0, 0, :25])
    assert np.array_equal(l[0, 0, :25], l_ref[0, 0, :25])


def test_out_rounding_floor_file_matches_the_oracle():
    # tests/golden/out_rounding_floor.txt is written by make_out_rounding_floor.py
    # from the oracle alone; re-derive the small workloads' lines here.
    import os

    from tests.golden import make_out_rounding_floor as mk

    rows = {}
    with open(mk.OUT) as f:
        for line in f:
            if not line.startswith("#"):
                name, *vals = line.split()
                rows[name] = vals
    assert set(rows) == set(workloads.WORKLOADS)
    for name in ("tiny_causal", "tiny_bshe_wide_scores"):
        fmax, n_floor, n_elig, amax = mk.floor_stats(workloads.WORKLOADS[name])
        n, a, f, nf, ne = rows[name]
        assert float(a) == pytest.approx(amax, rel=1e-6)
        assert float(f) == pytest.approx(fmax, rel=1e-6)
        assert (int(nf), int(ne)) == (n_floor, n_elig)
    # No named workload has an element that a bf16 output cannot bring within 1e-2.
    assert all(int(v[3]) == 0 for v in rows.values())
    assert os.path.basename(mk.OUT) == "out_rounding_floor.txt"
