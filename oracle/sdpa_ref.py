"""Plain fp64 CPU oracle for fused scaled-dot-product attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
and never calls it.  Everything is computed in float64 from the exact values
of the (bf16) inputs, one (batch, head) at a time, with the full score matrix
materialised.

What it computes
----------------
The definition of scaled-dot-product attention, softmax(Q K^T * scale + mask) V
(nvFuser issue 2278, which adds SDPA forward/backward nodes; forum thread
"Scaled_dot_product_attention", opening question), in the forward/backward
split of the nvFuser PR "DID loop split for SDPA" (``test_sdpa_loop_split``):

    attn, log_sumexp, seed, offset = sdpfa_fwd(q, k, v, dropout_p, is_causal, scale)
    dq, dk, dv = sdpfa_bwd(dout, q, k, v, attn, log_sumexp, dropout_p,
                           is_causal, seed, offset, scale)

Steps, per head, with s the scale:

1. ``scale=None`` means 1/sqrt(E) (the PR passes ``None``; reading: the usual
   SDPA default).
2. S = s * Q K^T (+ bias), shape [Sq, Sk].  The optional additive bias is the
   relative-position term the forum thread's opening question asks SDPA to
   accept and the attn_bias support the PyTorch PR "REDO of dropout support
   for mem eff" announces for the memory-efficient kernel; reading: it is added
   to the scaled scores before masking, and a -inf entry hides its key.
3. valid(i, j) = j <= i when causal (reading: top-left alignment, the plain
   lower-triangular mask; it also holds when Sq != Sk), else everywhere.
4. LSE_i = m_i + ln sum_{valid j} exp(S_ij - m_i), m_i the row max over valid
   j: natural log, of the scaled masked scores, before dropout.
5. P_ij = exp(S_ij - LSE_i) on valid entries, 0 elsewhere.
6. M_ij = keep(b, h, i, j) / (1 - p) when p > 0, else 1 (inverted dropout after
   the softmax; keep bits from ``philox_ref``).
7. O = (P * M) V.
8. Backward: dPd = dO V^T; dP = dPd * M; D_i = sum_j P_ij dP_ij;
   dS = P * (dP - D); dQ = s dS K; dK = s dS^T Q; dV = (P * M)^T dO.
9. Bias gradient (the forum thread's opening question wants the relative
   position term trained through SDPA): S = s Q K^T + bias, so the gradient
   with respect to the bias as head (b, h) sees it is dS itself, zero where
   the mask hides a score.  Where the bias broadcasts over a dimension,
   summing dS over it is the broadcast's own backward, outside attention.

D is formed as sum_j P dP, which equals rowsum(dO * O) in exact arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

from . import philox_ref


def resolve_scale(scale, E: int) -> float:
    """Step 1: ``None`` (or NaN) selects 1/sqrt(E)."""
    if scale is None or (isinstance(scale, float) and math.isnan(scale)):
        return 1.0 / math.sqrt(E)
    return float(scale)


def valid_mask(Sq: int, Sk: int, is_causal: bool, rows=None) -> np.ndarray:
    """Step 3: boolean [len(rows), Sk]; causal keeps key j for query i iff j <= i."""
    i = np.arange(Sq) if rows is None else np.asarray(rows)
    if not is_causal:
        return np.ones((len(i), Sk), dtype=bool)
    return np.arange(Sk)[None, :] <= i[:, None]


def dropout_multiplier(p: float, seed: int, offset: int, B: int, H: int, Sq: int, Sk: int,
                       b: int, h: int, rows=None) -> np.ndarray:
    """Step 6: keep/(1-p) with p > 0, else ones; shape [len(rows), Sk]."""
    n = Sq if rows is None else len(rows)
    if p == 0.0:
        return np.ones((n, Sk), dtype=np.float64)
    keep = philox_ref.keep_mask_head(seed, offset, p, B, H, Sq, Sk, b, h, rows=rows)
    return keep.astype(np.float64) / (1.0 - p)


def _as64(x) -> np.ndarray:
    """Exact float64 copy of an array-like (bf16 torch tensors are widened first)."""
    try:  # torch tensor
        import torch  # noqa: F401

        if hasattr(x, "detach"):
            return x.detach().to(device="cpu").double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def head_forward(qh, kh, vh, s: float, valid: np.ndarray, mult: np.ndarray, bias_h=None):
    """Steps 2, 4, 5, 7 on one head.  Returns (O [Sq,E], LSE [Sq], P [Sq,Sk])."""
    S = s * (qh @ kh.T)
    if bias_h is not None:
        S = S + bias_h
    masked = np.where(valid, S, -np.inf)
    m = masked.max(axis=1)
    lse = m + np.log(np.exp(masked - m[:, None]).sum(axis=1))
    P = np.where(valid, np.exp(S - lse[:, None]), 0.0)
    out = (P * mult) @ vh
    return out, lse, P


def head_backward(dOh, qh, kh, vh, s: float, valid: np.ndarray, mult: np.ndarray, bias_h=None,
                  want_ds: bool = False):
    """Steps 2-8 on one head.  Returns (dQ, dK, dV, D), and dS last with
    ``want_ds`` (step 9: the bias gradient).  The bias enters through P only:
    S = s Q K^T + bias, so dQ and dK keep their form."""
    _, _, P = head_forward(qh, kh, vh, s, valid, mult, bias_h)
    dPd = dOh @ vh.T
    dP = dPd * mult
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dq = s * (dS @ kh)
    dk = s * (dS.T @ qh)
    dv = (P * mult).T @ dOh
    if want_ds:
        return dq, dk, dv, D, dS
    return dq, dk, dv, D


def _heads(B: int, H: int, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def _bias64(bias, B: int, H: int, Sq: int, Sk: int):
    """The bias as float64 broadcast to [B, H, Sq, Sk], or None."""
    if bias is None:
        return None
    return np.broadcast_to(_as64(bias), (B, H, Sq, Sk))


def fwd(q, k, v, dropout_p: float = 0.0, is_causal: bool = False, scale=None,
        seed: int = 0, offset: int = 0, heads=None, bias=None):
    """Forward on logical [B, H, S, E] inputs.

    Returns ``(out [B,H,Sq,E], lse [B,H,Sq])`` in float64.  With ``heads`` (a
    list of (b, h)) only those heads are computed and the rest are NaN.
    ``bias`` (optional) broadcasts to [B, H, Sq, Sk].
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Sq, E = q.shape
    Sk = k.shape[2]
    s = resolve_scale(scale, E)
    bias = _bias64(bias, B, H, Sq, Sk)
    out = np.full((B, H, Sq, v.shape[3]), np.nan)
    lse = np.full((B, H, Sq), np.nan)
    valid = valid_mask(Sq, Sk, is_causal)
    for b, h in _heads(B, H, heads):
        mult = dropout_multiplier(dropout_p, seed, offset, B, H, Sq, Sk, b, h)
        out[b, h], lse[b, h], _ = head_forward(q[b, h], k[b, h], v[b, h], s, valid, mult,
                                               None if bias is None else bias[b, h])
    return out, lse


def fwd_rows(q, k, v, b: int, h: int, rows, dropout_p: float = 0.0, is_causal: bool = False,
             scale=None, seed: int = 0, offset: int = 0, bias=None):
    """Forward for selected query rows of head (b, h): ``(out [n,E], lse [n])``.

    Each row of attention depends only on its own query, so this equals the
    matching rows of :func:`fwd` and lets full-size problems be sampled.
    """
    B, H, Sq, E = q.shape
    Sk = k.shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    qh = _as64(q[b, h])[rows]
    kh, vh = _as64(k[b, h]), _as64(v[b, h])
    s = resolve_scale(scale, E)
    valid = valid_mask(Sq, Sk, is_causal, rows=rows)
    mult = dropout_multiplier(dropout_p, seed, offset, B, H, Sq, Sk, b, h, rows=rows)
    bias = _bias64(bias, B, H, Sq, Sk)
    out, lse, _ = head_forward(qh, kh, vh, s, valid, mult,
                               None if bias is None else bias[b, h][rows])
    return out, lse


def bwd(dout, q, k, v, dropout_p: float = 0.0, is_causal: bool = False, seed: int = 0,
        offset: int = 0, scale=None, heads=None, bias=None, want_dbias: bool = False):
    """Backward on logical [B, H, S, E] inputs: ``(dq, dk, dv)`` in float64.

    Computed from (dO, Q, K, V, p, seed, offset, causal, scale) alone; the
    forward's outputs are recomputed, never taken from the caller.  With
    ``want_dbias`` a fourth array follows: the bias gradient of step 9, shape
    [B, H, Sq, Sk] (NaN for heads not computed).
    """
    dout, q, k, v = _as64(dout), _as64(q), _as64(k), _as64(v)
    B, H, Sq, E = q.shape
    Sk = k.shape[2]
    s = resolve_scale(scale, E)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    valid = valid_mask(Sq, Sk, is_causal)
    bias = _bias64(bias, B, H, Sq, Sk)
    dbias = np.full((B, H, Sq, Sk), np.nan) if want_dbias else None
    for b, h in _heads(B, H, heads):
        mult = dropout_multiplier(dropout_p, seed, offset, B, H, Sq, Sk, b, h)
        r = head_backward(dout[b, h], q[b, h], k[b, h], v[b, h], s, valid, mult,
                          None if bias is None else bias[b, h], want_ds=want_dbias)
        dq[b, h], dk[b, h], dv[b, h] = r[:3]
        if want_dbias:
            dbias[b, h] = r[4]
    if want_dbias:
        return dq, dk, dv, dbias
    return dq, dk, dv
