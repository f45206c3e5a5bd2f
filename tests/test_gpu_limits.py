"""Row offsets at the edge of the kernels' 32-bit buffer offsets.

Within one (batch, head) slice the kernels address rows with 32-bit byte
offsets, and the ABI accepts a tensor while (S + 255) * row_stride * 2 +
E * 2 stays below 2^31 (the 255 rows cover loads issued past the last row,
which the buffer range check turns into zeros).  Here every tensor, outputs
included, is a view with the largest row stride that rule allows, so the
last rows sit just below 2 GiB into their slice; the results must match the
oracle on the logical values, and nothing may be written in the gaps between
the rows.  A stride one granule larger is refused.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import sdpa_ref
from tests._util import assert_grads, assert_lse, assert_out, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _max_row_stride(S, E):
    """Largest multiple of 8 elements with (S + 255) * stride * 2 + E * 2 < 2^31."""
    s = ((1 << 31) - 1 - 2 * E) // (2 * (S + 255))
    return s // 8 * 8


def _wide(x, stride):
    """A [1, 1, S, E] view of x's values whose rows are `stride` elements apart."""
    _, _, S, E = x.shape
    buf = torch.zeros((S - 1) * stride + E, dtype=x.dtype, device="cuda")
    v = buf.as_strided((1, 1, S, E), (buf.numel(), buf.numel(), stride, 1))
    v.copy_(x)
    return v


def _empty_wide(S, E, stride, dtype):
    buf = torch.full(((S - 1) * stride + E,), float("nan"), dtype=dtype, device="cuda")
    return buf.as_strided((1, 1, S, E), (buf.numel(), buf.numel(), stride, 1)), buf


def _only_the_view_written(view, buf):
    """Every element of the NaN-filled buffer outside the view is still NaN."""
    written = int((~torch.isnan(buf)).sum().item())
    assert written == view.numel(), f"{written} elements written, {view.numel()} in the view"


@pytest.mark.parametrize("Sq,Sk,E,causal", [(300, 300, 64, True), (200, 333, 128, False),
                                            (2048, 2048, 128, True), (4000, 3000, 64, False)])
def test_rows_just_below_two_gib(Sq, Sk, E, causal):
    sq_s, sk_s = _max_row_stride(Sq, E), _max_row_stride(Sk, E)
    say(f"row strides {sq_s} / {sk_s} elements: last row at "
        f"{(Sq - 1) * sq_s * 2 / 2**30:.3f} / {(Sk - 1) * sk_s * 2 / 2**30:.3f} GiB")
    q0, k0, v0, do0 = workloads.draw(1, 1, Sq, Sk, E, 91, 1.0, "BHSE", device="cuda")
    q, do = _wide(q0, sq_s), _wide(do0, sq_s)
    k, v = _wide(k0, sk_s), _wide(v0, sk_s)
    out, out_buf = _empty_wide(Sq, E, sq_s, torch.bfloat16)
    dq, dq_buf = _empty_wide(Sq, E, sq_s, torch.bfloat16)
    dk, dk_buf = _empty_wide(Sk, E, sk_s, torch.bfloat16)
    dv, dv_buf = _empty_wide(Sk, E, sk_s, torch.bfloat16)
    o, lse, s, off = sdpa.sdpa_fwd(q, k, v, 0.0, causal, None, out=out)
    sdpa.sdpa_bwd(do, q, k, v, out, lse, 0.0, causal, s, off, None, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref_out, ref_lse = sdpa_ref.fwd(q0, k0, v0, 0.0, causal)
    ref_dq, ref_dk, ref_dv = sdpa_ref.bwd(do0, q0, k0, v0, 0.0, causal)
    assert_out(host64(out), ref_out)
    assert_lse(host64(lse), ref_lse)
    assert_grads([("dq", host64(dq), ref_dq), ("dk", host64(dk), ref_dk),
                  ("dv", host64(dv), ref_dv)])
    # Nothing is stored between the rows (the gaps stay NaN), nor past the last row.
    for view, buf in ((out, out_buf), (dq, dq_buf), (dk, dk_buf), (dv, dv_buf)):
        _only_the_view_written(view, buf)
    del q, k, v, do, out, dq, dk, dv, out_buf, dq_buf, dk_buf, dv_buf
    torch.cuda.empty_cache()


def test_one_granule_more_is_refused():
    S, E = 300, 64
    st = _max_row_stride(S, E) + 8
    buf = torch.zeros((S - 1) * st + E, dtype=torch.bfloat16, device="cuda")
    q = buf.as_strided((1, 1, S, E), (buf.numel(), buf.numel(), st, 1))
    k = torch.zeros((1, 1, S, E), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError, match="2 GiB"):
        sdpa.sdpa_fwd(q, k, k.clone(), 0.0, True, None)
    del buf, q
    torch.cuda.empty_cache()
