"""Non-finite inputs on the GPU: the forward follows the definition.

A NaN or an infinity in query row i makes out row i NaN and LSE row i
non-finite (an infinity can leave every score of a short causal row at -inf,
whose log-sum-exp is -inf); a NaN in key row j makes NaN exactly the rows that
can see key j (with causal masking,
rows i >= j).  Every other row is bitwise the row of the clean call: rows never
exchange values in the forward, and a hidden score is replaced by -inf before
anything reads it.  The oracle obeys the same statement
(tests/test_oracle_sdpa.py); here the kernels are held to it through every
forward workgroup shape.
"""

import math

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from tests._util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _fwd(q, k, v, causal):
    out, lse, _, _ = sdpa.sdpa_fwd(q, k, v, 0.0, causal)
    torch.cuda.synchronize()
    return out.float(), lse


@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("E", [64, 128])
@pytest.mark.parametrize("bad", [math.nan, math.inf])
def test_non_finite_query_row(monkeypatch, shape, E, bad):
    say(f"non-finite query row: shape {shape} E{E} value {bad}")
    monkeypatch.setenv("SDPA14_FWD_SHAPE", str(shape))
    B, H, S = 1, 2, 600
    q, k, v, _ = workloads.draw(B, H, S, S, E, 39, 1.0, "BHSE", device="cuda")
    o_ref, l_ref = _fwd(q, k, v, True)
    rows = [0, 31, 33, 517, 599]
    q2 = q.clone()
    for r in rows:
        q2[0, 1, r, 5] = bad
    o, l = _fwd(q2, k, v, True)
    other = torch.ones(S, dtype=torch.bool, device="cuda")
    other[rows] = False
    assert torch.isnan(o[0, 1, rows]).all() and not torch.isfinite(l[0, 1, rows]).any()
    if math.isnan(bad):
        assert torch.isnan(l[0, 1, rows]).all()
    assert torch.equal(o[0, 1, other], o_ref[0, 1, other])
    assert torch.equal(l[0, 1, other], l_ref[0, 1, other])
    assert torch.equal(o[0, 0], o_ref[0, 0]) and torch.equal(l[0, 0], l_ref[0, 0])


@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("key", [0, 40, 333, 599])
def test_nan_key_row_causal(monkeypatch, shape, key):
    say(f"NaN key row {key}: shape {shape}")
    monkeypatch.setenv("SDPA14_FWD_SHAPE", str(shape))
    B, H, S, E = 2, 1, 600, 64
    q, k, v, _ = workloads.draw(B, H, S, S, E, 40, 1.0, "BHSE", device="cuda")
    o_ref, l_ref = _fwd(q, k, v, True)
    k2 = k.clone()
    k2[1, 0, key, 7] = math.nan
    o, l = _fwd(q, k2, v, True)
    assert torch.isnan(o[1, 0, key:]).all() and torch.isnan(l[1, 0, key:]).all()
    assert torch.equal(o[1, 0, :key], o_ref[1, 0, :key])
    assert torch.equal(l[1, 0, :key], l_ref[1, 0, :key])
    assert torch.equal(o[0], o_ref[0]) and torch.equal(l[0], l_ref[0])
