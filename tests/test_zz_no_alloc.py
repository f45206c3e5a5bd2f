"""The allocation-free backward (sdpa_bwd_noalloc) against sdpa_bwd_ext.

Both run the same kernels; the allocation-free call takes the row pass's
workspace from the library's device-resident scratch instead of from the
caller.  Its outputs must equal those of the workspace call bit for bit, on
consecutive calls whose sizes shrink (the scratch keeps the previous call's
contents), at the largest size it accepts, and with dropout and a bias.  Sizes
past that are refused before anything is enqueued.
"""

import ctypes
import math

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from scaled_dot_product_14_amd import _binding as bnd
from tests._util import gpu_available, say

needs_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _t(B, H, S, E=64):
    d = bnd.SdpaTensor()
    d.data, d.dtype = FAKE, 0
    for i, x in enumerate((B, H, S, E)):
        d.size[i] = x
    for i, x in enumerate((H * S * E, S * E, E, 1)):
        d.stride[i] = x
    return d


def test_max_rows_and_rejection_before_any_launch():
    lib = bnd.load_library()
    assert sdpa.sdpa_bwd_noalloc_max_rows() == 524288
    B, H, S = 1, 8, 65537  # one row past the maximum
    ts = [_t(B, H, S) for _ in range(8)]
    bnd.sdpa_set_rng_state(81, 82)
    rc = lib.sdpa_bwd_noalloc(*(ctypes.byref(t) for t in ts[:5]), FAKE, 0.0, 1, 0, 0, math.nan,
                              *(ctypes.byref(t) for t in ts[5:]), None, None)
    assert rc == bnd.SDPA_ERR_UNSUPPORTED
    assert "524288" in lib.sdpa_last_error().decode()
    assert bnd.sdpa_get_rng_state() == (81, 82)


def _both(q, k, v, do, p, causal, bias=None, rng=(0, 0)):
    sdpa.sdpa_set_rng_state(*rng)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    ref = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, bias=bias)
    got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    sdpa.sdpa_bwd_noalloc(do, q, k, v, out, lse, p, causal, s, o, None, *got, bias=bias)
    torch.cuda.synchronize()
    return ref, got


def _check(ref, got):
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), name


@pytest.mark.gpu
@needs_gpu
@pytest.mark.parametrize("first,second", [
    ((2, 12, 1024, 1024, 64, "BHSE", True, 0.0), (1, 2, 128, 128, 64, "BHSE", True, 0.0)),
    ((4, 16, 1000, 1000, 64, "BHSE", True, 0.1), (1, 3, 300, 257, 128, "BSHE", False, 0.2)),
])
def test_two_calls_in_a_row_second_smaller(first, second):
    for i, (B, H, Sq, Sk, E, layout, causal, p) in enumerate((first, second)):
        say(f"allocation-free backward call {i}: B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} "
            f"causal={causal} p={p}")
        q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 60 + i, 1.0, layout, device="cuda")
        ref, got = _both(q, k, v, do, p, causal, rng=(1234, 64 * i))
        _check(ref, got)


@pytest.mark.gpu
@needs_gpu
def test_largest_accepted_size_and_bias():
    B, H, Sq, Sk = 1, 8, 65536, 128  # B*H*Sq = 524288
    say(f"allocation-free backward at the largest size: B{B} H{H} Sq{Sq} Sk{Sk}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, 64, 70, 1.0, "BHSE", device="cuda")
    ref, got = _both(q, k, v, do, 0.0, False)
    _check(ref, got)
    say("allocation-free backward with a bias and dropout")
    q, k, v, do = workloads.draw(2, 2, 200, 200, 64, 71, 1.0, "BHSE", device="cuda")
    g = torch.Generator("cpu").manual_seed(72)
    bias = torch.randn((1, 2, 200, 200), generator=g).to(torch.bfloat16).to("cuda")
    ref, got = _both(q, k, v, do, 0.1, True, bias=bias, rng=(5, 6))
    _check(ref, got)
