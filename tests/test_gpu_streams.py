"""Calls on several streams at once give the results of the same calls in turn.

The library keeps no per-call state on the device beyond the caller's buffers
(the workspace is the caller's; the host RNG state is read under a lock when
a forward is enqueued), so forward and backward calls of different problems
enqueued on four streams, overlapping on the GPU, must return bitwise what
they return one after another on one stream.  Problems mix head dims, causal
masking, dropout and a bias, so launches of different kernels overlap.
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from tests._util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

PROBLEMS = [
    # (B, H, Sq, Sk, E, causal, p, bias)
    (2, 4, 512, 512, 64, True, 0.0, False),
    (1, 8, 300, 700, 128, False, 0.1, False),
    (2, 2, 1024, 1024, 64, True, 0.2, True),
    (1, 4, 257, 257, 96, True, 0.0, True),
]


def _setup(i, B, H, Sq, Sk, E, causal, p, bias):
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 200 + i, 1.0, "BHSE", device="cuda")
    b = None
    if bias:
        g = torch.Generator("cpu").manual_seed(300 + i)
        b = (torch.randn((Sq, (Sk + 7) // 8 * 8), generator=g) * 2).to(torch.bfloat16).to("cuda")[:, :Sk]
    bufs = dict(out=torch.empty_like(q), lse=torch.empty((B, H, Sq), dtype=torch.float32, device="cuda"),
                dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                ws=torch.empty(sdpa.sdpa_bwd_workspace_size(B, H, Sq), dtype=torch.uint8,
                               device="cuda"))
    return dict(q=q, k=k, v=v, do=do, bias=b, causal=causal, p=p, rng=(40 + i, 1000 * i), **bufs)


def _run(c):
    # The forward draws (seed, offset) from the host RNG state, set right
    # before it, so every run of a problem uses the same mask.
    sdpa.sdpa_set_rng_state(*c["rng"])
    _, _, s, o = sdpa.sdpa_fwd_ext(c["q"], c["k"], c["v"], c["p"], c["causal"], None, out=c["out"],
                                   lse=c["lse"], bias=c["bias"])
    sdpa.sdpa_bwd_ext(c["do"], c["q"], c["k"], c["v"], c["out"], c["lse"], c["p"], c["causal"],
                      s, o, None, c["dq"], c["dk"], c["dv"], c["ws"], bias=c["bias"])


def test_four_streams_match_one():
    cases = [_setup(i, *pr) for i, pr in enumerate(PROBLEMS)]
    for c in cases:
        _run(c)
    torch.cuda.synchronize()
    ref = [[c[n].clone() for n in ("out", "lse", "dq", "dk", "dv")] for c in cases]
    for rep in range(3):
        for c in cases:
            for n in ("out", "dq", "dk", "dv"):
                c[n].fill_(float("nan"))
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream() for _ in cases]
        for s_, c in zip(streams, cases):
            s_.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s_):
                _run(c)
        for s_ in streams:
            torch.cuda.current_stream().wait_stream(s_)
        torch.cuda.synchronize()
        for i, (c, r) in enumerate(zip(cases, ref)):
            for n, a in zip(("out", "lse", "dq", "dk", "dv"), r):
                assert torch.equal(c[n], a), f"problem {i} {n} differs on its own stream (rep {rep})"
        say(f"  rep {rep}: four streams match")
