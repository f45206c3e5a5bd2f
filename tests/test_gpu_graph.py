"""Forward + backward captured in a HIP graph replay the eager results.

bench.py times the step as a graph replay; this checks that replays give the
eager outputs bit for bit, several times in a row, with eager work and
synchronizations between the replays (the kernels are deterministic and
allocate nothing, so every replay must match exactly).
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from tests._util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("name", ["b2_h12_s1024_d64_causal", "tiny_bshe_wide_scores"])
def test_graph_replays_match_eager(name):
    say(f"graph replay {name}")
    w = workloads.WORKLOADS[name]
    q, k, v, do = workloads.make_inputs(w, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(sdpa.sdpa_bwd_workspace_size(w.B, w.H, w.Sq), 256), dtype=torch.uint8,
                     device="cuda")

    def step():
        sdpa.sdpa_set_rng_state(w.rng_seed, w.rng_offset)
        _, _, s, o = sdpa.sdpa_fwd(q, k, v, w.dropout_p, w.causal, None, out=out, lse=lse)
        sdpa.sdpa_bwd(do, q, k, v, out, lse, w.dropout_p, w.causal, s, o, None, dq=dq, dk=dk,
                      dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (out, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (out, lse, dq, dk, dv)):
            assert torch.equal(a, b), f"replay {rep} differs"
        # eager work between replays
        step()
        torch.cuda.synchronize()
        for a, b in zip(ref, (out, lse, dq, dk, dv)):
            assert torch.equal(a, b)
