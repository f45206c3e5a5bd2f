"""GPU tests of the extended calls: head-sharded dropout and device-resident RNG state.

Sharding: a call on a slice of the heads, told where the slice sits in the
whole problem (head_offset, heads_total), must draw the whole problem's keep
bits for those heads.  The oracle computes the whole problem (the absolute
Philox index of every element) and the shard's heads are compared with it.

Device RNG: with {seed, offset} in device memory the calls must equal the
host-state calls bit for bit, the state must advance by one forward's worth of
counters, and a captured forward + backward must draw the next mask on every
replay (the reason for keeping the state on the device).
"""

import pytest
import torch

import scaled_dot_product_14_amd as sdpa
import workloads
from oracle import philox_ref, sdpa_ref
from tests._util import assert_grads, assert_lse, assert_out, gpu_available, host64, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("B,H,S,E,causal,p,cuts", [
    (2, 4, 200, 64, True, 0.2, (0, 1, 4)),
    (1, 6, 130, 128, False, 0.3, (0, 2, 3, 6)),
])
def test_sharded_dropout_draws_the_whole_problem_mask(B, H, S, E, causal, p, cuts):
    say(f"sharded dropout B{B} H{H} S{S} E{E} causal={causal} p={p} cuts={cuts}")
    q, k, v, do = workloads.draw(B, H, S, S, E, 11, 1.0, "BHSE", device="cuda")
    seed, off = 2024, 777
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off)
    ref_dq, ref_dk, ref_dv = sdpa_ref.bwd(do, q, k, v, p, causal, seed, off, None)
    adv = philox_ref.offset_advance(B, H, S, S)
    for h0, h1 in zip(cuts[:-1], cuts[1:]):
        sl = (slice(None), slice(h0, h1))
        sdpa.sdpa_set_rng_state(seed, off)
        out, lse, s, o = sdpa.sdpa_fwd_ext(q[sl], k[sl], v[sl], p, causal, head_offset=h0,
                                           heads_total=H)
        assert (s, o) == (seed, off)
        assert sdpa.sdpa_get_rng_state() == (seed, off + adv)  # the whole problem's advance
        dq, dk, dv = sdpa.sdpa_bwd_ext(do[sl], q[sl], k[sl], v[sl], out, lse, p, causal, s, o,
                                       head_offset=h0, heads_total=H)
        torch.cuda.synchronize()
        say(f"  heads {h0}:{h1}")
        assert_out(host64(out), ref_out[sl], dtype=out.dtype)
        assert_lse(lse.cpu().double().numpy(), ref_lse[sl])
        assert_grads([("dq", host64(dq), ref_dq[sl]), ("dk", host64(dk), ref_dk[sl]),
                      ("dv", host64(dv), ref_dv[sl])])


def test_unsharded_options_equal_the_plain_calls():
    say("ext with head_offset 0, heads_total H equals sdpa_fwd / sdpa_bwd")
    q, k, v, do = workloads.draw(2, 3, 160, 160, 64, 12, 1.0, "BHSE", device="cuda")
    sdpa.sdpa_set_rng_state(9, 90)
    o1, l1, s1, f1 = sdpa.sdpa_fwd(q, k, v, 0.25, True)
    g1 = sdpa.sdpa_bwd(do, q, k, v, o1, l1, 0.25, True, s1, f1)
    sdpa.sdpa_set_rng_state(9, 90)
    o2, l2, s2, f2 = sdpa.sdpa_fwd_ext(q, k, v, 0.25, True, heads_total=3)
    g2 = sdpa.sdpa_bwd_ext(do, q, k, v, o2, l2, 0.25, True, s2, f2, heads_total=3)
    torch.cuda.synchronize()
    assert (s1, f1) == (s2, f2)
    for a, b in zip((o1, l1) + tuple(g1), (o2, l2) + tuple(g2)):
        assert torch.equal(a, b)


def _dev_state(seed, offset):
    return torch.tensor([seed, offset], dtype=torch.int64, device="cuda")


def test_device_rng_equals_host_rng():
    say("device RNG state: same bits as the host state, state advanced on the device")
    B, H, S, E, p = 1, 2, 256, 64, 0.3
    q, k, v, do = workloads.draw(B, H, S, S, E, 13, 1.0, "BHSE", device="cuda")
    seed, off = 4321, 1 << 40
    state, used = _dev_state(seed, off), torch.zeros(2, dtype=torch.int64, device="cuda")
    sdpa.sdpa_set_rng_state(1, 2)
    od, ld, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, True, rng_state=state, rng_used=used)
    assert (s, o) == (None, None)
    gd = sdpa.sdpa_bwd_ext(do, q, k, v, od, ld, p, True, rng_used=used)
    torch.cuda.synchronize()
    assert sdpa.sdpa_get_rng_state() == (1, 2)  # the host state is not touched
    assert used.tolist() == [seed, off]
    assert state.tolist() == [seed, off + philox_ref.offset_advance(B, H, S, S)]
    sdpa.sdpa_set_rng_state(seed, off)
    oh, lh, s, o = sdpa.sdpa_fwd(q, k, v, p, True)
    gh = sdpa.sdpa_bwd(do, q, k, v, oh, lh, p, True, s, o)
    torch.cuda.synchronize()
    for a, b in zip((od, ld) + tuple(gd), (oh, lh) + tuple(gh)):
        assert torch.equal(a, b)


def test_device_rng_without_dropout_leaves_state():
    q, k, v, _ = workloads.draw(1, 1, 64, 64, 64, 14, 1.0, "BHSE", device="cuda")
    state, used = _dev_state(5, 6), torch.full((2,), -1, dtype=torch.int64, device="cuda")
    sdpa.sdpa_fwd_ext(q, k, v, 0.0, True, rng_state=state, rng_used=used)
    torch.cuda.synchronize()
    assert state.tolist() == [5, 6] and used.tolist() == [-1, -1]


def test_graph_replays_draw_fresh_masks_from_device_state():
    say("captured fwd + bwd with device RNG: replay r uses offset o0 + r * advance")
    B, H, S, E, p = 2, 2, 192, 64, 0.2
    q, k, v, do = workloads.draw(B, H, S, S, E, 15, 1.0, "BHSE", device="cuda")
    seed, o0 = 77, 1000
    adv = philox_ref.offset_advance(B, H, S, S)
    state, used = _dev_state(seed, o0), torch.zeros(2, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(sdpa.sdpa_bwd_workspace_size(B, H, S), 256), dtype=torch.uint8,
                     device="cuda")

    def step():
        sdpa.sdpa_fwd_ext(q, k, v, p, True, out=out, lse=lse, rng_state=state, rng_used=used)
        sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, True, dq=dq, dk=dk, dv=dv, workspace=ws,
                          rng_used=used)

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
    state.copy_(_dev_state(seed, o0))
    torch.cuda.synchronize()

    previous = None
    for rep in range(3):
        for t in (out, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert used.tolist() == [seed, o0 + rep * adv]
        assert state.tolist() == [seed, o0 + (rep + 1) * adv]
        got = [t.clone() for t in (out, lse, dq, dk, dv)]
        # eager host-state reference at the offset this replay should have used
        sdpa.sdpa_set_rng_state(seed, o0 + rep * adv)
        oh, lh, s, o = sdpa.sdpa_fwd(q, k, v, p, True)
        gh = sdpa.sdpa_bwd(do, q, k, v, oh, lh, p, True, s, o)
        torch.cuda.synchronize()
        for a, b in zip(got, (oh, lh) + tuple(gh)):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"
        if previous is not None:
            assert not torch.equal(got[0], previous), "replays drew the same mask"
        previous = got[0]


def _bias(shape, Sk_pad, seed, scale=2.0, alibi=False):
    """bf16 bias of logical `shape` (..., Sq, Sk) whose rows are padded to Sk_pad."""
    Sq, Sk = shape[-2], shape[-1]
    g = torch.Generator("cpu").manual_seed(seed)
    full = torch.randn(tuple(shape[:-1]) + (Sk_pad,), generator=g) * scale
    if alibi:  # a relative-position term: -slope * |i - j|
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk_pad)[None, :]
        full = -0.05 * (i - j).abs().float().expand(tuple(shape[:-1]) + (Sk_pad,))
    return full.to(torch.bfloat16).to("cuda")[..., :Sk]


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,p,bshape,pad,heads", [
    (2, 3, 200, 200, 64, "BHSE", True, 0.0, "bhqk", 200, None),
    (1, 2, 130, 250, 128, "BHSE", False, 0.1, "1hqk", 256, None),
    (2, 2, 256, 256, 64, "BSHE", True, 0.0, "qk-alibi", 256, None),
    (4, 16, 1000, 1000, 64, "BHSE", True, 0.1, "1hqk", 1000, [(0, 0), (3, 15), (2, 7)]),
])
def test_bias_parity(B, H, Sq, Sk, E, layout, causal, p, bshape, pad, heads):
    say(f"bias {bshape} B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} p={p}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 16, 1.0, layout, device="cuda")
    if bshape == "bhqk":
        bias = _bias((B, H, Sq, Sk), pad, 17)
    elif bshape == "1hqk":
        bias = _bias((1, H, Sq, Sk), pad, 18)
    else:
        bias = _bias((Sq, Sk), pad, 19, alibi=True)
    seed, off = 31, 4096
    sdpa.sdpa_set_rng_state(seed, off)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    dq, dk, dv = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, bias=bias)
    torch.cuda.synchronize()
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off, heads=heads, bias=bias)
    ref_dq, ref_dk, ref_dv = sdpa_ref.bwd(do, q, k, v, p, causal, seed, off, None, heads=heads,
                                          bias=bias)
    sel = (slice(None),) if heads is None else (tuple(b for b, _ in heads), tuple(h for _, h in heads))
    assert_out(host64(out)[sel], ref_out[sel])
    assert_lse(lse.cpu().double().numpy()[sel], ref_lse[sel])
    assert_grads([("dq", host64(dq)[sel], ref_dq[sel]), ("dk", host64(dk)[sel], ref_dk[sel]),
                  ("dv", host64(dv)[sel], ref_dv[sel])])


def test_zero_bias_equals_no_bias():
    q, k, v, do = workloads.draw(2, 2, 192, 192, 64, 20, 1.0, "BHSE", device="cuda")
    zero = torch.zeros((192, 192), dtype=torch.bfloat16, device="cuda")
    o1, l1, s, f = sdpa.sdpa_fwd_ext(q, k, v, 0.0, True, bias=zero)
    g1 = sdpa.sdpa_bwd_ext(do, q, k, v, o1, l1, 0.0, True, s, f, bias=zero)
    o2, l2, s, f = sdpa.sdpa_fwd(q, k, v, 0.0, True)
    g2 = sdpa.sdpa_bwd(do, q, k, v, o2, l2, 0.0, True, s, f)
    torch.cuda.synchronize()
    # Same math up to the order of one multiply-add, so within rounding of bf16 outputs.
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-5
    for a, b in zip(g1, g2):
        assert (a.float() - b.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,p,with_bias", [
    (2, 3, 300, 300, 64, "BHSE", True, 0.1, False),
    (1, 4, 200, 333, 128, "BSHE", False, 0.0, True),
    (2, 12, 1024, 1024, 64, "BHSE", True, 0.0, False),
])
def test_inference_forward_against_the_oracle(B, H, Sq, Sk, E, layout, causal, p, with_bias):
    say(f"inference forward B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} p={p} "
        f"bias={with_bias}: no lse written, out against the oracle")
    q, k, v, _ = workloads.draw(B, H, Sq, Sk, E, 21, 1.0, layout, device="cuda")
    bias = None
    if with_bias:
        pad = (Sk + 7) // 8 * 8
        g = torch.Generator("cpu").manual_seed(35)
        bias = torch.randn((1, H, Sq, pad), generator=g).to(torch.bfloat16).to("cuda")[..., :Sk]
    seed, off = 3, 30
    sdpa.sdpa_set_rng_state(seed, off)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, p, causal, need_lse=False, bias=bias)
    torch.cuda.synchronize()
    assert lse is None and (s, o) == (seed, off)
    ref_out, _ = sdpa_ref.fwd(q, k, v, p, causal, None, seed, off, bias=bias)
    assert_out(host64(out), ref_out)
    # The training forward computes the same rows the same way.
    sdpa.sdpa_set_rng_state(seed, off)
    out2, _, _, _ = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_minus_infinity_bias_hides_keys_like_the_causal_mask():
    say("bias of -inf above the diagonal equals causal masking")
    B, H, S, E = 1, 2, 160, 64
    q, k, v, do = workloads.draw(B, H, S, S, E, 24, 1.0, "BHSE", device="cuda")
    tri = torch.ones(S, S, dtype=torch.bool, device="cuda").tril()
    bias = torch.zeros(S, S, dtype=torch.bfloat16, device="cuda").masked_fill(~tri, float("-inf"))
    o1, l1, s, f = sdpa.sdpa_fwd_ext(q, k, v, 0.0, False, bias=bias)
    g1 = sdpa.sdpa_bwd_ext(do, q, k, v, o1, l1, 0.0, False, s, f, bias=bias)
    torch.cuda.synchronize()
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, 0.0, True)
    ref_g = sdpa_ref.bwd(do, q, k, v, 0.0, True)
    assert_out(host64(o1), ref_out)
    assert_lse(l1.cpu().double().numpy(), ref_lse)
    assert_grads([(n, host64(a), r) for n, a, r in zip(("dq", "dk", "dv"), g1, ref_g)])


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 37), (37, 1), (3, 200)])
def test_bias_degenerate_sizes(Sq, Sk):
    say(f"bias with Sq={Sq} Sk={Sk}")
    B, H, E = 2, 2, 64
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 25, 1.0, "BHSE", device="cuda")
    pad = (Sk + 7) // 8 * 8
    g = torch.Generator("cpu").manual_seed(26)
    bias = (torch.randn((B, 1, Sq, pad), generator=g)).to(torch.bfloat16).to("cuda")[..., :Sk]
    for causal in (False, True):
        out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, 0.0, causal, bias=bias)
        grads = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, 0.0, causal, s, o, bias=bias)
        torch.cuda.synchronize()
        ref_out, ref_lse = sdpa_ref.fwd(q, k, v, 0.0, causal, bias=bias)
        ref_g = sdpa_ref.bwd(do, q, k, v, 0.0, causal, bias=bias)
        assert_out(host64(out), ref_out, dtype=out.dtype)
        assert_lse(lse.cpu().double().numpy(), ref_lse)
        assert_grads([(n, host64(a), r) for n, a, r in zip(("dq", "dk", "dv"), grads, ref_g)])


def test_everything_together_fp16_sharded_device_rng_bias():
    say("fp16 + head shard + device RNG + bias + dropout against the whole-problem oracle")
    B, H, S, E, p = 2, 4, 144, 64, 0.15
    q, k, v, do = (t.to(torch.float16) for t in
                   workloads.draw(B, H, S, S, E, 27, 1.0, "BHSE", device="cuda"))
    g = torch.Generator("cpu").manual_seed(28)
    bias = (torch.randn((1, H, S, S), generator=g)).to(torch.float16).to("cuda")
    seed, off = 555, 64
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, p, True, None, seed, off, bias=bias)
    ref_g = sdpa_ref.bwd(do, q, k, v, p, True, seed, off, None, bias=bias)
    h0, h1 = 1, 3
    sl = (slice(None), slice(h0, h1))
    state, used = _dev_state(seed, off), torch.zeros(2, dtype=torch.int64, device="cuda")
    out, lse, _, _ = sdpa.sdpa_fwd_ext(q[sl], k[sl], v[sl], p, True, head_offset=h0, heads_total=H,
                                       rng_state=state, rng_used=used, bias=bias[:, h0:h1])
    grads = sdpa.sdpa_bwd_ext(do[sl], q[sl], k[sl], v[sl], out, lse, p, True, head_offset=h0,
                              heads_total=H, rng_used=used, bias=bias[:, h0:h1])
    torch.cuda.synchronize()
    assert state.tolist() == [seed, off + philox_ref.offset_advance(B, H, S, S)]
    assert_out(host64(out), ref_out[sl], dtype=out.dtype)
    assert_lse(lse.cpu().double().numpy(), ref_lse[sl])
    assert_grads([(n, host64(a), r[sl]) for n, a, r in zip(("dq", "dk", "dv"), grads, ref_g)])


@pytest.mark.parametrize("B,H,Sq,Sk,E,layout,causal,f16,with_bias", [
    (4, 16, 1000, 1000, 64, "BHSE", True, False, False),
    (2, 3, 200, 330, 64, "BSHE", False, False, False),
    (1, 2, 130, 250, 128, "BHSE", False, True, True),
    (2, 2, 256, 256, 128, "BHSE", True, False, False),
    # Causal grids that take the split forward (32-row, four-share workgroups
    # with 32-key tiles for the last rows of each head).
    (2, 8, 640, 640, 64, "BSHE", True, True, True),
    (1, 12, 1024, 1024, 64, "BHSE", True, False, False),
])
def test_keep_bit_cache(B, H, Sq, Sk, E, layout, causal, f16, with_bias):
    say(f"keep-bit cache B{B} H{H} Sq{Sq} Sk{Sk} E{E} {layout} causal={causal} f16={f16} bias={with_bias}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 29, 1.0, layout, device="cuda")
    if f16:
        q, k, v, do = (workloads.to_layout(t.to(torch.float16), layout) for t in (q, k, v, do))
    bias = None
    if with_bias:
        pad = (Sk + 7) // 8 * 8
        g = torch.Generator("cpu").manual_seed(30)
        bias = torch.randn((1, H, Sq, pad), generator=g).to(q.dtype).to("cuda")[..., :Sk]
    p, seed, off = 0.2, 808, 96
    kb = torch.empty(sdpa.sdpa_keep_bits_size(B, H, Sq, Sk) // 4, dtype=torch.int32, device="cuda")
    sdpa.sdpa_set_rng_state(seed, off)
    o1, l1, s, f = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias, keep_bits=kb)
    g1 = sdpa.sdpa_bwd_ext(do, q, k, v, o1, l1, p, causal, s, f, bias=bias, keep_bits=kb)
    sdpa.sdpa_set_rng_state(seed, off)
    o2, l2, s, f = sdpa.sdpa_fwd_ext(q, k, v, p, causal, bias=bias)
    g2 = sdpa.sdpa_bwd_ext(do, q, k, v, o2, l2, p, causal, s, f, bias=bias)
    mask = sdpa.sdpa_debug_dropout_mask(seed, off, p, B, H, Sq, Sk)
    torch.cuda.synchronize()
    # Outputs and gradients are the same computation with the same mask.
    for a, b in zip((o1, l1) + tuple(g1), (o2, l2) + tuple(g2)):
        assert torch.equal(a, b)
    # The cached bits are the mask, wherever a row can see the key.
    W = kb.numel() // (B * H * Sq)
    words = kb.view(B, H, Sq, W).to(torch.int64) & 0xFFFFFFFF
    j = torch.arange(Sk, device="cuda")
    bits = (words[..., j // 32] >> (j % 32)) & 1
    visible = torch.ones(Sq, Sk, dtype=torch.bool, device="cuda")
    if causal:
        visible = visible.tril()
    assert torch.equal(bits.to(torch.uint8)[..., visible], mask[..., visible])


def _hidden_key_bias(kind: str, S: int) -> torch.Tensor:
    """[S, S] bias of 0 on visible keys and -inf on hidden ones; every row keeps
    its own key.  'window': keys i-15 .. i+15; 'blocks': 48-key diagonal blocks."""
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    if kind == "window":
        vis = (j - i).abs() <= 15
    else:
        vis = (i // 48) == (j // 48)
    b = torch.zeros(S, S).masked_fill(~vis, float("-inf"))
    return b.to(torch.bfloat16).to("cuda")


@pytest.mark.parametrize("shape", [1, 2, 3, 4])
@pytest.mark.parametrize("kind", ["window", "blocks"])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_whose_first_tiles_are_all_hidden(monkeypatch, shape, kind, causal):
    # Rows of one wave reach their first visible key in different tiles, and
    # with key shares some share of a row sees no visible key at all: the
    # online softmax and the share merge must not turn -inf - -inf into NaN.
    say(f"hidden-key bias {kind} causal={causal} forward shape {shape}")
    monkeypatch.setenv("SDPA14_FWD_SHAPE", str(shape))
    B, H, S, E = 1, 2, 304, 64
    q, k, v, do = workloads.draw(B, H, S, S, E, 36, 1.0, "BHSE", device="cuda")
    bias = _hidden_key_bias(kind, S)
    out, lse, s, o = sdpa.sdpa_fwd_ext(q, k, v, 0.0, causal, bias=bias)
    grads = sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, 0.0, causal, s, o, bias=bias)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ref_out, ref_lse = sdpa_ref.fwd(q, k, v, 0.0, causal, bias=bias)
    ref_g = sdpa_ref.bwd(do, q, k, v, 0.0, causal, bias=bias)
    assert_out(host64(out), ref_out)
    assert_lse(lse.cpu().double().numpy(), ref_lse)
    assert_grads([(n, host64(a), r) for n, a, r in zip(("dq", "dk", "dv"), grads, ref_g)])


@pytest.mark.parametrize("B,H,Sq,Sk,E,causal,p", [
    (2, 3, 300, 300, 64, True, 0.1),
    (1, 2, 130, 250, 128, False, 0.0),
])
def test_backward_in_two_parts_equals_one_call(B, H, Sq, Sk, E, causal, p):
    say(f"backward as row pass, then main kernel: B{B} H{H} Sq{Sq} Sk{Sk} E{E}")
    q, k, v, do = workloads.draw(B, H, Sq, Sk, E, 33, 1.0, "BHSE", device="cuda")
    sdpa.sdpa_set_rng_state(9, 90)
    out, lse, s, o = sdpa.sdpa_fwd(q, k, v, p, causal)
    ref = sdpa.sdpa_bwd(do, q, k, v, out, lse, p, causal, s, o)
    ws = torch.empty(sdpa.sdpa_bwd_workspace_size(B, H, Sq), dtype=torch.uint8, device="cuda")
    got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, None, *got, workspace=ws, bwd_parts=1)
    assert all(torch.isnan(t.float()).all() for t in got)  # the row pass writes no gradient
    sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, p, causal, s, o, None, *got, workspace=ws, bwd_parts=2)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
