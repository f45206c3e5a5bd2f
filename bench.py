"""Benchmark of the fused SDPA hot path on one MI355X.

A step is one forward plus one backward (every kernel of the path) over the
b2 h12 s1024 d64 causal bf16 workload (the shape of the nvFuser test
``test_sdpa_loop_split``), with inputs resident in HBM before timing starts.

Prints ONE JSON line:
  value         whole-step TFLOP/s, counted FLOPs (forward 4*B*H*Sq*Sk*E, halved
                when causal; backward 2.5x forward) over the timed step time: K
                steps as replays of a HIP graph of up to 20 back-to-back steps
                (ms_per_step_one_step_graph: a graph of one step, replayed K times)
  fwd / bwd     the same for the forward and the backward alone, each timed as
                a HIP graph of back-to-back calls replayed between events on the
                launch stream, and their fraction of the bf16 dense MFMA peak
                (eager_us: the same calls issued from Python one by one)
  kernels       average duration of one forward (one kernel) and one backward
                (row pass + main kernel) from those graph replays
  kernels_bracketed  the same from HIP events the library records around each of
                its launches (the brackets' own cost included)
  roofline      the dominant kernel against its roofline
  cpu_baseline  the fp64 CPU oracle on the host cores (a reported baseline)

Options: --steps K --warmup W --gpus N (N must be 1), --no-cpu-baseline,
--workload NAME, --shape B,H,Sq,Sk,E,causal[,p], --bias {none,qk,bhqk} (an additive bias through the
extended calls), --dbias (with a bias: the backward also writes the [B, H, Sq, Sk] bias
gradient), --copy-bytes N (time a plain device copy of N bytes instead, for calibrating
hardware byte counters).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = "fwd / bwd TFLOP/s and % bf16 MFMA peak at b2 h12 s1024 d64 causal"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b2_h12_s1024_d64_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent on the oracle baseline")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--keep-bits", action="store_true",
                    help="with dropout: the forward keeps its mask bits for the backward "
                         "(extended calls) instead of the backward regenerating them")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache kernel timing (input sets rotated past the caches)")
    ap.add_argument("--bias", choices=("none", "qk", "bhqk"), default="none",
                    help="add an additive bf16 bias: [Sq, Sk] broadcast over batch and heads, "
                         "or a full [B, H, Sq, Sk] (drawn N(0, 4)); timed through the extended calls")
    ap.add_argument("--dbias", action="store_true",
                    help="with --bias: the backward also writes the full [B, H, Sq, Sk] bias gradient")
    ap.add_argument("--shape", default="",
                    help="B,H,Sq,Sk,E,causal[,p] instead of a named workload (exploration)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "fwd": ["fwd.hip", "lds_ring.h", "device_common.h", "philox.h", "kernels.h", "occupancy.h"],
    "bwd_main": ["bwd.hip", "bwd_e128.hip", "bwd_kernels.h", "lds_ring.h", "device_common.h",
                 "philox.h", "kernels.h"],
    "bwd_rows": ["bwd.hip", "bwd_kernels.h", "device_common.h", "kernels.h"],
}


def source_hash(kernel: str) -> str:
    """sha256 over the sources a kernel is built from (to tell stale counters)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "scaled_dot_product_14_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == source_hash(kernel) else None


def copy_calibration(nbytes: int, steps: int):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": nbytes, "launches": steps, "s_per_copy": dt,
                      "GBps_read_plus_write": 2 * nbytes / dt / 1e9}), flush=True)


def timed_loop(fn, steps: int):
    import torch
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


def capture(step, before_capture):
    """HIP graph of one call of step, captured after warm-up on a side stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    before_capture()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph


def replayed_launches(fn, launches: int, steps: int):
    """Average duration (ms) of one call of fn, from a HIP graph of `launches`
    back-to-back calls replayed so that about `steps` calls are timed, between
    events on the stream the library launches on (the current stream)."""
    import torch
    graph = capture(lambda: [fn() for _ in range(launches)], lambda: None)
    graph.replay()
    reps = max(1, steps // launches)
    return timed_loop(graph.replay, reps) / launches


def cpu_baseline(w, q, k, v, do, min_seconds: float):
    """Oracle forward + backward on whole heads until min_seconds of CPU time."""
    from oracle import sdpa_ref

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = int(os.environ.get("OMP_NUM_THREADS", "1")), "unknown"
    qc, kc, vc, dc = (t.cpu() for t in (q, k, v, do))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_head = w.fwd_flops() / len(heads) * 3.5  # forward + backward counted FLOPs
    done, flops, t0 = 0, 0.0, time.perf_counter()
    while True:
        b, h = heads[done % len(heads)]
        sdpa_ref.fwd(qc, kc, vc, w.dropout_p, w.causal, heads=[(b, h)])
        sdpa_ref.bwd(dc, qc, kc, vc, w.dropout_p, w.causal, heads=[(b, h)])
        done += 1
        flops += per_head
        if time.perf_counter() - t0 >= min_seconds and done >= 2:
            break
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(cores, threads),
            "kind": "oracle",
            "sample": f"{done} whole heads (of {len(heads)}) of the same workload, fp64 numpy "
                      f"forward + backward, {dt:.1f} s wall; BLAS {blas} with {threads} threads "
                      f"on {cores} visible cores"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: heads shard across GPUs with no exchange, so one GPU's share is "
              "the same kernel on fewer heads.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return

    sys.path.insert(0, ROOT)
    import scaled_dot_product_14_amd as sdpa
    import workloads

    if args.shape:
        f = args.shape.split(",")
        B, H, Sq, Sk, E, causal = (int(x) for x in f[:6])
        p = float(f[6]) if len(f) > 6 else 0.0
        w = workloads.Workload(f"shape_{args.shape}", B, H, Sq, Sk, E, "BHSE", bool(causal), p,
                               7, rng_seed=1234 if p > 0 else 0)
    else:
        w = workloads.WORKLOADS[args.workload]
    log(f"workload {w}")
    q, k, v, do = workloads.make_inputs(w, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(sdpa.sdpa_bwd_workspace_size(w.B, w.H, w.Sq), 256), dtype=torch.uint8,
                     device="cuda")
    sdpa.sdpa_set_rng_state(w.rng_seed, w.rng_offset)
    state = {}
    bias = None
    if args.bias != "none":
        gb = torch.Generator("cpu").manual_seed(8)
        bshape = (w.Sq, w.Sk) if args.bias == "qk" else (w.B, w.H, w.Sq, w.Sk)
        bias = (torch.randn(bshape, generator=gb) * 2.0).to(torch.bfloat16).to("cuda")
    dbias = None
    if args.dbias:
        if bias is None:
            raise SystemExit("--dbias needs --bias")
        dbias = torch.empty((w.B, w.H, w.Sq, -(-w.Sk // 8) * 8), dtype=torch.bfloat16,
                            device="cuda")[..., :w.Sk]

    keep = None
    if args.keep_bits:
        keep = torch.empty(sdpa.sdpa_keep_bits_size(w.B, w.H, w.Sq, w.Sk) // 4, dtype=torch.int32,
                           device="cuda")

    def fwd():
        if bias is None and keep is None:
            _, _, s, o = sdpa.sdpa_fwd(q, k, v, w.dropout_p, w.causal, None, out=out, lse=lse)
        else:
            _, _, s, o = sdpa.sdpa_fwd_ext(q, k, v, w.dropout_p, w.causal, None, out=out,
                                           lse=lse, bias=bias, keep_bits=keep)
        state["so"] = (s, o)

    def bwd(parts=0):
        s, o = state["so"]
        if bias is None and keep is None and parts == 0:
            sdpa.sdpa_bwd(do, q, k, v, out, lse, w.dropout_p, w.causal, s, o, None, dq=dq,
                          dk=dk, dv=dv, workspace=ws)
        else:
            sdpa.sdpa_bwd_ext(do, q, k, v, out, lse, w.dropout_p, w.causal, s, o, None, dq=dq,
                              dk=dk, dv=dv, workspace=ws, bias=bias, keep_bits=keep,
                              bwd_parts=parts, dbias=dbias)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warm-up done")

    # The step's kernels replayed from a HIP graph captured once: the timed work
    # is the same forward and backward, without the Python launch path.  The
    # graph holds n_graph back-to-back steps (the largest divisor of K up to
    # 20), so the K timed steps are K / n_graph replays: each graph launch
    # leaves the GPU idle for several microseconds at its boundary, which a
    # training step's graph (many layers per launch) does not pay per
    # attention call.  The one-step graph is timed beside it.
    # With dropout each captured step draws the next offset from the host RNG
    # state and every replay reuses those captured offsets, so the eager
    # reference runs the same n_graph steps from the same starting state: the
    # buffers then hold the last step's results on both sides.
    n_graph = max(d for d in range(1, min(args.steps, 20) + 1) if args.steps % d == 0)
    graph = capture(lambda: [step() for _ in range(n_graph)],
                    lambda: sdpa.sdpa_set_rng_state(w.rng_seed, w.rng_offset))
    sdpa.sdpa_set_rng_state(w.rng_seed, w.rng_offset)
    for _ in range(n_graph):
        step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, dq, dk, dv)]
    for t in (out, dq, dk, dv):
        t.zero_()
    graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(eager, (out, lse, dq, dk, dv)))
    if not same:
        raise RuntimeError("graph replay differs from the eager step")
    ms_step = timed_loop(graph.replay, args.steps // n_graph) / n_graph
    log(f"timed {args.steps} graph-replayed steps ({n_graph} per graph): {ms_step * 1e3:.2f} us/step")
    graph1 = capture(step, lambda: sdpa.sdpa_set_rng_state(w.rng_seed, w.rng_offset))
    ms_step_1 = timed_loop(graph1.replay, args.steps)
    log(f"timed {args.steps} one-step graph replays: {ms_step_1 * 1e3:.2f} us/step")
    ms_eager = timed_loop(step, args.steps)
    log(f"timed {args.steps} eager steps: {ms_eager * 1e3:.2f} us/step")
    # Forward-only and backward-only: graphs of back-to-back launches replayed
    # (a forward is one kernel, a backward the row pass plus the main kernel).
    # The same passes issued from Python one by one are reported beside them;
    # at this size their host launch path costs about as much as the kernels.
    per_graph = 20
    ms_fwd = replayed_launches(fwd, per_graph, args.steps)
    ms_bwd = replayed_launches(bwd, per_graph, args.steps)
    log(f"graph-replayed launches: fwd {ms_fwd * 1e3:.2f} us, bwd {ms_bwd * 1e3:.2f} us")
    ms_fwd_eager = timed_loop(fwd, args.steps)
    ms_bwd_eager = timed_loop(bwd, args.steps)
    log(f"eager launches: fwd {ms_fwd_eager * 1e3:.2f} us, bwd {ms_bwd_eager * 1e3:.2f} us")
    # The backward's two kernels on their own: event pairs the library records
    # around each launch, captured as graph nodes in a graph of back-to-back
    # backward calls.
    ms_rows = replayed_launches(lambda: bwd(parts=1), per_graph, args.steps)
    ms_main = replayed_launches(lambda: bwd(parts=2), per_graph, args.steps)
    n_main = n_rows = per_graph * max(1, args.steps // per_graph)
    log(f"graph-replayed backward kernels: row pass {ms_rows * 1e3:.2f} us, "
        f"main {ms_main * 1e3:.2f} us")
    rows_bytes = w.B * w.H * w.Sq * (4 * w.E + 12)  # dO, O (bf16) and LSE read; -D, L written
    kern = {"fwd": {"avg_us": ms_fwd * 1e3, "launches": per_graph * max(1, args.steps // per_graph),
                    "timing": "graph of back-to-back forward calls, events on the launch stream"},
            "bwd_main": {"avg_us": ms_main * 1e3, "launches": n_main,
                         "timing": "graph of back-to-back main-kernel launches (backward calls "
                                   "with bwd_parts = 2 on a filled workspace), events on the "
                                   "launch stream"},
            "bwd_rows": {"avg_us": ms_rows * 1e3, "launches": n_rows,
                         "timing": "graph of back-to-back row passes (bwd_parts = 1), events "
                                   "on the launch stream",
                         "algorithmic_bytes": rows_bytes,
                         "GBps": rows_bytes / (ms_rows * 1e-3) / 1e9,
                         "frac_hbm_peak": rows_bytes / (ms_rows * 1e-3) / 1e9 / PEAK_HBM_GBS}}

    # Per-launch brackets: events recorded by the library around each of its
    # launches (their own cost, ~1-2 us per launch, is inside the figure).
    names = {sdpa.KERNEL_FWD: "fwd", sdpa.KERNEL_BWD: "bwd_main", sdpa.KERNEL_BWD_ROWS: "bwd_rows"}
    for kind in names:
        sdpa.sdpa_profile_read(kind)
    sdpa.sdpa_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sdpa.sdpa_profile_enable(False)
    bracketed = {}
    for kind, name in names.items():
        tot, n = sdpa.sdpa_profile_read(kind)
        bracketed[name] = {"avg_us": tot / max(n, 1) * 1e3, "launches": n}
    log(f"bracketed kernel averages (us): "
        f"{ {k_: round(v_['avg_us'], 2) for k_, v_ in bracketed.items()} }")

    # Cold cache: the same kernels on input sets rotated so that each launch
    # finds its inputs outside the 4 MB L2s and the 256 MB last-level cache
    # (more than 512 MB of distinct inputs per rotation).
    cold = None
    if not args.no_cold and bias is None and keep is None:
        set_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, do, out))
        n_sets = max(2, -(-2 * 256 * 2**20 // set_bytes) + 1)
        sets = []
        for i in range(n_sets):
            qi, ki, vi, doi = (t.clone() for t in (q, k, v, do))
            sets.append((qi, ki, vi, doi, torch.empty_like(q),
                         torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")))
        for kind in names:
            sdpa.sdpa_profile_read(kind)
        sdpa.sdpa_profile_enable(True)
        reps = max(1, 200 // n_sets)
        for _ in range(reps):
            for qi, ki, vi, doi, oi, li in sets:
                _, _, s_, o_ = sdpa.sdpa_fwd(qi, ki, vi, w.dropout_p, w.causal, None, out=oi, lse=li)
                sdpa.sdpa_bwd(doi, qi, ki, vi, oi, li, w.dropout_p, w.causal, s_, o_, None, dq=dq,
                              dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        sdpa.sdpa_profile_enable(False)
        cold = {"input_sets": n_sets, "bytes_per_set": set_bytes}
        for kind, name in names.items():
            tot, n = sdpa.sdpa_profile_read(kind)
            cold[name + "_avg_us"] = tot / max(n, 1) * 1e3
        del sets
        log(f"cold-cache kernel averages (us): fwd {cold['fwd_avg_us']:.2f}, "
            f"bwd main {cold['bwd_main_avg_us']:.2f}, row pass {cold['bwd_rows_avg_us']:.2f} "
            f"over {n_sets} input sets")

    f_fwd, f_bwd = w.fwd_flops(), w.bwd_flops()
    kern["fwd"]["algorithmic_tflop"] = f_fwd / 1e12
    kern["bwd_main"]["algorithmic_tflop"] = f_bwd / 1e12  # the row pass has no products
    for name in ("fwd", "bwd_main"):
        kk = kern[name]
        kk["tflops"] = kk["algorithmic_tflop"] / (kk["avg_us"] * 1e-6)
        kk["frac_peak"] = kk["tflops"] / PEAK_BF16_TFLOPS
    # The dominant kernel: the one of the two contraction kernels with the
    # longest launch (the backward main kernel at every workload measured).
    dominant = max(("fwd", "bwd_main"), key=lambda n: kern[n]["avg_us"])
    dk_ = kern[dominant]
    names_k = {"fwd": "forward kernel", "bwd_main": "backward main kernel (bwd_kernel)"}
    roof = {"kernel": names_k[dominant], "bound": "mfma", "achieved": dk_["tflops"],
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": dk_["frac_peak"],
            "traffic": measured_traffic(w.name, dominant) if bias is None and keep is None else None}

    result = {
        "metric": METRIC,
        "value": (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.Sq, "Sk": w.Sk, "E": w.E,
                   "layout": w.layout, "causal": w.causal, "dropout_p": w.dropout_p,
                   "bias": args.bias, "dbias": bool(args.dbias), "keep_bits": bool(args.keep_bits),
                   "cache": "warm (same buffers every step)"},
        "timing": f"replays of a HIP graph of {n_graph} back-to-back steps, K / {n_graph} "
                  "replays between events on the launch stream (ms_per_step_one_step_graph: "
                  "a graph of one step replayed K times; eager_ms_per_step: the same step "
                  "issued from Python each time)",
        "steps_per_graph": n_graph,
        "ms_per_step_one_step_graph": ms_step_1,
        "eager_ms_per_step": ms_eager,
        "fwd": {"tflops": f_fwd / (ms_fwd * 1e-3) / 1e12, "us": ms_fwd * 1e3,
                "frac_peak": f_fwd / (ms_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "eager_us": ms_fwd_eager * 1e3},
        "bwd": {"tflops": f_bwd / (ms_bwd * 1e-3) / 1e12, "us": ms_bwd * 1e3,
                "frac_peak": f_bwd / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "eager_us": ms_bwd_eager * 1e3},
        "kernels": kern,
        "kernels_bracketed": bracketed,
        "kernels_cold_cache": cold,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, do, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
