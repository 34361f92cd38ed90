#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C1]

A step is one whole-layer forward (router -> permute -> grouped SwiGLU experts and the
shared MLP -> combine) over one batch of seeded synthetic tokens resident in HBM. Prints
one JSON line: whole-layer tokens/s, the expert-GEMM TFLOP/s, the roofline of the
dominant kernel (the gate/up pass: routed experts with gathered rows plus the shared
MLP, one persistent launch, SwiGLU fused), per-stage times and the CPU oracle timed on a
bounded sample of the same workload.

Timing: W warm-up steps, then the K timed steps as K forward calls captured in one HIP
graph and replayed once between synchronizations (value, ms_per_step); beside it the
same forward with one graph replay per step (mean over K, and the median of at least 50
individually timed replays), and eager launches. Stage times are medians of 50 graph
replays, each replay holding several back-to-back calls (5 for the expert passes, 10 for
the short stages) and timed per call, so that a replay's own launch and events stay out
of one call's time. --profile-forward N only replays the one-step graph N times, for a
kernel trace of forward steps alone; --profile-backward N does the same for the
fixed-router backward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE fwd tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak), 64e K=4"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_gemm_amd", "csrc", "gemm_stream.hip")
GEMM_CALLS = 5  # expert-pass launches per timed graph replay
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "experts_gateup_olmo64e_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(a, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def gemm_source_sha() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 --pmc
    summary, or None if absent, taken on another workload (name and shapes, as the bench
    line labels it) or from a different version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != gemm_source_sha():
        return None
    if str(t.get("workload", "")).split(",")[0].strip() != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def capture(torch, fn, calls: int = 1):
    """fn() called `calls` times, captured once in a HIP graph (warmed on a side stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm (not captured)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    return g


def replay_times(torch, g, reps: int) -> list:
    """GPU time (ms) of each of `reps` back-to-back replays of graph g, every replay
    bracketed by its own pair of events on the replay stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def time_median(torch, fn, reps: int, calls: int = 1) -> float:
    """Median GPU time (ms) of one fn() call: `reps` timed replays of a graph holding
    `calls` calls (several calls per replay for kernels of a few microseconds, so that a
    replay's launch does not enter its own timing)."""
    g = capture(torch, fn, calls)
    return float(np.median(replay_times(torch, g, reps))) / calls


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gfx_clock_during(torch, g, seconds: float):
    """Median shader (GFX) clock in MHz sampled through amdsmi while graph g replays
    back to back for about `seconds`, over the samples taken while the GPU was busy;
    None where amdsmi is not available or too few samples were."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
    except Exception:  # pragma: no cover - no SMI library or device
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                samples.append(float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]))
            except Exception:
                pass
            time.sleep(0.005)

    one = float(np.median(replay_times(torch, g, 5)))
    n = max(20, int(seconds * 1e3 / max(one, 1e-3)))
    th = threading.Thread(target=sample, daemon=True)
    th.start()
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    keep = samples[len(samples) // 5:]  # drop the ramp at the start of the window
    # samples taken while the GPU sat idle between replays read the idle clock: keep the
    # busy ones (within half of the highest reading)
    if keep:
        top = max(keep)
        keep = [c for c in keep if c >= 0.5 * top]
    return float(np.median(keep)) if len(keep) >= 5 else None


def time_cold(torch, fn, reps: int, scratch) -> float:
    """Median GPU time (ms) of single fn() calls, each after a read of `scratch` (larger
    than the 256 MB Infinity Cache) that leaves neither L2 nor the MALL holding fn's
    inputs. A read, not a write: evicting dirty lines would put write-back traffic inside
    the timed call."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for i in range(reps):
        scratch.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def cpu_baseline(inp, sample_tokens: int):
    """The oracle as it stands, on the first `sample_tokens` tokens of the workload."""
    import oracle.moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    c = inp.cfg
    x = inp.as_float(inp.x[:sample_tokens])
    cap = -1 if c.capacity_factor is None else O.capacity_from_factor(c.capacity_factor, c.K, sample_tokens, c.N)
    spec = O.LayerSpec(N=c.N, K=c.K, score=c.score, renorm=c.renorm, alpha=c.alpha, s=c.s, capacity=cap)
    times = []
    # at least 3 runs and about 10 s of oracle work in all (at most 15 runs)
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 15):
        t0 = time.perf_counter()
        O.forward(spec, x, inp.as_float(inp.w_router), inp.expert_f32, inp.shared_f32(),
                  logit_bias=inp.logit_bias,
                  w_shared_gate=None if inp.w_shared_gate is None else inp.as_float(inp.w_shared_gate))
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{sample_tokens} of {inp.x.shape[0]} tokens of the same layer (all {c.N} experts), fp64 "
                      f"NumPy forward only, median of {len(times)} runs of {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C1")
    ap.add_argument("--tokens", type=int, default=0, metavar="T",
                    help="run the workload's layer on T tokens instead of its own count "
                         "(the workload label names T)")
    ap.add_argument("--stage-reps", type=int, default=50,
                    help="timed replays per stage (the median is reported)")
    ap.add_argument("--profile-backward", type=int, default=0, metavar="N",
                    help="only replay a captured fixed-router backward N times after one forward "
                         "(bf16 workloads; for a kernel trace of backward calls alone)")
    ap.add_argument("--profile-forward", type=int, default=0, metavar="N",
                    help="only replay the captured forward N times after the warmup (for a "
                         "kernel trace of forward steps alone) and print one timing line")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP graph replays of the forward")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the layer runs "
              "unsharded on a single MI355X; expert-parallel sharding across GPUs is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_gemm_amd import synth
    from mixture_experts_layer_gemm_amd import moe

    cfg = synth.get_config(args.workload)
    if args.tokens > 0:
        import dataclasses
        cfg = dataclasses.replace(cfg, T=args.tokens)
    log(f"generating {cfg.name} inputs (T={cfg.T}) ...")
    t0 = time.time()
    inp = synth.make_inputs(cfg)
    log(f"  {time.time() - t0:.1f} s; uploading")
    dt = cfg.dtype
    x = to_device(inp.x, dt, torch)
    w_router = to_device(inp.w_router, dt, torch)
    w_gate, w_up, w_down = (to_device(a, dt, torch) for a in (inp.w_gate, inp.w_up, inp.w_down))
    shared = [tuple(to_device(w, dt, torch) for w in s) for s in inp.shared] or None
    bias = None if inp.logit_bias is None else torch.from_numpy(inp.logit_bias).cuda()
    gate = None if inp.w_shared_gate is None else to_device(inp.w_shared_gate, dt, torch)
    T, d, N, K, d_r = cfg.T, cfg.d_model, cfg.N, cfg.K, cfg.d_r
    workload_label = f"{cfg.name}: T={T} d_model={d} N={N} K={K} d_r={d_r} d_s={cfg.d_s}"
    cap = moe.capacity_from_factor(cfg.capacity_factor, K, T, N) if cfg.capacity_factor is not None else -1
    layer = moe.MoELayer(x, w_router, w_gate, w_up, w_down, K, score=cfg.score, renorm=cfg.renorm,
                         alpha=cfg.alpha, s=cfg.s, capacity=cap, logit_bias=bias, w_shared_gate=gate,
                         shared=shared, keep_intermediates=True)
    torch.cuda.synchronize()

    log(f"warmup {args.warmup}, timed {args.steps} steps")
    for _ in range(args.warmup):
        layer.forward()
    torch.cuda.synchronize()

    def timed(step):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    if args.profile_backward > 0:
        if dt != "bf16":
            print("the backward is bf16 only", file=sys.stderr)
            sys.exit(2)
        layer_t = moe.MoELayer(x, w_router, w_gate, w_up, w_down, K, score=cfg.score,
                               renorm=cfg.renorm, alpha=cfg.alpha, s=cfg.s, capacity=cap,
                               logit_bias=bias, w_shared_gate=gate, shared=shared, trainable=True)
        layer_t.forward()
        dy = torch.randn(T, d, device=x.device, dtype=torch.float32).to(torch.bfloat16)
        gb = capture(torch, lambda: layer_t.backward(dy))
        for _ in range(args.warmup):
            gb.replay()
        torch.cuda.synchronize()
        t = replay_times(torch, gb, args.profile_backward)
        print(json.dumps({"mode": "backward graph replays only", "workload": cfg.name,
                          "replays": len(t), "ms_median": round(float(np.median(t)), 4),
                          "ms_mean": round(float(np.mean(t)), 4)}), flush=True)
        return

    # the forward captured once in a HIP graph; each step is one replay
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward()
    if args.profile_forward > 0:
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t = replay_times(torch, graph, args.profile_forward)
        print(json.dumps({"mode": "forward graph replays only", "workload": cfg.name,
                          "replays": len(t), "ms_median": round(float(np.median(t)), 4),
                          "ms_mean": round(float(np.mean(t)), 4)}), flush=True)
        return

    # eager: every step enqueues the forward's kernels one by one
    ms_eager = timed(layer.forward)
    for _ in range(args.warmup):
        graph.replay()
    # one forward per graph replay: each step pays the replay's launch
    ms_each = timed(graph.replay)
    ms = ms_eager
    if not args.eager:
        # the timed K steps: K forward calls captured back to back in one graph and
        # replayed once, as the layers of a model step run back to back
        graph_k = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_k):
            for _ in range(args.steps):
                layer.forward()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        graph_k.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        del graph_k
    tokens_per_s = T / (ms / 1e3)
    # per-step spread: one forward per replay, every replay timed on its own, at least 50
    step_times = replay_times(torch, graph, max(50, args.steps))
    ms_median = float(np.median(step_times))

    # ---- per-stage timing on the layer's own buffers ------------------------------
    o = layer.out
    R = int(o["offsets"][-1].item())
    esz = 2 if dt == "bf16" else 4
    rows = layer.rows
    reps = args.stage_reps
    log("stage timings")
    st = {}
    pk = layer.weights_packed
    lw = layer.tensors                 # the layer's own (packed) weights
    sm = layer.shared_mlp
    d_s = 0 if sm is None else sm[0].shape[0]
    bufs = dict(h_perm=o["h_perm"], f_perm=o["f_perm"],
                h_shared=torch.empty(T, d_s, dtype=x.dtype, device=x.device) if d_s else None,
                g=torch.empty(T, d, dtype=x.dtype, device=x.device) if d_s else None)

    def experts(pass_, with_shared=True):
        return lambda: moe.moe_experts(x, o["row_token"], o["offsets"], rows, lw["w_gate"],
                                       lw["w_up"], lw["w_down"], shared=sm if with_shared else None,
                                       out=bufs, packed=pk, pass_=pass_)
    # the dominant kernel: the gate/up pass (routed experts + shared MLP, one launch), each
    # replay timed with events on the stream it runs on; medians over `reps` replays of a
    # graph of GEMM_CALLS back-to-back launches, per launch (as the forward runs them: a
    # replay's own launch and events would otherwise enter one launch's time)
    st["experts_gateup_ms"] = time_median(torch, experts(1), reps, calls=GEMM_CALLS)
    st["experts_down_ms"] = time_median(torch, experts(2), reps, calls=GEMM_CALLS)
    # the same passes with the routed experts alone and the shared MLP alone
    apart = {"routed_gateup_ms": time_median(torch, experts(1, False), reps, calls=GEMM_CALLS),
             "routed_down_ms": time_median(torch, experts(2, False), reps, calls=GEMM_CALLS)}
    if sm is not None:
        apart["shared_gateup_ms"] = time_median(torch, lambda: moe.moe_grouped_gemm(
            x, None, sm[0][None], sm[1][None], out=bufs["h_shared"], swiglu=True, packed=pk),
            reps, calls=GEMM_CALLS)
        apart["shared_down_ms"] = time_median(torch, lambda: moe.moe_grouped_gemm(
            bufs["h_shared"], None, sm[2][None], out=bufs["g"], swiglu=False, packed=pk),
            reps, calls=GEMM_CALLS)
    # shader clock while the gate/up pass replays back to back for about a second
    clock_mhz = gfx_clock_during(torch, capture(torch, experts(1)), 1.0)
    st["route_ms"] = time_median(torch, lambda: moe.moe_route(
        x, w_router, K, score=cfg.score, renorm=cfg.renorm, alpha=cfg.alpha, logit_bias=bias,
        w_shared_gate=gate, want_counts=False), reps, calls=10)
    idx = o["topk_idx"]
    st["permute_ms"] = time_median(torch, lambda: moe.moe_permute(x, idx, N, cap, copy_rows=False),
                                   reps, calls=10)
    y2 = torch.empty_like(layer.y)
    st["combine_ms"] = time_median(torch, lambda: moe.moe_combine(
        o["f_perm"], o["dest_row"], o["topk_r"], o.get("g"), s=cfg.s, s_tok=o.get("s_tok"), y=y2),
        reps, calls=10)

    # the same three stages with cold caches (a 512 MB read before each call)
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=x.device)
    cold = {}
    cold["route_ms"] = time_cold(torch, lambda: moe.moe_route(
        x, w_router, K, score=cfg.score, renorm=cfg.renorm, alpha=cfg.alpha, logit_bias=bias,
        w_shared_gate=gate, want_counts=False), reps, scratch)
    cold["permute_ms"] = time_cold(torch, lambda: moe.moe_permute(x, idx, N, cap, copy_rows=False),
                                   reps, scratch)
    cold["combine_ms"] = time_cold(torch, lambda: moe.moe_combine(
        o["f_perm"], o["dest_row"], o["topk_r"], o.get("g"), s=cfg.s, s_tok=o.get("s_tok"), y=y2),
        reps, scratch)
    del scratch

    # next rows on the same batch: balance statistics, rank-wide capacity (8 destinations
    # of N/8 experts, capacity factor 1), biased selection and the bias controller
    nx = {}
    z_l = o["logits"]
    nx["balance_stats_ms"] = time_median(torch, lambda: moe.moe_balance_stats(
        z_l, o["C_req"], o["C_keep"], o["dest_row"], o["topk_r"], score=cfg.score), reps, calls=10)
    grp = N // 8 if N % 8 == 0 else N
    rcap = moe.rank_capacity_from_factor(1.0, K, -(-T // (N // grp)))
    nx["permute_rank_capacity_ms"] = time_median(torch, lambda: moe.moe_permute(
        x, idx, N, rcap, copy_rows=False, capacity_group=grp), reps, calls=10)
    eb = torch.linspace(-0.5, 0.5, N, device=x.device, dtype=torch.float32)
    nx["route_biased_ms"] = time_median(torch, lambda: moe.moe_route(
        x, w_router, K, score=cfg.score, renorm=cfg.renorm, alpha=cfg.alpha, logit_bias=bias,
        w_shared_gate=gate, want_counts=False, expert_bias=eb), reps, calls=10)
    acc = o["C_req"].clone()
    nx["bias_update_ms"] = time_median(torch, lambda: moe.moe_bias_update(acc, eb, 1e-3, reset=False),
                                       reps, calls=10)
    nx_bytes = {"balance_stats": T * N * 4 + T * K * 8 + 8 * N}
    # f4: fixed-router backward on the same batch (recompute A, B; dH; dX; weight gradients)
    bwd_flops = None
    if dt == "bf16":
        layer_t = moe.MoELayer(x, w_router, w_gate, w_up, w_down, K, score=cfg.score,
                               renorm=cfg.renorm, alpha=cfg.alpha, s=cfg.s, capacity=cap,
                               logit_bias=bias, w_shared_gate=gate, shared=shared, trainable=True)
        layer_t.forward()
        dy = torch.randn(T, d, device=x.device, dtype=torch.float32).to(torch.bfloat16)
        nx["backward_ms"] = time_median(torch, lambda: layer_t.backward(dy), max(5, reps // 5))
        R_t = int(layer_t.out["offsets"][-1].item())
        bwd_flops = 16.0 * R_t * d * d_r + 16.0 * T * d * (layer_t.shared_mlp[0].shape[0]
                                                           if layer_t.shared_mlp else 0)
        del layer_t

    # algorithmic work (each counted once): flops of the contractions; bytes = weights of
    # the active experts and the shared MLP, x read once, h written once
    act_experts = int((o["C_keep"] > 0).sum().item())
    flops_gateup = 4.0 * R * d * d_r + 4.0 * T * d * d_s
    flops_experts = 6.0 * R * d * d_r + 6.0 * T * d * d_s
    bytes_gateup = esz * (2 * act_experts * d_r * d + 2 * d_s * d + T * d + R * d_r + T * d_s)
    t_gateup = st["experts_gateup_ms"] * 1e-3
    expert_tflops = flops_experts / ((st["experts_gateup_ms"] + st["experts_down_ms"]) * 1e-3) / 1e12
    t_mfma = flops_gateup / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = bytes_gateup / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:   # the binding roofline of this shape
        roof = {"bound": "hbm", "achieved": round(bytes_gateup / t_gateup / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops_gateup / t_gateup / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(workload_label)
    stage_bytes = {
        "route": T * d * esz + N * d * esz + T * K * 8,
        # count: idx in, ranks out; map: idx + ranks in, dest_row + row_token out
        "permute": T * K * 20 + R * 4,
        "combine": R * d * esz + (2 if d_s else 1) * T * d * esz + T * K * 8,
    }
    hbm = {k: b / (st[k + "_ms"] * 1e-3) / 1e9 for k, b in stage_bytes.items()}
    hbm_cold = {k: b / (cold[k + "_ms"] * 1e-3) / 1e9 for k, b in stage_bytes.items()}
    # the persistent GEMM takes two row halves (8 waves, 2 weight stages in flight) when
    # the packed bound holds at least 1024 rows per group, else one (4 waves, 4 stages)
    rh2 = rows >= 1024 * N
    kernel_label = ("gate/up pass: routed experts (gathered rows) + shared MLP, SwiGLU fused "
                    "(gemm_stream_kernel<2,4,%s,1>)" % ("2,2" if rh2 else "4,1")) if pk else \
        "routed gate/up grouped GEMM (row-major weights)"
    routed_flops = 6.0 * R * d * d_r
    t_routed = (apart["routed_gateup_ms"] + apart["routed_down_ms"]) * 1e-3
    gemm = {"routed_kept_tflops": round(routed_flops / t_routed / 1e12, 1),
            "routed_kept_frac_bf16_peak": round(routed_flops / t_routed / 1e12 / PEAK_BF16_TFLOPS, 4),
            "passes_ms": {k.replace("_ms", ""): round(v, 4) for k, v in apart.items()}}
    if d_s:
        shared_flops = 6.0 * T * d * d_s
        t_sh = (apart["shared_gateup_ms"] + apart["shared_down_ms"]) * 1e-3
        gemm["shared_tflops"] = round(shared_flops / t_sh / 1e12, 1)
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_one_per_replay": round(ms_each, 4),
        "ms_per_step_one_per_replay_median": round(ms_median, 4),
        "step_reps": len(step_times),
        "launch": "eager" if args.eager else "hip_graph: the K timed steps captured in one graph",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else "f32",
        "data": "synthetic: seeded normals (x ~ N(0,1), weights ~ N(0, %g)), bf16-rounded" % cfg.std_w,
        "config": {"workload": workload_label,
                   "T": T, "d_model": d, "N": N, "K": K, "d_r": d_r, "d_s": cfg.d_s,
                   "score": ["softmax", "sigmoid", "softmax_selected"][cfg.score],
                   "renorm": cfg.renorm, "alpha": cfg.alpha, "capacity": cap,
                   "kept_routes": R, "active_experts": act_experts},
        "expert_gemm_tflops": round(expert_tflops, 1),
        "expert_gemm_frac_bf16_peak": round(expert_tflops / PEAK_BF16_TFLOPS, 4),
        # the routed experts (kept routes only) and the shared MLP run in the same two
        # launches, so the rate above is over both; their flops apart:
        "expert_gemm_gflop": {"routed_kept": round(6.0 * R * d * d_r / 1e9, 1),
                              "shared": round(6.0 * T * d * d_s / 1e9, 1)},
        # the same work in launches of its own: the routed experts alone (6 d d_r per kept
        # route over their two passes) and the shared MLP alone
        "grouped_gemm_apart": gemm,
        "shader_clock_mhz": None if clock_mhz is None else round(clock_mhz),
        "peak_bf16_at_clock_tflops": (None if clock_mhz is None else
                                      round(PEAK_BF16_TFLOPS * clock_mhz / 2400.0, 1)),
        "stage_timing": f"median of {reps} graph replays per stage, per call (expert passes: "
                        f"{GEMM_CALLS} calls per replay; route, permute, combine and the short "
                        "next rows: 10)",
        "roofline": dict(kernel=kernel_label,
                         time="median of %d replays of %d back-to-back launches, per launch"
                              % (reps, GEMM_CALLS),
                         **roof, algorithmic_bytes=bytes_gateup, flops_per_launch=flops_gateup,
                         mfma_tflops=round(flops_gateup / t_gateup / 1e12, 1),
                         mfma_frac=round(flops_gateup / t_gateup / 1e12 / PEAK_BF16_TFLOPS, 4)),
        "stages_ms": {k.replace("_ms", ""): round(v, 4) for k, v in st.items()},
        "stages_hbm_frac": {k: round(v / PEAK_HBM_GBS, 3) for k, v in hbm.items()},
        "stages_ms_cold": {k.replace("_ms", ""): round(v, 4) for k, v in cold.items()},
        "stages_hbm_frac_cold": {k: round(v / PEAK_HBM_GBS, 3) for k, v in hbm_cold.items()},
        "next_rows_ms": {k.replace("_ms", ""): round(v, 4) for k, v in nx.items()},
        "backward_tflops": (round(bwd_flops / (nx["backward_ms"] * 1e-3) / 1e12, 1)
                            if bwd_flops else None),
        "next_rows_hbm_frac": {"balance_stats": round(
            nx_bytes["balance_stats"] / (nx["balance_stats_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)},
    }
    # what a plain streaming read reaches on this GPU (row sums over 1 GiB of fp32 that no
    # cache holds), the practical ceiling beside the 8 TB/s spec figure
    probe = torch.ones(256 << 20, dtype=torch.float32, device=x.device).view(-1, 4096)
    probe.sum(dim=1)
    torch.cuda.synchronize()
    pt = []
    for _ in range(5):   # eager: a torch reduction is not captured in a graph here
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        probe.sum(dim=1)
        e1.record()
        torch.cuda.synchronize()
        pt.append(e0.elapsed_time(e1))
    probe_ms = float(np.median(pt))
    out["hbm_read_probe_gbs"] = round(probe.numel() * 4 / (probe_ms * 1e-3) / 1e9, 1)
    del probe
    torch.cuda.synchronize()
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=x.device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = args.copy_probe_mib << 20
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_sample_tokens, T))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
