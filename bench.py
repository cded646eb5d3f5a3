#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

A step is one moe_chunked_forward call: routing metadata for every chunk,
then per chunk pair, on one HIP stream: one gate/up GEMM + SwiGLU launch over
both chunks' rows that gathers its rows straight from hidden_states (the
permute fused into its row addressing), one down GEMM launch, and the two
chunks' weighted combines.  The per-chunk schedule (every chunk runs permute,
FFN and combine on its own stream, two streams alternating) is timed beside it.  Inputs are seeded
synthetic data already resident in HBM when the timed region starts.

Prints ONE JSON line: MoE-layer tokens/s (T / seconds per step), the roofline
of the dominant kernel (the gate/up grouped GEMM) measured live with HIP
events on the stream it runs on, and the CPU oracle timed on the host cores on
a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--num-chunks N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s (permute+expert GEMM+combine); % HBM / % MFMA peak"
HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}  # dense FLOP/s (fp32: matrix/vector peak)
GATE_UP_SRCS = tuple(os.path.join(ROOT, "combine_top_route_expert_amd", "csrc", f)
                     for f in ("gemm_bf16.hip", "moe_internal.h"))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(paths=GATE_UP_SRCS):
    """Hash of the code the gate/up kernel is built from, comments and blank
    space dropped, so that an edit of a comment keeps the recorded counters."""
    import re
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def make_inputs(cfg, torch, synth):
    import numpy as np
    idx, w = synth.routing(cfg)
    hidden = synth.hidden_states(cfg, "cuda")
    wgu, wd = synth.all_expert_weights(cfg, "cuda")
    torch.cuda.synchronize()
    return {"hidden": hidden, "idx": torch.from_numpy(idx).cuda(),
            "w": torch.from_numpy(w).cuda(), "wgu": wgu, "wd": wd,
            "idx_np": idx, "w_np": w, "counts": np.bincount(idx.ravel(), minlength=cfg.E)}


def time_layer(moe, torch, shape, inp, steps, warmup, two_streams=True,
               schedule=None):
    cfg_dtype = shape.torch_dtype
    out = torch.empty((shape.T, shape.H), dtype=cfg_dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else None

    def step():
        if schedule is None:
            moe.moe_chunked_forward(shape, inp["hidden"], inp["idx"], inp["w"], inp["wgu"],
                                    inp["wd"], out, ws, err, s0=s0, s1=s1)
        else:
            moe.moe_chunked_forward_schedule(shape, inp["hidden"], inp["idx"], inp["w"],
                                             inp["wgu"], inp["wd"], out, ws, err, s0=s0, s1=s1,
                                             schedule=schedule)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s0)
    for _ in range(steps):
        step()
    e1.record(s0)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"wall_ms": wall_ms, "event_ms": e0.elapsed_time(e1) / steps,
            "workspace_bytes": ws.numel(), "dev_error": int(err.item())}


def time_backward(moe, torch, shape, inp, steps, warmup):
    """Average time of moe_chunked_backward (forward recomputed per chunk pair)."""
    dt = shape.torch_dtype
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I
    go = inp["hidden"]  # any [T,H] tensor of the layer dtype serves as the upstream gradient
    gh = torch.empty((T, H), dtype=dt, device="cuda")
    gw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    gwgu = torch.empty((E, 2 * I, H), dtype=torch.float32, device="cuda")
    gwd = torch.empty((E, H, I), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_backward_workspace_size(shape), dtype=torch.uint8, device="cuda")
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()

    def step():
        moe.moe_chunked_backward(shape, inp["hidden"], inp["idx"], inp["w"], inp["wgu"], inp["wd"],
                                 go, gh, gw, gwgu, gwd, ws, None, s0=s0, s1=s1)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del gwgu, gwd
    return ms, ws.numel()


def time_graph(moe, torch, shape, inp, steps):
    """The same layer step captured once in a HIP graph and replayed: removes the
    host launch cost and the gaps between the step's kernels."""
    out = torch.empty((shape.T, shape.H), dtype=shape.torch_dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        moe.moe_chunked_forward(shape, inp["hidden"], inp["idx"], inp["w"], inp["wgu"], inp["wd"],
                                out, ws, None, s0=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_chunked_forward(shape, inp["hidden"], inp["idx"], inp["w"], inp["wgu"], inp["wd"],
                                out, ws, None, s0=torch.cuda.current_stream())
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def per_step_times(moe, torch, shape, inp, reps, flush_bytes=0):
    """Median and minimum of single-step times (HIP events around each step).  With
    flush_bytes > 0 a scratch buffer of that size is written before every step,
    outside the timed window, so L2 and MALL start cold."""
    out = torch.empty((shape.T, shape.H), dtype=shape.torch_dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    times = []
    for i in range(reps + 2):
        if scratch is not None:
            scratch.fill_(i & 0xff)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s0)
        moe.moe_chunked_forward(shape, inp["hidden"], inp["idx"], inp["w"], inp["wgu"], inp["wd"],
                                out, ws, None, s0=s0, s1=s1)
        e1.record(s0)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    times.sort()
    return {"median_ms": times[len(times) // 2], "min_ms": times[0], "reps": reps,
            "flush_bytes": flush_bytes}


def kernel_times(moe, torch, shape, inp, reps):
    """Average duration of each launch the layer makes for its first chunk pair
    (route_meta for all chunks; permute and combine of chunk 0; the gate_up and
    down launches over chunks 0 and 1), HIP events on the stream the kernels
    run on (torch's current stream)."""
    T, k, E, N, G, H, I = shape.T, shape.k, shape.E, shape.N, shape.G, shape.H, shape.I
    dt = shape.torch_dtype
    i32 = dict(dtype=torch.int32, device="cuda")
    counts = torch.empty((N, E), **i32)
    offsets = torch.empty((N, E + 1), **i32)
    splits = torch.empty((N, G), **i32)
    src_row = torch.empty(T * k, **i32)
    dst_row = torch.empty(T * k, **i32)
    err = torch.empty(1, **i32)
    mws = torch.empty(moe.moe_route_meta_workspace_size(shape), dtype=torch.uint8, device="cuda")
    rows = []
    for c in range(min(N, 2)):
        t0, t1 = moe.moe_chunk_range(shape, c)
        rows.append((t1 - t0) * k)
    if len(rows) < 2:
        rows.append(0)
    xp = [torch.empty((max(r, 1), H), dtype=dt, device="cuda") for r in rows]
    act = torch.empty((rows[0] + rows[1], I), dtype=dt, device="cuda")
    out = torch.empty((T, H), dtype=dt, device="cuda")
    s = torch.cuda.current_stream()
    x1 = xp[1] if rows[1] else None
    calls = {
        "route_meta": lambda: moe.moe_route_meta(shape, inp["idx"], counts, offsets, splits,
                                                 src_row, dst_row, err, mws, s),
        "permute": lambda: moe.moe_permute(shape, 0, inp["hidden"], dst_row, xp[0], s),
        "gate_up": lambda: moe.moe_expert_gate_up_gather_pair(shape, 0, inp["hidden"], src_row,
                                                              offsets, inp["wgu"], act, s),
        "down": lambda: moe.moe_expert_down_pair(shape, 0, act, offsets, inp["wd"], xp[0], x1, s),
        "combine": lambda: moe.moe_unpermute_combine(shape, 0, xp[0], dst_row, inp["w"], out, s),
    }
    res = {}
    for name, fn in calls.items():
        fn()
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / reps  # microseconds per launch
    cp = counts[:2].sum(0).cpu()
    return res, int(cp.sum().item()), int((cp > 0).sum().item()), rows


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3)


def load_traffic(config_name, N):
    """HBM bytes per gate/up launch from committed rocprofv3 --pmc counters, if they
    were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"gate_up_gemm_{config_name}_N{N}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inp, synth, target_s=15.0):
    """The oracle, as it stands, on a bounded prefix of the same workload."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    hid = synth.to_f64(inp["hidden"])
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = (synth.to_f64(inp["wgu"][e]), synth.to_f64(inp["wd"][e]))
        return cache[e]

    def run(ts):
        for e in np.unique(inp["idx_np"][:ts]):
            get(int(e))  # input conversion happens outside the timed region
        t = time.perf_counter()
        oracle.moe_forward(hid[:ts], inp["idx_np"][:ts], inp["w_np"][:ts], get, cfg.E, cfg.I,
                           cfg.groups, 1)
        return time.perf_counter() - t

    ts = min(cfg.T, 128)
    el = run(ts)
    while el < target_s / 3 and ts < cfg.T:
        ts = min(cfg.T, max(ts * 2, int(ts * target_s / max(el, 1e-3))))
        el = run(ts)
    # a sample that finishes quickly is repeated until about target_s/1.5 of CPU work
    reps, total = 1, el
    while total < target_s / 1.5:
        total += run(ts)
        reps += 1
    return {"value": ts * reps / total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {ts} of {cfg.T} tokens of {cfg.name} (N=1), float64 numpy oracle, "
                      f"{reps} run(s), {total:.1f} s; expert weights converted to float64 outside "
                      f"the timing"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="bf16_e64_zipf")
    ap.add_argument("--num-chunks", type=int, default=2)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this MoE layer build runs on one "
              "GPU only (no multi-GPU path); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_top_route_expert_amd as moe
    import synth

    moe.load_library()
    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    N = args.num_chunks
    log(f"inputs {cfg.name}")
    inp = make_inputs(cfg, torch, synth)
    shape = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.groups, N, cfg.dtype)

    # one common warm-up (clocks, caches, allocator) before any timed run: at
    # least 20 steps and one second, since the GPU reaches its steady clock only
    # after some 100 ms of load (a first timed run right after 20 steps measured
    # 8% slower than the next ones)
    log("warm-up")
    t_warm = time.perf_counter()
    time_layer(moe, torch, shape, inp, 1, max(args.warmup, 20))
    while time.perf_counter() - t_warm < 1.0:
        time_layer(moe, torch, shape, inp, 1, 50)
    log(f"layer N={N}")
    main_run = time_layer(moe, torch, shape, inp, args.steps, args.warmup)
    log(f"layer N=1 (reference)")
    shape1 = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.groups, 1, cfg.dtype)
    run1 = time_layer(moe, torch, shape1, inp, args.steps, args.warmup, two_streams=False)
    log(f"layer N={N}, per-chunk schedule")
    run_pc = time_layer(moe, torch, shape, inp, args.steps, args.warmup,
                        schedule=moe.MOE_SCHEDULE_PER_CHUNK)
    log("layer replayed from a HIP graph")
    graph_ms = time_graph(moe, torch, shape, inp, args.steps)
    log("single steps, warm and with L2/MALL flushed")
    warm = per_step_times(moe, torch, shape, inp, 20)
    cold = per_step_times(moe, torch, shape, inp, 20, flush_bytes=1 << 30)
    log(f"backward N={N}")
    bwd_ms, bwd_ws = time_backward(moe, torch, shape, inp, max(5, args.steps // 5), 2)
    log("per-kernel timing")
    kt, rows0, e_act0, chunk_rows = kernel_times(moe, torch, shape, inp, args.kernel_reps)
    copy_bw = copy_bandwidth(torch)

    s = cfg.elem_bytes
    H, I = cfg.H, cfg.I
    A_valid = int(inp["counts"].sum())
    # the gate/up launch reads each of the pair's tokens' rows (gathered from
    # hidden_states), every active expert's weights once, and writes act
    pair_tokens = min(cfg.T, 2 * -(-cfg.T // N)) if N >= 2 else cfg.T
    gu_bytes = pair_tokens * H * s + e_act0 * 2 * I * H * s + rows0 * I * s
    gu_flops = 2.0 * rows0 * H * 2 * I
    gu_s = kt["gate_up"] * 1e-6
    peak_f = MFMA_PEAK[cfg.dtype]
    if gu_bytes / HBM_PEAK >= gu_flops / peak_f:
        roof = {"bound": "hbm", "achieved": gu_bytes / gu_s / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gu_flops / gu_s / 1e12, "peak": peak_f / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    traffic = load_traffic(cfg.name, N)
    roof["traffic"] = traffic
    roof["kernel"] = ("grouped_gemm_bf16<gate_up> (moe_expert_gate_up_gather_pair), chunks 0-1"
                      if N >= 2 else
                      "grouped_gemm_bf16<gate_up> (moe_expert_gate_up_gather_pair), chunk 0")
    roof["rows_per_launch"] = rows0
    roof["algorithmic_bytes_per_launch"] = gu_bytes
    roof["algorithmic_flop_per_launch"] = gu_flops
    roof["avg_launch_us"] = kt["gate_up"]
    roof["mfma_frac"] = gu_flops / gu_s / peak_f

    # every launch the layer makes for its first chunk pair, against its own
    # roofline: algorithmic bytes (and flop) per launch / the launch's time
    tok0 = chunk_rows[0] // cfg.k  # tokens of chunk 0
    dn_bytes = rows0 * I * s + e_act0 * H * I * s + rows0 * H * s
    per_kernel = {
        "route_meta": (12 * cfg.T * cfg.k, 0.0, "all chunks: ids read once, src_row and dst_row written"),
        "permute": (tok0 * H * s + chunk_rows[0] * H * s + 4 * chunk_rows[0], 0.0,
                    "chunk 0 (per-chunk schedule; the pair-fused layer gathers in gate_up)"),
        "gate_up": (gu_bytes, gu_flops, "chunks 0-1, rows gathered from hidden_states"),
        "down": (dn_bytes, 2.0 * rows0 * H * I, "chunks 0-1"),
        "combine": (chunk_rows[0] * H * s + tok0 * H * s + 8 * chunk_rows[0], 0.0, "chunk 0"),
    }
    kernels_roofline = {}
    for name, (nbytes, flop, what) in per_kernel.items():
        sec = kt[name] * 1e-6
        r = {"us": kt[name], "bytes": nbytes, "GBps": nbytes / sec / 1e9,
             "hbm_frac": nbytes / sec / HBM_PEAK, "launch": what}
        if flop:
            r.update({"flop": flop, "TFLOPs": flop / sec / 1e12, "mfma_frac": flop / sec / peak_f})
        kernels_roofline[name] = r

    ms = main_run["wall_ms"]
    line = {
        "metric": METRIC, "value": cfg.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": H, "E": cfg.E, "top_k": cfg.k,
                   "I": I, "num_chunks": N, "streams": 1, "schedule": "pair_fused",
                   "groups": cfg.groups},
        "roofline": roof,
        "kernels_us": kt,
        "kernels_roofline": kernels_roofline,
        "event_ms_per_step": main_run["event_ms"],
        "unchunked": {"ms_per_step": run1["wall_ms"], "value": cfg.T / (run1["wall_ms"] * 1e-3)},
        "per_chunk_schedule": {"ms_per_step": run_pc["wall_ms"],
                               "value": cfg.T / (run_pc["wall_ms"] * 1e-3)},
        "hip_graph": {"ms_per_step": graph_ms, "value": cfg.T / (graph_ms * 1e-3),
                      "note": "the same step captured once and replayed"},
        "single_step": {"warm": warm, "cold": cold},
        "backward": {"ms_per_step": bwd_ms, "value": cfg.T / (bwd_ms * 1e-3),
                     "flop_per_step": 18.0 * A_valid * H * I,
                     "tflops": 18.0 * A_valid * H * I / (bwd_ms * 1e-3) / 1e12,
                     "workspace_bytes": bwd_ws,
                     "note": "moe_chunked_backward: forward recomputed per chunk pair, "
                             "grads of hidden_states, top_k_weights (fp32) and both expert "
                             "weight tensors (fp32); flop = 18*A*H*I"},
        "workspace_bytes": {"N": main_run["workspace_bytes"], "N1": run1["workspace_bytes"],
                            "slots_model_N": min(N, 2) * -(-cfg.T // N) * cfg.k * (H + I) * s},
        "copy_bandwidth_GBps": copy_bw / 1e9,
        "expert_load": {"max_over_mean": float(inp["counts"].max() / inp["counts"].mean()),
                        "empty_experts": int((inp["counts"] == 0).sum())},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, synth)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
