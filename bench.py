#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

A step is one moe_chunked_forward call: routing metadata for every chunk,
then per chunk pair, on one HIP stream: one gate/up GEMM + SwiGLU launch over
both chunks' rows that gathers its rows straight from hidden_states (the
permute fused into its row addressing), one down GEMM launch, and the two
chunks' weighted combines.  Inputs are seeded synthetic data already resident
in HBM when the timed region starts.

Headline (default): the DeepSeek-V3-shaped layer (T=4096, H=7168, E=256
routed experts, top-8, I=2048, bf16, all experts on this GPU), num_chunks=1.
`value` is T / (mean time of K single steps, each started with L2 and MALL
flushed by writing a 1 GiB scratch buffer outside its HIP-event window).
Back-to-back (pipelined) steps, a replayed HIP graph, the per-chunk two-stream
schedule, the backward and a num_chunks sweep of the packed 16k-token layer
(time and requested workspace against the W_pair model) are reported beside
it.

Prints ONE JSON line: MoE-layer tokens/s, the roofline of the dominant kernel
(the gate/up grouped GEMM) measured live with HIP events on the stream it runs
on, and the CPU oracle timed on the host cores on a bounded sample of the same
workload.

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


_STREAM_PAIR = []


def stream_pair(torch):
    """The two streams of the two-stream schedules: the first two streams the
    process takes from torch's stream pool, created once and reused.  HIP runs
    its streams on a few hardware queues (four by default); the null stream holds
    the first, the next streams created each get one of their own, and later ones
    share them.  Two streams on one queue run their kernels one after another, so
    a pair taken later could serialise the schedule (a kernel trace showed an
    arbitrary pool stream on the null stream's queue)."""
    if not _STREAM_PAIR:
        _STREAM_PAIR.extend((torch.cuda.Stream(), torch.cuda.Stream()))
    return _STREAM_PAIR[0], _STREAM_PAIR[1]


def time_layer(moe, torch, shape, inp, steps, warmup, two_streams=True,
               schedule=None):
    cfg_dtype = shape.torch_dtype
    out = torch.empty((shape.T, shape.H), dtype=cfg_dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if two_streams:
        s0, s1 = stream_pair(torch)
    else:
        s0, s1 = torch.cuda.current_stream(), None

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


def per_step_times(moe, torch, shape, inp, reps, flush_bytes=0, warmup=2):
    """Single-step times: HIP events on s0 around each of `reps` steps, with a
    device synchronisation on both sides of every step.  With flush_bytes > 0 a
    scratch buffer of that size is written before every step, outside its
    event window, so L2 and MALL start cold.  Returns the mean (the headline
    rate uses it), median and minimum."""
    out = torch.empty((shape.T, shape.H), dtype=shape.torch_dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    times = []
    t_wall = 0.0
    for i in range(reps + warmup):
        if scratch is not None:
            scratch.fill_(i & 0xff)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(s0)
        moe.moe_chunked_forward(shape, inp["hidden"], inp["idx"], inp["w"], inp["wgu"], inp["wd"],
                                out, ws, err, s0=s0, s1=s1)
        e1.record(s0)
        torch.cuda.synchronize()
        if i >= warmup:
            t_wall += time.perf_counter() - t0
            times.append(e0.elapsed_time(e1))
    srt = sorted(times)
    return {"mean_ms": sum(times) / len(times), "median_ms": srt[len(srt) // 2],
            "min_ms": srt[0], "max_ms": srt[-1], "reps": reps, "flush_bytes": flush_bytes,
            "wall_ms_mean": t_wall * 1e3 / reps, "dev_error": int(err.item()),
            "workspace_bytes": ws.numel()}


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


def cpu_info():
    """Host cores the process may use, and the CPU model."""
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        usable = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"nproc": usable, "cpu_count": os.cpu_count(), "cpu_model": model}


def cpu_baseline(cfg, inp, synth, torch, target_s=12.0, max_runs=4):
    """The oracle, as it stands, on a bounded prefix of the same workload (N=1).

    Expert weights are handed to the oracle one expert at a time as exact
    float64 copies (converted on the device, then copied to the host), and
    nothing is cached, so host memory stays bounded for every workload; the
    time spent in those conversions is measured and left out of the oracle's
    time.  The prefix grows until the oracle works about target_s / 3 seconds
    (at most max_runs runs)."""
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    hid = synth.to_f64(inp["hidden"])
    conv = [0.0, 0]

    def get(e):
        t = time.perf_counter()
        pair = (inp["wgu"][e].to(torch.float64).cpu().numpy(),
                inp["wd"][e].to(torch.float64).cpu().numpy())
        conv[0] += time.perf_counter() - t
        conv[1] += 1
        return pair

    def run(ts):
        log(f"  oracle on the first {ts} tokens")
        conv[0], conv[1] = 0.0, 0
        t = time.perf_counter()
        oracle.moe_forward(hid[:ts], inp["idx_np"][:ts], inp["w_np"][:ts], get, cfg.E, cfg.I,
                           cfg.groups, 1)
        return time.perf_counter() - t - conv[0], conv[1]

    ts = min(cfg.T, 16)
    el, n_exp = run(ts)
    runs = 1
    while el < target_s / 3 and ts < cfg.T and runs < max_runs:
        ts = min(cfg.T, max(ts * 2, int(ts * target_s / max(el, 1e-3))))
        el, n_exp = run(ts)
        runs += 1
    reps, total = 1, el
    while total < target_s / 1.5 and runs < max_runs:
        more, _ = run(ts)
        total += more
        reps += 1
        runs += 1
    d = {"value": ts * reps / total, "unit": "tokens/s", "cores": int(threads),
         "kind": "oracle",
         "sample": f"first {ts} of {cfg.T} tokens of {cfg.name} (N=1; {n_exp} experts touched), "
                   f"float64 numpy oracle (oracle.moe_forward), {reps} timed run(s), "
                   f"{total:.1f} s of oracle time; each expert's weights converted to float64 "
                   f"one expert at a time, outside the timing"}
    d.update(cpu_info())
    d["blas_threads"] = int(threads)
    return d


def chunk_sweep(moe, torch, synth, name, Ns, steps):
    """num_chunks sweep of one workload: time per step of both schedules and the
    workspace the library requests, against the W_pair model
    min(N, 2) * ceil(T/N) * k * (H + I) * element bytes (the pair residency of
    the Chunk MoE key formulas; H + I because y overwrites the dead x_perm)."""
    cfg = synth.CONFIGS[name]
    log(f"chunk sweep inputs {name}")
    inp = make_inputs(cfg, torch, synth)
    s = cfg.elem_bytes
    res = {"workload": name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
           "points": []}
    for N in Ns:
        shape = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.groups, N, cfg.dtype)
        log(f"chunk sweep {name} N={N}")
        time_layer(moe, torch, shape, inp, 1, 5)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fused = time_layer(moe, torch, shape, inp, steps, 3)
        peak = torch.cuda.max_memory_allocated() - base
        per_chunk = time_layer(moe, torch, shape, inp, steps, 3,
                               schedule=moe.MOE_SCHEDULE_PER_CHUNK)
        model = min(N, 2) * -(-cfg.T // N) * cfg.k * (cfg.H + cfg.I) * s
        res["points"].append({
            "N": N, "ms_pair_fused": fused["wall_ms"], "ms_per_chunk_two_streams": per_chunk["wall_ms"],
            "tokens_per_s_pair_fused": cfg.T / (fused["wall_ms"] * 1e-3),
            "workspace_requested_bytes": fused["workspace_bytes"],
            "w_pair_model_bytes": model,
            "workspace_over_model": fused["workspace_bytes"] / model,
            "peak_alloc_workspace_and_out_bytes": peak})
    del inp
    torch.cuda.empty_cache()
    return res


def vendor_dense_gemm(torch, reps=20):
    """Context for the matrix-core fractions: the vendor library's dense bf16 GEMM
    (torch.matmul on contiguous 2-D operands, hipBLASLt underneath) on the shapes
    of the MFMA-bound expert launches, one expert's worth: the two-expert skew's
    gate/up (4000 x 7168 by 7168 x 4096) and down (4000 x 2048 by 2048 x 7168),
    and a dense 16384 x 2048 by 2048 x 1536 (the packed 16k-token gate/up if all
    rows went to one expert).  Not on the layer's path."""
    res = {}
    for name, (m, kk, n) in {"skew_gate_up_one_expert": (4000, 7168, 4096),
                             "skew_down_one_expert": (4000, 2048, 7168),
                             "packed16k_gate_up_dense": (16384, 2048, 1536)}.items():
        a = torch.randn(m, kk, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(kk, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        flop = 2.0 * m * kk * n
        res[name] = {"m": m, "k": kk, "n": n, "us": sec * 1e6, "TFLOPs": flop / sec / 1e12,
                     "mfma_frac": flop / sec / MFMA_PEAK["bf16"]}
        del a, b
    return res


def prefetch_ab(moe, torch, synth, name, base_cfg, base_inp, rounds=3, steps=20):
    """The pair-fused schedule with and without the weight warm-up on a second
    stream (MOE_SCHEDULE_PAIR_FUSED_PREFETCH), interleaved over `rounds`, on one
    workload; its expert weights are reused from the headline inputs when they are
    the same tensors."""
    cfg = synth.CONFIGS[name]
    same_w = (cfg.weight_seed, cfg.E, cfg.H, cfg.I, cfg.dtype) == \
        (base_cfg.weight_seed, base_cfg.E, base_cfg.H, base_cfg.I, base_cfg.dtype)
    if name == base_cfg.name:
        inp = base_inp
    else:
        import numpy as np
        idx, w = synth.routing(cfg)
        inp = {"hidden": synth.hidden_states(cfg, "cuda"), "idx": torch.from_numpy(idx).cuda(),
               "w": torch.from_numpy(w).cuda()}
        if same_w:
            inp["wgu"], inp["wd"] = base_inp["wgu"], base_inp["wd"]
        else:
            inp["wgu"], inp["wd"] = synth.all_expert_weights(cfg, "cuda")
    shape = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.groups, cfg.num_chunks[0],
                           cfg.dtype)
    res = {"default": [], "prefetch": []}
    for _ in range(rounds):
        res["default"].append(time_layer(moe, torch, shape, inp, steps, 3)["wall_ms"])
        res["prefetch"].append(time_layer(moe, torch, shape, inp, steps, 3,
                                          schedule=moe.MOE_SCHEDULE_PAIR_FUSED_PREFETCH)["wall_ms"])
    med = {k: sorted(v)[len(v) // 2] for k, v in res.items()}
    return {"workload": name, "num_chunks": shape.N, "ms_default": res["default"],
            "ms_prefetch": res["prefetch"], "median_default_ms": med["default"],
            "median_prefetch_ms": med["prefetch"],
            "prefetch_over_default": med["prefetch"] / med["default"],
            "note": "back-to-back steps; the prefetch schedule warms the first 128 bytes of every "
                    "gate/up weight row on s1 during the metadata pass"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3_e256")
    ap.add_argument("--num-chunks", type=int, default=1)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--sweep-config", default="packed16k_e128",
                    help="workload of the num_chunks sweep ('' to skip it)")
    ap.add_argument("--sweep-chunks", default="1,2,4,8")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-prefetch-ab", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this MoE layer build runs on one "
              "GPU only (no multi-GPU path); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_top_route_expert_amd as moe
    import synth

    moe.load_library()
    torch.cuda.set_device(0)
    stream_pair(torch)  # before any other stream, so that each gets a hardware queue
    cfg = synth.CONFIGS[args.config]
    N = args.num_chunks
    log(f"inputs {cfg.name}")
    inp = make_inputs(cfg, torch, synth)
    shape = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.groups, N, cfg.dtype)

    # one common warm-up (clocks, caches, allocator) before any timed run: the
    # W warm-up steps, then more until one second has passed, since the GPU
    # reaches its steady clock only after some 100 ms of load (a first timed run
    # right after 20 short steps measured 8% slower than the next ones)
    log("warm-up")
    t_warm = time.perf_counter()
    time_layer(moe, torch, shape, inp, 1, max(args.warmup, 1))
    while time.perf_counter() - t_warm < 1.0:
        time_layer(moe, torch, shape, inp, 1, 10)
    log(f"headline: {args.steps} single steps, L2/MALL flushed before each, N={N}")
    cold = per_step_times(moe, torch, shape, inp, args.steps, flush_bytes=1 << 30)
    log("single steps, warm")
    warm = per_step_times(moe, torch, shape, inp, args.steps)
    log("back-to-back steps")
    piped = time_layer(moe, torch, shape, inp, args.steps, args.warmup)
    log(f"per-chunk schedule, N={N}")
    run_pc = time_layer(moe, torch, shape, inp, args.steps, args.warmup,
                        schedule=moe.MOE_SCHEDULE_PER_CHUNK)
    log("layer replayed from a HIP graph")
    graph_ms = time_graph(moe, torch, shape, inp, args.steps)
    bwd = None
    if not args.no_backward:
        log(f"backward N={N}")
        bwd_steps = max(3, args.steps // 10)
        bwd_ms, bwd_ws = time_backward(moe, torch, shape, inp, bwd_steps, 1)
        A_valid = int(inp["counts"].sum())
        bwd = {"ms_per_step": bwd_ms, "value": cfg.T / (bwd_ms * 1e-3), "steps": bwd_steps,
               "flop_per_step": 18.0 * A_valid * cfg.H * cfg.I,
               "tflops": 18.0 * A_valid * cfg.H * cfg.I / (bwd_ms * 1e-3) / 1e12,
               "workspace_bytes": bwd_ws,
               "note": "moe_chunked_backward: forward recomputed per chunk pair, grads of "
                       "hidden_states, top_k_weights (fp32) and both expert weight tensors "
                       "(fp32); flop = 18*A*H*I"}
        torch.cuda.empty_cache()
    log("per-kernel timing")
    kt, rows0, e_act0, chunk_rows = kernel_times(moe, torch, shape, inp, args.kernel_reps)
    copy_bw = copy_bandwidth(torch)

    s = cfg.elem_bytes
    H, I = cfg.H, cfg.I
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
    roof["traffic"] = load_traffic(cfg.name, N)
    roof["kernel"] = ("grouped_gemm_bf16<gate_up> (moe_expert_gate_up_gather_pair), chunks 0-1"
                      if N >= 2 else
                      "grouped_gemm_bf16<gate_up> (moe_expert_gate_up_gather_pair), chunk 0")
    roof["rows_per_launch"] = rows0
    roof["active_experts"] = e_act0
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

    ms = cold["mean_ms"]
    line = {
        "metric": METRIC, "value": cfg.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": H, "E": cfg.E, "top_k": cfg.k,
                   "I": I, "num_chunks": N, "streams": 1, "schedule": "pair_fused",
                   "groups": cfg.groups,
                   "timing": "mean of K single steps, each after a 1 GiB L2/MALL flush, "
                             "HIP events on s0 with a device sync on both sides"},
        "roofline": roof,
        "kernels_us": kt,
        "kernels_roofline": kernels_roofline,
        "single_step": {"cold": cold, "warm": warm},
        "pipelined": {"ms_per_step": piped["wall_ms"], "value": cfg.T / (piped["wall_ms"] * 1e-3),
                      "event_ms_per_step": piped["event_ms"],
                      "note": "K steps back to back between two device synchronisations"},
        "per_chunk_schedule": {"ms_per_step": run_pc["wall_ms"],
                               "value": cfg.T / (run_pc["wall_ms"] * 1e-3),
                               "note": "permute, gate_up, down, combine per chunk on stream c%2"},
        "hip_graph": {"ms_per_step": graph_ms, "value": cfg.T / (graph_ms * 1e-3),
                      "note": "the same step captured once and replayed"},
        "backward": bwd,
        "workspace_bytes": {"requested": cold["workspace_bytes"],
                            "slots_model": min(N, 2) * -(-cfg.T // N) * cfg.k * (H + I) * s},
        "copy_bandwidth_GBps": copy_bw / 1e9,
        "expert_load": {"max_over_mean": float(inp["counts"].max() / inp["counts"].mean()),
                        "empty_experts": int((inp["counts"] == 0).sum())},
    }
    log("vendor dense GEMM reference")
    line["vendor_dense_gemm_bf16"] = vendor_dense_gemm(torch)
    if not args.no_prefetch_ab:
        log("prefetch schedule A/B")
        line["prefetch_schedule_ab"] = [prefetch_ab(moe, torch, synth, n, cfg, inp)
                                        for n in ("decode_t64", cfg.name)]
    if args.sweep_config:
        Ns = [int(x) for x in args.sweep_chunks.split(",") if x]
        line["chunk_sweep"] = chunk_sweep(moe, torch, synth, args.sweep_config, Ns,
                                          max(5, args.steps // 2))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, synth, torch)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
