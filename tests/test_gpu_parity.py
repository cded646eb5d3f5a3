"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Integer outputs (counts, offsets, splits, src_row, dst_row, dropped-id count)
and the permute are compared bit-exactly.  Floating outputs are compared with
the row-wise inf-norm relative error
    max_t ||gpu_t - oracle_t||_inf / max(||oracle_t||_inf, 1e-30)
against 1e-5 for fp32 workloads and 2e-2 for bf16 workloads (fp32 accumulate,
act / y / out each rounded to bf16 once).  GPU chunked output must equal GPU
unchunked output bit for bit.  Small workloads are compared on every row; the
large ones on every metadata entry, every permuted row, and sampled experts and
tokens that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import combine_top_route_expert_amd as moe
import oracle
import synth
from gpu_layer import build_layer, f64, run_forward, run_route_meta, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
C = synth.CONFIGS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


_layers = {}


def layer_for(name, T=None):
    key = (name, T)
    if key not in _layers:
        if len(_layers) > 3:
            _layers.clear()
        cfg = C[name] if T is None else C[name].with_tokens(T)
        _layers[key] = build_layer(cfg)
    return _layers[key]


def sample_tokens(T, n=6, seed=0):
    rng = np.random.default_rng(seed)
    base = {0, T - 1, T // 2}
    base.update(int(x) for x in rng.integers(0, T, size=max(0, n - 3)))
    return sorted(base)


# --------------------------------------------------------------------- inputs
def test_generator_same_bits_on_device():
    key = synth.stream_key(3, synth.S_W_GATE_UP, 5)
    for n, start in [(1000, 0), (1 << 20, 77)]:
        say(f"generator normal n={n}")
        assert torch.equal(synth.normal(key, n, 0.02, "cuda", start).cpu(),
                           synth.normal(key, n, 0.02, "cpu", start))
    assert torch.equal(synth.uniform(key, 5000, "cuda").cpu(), synth.uniform(key, 5000, "cpu"))
    cfg = C["bf16_e64_zipf"]
    assert torch.equal(synth.expert_gate_up(cfg, 3, "cuda").cpu(),
                       synth.expert_gate_up(cfg, 3, "cpu"))
    assert torch.equal(synth.hidden_states(cfg.with_tokens(64), "cuda").cpu(),
                       synth.hidden_states(cfg.with_tokens(64), "cpu"))


# --------------------------------------------------------------------- a1 metadata
META_CASES = [
    ("tiny_f32", 1, None), ("bf16_e64_zipf", 1, None), ("bf16_e64_zipf", 2, None),
    ("dsv3_e256", 1, 16), ("dsv3_e256", 1, 8), ("dsv3_e256", 3, 16),
    ("packed16k_e128", 1, None), ("packed16k_e128", 2, None), ("packed16k_e128", 4, None),
    ("packed16k_e128", 8, None), ("decode_t64", 1, 16), ("t3_n4", 4, 16), ("t3_n4", 1, 16),
    ("skew_two_experts", 1, 16),
]


def _check_meta(idx_np, E, G, N, T, k, H=128, I=256, dtype="f32"):
    shape = moe.make_shape(T, H, E, k, I, G, N, dtype)
    say(f"route_meta T={T} k={k} E={E} G={G} N={N}")
    got = run_route_meta(torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).cuda()
                         if T else torch.empty(0, dtype=torch.int32, device="cuda"), shape)
    want = oracle.route_meta(np.asarray(idx_np).reshape(T, k), E, G, N)
    for key in ("counts", "offsets", "group_splits", "src_row", "dst_row"):
        assert np.array_equal(got[key].reshape(want[key].shape), want[key]), key
    assert int(got["dev_error"][0]) == want["n_invalid"]


@pytest.mark.parametrize("name,N,G", META_CASES)
def test_route_meta_bit_exact(name, N, G):
    cfg = C[name]
    idx_np, _ = synth.routing(cfg)
    _check_meta(idx_np, cfg.E, cfg.groups if G is None else G, N, cfg.T, cfg.k, cfg.H, cfg.I,
                cfg.dtype)


@pytest.mark.parametrize("T,k,E,G,N,bad", [
    (777, 3, 6, 3, 5, 0.1),      # E not a power of two, dropped ids, ragged chunks
    (100, 64, 1024, 16, 1, 0.0),  # largest k and E
    (4000, 2, 1, 1, 3, 0.05),    # one expert
    (3, 8, 256, 16, 7, 0.0),     # more chunks than tokens
    (1, 1, 8, 1, 1, 0.0),
    (2500, 8, 256, 16, 2, 1.0),  # every id dropped
    (0, 8, 256, 16, 4, 0.0),     # no tokens
    (20000, 8, 64, 4, 2, 0.05),   # chunks of 80000 assignments (several per segment plan)
    (300, 64, 1024, 16, 3, 0.02),  # largest E with dropped ids and three chunks
    (5000, 8, 512, 8, 2, 0.03),
    (16384, 8, 96, 3, 2, 0.01),    # E not a power of two, 65536 assignments per chunk
    # either side of the metadata paths' limits: one launch up to 8192
    # assignments per chunk (E <= 512), two up to 32768, both only up to 65536
    # assignments in all, three otherwise
    (1024, 8, 64, 1, 1, 0.02),     # 8192 in one chunk: one launch
    (1025, 8, 64, 1, 1, 0.02),     # 8200: two launches
    (8192, 8, 512, 8, 8, 0.01),    # 8 x 8192 = 65536, E = 512: one launch
    (8193, 8, 512, 8, 8, 0.01),    # 65544 in all: three launches
    (8200, 8, 256, 16, 9, 0.01),   # 65600 in all: three launches
    (900, 8, 513, 27, 1, 0.01),    # E = 513: two launches
    (1000, 13, 37, 1, 3, 0.05),    # one launch, ragged slices and chunks
    (4096, 8, 256, 16, 2, 0.01),   # 2 x 16384: two launches
    (4096, 16, 1024, 16, 2, 0.01),  # 2 x 32768, E = 1024 (segments of 2048): two launches
    (4097, 16, 1024, 16, 2, 0.0),  # 32784 per chunk, 65552 in all: three launches
    (3000, 7, 96, 3, 1, 0.2),      # 21000 in one chunk, many dropped: two launches
])
def test_route_meta_edge_cases(T, k, E, G, N, bad):
    rng = np.random.default_rng(T + k + E)
    idx = rng.integers(0, E, size=(T, k))
    if bad:
        m = rng.random((T, k)) < bad
        idx[m] = rng.choice([-1, E, E + 3, -(1 << 30)], size=int(m.sum()))
    _check_meta(idx.astype(np.int32), E, G, N, T, k)


def _random_meta_shapes(n, seed):
    """Seeded shapes spread over both metadata paths: chunk sizes around the
    one-launch limit (8192 assignments per chunk, 65536 in all), E up to 1024
    with G dividing E, empty and ragged chunks, dropped ids."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.choice([1, 2, 5, 8, 37, 64, 96, 128, 256, 500, 512, 513, 1024]))
        G = int(rng.choice([g for g in (1, 2, 3, 4, 8, 16, 27) if E % g == 0]))
        k = int(rng.choice([1, 2, 3, 4, 6, 8, 13]))
        N = int(rng.choice([1, 2, 3, 4, 5, 8, 9]))
        per_chunk = int(rng.choice([1, 100, 4000, 8192, 8193, 12000]))
        T = max(0, min(per_chunk * N // k + int(rng.integers(-3, 4)), 70000 // k))
        bad = float(rng.choice([0.0, 0.0, 0.01, 0.3]))
        out.append((T, k, E, G, N, bad))
    return out


@pytest.mark.parametrize("T,k,E,G,N,bad", _random_meta_shapes(24, 2024))
def test_route_meta_random_shapes(T, k, E, G, N, bad):
    rng = np.random.default_rng(T * 31 + k * 7 + E + N)
    idx = rng.integers(0, E, size=(T, k))
    if bad and T:
        m = rng.random((T, k)) < bad
        idx[m] = rng.choice([-1, E, 1 << 20], size=int(m.sum()))
    _check_meta(idx.astype(np.int32), E, G, N, T, k)


# --------------------------------------------------------------------- a2 permute
@pytest.mark.parametrize("name,N", [("tiny_f32", 1), ("bf16_e64_zipf", 2), ("dsv3_e256", 1),
                                    ("packed16k_e128", 4), ("t3_n4", 4)])
def test_permute_bit_exact(name, N):
    L = layer_for(name)
    cfg = L.cfg
    shape = L.shape(N)
    meta = run_route_meta(L.idx, shape)
    want = oracle.route_meta(L.idx_np, cfg.E, shape.G, N)
    dst = torch.from_numpy(meta["dst_row"]).cuda()
    for c in range(N):
        t0, t1 = moe.moe_chunk_range(shape, c)
        rows = (t1 - t0) * cfg.k
        valid = int(want["offsets"][c, cfg.E])
        # one canary row past the chunk's rows
        xp = torch.empty((rows + 1, cfg.H), dtype=cfg.torch_dtype, device="cuda")
        xp.view(torch.int16 if cfg.dtype == "bf16" else torch.int32).fill_(-12345)
        say(f"permute {name} N={N} chunk={c}")
        moe.moe_permute(shape, c, L.hidden, dst, xp)
        torch.cuda.synchronize()
        src = torch.from_numpy(want["src_row"][t0 * cfg.k:t0 * cfg.k + valid] // cfg.k).cuda()
        expect = L.hidden.index_select(0, src.long())  # the oracle's permutation applied
        assert torch.equal(xp[:valid], expect)
        canary = xp[valid:].view(torch.int16 if cfg.dtype == "bf16" else torch.int32)
        assert bool((canary == -12345).all())


# --------------------------------------------------------------------- a3/a4 expert FFN
def _chunk_pipeline(L, shape, c):
    """GPU route_meta + permute + gate_up + down for one chunk, through the C ABI."""
    cfg = L.cfg
    meta = run_route_meta(L.idx, shape)
    t0, t1 = moe.moe_chunk_range(shape, c)
    rows = (t1 - t0) * cfg.k
    dst = torch.from_numpy(meta["dst_row"]).cuda()
    off = torch.from_numpy(meta["offsets"]).cuda()
    xp = torch.zeros((rows, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    act = torch.zeros((rows, cfg.I), dtype=cfg.torch_dtype, device="cuda")
    y = torch.zeros((rows, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    say(f"expert ffn {cfg.name} N={shape.N} chunk={c}")
    moe.moe_permute(shape, c, L.hidden, dst, xp)
    moe.moe_expert_gate_up(shape, c, xp, off, L.wgu, act)
    moe.moe_expert_down(shape, c, act, off, L.wd, y)
    torch.cuda.synchronize()
    return meta, act, y


@pytest.mark.parametrize("name,N,n_experts", [
    ("tiny_f32", 1, None), ("bf16_e64_zipf", 2, 6), ("dsv3_e256", 1, 3),
    ("packed16k_e128", 2, 4), ("skew_two_experts", 1, 2), ("decode_t64", 1, 4),
])
def test_expert_ffn_vs_oracle(name, N, n_experts):
    L = layer_for(name)
    cfg = L.cfg
    shape = L.shape(N)
    c = N - 1  # the last chunk: ragged when T % N != 0
    meta, act, y = _chunk_pipeline(L, shape, c)
    want = oracle.route_meta(L.idx_np, cfg.E, shape.G, N)
    t0, _ = moe.moe_chunk_range(shape, c)
    off = want["offsets"][c]
    active = [e for e in range(cfg.E) if off[e + 1] > off[e]]
    if n_experts is not None:
        # the largest expert, the smallest, and evenly spaced others
        by_size = sorted(active, key=lambda e: off[e + 1] - off[e])
        pick = {by_size[0], by_size[-1]}
        pick.update(by_size[i] for i in np.linspace(0, len(by_size) - 1, n_experts).astype(int))
        active = sorted(pick)
    hid = L.hidden64()
    tol = TOL[cfg.dtype]
    for e in active:
        lo, hi = int(off[e]), int(off[e + 1])
        xs = oracle.permute(hid, want["src_row"][t0 * cfg.k + lo:t0 * cfg.k + hi], cfg.k, hi - lo)
        wgu, wd = L.expert64(e)
        ref_act = oracle.expert_act(xs, wgu, cfg.I)
        ref_y = oracle.expert_ffn(xs, [0, hi - lo], lambda _: (wgu, wd), cfg.I)
        err_a = oracle.row_rel_err(f64(act[lo:hi]), ref_act)
        err_y = oracle.row_rel_err(f64(y[lo:hi]), ref_y)
        assert err_a <= tol, (e, err_a)
        assert err_y <= tol, (e, err_y)


# --------------------------------------------------------------------- whole layer
FULL_CASES = [("tiny_f32", 1, None), ("t3_n4", 4, None), ("t3_n4", 1, None),
              ("bf16_e64_zipf", 1, 1024), ("bf16_e64_zipf", 2, 1000),
              ("odd_dims_bf16", 1, None), ("odd_dims_bf16", 3, None), ("odd_dims_f32", 4, None),
              # full sizes, every row: the DeepSeek-V3-shaped layer as the bench runs it (one
              # chunk, 4096 tokens, 256 experts of 95-160 rows), the decode batch, the skew
              ("decode_t64", 1, None), ("skew_two_experts", 1, None), ("dsv3_e256", 1, None),
              # the Zipf workloads at full size: the bench's earlier headline at N=2, and the
              # packed 16k-token layer unchunked and at N=8 (four chunk pairs)
              ("bf16_e64_zipf", 2, None), ("packed16k_e128", 1, None), ("packed16k_e128", 8, None)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,N,T", FULL_CASES)
def test_forward_every_row_vs_oracle(name, N, T):
    """Every output row against the chunked float64 oracle (its experts streamed
    one at a time for the E = 256 workloads)."""
    L = layer_for(name, T)
    cfg = L.cfg
    say(f"forward every row {name} T={cfg.T} N={N}")
    out, err = run_forward(L, L.shape(N))
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, N)
    assert err == meta["n_invalid"] == 0
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL[cfg.dtype], e


def _routing_with_counts(counts, T, k, seed=5):
    """top_k_index whose expert e receives counts[e] of the T * k slots, every
    token's k experts distinct (the slots sorted by expert, filled column by
    column: a run of at most T equal ids never lands twice in one token)."""
    assert sum(counts) == T * k and max(counts) <= T
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    idx = ids.reshape(k, T).T.copy()
    rng = np.random.default_rng(seed)
    idx = idx[rng.permutation(T)]  # tokens in random order, counts unchanged
    assert all(len(set(r)) == k for r in idx.tolist())
    return idx


@pytest.mark.parametrize("N", [1, 2])
def test_compact_tile_row_classes_every_row(N):
    """Experts at every row count around the compact tiles' class bounds (1,
    31-33, 63-65, 127-129, 159-161; a single-tile expert's rows split over both
    wave rows) and around one wide tile (255-257), and larger experts whose last
    m-tile falls in each class (276, 306, 356, 406, 456, 641 rows: tails of 20,
    50, 100, 150, 200, 129 rows on one wave row), in a launch large enough for
    the 256 x 256 instance (5200 rows).  Every output row against the oracle."""
    counts = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 159, 160, 161, 255, 256, 257,
              276, 306, 356, 406, 456, 641, 200, 200, 200, 200, 38, 0, 0, 0]
    T, k = 650, 8
    cfg = C["bf16_e64_zipf"].with_(T=T, E=len(counts), k=k, H=512, I=256)
    idx = _routing_with_counts(counts, T, k)
    _, w = synth.routing(cfg)
    L = build_layer(cfg, idx, w)
    say(f"compact row classes N={N}")
    out, err = run_forward(L, L.shape(N))
    ref, meta = oracle.moe_forward(L.hidden64(), idx, w, L.expert64, cfg.E, cfg.I, 1, N)
    assert err == meta["n_invalid"] == 0
    np.testing.assert_array_equal(meta["counts"].sum(axis=0), counts)
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL["bf16"], e


def _random_forward_cases(n=12, seed=2024):
    """Seeded random layer shapes: every third one has at least 4096 assignments
    (the 256 x 256 instance with its load roles and compact tiles), the others
    run the 64 x 128 instance; H and I multiples of 64, any E, k, T and N."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        big = i % 3 == 0
        k = int(rng.integers(1, 9))
        E = int(rng.integers(max(k, 2), 300))
        T = int(rng.integers(4096 // k + 1, 4096 // k + 400)) if big else int(rng.integers(1, 700))
        H = 64 * int(rng.integers(1, 9 if big else 17))
        I = 64 * int(rng.integers(1, 7 if big else 9))
        N = int(rng.integers(1, 6))
        cases.append((T, H, E, k, I, N))
    return cases


@pytest.mark.parametrize("T,H,E,k,I,N", _random_forward_cases())
def test_forward_random_shapes_every_row(T, H, E, k, I, N):
    """Random shapes (Zipf-skewed routing, bf16): every row against the oracle,
    and the chunked output equal to the unchunked one bit for bit."""
    cfg = C["bf16_e64_zipf"].with_(T=T, E=E, k=k, H=H, I=I, seed=T + E, weight_seed=H + I)
    L = build_layer(cfg)
    say(f"random shape T={T} H={H} E={E} k={k} I={I} N={N}")
    out, err = run_forward(L, L.shape(N))
    assert err == 0
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, N)
    assert meta["n_invalid"] == 0
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL["bf16"], e
    if N > 1:
        out1, _ = run_forward(L, L.shape(1))
        assert torch.equal(out1, out)


def _random_forward_cases_f32(n=6, seed=2025):
    """Seeded random fp32 layer shapes: H and I multiples of 4 (the fp32 path's
    only alignment), any E, k, T and N."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        k = int(rng.integers(1, 9))
        E = int(rng.integers(max(k, 2), 200))
        T = int(rng.integers(1, 1500))
        H = 4 * int(rng.integers(1, 129))
        I = 4 * int(rng.integers(1, 97))
        N = int(rng.integers(1, 6))
        cases.append((T, H, E, k, I, N))
    return cases


@pytest.mark.parametrize("T,H,E,k,I,N", _random_forward_cases_f32())
def test_forward_random_shapes_f32_every_row(T, H, E, k, I, N):
    """Random fp32 shapes: every row against the oracle (fp32 tolerance), and the
    chunked output equal to the unchunked one bit for bit."""
    cfg = C["odd_dims_f32"].with_(T=T, E=E, k=k, H=H, I=I, groups=1, seed=T + E,
                                  weight_seed=H + I)
    L = build_layer(cfg)
    say(f"random fp32 shape T={T} H={H} E={E} k={k} I={I} N={N}")
    out, err = run_forward(L, L.shape(N))
    assert err == 0
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, N)
    assert meta["n_invalid"] == 0
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL["f32"], e
    if N > 1:
        out1, _ = run_forward(L, L.shape(1))
        assert torch.equal(out1, out)


@pytest.mark.parametrize("H,I", [(64, 128), (192, 64), (128, 192), (192, 256)])
def test_wide_tile_few_k_steps_every_row(H, I):
    """The 256 x 256 one-tile kernel with 1 to 4 K steps of 64 (its load roles
    issue the first A stage and two B stages before the loop, then A one step
    and B two steps ahead, so the shortest loops skip those issues and change
    the final waits): gate/up K = H (1 or 3 steps on the wide tile; I = 64 and
    192 run gate/up on the 64 x 128 tile), down K = I (1 to 4 steps), over 4096
    rows of 8 experts (wide tiles with ragged tails).  Every row against the
    oracle; N = 2 equals N = 1 bit for bit."""
    cfg = C["bf16_e64_zipf"].with_(T=1024, E=8, k=4, H=H, I=I)
    L = build_layer(cfg)
    say(f"wide tile few K steps H={H} I={I}")
    out, err = run_forward(L, L.shape(1))
    assert err == 0
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, 1)
    assert meta["n_invalid"] == 0 and meta["counts"].max() > 256
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL["bf16"], e
    out2, _ = run_forward(L, L.shape(2))
    assert torch.equal(out2, out)


@pytest.mark.parametrize("I", [64, 128])
def test_tile_loop_few_k_steps_every_row(I):
    """The tile-loop form of the 256 x 256 kernel (4096 rows over E = 256, so the
    grid is capped and workgroups take several tiles) with its load roles at one
    and two K steps: the down GEMM with K = I = 64 and 128 over H = 2048 (eight
    n-tiles).  Every row against the oracle; N = 2 equals N = 1 bit for bit."""
    cfg = C["bf16_e64_zipf"].with_(T=1024, E=256, k=4, H=2048, I=I)
    L = build_layer(cfg)
    say(f"tile loop few K steps I={I}")
    out, err = run_forward(L, L.shape(1))
    assert err == 0
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, 1)
    assert meta["n_invalid"] == 0
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL["bf16"], e
    out2, _ = run_forward(L, L.shape(2))
    assert torch.equal(out2, out)


@pytest.mark.parametrize("name,kw", [
    ("odd_dims_bf16", dict(T=50, k=64, E=96, H=128, I=128, groups=2)),
    ("odd_dims_f32", dict(T=29, k=64, E=70, H=36, I=20, groups=1)),
])
def test_forward_largest_top_k(name, kw):
    """top_k = 64, the largest the library accepts: each token's combine sums 64
    rows.  Every row against the oracle; chunked (N = 3) equals unchunked bit
    for bit."""
    cfg = C[name].with_(**kw)
    L = build_layer(cfg)
    say(f"top_k=64 {name} N=1")
    out, err = run_forward(L, L.shape(1))
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, 1)
    assert err == meta["n_invalid"] == 0
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL[cfg.dtype], e
    say(f"top_k=64 {name} N=3")
    out3, _ = run_forward(L, L.shape(3))
    assert torch.equal(out3, out)


def test_forward_largest_expert_count():
    """E = 1024, the largest the library accepts, 4800 rows: the tile map
    numbers 16 experts per lane, the 256x256 gate/up runs its tile-loop form
    (the bound counts up to 1024 partial m-tiles) and the down its one-tile
    form; N = 4 runs pairs of 2400 rows with the 64x128 kernel.  Every row
    against the oracle; both give the same bits."""
    cfg = C["odd_dims_bf16"].with_(T=600, k=8, E=1024, H=128, I=256, groups=16)
    L = build_layer(cfg)
    say("E=1024 N=1")
    out, err = run_forward(L, L.shape(1))
    ref, meta = oracle.moe_forward(L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I,
                                   cfg.groups, 1)
    assert err == meta["n_invalid"] == 0
    e = oracle.row_rel_err(f64(out), ref)
    assert e <= TOL[cfg.dtype], e
    say("E=1024 N=4")
    out4, _ = run_forward(L, L.shape(4))
    assert torch.equal(out4, out)


SAMPLED_CASES = [("bf16_e64_zipf", 2, 24), ("dsv3_e256", 3, 24), ("packed16k_e128", 4, 48),
                 ("packed16k_e128", 8, 16), ("skew_two_experts", 1, 64)]


@pytest.mark.parametrize("name,N,n_tok", SAMPLED_CASES)
def test_forward_sampled_tokens_vs_oracle(name, N, n_tok):
    L = layer_for(name)
    cfg = L.cfg
    out, err = run_forward(L, L.shape(N))
    assert err == 0
    toks = sample_tokens(cfg.T, n_tok)
    ref = oracle.moe_tokens(toks, L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I)
    e = oracle.row_rel_err(f64(out[toks]), ref)
    assert e <= TOL[cfg.dtype], e
    assert not torch.isnan(out.float()).any()


@pytest.mark.parametrize("name,Ns", [("bf16_e64_zipf", (2,)), ("packed16k_e128", (2, 4, 8)),
                                     ("t3_n4", (4,)), ("dsv3_e256", (3,)),
                                     ("tiny_f32", (2, 5)), ("odd_dims_bf16", (3,)),
                                     ("odd_dims_f32", (4,))])
def test_chunked_equals_unchunked_bitwise(name, Ns):
    L = layer_for(name)
    base, _ = run_forward(L, L.shape(1), two_streams=False)
    for N in Ns:
        for sched in (moe.MOE_SCHEDULE_PAIR_FUSED, moe.MOE_SCHEDULE_PER_CHUNK,
                      moe.MOE_SCHEDULE_PAIR_FUSED_PREFETCH, moe.MOE_SCHEDULE_EXPERT_HALVES):
            for two in (True, False):
                say(f"chunked {name} N={N} schedule={sched} two_streams={two}")
                out, _ = run_forward(L, L.shape(N), two_streams=two, schedule=sched)
                assert torch.equal(out, base), (N, sched, two)


@pytest.mark.parametrize("name,N", [("decode_t64", 1), ("bf16_e64_zipf", 2), ("tiny_f32", 3)])
def test_prefetch_schedule_same_bits_and_oracle(name, N):
    """The weight-prefetch schedule (gate/up weight heads warmed on s1 during the
    metadata pass) gives the bits of the default schedule, and sampled tokens
    match the oracle."""
    L = layer_for(name)
    cfg = L.cfg
    say(f"prefetch schedule {name} N={N}: default")
    base, _ = run_forward(L, L.shape(N), two_streams=False)
    say(f"prefetch schedule {name} N={N}: prefetch on s1")
    out, err = run_forward(L, L.shape(N), two_streams=True,
                           schedule=moe.MOE_SCHEDULE_PAIR_FUSED_PREFETCH)
    assert err == 0
    assert torch.equal(out, base)
    toks = sample_tokens(cfg.T, 16)
    ref = oracle.moe_tokens(toks, L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I)
    e = oracle.row_rel_err(f64(out[toks]), ref)
    assert e <= TOL[cfg.dtype], e


@pytest.mark.parametrize("name,N", [("dsv3_e256", 1), ("decode_t64", 1), ("bf16_e64_zipf", 2),
                                    ("skew_two_experts", 1), ("odd_dims_f32", 3)])
def test_expert_halves_schedule_same_bits_and_oracle(name, N):
    """The expert-halves schedule (each expert GEMM launched over experts
    [0, E/2) and [E/2, E), the first half's down on s1 beside the second half's
    gate_up on s0) gives the bits of the default schedule, and sampled tokens
    match the oracle."""
    L = layer_for(name)
    cfg = L.cfg
    say(f"expert halves {name} N={N}: default")
    base, _ = run_forward(L, L.shape(N), two_streams=False)
    say(f"expert halves {name} N={N}: halves on s0 and s1")
    out, err = run_forward(L, L.shape(N), two_streams=True,
                           schedule=moe.MOE_SCHEDULE_EXPERT_HALVES)
    assert err == 0
    assert torch.equal(out, base)
    toks = sample_tokens(cfg.T, 16)
    ref = oracle.moe_tokens(toks, L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I)
    e = oracle.row_rel_err(f64(out[toks]), ref)
    assert e <= TOL[cfg.dtype], e


def test_tile_loop_several_tiles_per_workgroup():
    """4096 rows over E = 256 mostly small experts: the 256x256 grouped GEMMs
    run their tile-loop variant with the grid capped to 128 workgroups per XCD,
    so every workgroup takes several m-tiles (about 4 for gate/up, 7 for down).
    N = 4 runs pairs of 2048 rows with the 64x128 one-tile kernel.  The two
    outputs must be the same bits, and sampled tokens must match the oracle."""
    L = layer_for("decode_t64", 512)
    cfg = L.cfg
    say("tile loop: decode shape T=512 N=1")
    base, err = run_forward(L, L.shape(1), two_streams=False)
    assert err == 0
    say("tile loop: decode shape T=512 N=4")
    out4, _ = run_forward(L, L.shape(4), two_streams=False)
    assert torch.equal(out4, base)
    toks = sample_tokens(cfg.T, 12)
    ref = oracle.moe_tokens(toks, L.hidden64(), L.idx_np, L.w_np, L.expert64, cfg.E, cfg.I)
    e = oracle.row_rel_err(f64(base[toks]), ref)
    assert e <= 2e-2, e


PAIR_CASES = [("bf16_e64_zipf", 2, 0), ("tiny_f32", 3, 0), ("tiny_f32", 3, 2), ("t3_n4", 4, 2),
              ("packed16k_e128", 4, 2), ("dsv3_e256", 3, 0), ("dsv3_e256", 3, 2),
              ("decode_t64", 2, 0)]


@pytest.mark.parametrize("name,N,c", PAIR_CASES)
def test_expert_ffn_pair_bitwise(name, N, c):
    """One launch pair over chunks c and c+1 == moe_expert_ffn on each chunk, bit
    for bit; act holds the pair's rows grouped by expert; rows past each chunk's
    valid rows are not written."""
    L = layer_for(name)
    cfg = L.cfg
    shape = L.shape(N)
    meta = run_route_meta(L.idx, shape)
    dst = torch.from_numpy(meta["dst_row"]).cuda()
    off = torch.from_numpy(meta["offsets"]).cuda()
    dt = cfg.torch_dtype
    chunks = [c] + ([c + 1] if c + 1 < N else [])
    rows = {}
    xp, ref_act, ref_y = {}, {}, {}
    for cc in chunks:
        t0, t1 = moe.moe_chunk_range(shape, cc)
        rows[cc] = (t1 - t0) * cfg.k
        xp[cc] = torch.empty((rows[cc], cfg.H), dtype=dt, device="cuda")
        if rows[cc]:
            moe.moe_permute(shape, cc, L.hidden, dst, xp[cc])
            ref_act[cc] = torch.empty((rows[cc], cfg.I), dtype=dt, device="cuda")
            ref_y[cc] = torch.empty((rows[cc], cfg.H), dtype=dt, device="cuda")
            say(f"ffn {name} N={N} chunk={cc}")
            moe.moe_expert_ffn(shape, cc, xp[cc], off, L.wgu, L.wd, ref_act[cc], ref_y[cc])
    r1 = rows.get(c + 1, 0)
    act = torch.full((rows[c] + r1, cfg.I), 555.0, dtype=dt, device="cuda")
    y0 = torch.full((rows[c] + 3, cfg.H), 777.0, dtype=dt, device="cuda")
    y1 = torch.full((r1 + 3, cfg.H), 777.0, dtype=dt, device="cuda") if r1 else None
    say(f"ffn_pair {name} N={N} chunk={c}")
    moe.moe_expert_ffn_pair(shape, c, xp[c], xp.get(c + 1) if r1 else None, off, L.wgu, L.wd,
                            act, y0, y1)
    torch.cuda.synchronize()
    o0 = meta["offsets"][c]
    o1 = meta["offsets"][c + 1] if r1 else np.zeros_like(o0)
    valid0, valid1 = int(o0[-1]), int(o1[-1])
    assert torch.equal(y0[:valid0], ref_y[c][:valid0])
    assert bool((y0[valid0:] == 777.0).all())
    if r1:
        assert torch.equal(y1[:valid1], ref_y[c + 1][:valid1])
        assert bool((y1[valid1:] == 777.0).all())
    for e in range(cfg.E):
        n0, n1 = int(o0[e + 1] - o0[e]), int(o1[e + 1] - o1[e])
        b = int(o0[e] + o1[e])
        assert torch.equal(act[b:b + n0], ref_act[c][int(o0[e]):int(o0[e]) + n0]), e
        if n1:
            assert torch.equal(act[b + n0:b + n0 + n1], ref_act[c + 1][int(o1[e]):int(o1[e]) + n1]), e
    assert bool((act[valid0 + valid1:] == 555.0).all())
    # the gate_up with the permute fused (rows gathered from hidden_states)
    src = torch.from_numpy(meta["src_row"]).cuda()
    act2 = torch.full_like(act, 555.0)
    say(f"gate_up_gather_pair {name} N={N} chunk={c}")
    moe.moe_expert_gate_up_gather_pair(shape, c, L.hidden, src, off, L.wgu, act2)
    torch.cuda.synchronize()
    assert torch.equal(act2, act)


@pytest.mark.parametrize("name,N", [("bf16_e64_zipf", 2), ("odd_dims_bf16", 3)])
def test_gate_up_pair_rows_over_4gib_apart(name, N):
    """The pair gate/up copies its stages with 32-bit offsets from one base when
    both chunks' rows fit a 4 GiB window, else with 64-bit addresses: two row
    buffers more than 4 GiB apart take the second form and must give the same
    bits as the same rows side by side (256x256 tile for the Zipf workload,
    64x128 for the odd sizes)."""
    L = layer_for(name)
    cfg = L.cfg
    shape = L.shape(N)
    meta = run_route_meta(L.idx, shape)
    dst = torch.from_numpy(meta["dst_row"]).cuda()
    off = torch.from_numpy(meta["offsets"]).cuda()
    dt = cfg.torch_dtype
    n = []
    for cc in (0, 1):
        t0, t1 = moe.moe_chunk_range(shape, cc)
        n.append((t1 - t0) * cfg.k)
    row_bytes = cfg.H * 2
    gap = (1 << 32) + 4096
    big = torch.empty(n[0] * row_bytes + gap + n[1] * row_bytes, dtype=torch.uint8, device="cuda")
    far = [big[:n[0] * row_bytes].view(dt).view(n[0], cfg.H),
           big[n[0] * row_bytes + gap:].view(dt).view(n[1], cfg.H)]
    near = torch.empty((n[0] + n[1], cfg.H), dtype=dt, device="cuda")
    near = [near[:n[0]], near[n[0]:]]
    for cc in (0, 1):
        moe.moe_permute(shape, cc, L.hidden, dst, near[cc])
        far[cc].copy_(near[cc])
    acts = []
    for xs in (near, far):
        act = torch.full((n[0] + n[1], cfg.I), 555.0, dtype=dt, device="cuda")
        say(f"gate_up_pair {name} N={N} rows {'far apart' if xs is far else 'adjacent'}")
        moe.moe_expert_gate_up_pair(shape, 0, xs[0], xs[1], off, L.wgu, act)
        acts.append(act)
    torch.cuda.synchronize()
    assert torch.equal(acts[0], acts[1])
    del big


def test_run_twice_identical():
    L = layer_for("packed16k_e128")
    a, _ = run_forward(L, L.shape(2))
    b, _ = run_forward(L, L.shape(2))
    assert torch.equal(a, b)


def test_steps_compose_to_forward():
    """route_meta + per-chunk permute / gate_up / down / combine == chunked_forward."""
    L = layer_for("bf16_e64_zipf")
    cfg = L.cfg
    shape = L.shape(2)
    fwd, _ = run_forward(L, shape)
    meta = run_route_meta(L.idx, shape)
    dst = torch.from_numpy(meta["dst_row"]).cuda()
    off = torch.from_numpy(meta["offsets"]).cuda()
    out = torch.zeros_like(fwd)
    for c in range(2):
        t0, t1 = moe.moe_chunk_range(shape, c)
        rows = (t1 - t0) * cfg.k
        xp = torch.empty((rows, cfg.H), dtype=cfg.torch_dtype, device="cuda")
        act = torch.empty((rows, cfg.I), dtype=cfg.torch_dtype, device="cuda")
        moe.moe_permute(shape, c, L.hidden, dst, xp)
        moe.moe_expert_ffn(shape, c, xp, off, L.wgu, L.wd, act, xp)
        moe.moe_unpermute_combine(shape, c, xp, dst, L.w, out)
    torch.cuda.synchronize()
    assert torch.equal(out, fwd)
    # the same with the pair-fused FFN
    xps = []
    for c in range(2):
        t0, t1 = moe.moe_chunk_range(shape, c)
        xps.append(torch.empty(((t1 - t0) * cfg.k, cfg.H), dtype=cfg.torch_dtype, device="cuda"))
        moe.moe_permute(shape, c, L.hidden, dst, xps[c])
    act = torch.empty((cfg.T * cfg.k, cfg.I), dtype=cfg.torch_dtype, device="cuda")
    moe.moe_expert_ffn_pair(shape, 0, xps[0], xps[1], off, L.wgu, L.wd, act, xps[0], xps[1])
    out2 = torch.zeros_like(fwd)
    for c in range(2):
        moe.moe_unpermute_combine(shape, c, xps[c], dst, L.w, out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, fwd)


def test_dropped_ids_and_canary_rows():
    """Out-of-range ids are dropped and counted; a token with every slot dropped
    gets zeros; rows past T are never written."""
    cfg = C["tiny_f32"]
    idx, w = synth.routing(cfg)
    idx = idx.copy()
    idx[5, :] = -1
    idx[9, 1] = cfg.E
    idx[200, 0] = 1 << 20
    L = build_layer(cfg, idx, w)
    for N, sched in ((1, None), (3, moe.MOE_SCHEDULE_PAIR_FUSED), (3, moe.MOE_SCHEDULE_PER_CHUNK)):
        out = torch.full((cfg.T + 2, cfg.H), 777.0, dtype=cfg.torch_dtype, device="cuda")
        got, err = run_forward(L, L.shape(N), out=out, schedule=sched)
        ref, meta = oracle.moe_forward(L.hidden64(), idx, w, L.expert64, cfg.E, cfg.I, 1, N)
        assert err == meta["n_invalid"] == cfg.k + 2
        assert oracle.row_rel_err(f64(got[:cfg.T]), ref) <= TOL["f32"]
        assert bool((got[5] == 0).all())
        assert bool((got[cfg.T:] == 777.0).all())


def test_zero_tokens():
    cfg = C["tiny_f32"].with_tokens(0)
    shape = moe.make_shape(0, cfg.H, cfg.E, cfg.k, cfg.I, 1, 3, cfg.dtype)
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    z = torch.empty(0, device="cuda")
    say("zero tokens")
    moe.moe_chunked_forward(shape, z, torch.empty(0, dtype=torch.int32, device="cuda"), z,
                            torch.zeros(cfg.E * 2 * cfg.I * cfg.H, device="cuda"),
                            torch.zeros(cfg.E * cfg.H * cfg.I, device="cuda"), z, ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def test_forward_and_backward_in_hip_graph():
    """The pair-fused forward and the backward issue only kernels on s0 (no
    events, memsets or host reads), so they can be captured in a HIP graph; every
    replay, with eager work and synchronisations between replays, gives the
    eager bits."""
    L = layer_for("bf16_e64_zipf", 1024)
    cfg = L.cfg
    shape = L.shape(2)
    eager, _ = run_forward(L, shape)
    out = torch.zeros_like(eager)
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    bshape = L.shape(2)
    gh = torch.zeros((cfg.T, cfg.H), dtype=cfg.torch_dtype, device="cuda")
    gw = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    gwgu = torch.zeros((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.float32, device="cuda")
    gwd = torch.zeros((cfg.E, cfg.H, cfg.I), dtype=torch.float32, device="cuda")
    bws = torch.empty(moe.moe_backward_workspace_size(bshape), dtype=torch.uint8, device="cuda")
    go = L.hidden  # any [T,H] tensor of the layer dtype
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # warm-up on the capture stream
        moe.moe_chunked_forward(shape, L.hidden, L.idx, L.w, L.wgu, L.wd, out, ws, s0=s)
        moe.moe_chunked_backward(bshape, L.hidden, L.idx, L.w, L.wgu, L.wd, go, gh, gw, gwgu, gwd,
                                 bws, s0=s)
    torch.cuda.synchronize()
    ref_b = [t.clone() for t in (gh, gw, gwgu, gwd)]
    g = torch.cuda.CUDAGraph()
    say("capture forward + backward")
    with torch.cuda.graph(g, stream=s):
        moe.moe_chunked_forward(shape, L.hidden, L.idx, L.w, L.wgu, L.wd, out, ws,
                                s0=torch.cuda.current_stream())
        moe.moe_chunked_backward(bshape, L.hidden, L.idx, L.w, L.wgu, L.wd, go, gh, gw, gwgu, gwd,
                                 bws, s0=torch.cuda.current_stream())
    for rep in range(4):
        out.fill_(float("nan"))
        gh.fill_(float("nan"))
        gwgu.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        for got, want in zip((gh, gw, gwgu, gwd), ref_b):
            assert torch.equal(got, want), rep
        # eager work between replays
        run_forward(L, shape)


@pytest.mark.parametrize("schedule", [moe.MOE_SCHEDULE_PER_CHUNK, moe.MOE_SCHEDULE_EXPERT_HALVES,
                                      moe.MOE_SCHEDULE_PAIR_FUSED_PREFETCH])
def test_two_stream_schedules_in_hip_graph(schedule):
    """The two-stream schedules order s1 after s0 and s0 after s1 with event
    record / wait pairs only (no memsets or host reads), so a capture on s0
    takes s1's work in and joins it back: every replay, with eager work and
    synchronisations between replays, gives the eager bits."""
    L = layer_for("bf16_e64_zipf", 1024)
    shape = L.shape(4)
    eager, _ = run_forward(L, L.shape(1))
    out = torch.zeros_like(eager)
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    s, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # warm-up on the capture stream (creates the library's events)
        moe.moe_chunked_forward_schedule(shape, L.hidden, L.idx, L.w, L.wgu, L.wd, out, ws,
                                         s0=s, s1=s1, schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
    g = torch.cuda.CUDAGraph()
    say(f"capture schedule {schedule}")
    with torch.cuda.graph(g, stream=s):
        moe.moe_chunked_forward_schedule(shape, L.hidden, L.idx, L.w, L.wgu, L.wd, out, ws,
                                         s0=torch.cuda.current_stream(), s1=s1,
                                         schedule=schedule)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        run_forward(L, shape)  # eager work between replays
