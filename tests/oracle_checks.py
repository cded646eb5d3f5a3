"""Pins of the CPU oracle to facts outside itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix: closed forms, library routines that are
not the ones the oracle uses, brute force over every small input, invariants,
and the page's own figures (tests/golden/).  test_oracle_pins.py runs them all;
test_oracle_mutations.py plants mistakes in the oracle and checks that some pin
fails for each.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

import oracle.moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- a0 chunks
def check_chunk_bounds():
    """T_chunk = ceil(T/N) [Chunk MoE page, key formulas]; exactly N chunks that
    tile [0, T) in order; the page's empty tail chunk (T=3, N=4)."""
    for T in range(0, 41):
        for N in range(1, 11):
            b = om.chunk_bounds(T, N)
            assert len(b) == N
            pos = 0
            for t0, t1 in b:
                assert t0 == pos and t1 >= t0
                pos = t1
            assert pos == T
            sizes = [t1 - t0 for t0, t1 in b]
            # the common size is the least s with N*s >= T, found by search
            s = next(s for s in range(T + 1) if s * N >= T)
            assert sizes[0] == s
            nz = [x for x in sizes if x]
            assert all(x == s for x in nz[:-1]) and (not nz or 0 < nz[-1] <= s)
            assert all(x == 0 for x in sizes[len(nz):])
    assert om.chunk_bounds(3, 4) == [(0, 1), (1, 2), (2, 3), (3, 3)]
    assert [t1 - t0 for t0, t1 in om.chunk_bounds(16384, 4)] == [4096] * 4
    assert [t1 - t0 for t0, t1 in om.chunk_bounds(10, 4)] == [3, 3, 3, 1]


def check_resolve_num_chunks():
    """Guide step 3 of the Chunk MoE page (golden cases) plus chunk_size alone."""
    for case in _golden("chunk_moe_page_facts.json")["guide_step3_chunk_rule"]:
        n, w = om.resolve_num_chunks(16384, case["num_chunks"], case["chunk_size"])
        assert (n, w) == (case["N"], case["warned"]), case
    assert om.resolve_num_chunks(16384, 0, 4096) == (4, False)
    assert om.resolve_num_chunks(16385, 0, 4096) == (5, False)
    assert om.resolve_num_chunks(0, 0, 4096) == (1, False)


def check_w_pair():
    """W_pair = O(2 x ceil(T/N)): no drop at N=2, half at N=4 (golden, page figures)."""
    facts = _golden("chunk_moe_page_facts.json")["facts"]["pair_resident_fraction_of_unchunked"]
    T, k = 16384, 8
    full = om.w_pair_rows(T, 1, k)
    assert full == T * k
    for n, frac in facts.items():
        assert om.w_pair_rows(T, int(n), k) / full == frac


# ---------------------------------------------------------------- a1 metadata
def _random_index(rng, T, k, E, invalid_frac=0.0):
    idx = rng.integers(0, E, size=(T, k))
    if invalid_frac:
        bad = rng.random((T, k)) < invalid_frac
        idx[bad] = rng.choice([-1, E, E + 7, -100], size=int(bad.sum()))
    return idx.astype(np.int32)


def _meta_vs_library(idx, E, G, N):
    """Counts by np.bincount, offsets by np.cumsum, permutation by numpy's stable
    argsort (the oracle itself uses Python's sorted and plain loops)."""
    m = om.route_meta(idx, E, G, N)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    tc = -(-T // N)
    tot_invalid = 0
    for c in range(N):
        t0, t1 = min(T, c * tc), min(T, (c + 1) * tc)
        f0, f1 = t0 * k, t1 * k
        seg = flat[f0:f1]
        ok = (seg >= 0) & (seg < E)
        tot_invalid += int((~ok).sum())
        cnt = np.bincount(seg[ok], minlength=E)
        assert np.array_equal(m["counts"][c], cnt)
        assert np.array_equal(m["offsets"][c], np.concatenate([[0], np.cumsum(cnt)]))
        assert np.array_equal(m["group_splits"][c], cnt.reshape(max(G, 1), -1).sum(1))
        keyed = np.where(ok, seg, E + 1)  # dropped ids sort last
        order = np.argsort(keyed, kind="stable")[: int(ok.sum())] + f0
        nv = int(ok.sum())
        assert np.array_equal(m["src_row"][f0:f0 + nv], order)
        assert np.all(m["src_row"][f0 + nv:f1] == -1)
        d = m["dst_row"][f0:f1]
        assert np.all(d[~ok] == -1)
        assert np.array_equal(np.sort(d[ok]), np.arange(nv))
        assert np.array_equal(m["src_row"][f0 + d[ok]], np.arange(f0, f1)[ok])
    assert m["n_invalid"] == tot_invalid
    assert int(m["counts"].sum()) == T * k - tot_invalid
    return m


def check_route_meta_library():
    rng = np.random.default_rng(11)
    for (T, k, E, G, N, bad) in [(50, 2, 8, 1, 1, 0.0), (50, 2, 8, 4, 3, 0.1),
                                 (97, 8, 256, 16, 4, 0.02), (33, 4, 64, 8, 7, 0.0),
                                 (3, 8, 256, 16, 4, 0.0), (1, 1, 1, 1, 1, 0.0),
                                 (40, 3, 5, 5, 40, 0.2), (40, 3, 5, 1, 45, 0.0)]:
        _meta_vs_library(_random_index(rng, T, k, E, bad), E, G, N)


def check_route_meta_bruteforce():
    """Every index table over {-1, 0, 1, 2} (E=3) for T=3, k=2, with N = 1, 2, 3:
    the defining properties of a stable permute checked one by one."""
    E = 3
    for tab in itertools.product([-1, 0, 1, 2], repeat=6):
        idx = np.array(tab, np.int32).reshape(3, 2)
        for N in (1, 2, 3):
            m = om.route_meta(idx, E, 1, N)
            tc = -(-3 // N)
            for c in range(N):
                t0, t1 = min(3, c * tc), min(3, (c + 1) * tc)
                fs = range(t0 * 2, t1 * 2)
                valid = [f for f in fs if 0 <= tab[f] < E]
                rows = [int(m["src_row"][t0 * 2 + r]) for r in range(len(valid))]
                assert sorted(rows) == valid
                for a, b in zip(rows, rows[1:]):
                    assert tab[a] < tab[b] or (tab[a] == tab[b] and a < b)
                for r, f in enumerate(rows):
                    assert m["dst_row"][f] == r
                for f in fs:
                    if f not in valid:
                        assert m["dst_row"][f] == -1
                for e in range(E + 1):
                    assert m["offsets"][c][e] == sum(1 for f in valid if tab[f] < e)
            assert m["n_invalid"] == sum(1 for v in tab if not 0 <= v < E)


# ---------------------------------------------------------------- FFN
def _scalar_silu(z):
    return z / (1.0 + math.exp(-z))


def check_silu():
    assert om.silu(np.array([0.0]))[0] == 0.0
    assert abs(om.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(om.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    z = np.linspace(-30, 30, 601)
    # sigmoid(z) + sigmoid(-z) = 1  =>  silu(z) - silu(-z) = z
    assert np.allclose(om.silu(z) - om.silu(-z), z, rtol=0, atol=1e-12)
    assert abs(om.silu(np.array([-800.0]))[0]) < 1e-300


def check_ffn_closed_form():
    """H = I, W_g = a*Id, W_u = b*Id, W_d = a permutation P: y = P (silu(a x) * b x).
    Distinguishes gate from up, W_d from its transpose, and the activation."""
    H = I = 8
    a, b = 1.7, -0.6
    P = np.eye(H)[[3, 0, 6, 1, 7, 2, 5, 4]]  # not symmetric
    wgu = np.concatenate([a * np.eye(I), b * np.eye(I)], axis=0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, H))
    y = om.expert_ffn(x, [0, 5], lambda e: (wgu, P), I)
    want = np.stack([P @ np.array([_scalar_silu(a * v) * b * v for v in row]) for row in x])
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


def _bruteforce_ffn_row(x, wgu, wd, I):
    H = len(x)
    act = []
    for i in range(I):
        g = sum(wgu[i][h] * x[h] for h in range(H))
        u = sum(wgu[I + i][h] * x[h] for h in range(H))
        act.append(_scalar_silu(g) * u)
    return [sum(wd[h][i] * act[i] for i in range(I)) for h in range(H)]


def _tiny_layer(rng, T=7, H=5, I=3, E=3, k=2):
    idx = _random_index(rng, T, k, E)
    w = rng.random((T, k))
    x = rng.standard_normal((T, H))
    experts = [(rng.standard_normal((2 * I, H)), rng.standard_normal((H, I))) for _ in range(E)]
    return idx, w, x, experts


def check_ffn_bruteforce():
    """Whole layer on tiny inputs against scalar Python loops (math.exp)."""
    rng = np.random.default_rng(5)
    for N in (1, 2, 4):
        idx, w, x, ex = _tiny_layer(rng)
        T, k = idx.shape
        out, _ = om.moe_forward(x, idx, w, lambda e: ex[e], E=3, I=3, G=1, N=N)
        for t in range(T):
            want = [0.0] * x.shape[1]
            for j in range(k):
                yr = _bruteforce_ffn_row(list(x[t]), ex[idx[t, j]][0], ex[idx[t, j]][1], 3)
                want = [a + w[t, j] * b for a, b in zip(want, yr)]
            assert np.allclose(out[t], want, rtol=1e-12, atol=1e-12), (N, t)


# ---------------------------------------------------------------- permute / combine
def check_identity_k1():
    """k=1, unit weights, y := x_perm: unpermute(permute(x)) == x exactly."""
    rng = np.random.default_rng(7)
    T, H, E = 37, 6, 5
    x = rng.standard_normal((T, H))
    idx = _random_index(rng, T, 1, E)
    for N in (1, 3):
        m = om.route_meta(idx, E, 1, N)
        tc = -(-T // N)
        for c in range(N):
            t0, t1 = min(T, c * tc), min(T, (c + 1) * tc)
            rows = int(m["offsets"][c, E])
            xp = om.permute(x, m["src_row"][t0:t1], 1, rows)
            back = om.unpermute_combine(xp, m["dst_row"][t0:t1], np.ones((t1 - t0, 1)))
            assert np.array_equal(back, x[t0:t1])


def check_identical_experts_dense():
    """All experts equal and sum_j w = 1: the layer equals the dense FFN whatever
    the routing (scalar loops for the dense FFN)."""
    rng = np.random.default_rng(9)
    T, H, I, E, k = 9, 4, 3, 6, 3
    wgu = rng.standard_normal((2 * I, H))
    wd = rng.standard_normal((H, I))
    x = rng.standard_normal((T, H))
    idx = _random_index(rng, T, k, E)
    w = rng.random((T, k))
    w /= w.sum(1, keepdims=True)
    out, _ = om.moe_forward(x, idx, w, lambda e: (wgu, wd), E, I, 1, 2)
    for t in range(T):
        assert np.allclose(out[t], _bruteforce_ffn_row(list(x[t]), wgu, wd, I), rtol=1e-12,
                           atol=1e-12)


def check_weights_linear_and_dropped_slots():
    """Output is linear in top_k_weights, a zero-weight slot equals a dropped slot,
    and each slot's weight multiplies its own expert's output."""
    rng = np.random.default_rng(13)
    idx, w, x, ex = _tiny_layer(rng, T=11, E=4, k=3)
    get = lambda e: ex[e]  # noqa: E731
    o1, _ = om.moe_forward(x, idx, w, get, 4, 3)
    o2, _ = om.moe_forward(x, idx, 2.5 * w, get, 4, 3)
    assert np.allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-12)
    w0 = w.copy()
    w0[:, 1] = 0.0
    idx_drop = idx.copy()
    idx_drop[:, 1] = -1
    a, _ = om.moe_forward(x, idx, w0, get, 4, 3)
    b, m = om.moe_forward(x, idx_drop, w, get, 4, 3)
    assert m["n_invalid"] == idx.shape[0]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # one-hot weights pick out a single slot's expert output
    wj = np.zeros_like(w)
    wj[:, 2] = 1.0
    o, _ = om.moe_forward(x, idx, wj, get, 4, 3)
    for t in range(idx.shape[0]):
        e = idx[t, 2]
        assert np.allclose(o[t], _bruteforce_ffn_row(list(x[t]), ex[e][0], ex[e][1], 3),
                           rtol=1e-12, atol=1e-12)


def check_plain_definition_vs_chunked():
    """moe_tokens (direct definition, no permute) against moe_forward at N = 1, 3, 8."""
    rng = np.random.default_rng(17)
    T, H, I, E, k = 41, 16, 12, 7, 3
    idx = _random_index(rng, T, k, E, 0.05)
    w = rng.random((T, k)).astype(np.float32)
    x = rng.standard_normal((T, H))
    ex = [(rng.standard_normal((2 * I, H)) * 0.3, rng.standard_normal((H, I)) * 0.3)
          for _ in range(E)]
    direct = om.moe_tokens(range(T), x, idx, w, lambda e: ex[e], E, I)
    for N in (1, 3, 8, 50):
        out, _ = om.moe_forward(x, idx, w, lambda e: ex[e], E, I, 1, N)
        assert np.allclose(out, direct, rtol=1e-12, atol=1e-12), N


# ---------------------------------------------------------------- backward
def check_silu_grad():
    """silu'(0) = 1/2 exactly, and central differences of the scalar silu."""
    assert om.silu_grad(np.array([0.0]))[0] == 0.5
    for z in (-7.5, -2.0, -0.3, 0.4, 1.0, 3.3, 9.0):
        h = 1e-6
        fd = (_scalar_silu(z + h) - _scalar_silu(z - h)) / (2 * h)
        assert abs(om.silu_grad(np.array([z]))[0] - fd) < 1e-8, z


def _bruteforce_loss(x, idx, w, experts, I, grad_out):
    """sum_t grad_out[t] . out[t] with out from scalar Python loops (no oracle code)."""
    T, k = idx.shape
    total = 0.0
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if not 0 <= e < len(experts):
                continue
            yr = _bruteforce_ffn_row(list(x[t]), experts[e][0], experts[e][1], I)
            total += float(w[t, j]) * sum(a * b for a, b in zip(grad_out[t], yr))
    return total


def check_backward_finite_differences():
    """moe_backward against central differences of the scalar-loop forward, for
    every input: hidden_states, top_k_weights, w_gate_up and w_down.  The index
    table has a dropped slot and a token routed twice to one expert."""
    rng = np.random.default_rng(23)
    T, H, I, E, k = 5, 4, 3, 3, 2
    idx = _random_index(rng, T, k, E)
    idx[1, 1] = -1
    idx[2, :] = 2
    w = rng.random((T, k))
    x = rng.standard_normal((T, H))
    ex = [[rng.standard_normal((2 * I, H)), rng.standard_normal((H, I))] for _ in range(E)]
    go = rng.standard_normal((T, H))
    h = 1e-6

    def fd(arr, pos):
        old = arr[pos]
        arr[pos] = old + h
        lp = _bruteforce_loss(x, idx, w, ex, I, go)
        arr[pos] = old - h
        lm = _bruteforce_loss(x, idx, w, ex, I, go)
        arr[pos] = old
        return (lp - lm) / (2 * h)

    for N in (1, 2):
        b = om.moe_backward(x, idx, w, lambda e: (ex[e][0], ex[e][1]), E, I, go, 1, N)
        for pos in np.ndindex(x.shape):
            assert abs(b["grad_hidden"][pos] - fd(x, pos)) < 1e-6, ("hidden", N, pos)
        for pos in np.ndindex(w.shape):
            want = fd(w, pos)
            assert abs(b["grad_w"][pos] - want) < 1e-6, ("w", N, pos)
        for e in range(E):
            gwgu = b["grad_wgu"].get(e, np.zeros((2 * I, H)))
            gwd = b["grad_wd"].get(e, np.zeros((H, I)))
            for pos in np.ndindex(ex[e][0].shape):
                assert abs(gwgu[pos] - fd(ex[e][0], pos)) < 1e-6, ("wgu", N, e, pos)
            for pos in np.ndindex(ex[e][1].shape):
                assert abs(gwd[pos] - fd(ex[e][1], pos)) < 1e-6, ("wd", N, e, pos)


def check_backward_views_and_chunking():
    """The per-token and per-expert backward views equal moe_backward, and the
    gradient does not depend on the chunk count."""
    rng = np.random.default_rng(29)
    T, H, I, E, k = 23, 8, 6, 5, 3
    idx = _random_index(rng, T, k, E, 0.05)
    w = rng.random((T, k))
    x = rng.standard_normal((T, H))
    ex = [(rng.standard_normal((2 * I, H)) * 0.4, rng.standard_normal((H, I)) * 0.4)
          for _ in range(E)]
    get = lambda e: ex[e]  # noqa: E731
    go = rng.standard_normal((T, H))
    ref = om.moe_backward(x, idx, w, get, E, I, go, 1, 1)
    gh, gw = om.moe_tokens_backward(range(T), x, idx, w, get, E, I, go)
    assert np.allclose(gh, ref["grad_hidden"], rtol=1e-12, atol=1e-12)
    assert np.allclose(gw, ref["grad_w"], rtol=1e-12, atol=1e-12)
    for e in range(E):
        gwgu, gwd = om.expert_weight_grads(e, x, idx, w, get, I, go)
        assert np.allclose(gwgu, ref["grad_wgu"].get(e, 0 * gwgu), rtol=1e-12, atol=1e-12), e
        assert np.allclose(gwd, ref["grad_wd"].get(e, 0 * gwd), rtol=1e-12, atol=1e-12), e
    for N in (2, 4, 30):
        b = om.moe_backward(x, idx, w, get, E, I, go, 1, N)
        for key in ("grad_hidden", "grad_w"):
            assert np.allclose(b[key], ref[key], rtol=1e-12, atol=1e-12), (N, key)
        for e in ref["grad_wgu"]:
            assert np.allclose(b["grad_wgu"][e], ref["grad_wgu"][e], rtol=1e-12, atol=1e-12)
            assert np.allclose(b["grad_wd"][e], ref["grad_wd"][e], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- parity metric
def check_row_rel_err():
    """The comparison metric, on hand-computed 3 x 4 cases: the row-wise
    inf-norm relative error max_t max_h |g - r| / max(max_h |r|, 1e-30) (the
    reading taken for the unnamed norm of the tolerances).  The cases are built
    so that the whole-array ratio, the elementwise ratio and a signed
    difference all give other values."""
    ref = np.array([[10.0, 0.01, 0.0, 0.0],
                    [0.0, 1.0, 0.0, 0.0],
                    [0.0, 0.0, 0.0, 0.0]])
    got = np.array([[10.5, 0.02, 0.0, 0.0],   # row error 0.5 / 10 = 0.05 (elementwise: 1.0)
                    [0.0, 1.25, 0.0, 0.0],    # row error 0.25 / 1 = 0.25
                    [0.0, 0.0, 0.0, 0.0]])    # zero row, exact: 0
    # by hand: max(0.05, 0.25, 0) = 0.25; whole-array ratio would be 0.5 / 10 = 0.05
    assert om.row_rel_err(got, ref) == 0.25
    # the metric is symmetric in the row it measures, not in its arguments:
    # swapping them divides by the other row's norm (0.25 / 1.25 = 0.2 for row 1)
    assert om.row_rel_err(ref, got) == max(0.5 / 10.5, 0.25 / 1.25)
    # a sign flip: |(-1) - 1| / 1 = 2 (a signed difference would give 0 there)
    flip = got.copy()
    flip[1, 1] = -1.0
    assert om.row_rel_err(flip, ref) == 2.0
    # a below-reference error only: |0.75 - 1| / 1 = 0.25 (a signed max would miss it)
    low = ref.copy()
    low[1, 1] = 0.75
    assert om.row_rel_err(low, ref) == 0.25
    # an all-zero reference row is measured against the floor 1e-30
    tiny = ref.copy()
    tiny[2, 2] = 2e-31
    assert math.isclose(om.row_rel_err(tiny, ref), 0.2, rel_tol=1e-12)
    # identical arrays and no rows give 0
    assert om.row_rel_err(ref, ref) == 0.0
    assert om.row_rel_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    # a NaN or infinity fails every tolerance
    bad = got.copy()
    bad[2, 3] = np.nan
    assert not om.row_rel_err(bad, ref) <= 1e30
    bad[2, 3] = np.inf
    assert not om.row_rel_err(bad, ref) <= 1e30
    # one row against three is an error, not a broadcast comparison
    for g, r in ((got[:1], ref), (got, ref[:, :3]), (got[0], ref[0])):
        try:
            om.row_rel_err(g, r)
        except ValueError:
            continue
        raise AssertionError(f"row_rel_err accepted shapes {np.shape(g)} and {np.shape(r)}")


ALL_CHECKS = [
    check_chunk_bounds, check_resolve_num_chunks, check_w_pair, check_route_meta_library,
    check_route_meta_bruteforce, check_silu, check_ffn_closed_form, check_ffn_bruteforce,
    check_identity_k1, check_identical_experts_dense, check_weights_linear_and_dropped_slots,
    check_plain_definition_vs_chunked, check_silu_grad, check_backward_finite_differences,
    check_backward_views_and_chunking, check_row_rel_err,
]
