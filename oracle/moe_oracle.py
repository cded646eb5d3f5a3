"""CPU oracle of the MoE layer's dispatch / expert / combine path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in ``oracle/``;
the GPU library and its Python binding never do.  The oracle shares no code with
the GPU path: it is plain numpy in float64, written from the pages' description
of the method, slow on purpose and meant to be read against the pages by eye.

Sources (page title, then the section each function follows):

* [ChunkMoE] "昇腾MindSpeed分块专家计算Chunk MoE:让通信藏进计算、显存轻装上阵"
  (MindSpeed Chunk MoE article): sections "核心原理" (core principle: the
  standard dispatcher permutes, exchanges, runs the experts, exchanges back and
  unpermutes), the timing-diagram section (inputs ``hidden_states``,
  ``top_k_index``, ``top_k_weights`` cut along the token dimension; per chunk
  permute -> dispatch -> expert -> combine -> unpermute; batched metadata for all
  chunks; empty chunks still run), "一组关键公式" (key formulas:
  T_chunk = ceil(T/N), W_pair = O(2 x T_chunk)) and "操作指南" step 3 (the
  moe_num_chunks / moe_chunk_size rule).
* [MindSpore] "昇思MindSpore MoE模型性能优化方案" news page (2025-12-12),
  section "# 02 AlltoAllV收发异构复用特性": the per-destination send/receive
  lists of dispatch are reused by combine.
* [CANN-blog] MoE communication blog, section 4.2 (mixed precision): router
  probabilities stay fp32.

Readings where the pages are silent:

* expert FFN = SwiGLU without bias: FFN_e(x) = W_d[e] (silu(W_g[e] x) * (W_u[e] x)),
  silu(z) = z / (1 + e^-z); ``w_gate_up[e]`` is [2I, H] (gate rows first),
  ``w_down[e]`` is [H, I];
* ``top_k_weights`` scale each expert's output in the unpermute sum and are used
  as given (no renormalisation inside the layer);
* the permute is stable: rows of one expert keep ascending flat index
  f = t*k + j; offsets, ranks and rows are chunk-local;
* an expert id outside [0, E) is dropped (no row, no contribution) and counted;
* send splits to G destination groups of E/G contiguous experts are sums of the
  per-expert counts.

Backward (the gradient of the same layer, with the forward of every chunk
recomputed in the backward pass as the guide's chunk_moe_recompute option does,
[ChunkMoE, "操作指南" step 3 and the timing-diagram section, whose backward
mirrors the forward chunk by chunk]): ``silu_grad``, ``moe_backward``,
``moe_tokens_backward``, ``expert_weight_grads``.  Pinned by central finite
differences of the forward oracle.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

__all__ = [
    "chunk_bounds", "resolve_num_chunks", "w_pair_rows", "route_meta", "permute",
    "silu", "expert_act", "expert_ffn", "unpermute_combine", "moe_forward", "moe_tokens",
    "silu_grad", "moe_backward", "moe_tokens_backward", "expert_weight_grads",
    "row_rel_err",
]


# --------------------------------------------------------------------------
# a0: chunk split   [ChunkMoE, "一组关键公式": T_chunk = ceil(T/N)]
# --------------------------------------------------------------------------
def chunk_bounds(T: int, N: int) -> List[Tuple[int, int]]:
    """Token ranges [t0, t1) of the N chunks; each holds T_chunk = ceil(T/N)
    tokens except the tail, and trailing chunks may be empty (the page keeps such
    empty chunks in the pipeline)."""
    if N < 1:
        raise ValueError("N must be >= 1")
    tc = -(-T // N)  # ceil(T / N)
    return [(min(T, c * tc), min(T, (c + 1) * tc)) for c in range(N)]


def resolve_num_chunks(T: int, num_chunks: int, chunk_size: int) -> Tuple[int, bool]:
    """[ChunkMoE, "操作指南" step 3]: set only one of moe_num_chunks and
    moe_chunk_size; if both are positive, moe_num_chunks wins and a warning is
    raised; if neither is positive the tokens are not split.  A chunk size alone
    means ceil(T / chunk_size) chunks.  Returns (N, warned)."""
    if num_chunks > 0:
        return num_chunks, chunk_size > 0
    if chunk_size > 0:
        return max(1, -(-T // chunk_size)), False
    return 1, False


def w_pair_rows(T: int, N: int, k: int) -> int:
    """Rows a chunk pair keeps resident: the W_pair = O(2 x ceil(T/N)) relation of
    [ChunkMoE, "一组关键公式"], counted in permuted rows (k per token).  With one
    chunk only that chunk is resident."""
    return min(N, 2) * (-(-T // N)) * k


# --------------------------------------------------------------------------
# a1: routing metadata, for every chunk at once
#     [ChunkMoE, timing-diagram section: batched metadata for all chunks;
#      MindSpore "# 02": per-destination send lists]
# --------------------------------------------------------------------------
def route_meta(top_k_index: np.ndarray, E: int, G: int, N: int) -> Dict[str, np.ndarray]:
    """Per chunk c:

    * counts[c][e]      number of the chunk's assignments routed to expert e
    * offsets[c][0..E]  exclusive prefix sum of counts (offsets[c][E] = valid rows)
    * group_splits[c][g] rows sent to destination group g (experts
                        [g*E/G, (g+1)*E/G))
    * src_row[t0*k + r] flat assignment index f = t*k + j held by chunk row r
                        (-1 past the valid rows)
    * dst_row[f]        chunk row of assignment f (-1 for a dropped id)
    * n_invalid         number of dropped assignments (ids outside [0, E))

    Rows are ordered by a stable comparison sort on the expert id, so rows of one
    expert keep ascending f (token, then slot)."""
    idx = np.asarray(top_k_index)
    T, k = idx.shape
    G = max(G, 1)
    if E % G:
        raise ValueError("E must be a multiple of G")
    flat = idx.reshape(-1).tolist()
    A = T * k
    counts = np.zeros((N, E), np.int64)
    offsets = np.zeros((N, E + 1), np.int64)
    splits = np.zeros((N, G), np.int64)
    src_row = np.full(A, -1, np.int64)
    dst_row = np.full(A, -1, np.int64)
    n_invalid = 0
    for c, (t0, t1) in enumerate(chunk_bounds(T, N)):
        f0, f1 = t0 * k, t1 * k
        valid = [f for f in range(f0, f1) if 0 <= flat[f] < E]
        n_invalid += (f1 - f0) - len(valid)
        order = sorted(valid, key=lambda f: flat[f])  # Python's sort is stable
        for r, f in enumerate(order):
            src_row[f0 + r] = f
            dst_row[f] = r
            counts[c, flat[f]] += 1
        run = 0
        for e in range(E):
            offsets[c, e] = run
            run += counts[c, e]
        offsets[c, E] = run
        per = E // G
        for g in range(G):
            splits[c, g] = sum(counts[c, e] for e in range(g * per, (g + 1) * per))
    return {"counts": counts, "offsets": offsets, "group_splits": splits,
            "src_row": src_row, "dst_row": dst_row, "n_invalid": n_invalid}


# --------------------------------------------------------------------------
# a2: permute   [ChunkMoE, "核心原理" and timing-diagram section]
# --------------------------------------------------------------------------
def permute(hidden: np.ndarray, src_row_chunk: np.ndarray, k: int, rows: int) -> np.ndarray:
    """Expert-contiguous copy of one chunk: row r holds the token of assignment
    src_row_chunk[r], i.e. hidden[src_row_chunk[r] // k], for r < rows."""
    return np.asarray(hidden, np.float64)[np.asarray(src_row_chunk[:rows]) // k]


# --------------------------------------------------------------------------
# a3 + a4: expert FFN (SwiGLU) on each expert's contiguous rows
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


ExpertGetter = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def expert_ffn(x_perm: np.ndarray, offsets_c: Sequence[int], get_expert: ExpertGetter,
               I: int) -> np.ndarray:
    """y[r] = W_d[e] (silu(W_g[e] x_r) * (W_u[e] x_r)) for the rows
    [offsets_c[e], offsets_c[e+1]) of each expert e; get_expert(e) returns
    (w_gate_up[e] [2I,H], w_down[e] [H,I]) as float64."""
    x_perm = np.asarray(x_perm, np.float64)
    E = len(offsets_c) - 1
    rows = int(offsets_c[E])
    y = np.zeros((rows, x_perm.shape[1] if rows else 0), np.float64)
    for e in range(E):
        lo, hi = int(offsets_c[e]), int(offsets_c[e + 1])
        if hi == lo:
            continue
        wgu, wd = get_expert(e)
        y[lo:hi] = expert_act(x_perm[lo:hi], wgu, I) @ wd.T
    return y


def expert_act(xs: np.ndarray, wgu: np.ndarray, I: int) -> np.ndarray:
    """SwiGLU activation of one expert's rows: silu(xs W_g^T) * (xs W_u^T), with
    W_g = wgu[:I] and W_u = wgu[I:2I]."""
    xs = np.asarray(xs, np.float64)
    gate = xs @ wgu[:I].T
    up = xs @ wgu[I:2 * I].T
    return silu(gate) * up


# --------------------------------------------------------------------------
# a5: unpermute + top_k_weights-weighted combine
#     [ChunkMoE, timing-diagram section; MindSpore "# 02": combine reuses the
#      dispatch lists, here dst_row; CANN-blog 4.2: weights kept in fp32]
# --------------------------------------------------------------------------
def unpermute_combine(y: np.ndarray, dst_row_chunk: np.ndarray,
                      weights_chunk: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y[dst_row[t*k+j]], slots j in ascending order,
    dropped slots (dst_row = -1) contribute nothing.  Indices are chunk-local."""
    w = np.asarray(weights_chunk, np.float64)
    tc, k = w.shape
    d = np.asarray(dst_row_chunk).reshape(tc, k)
    H = y.shape[1] if y.ndim == 2 and y.shape[0] else 0
    out = np.zeros((tc, H), np.float64)
    for j in range(k):
        keep = d[:, j] >= 0
        out[keep] += w[keep, j, None] * y[d[keep, j]]
    return out


# --------------------------------------------------------------------------
# whole layer, chunked
# --------------------------------------------------------------------------
def moe_forward(hidden: np.ndarray, top_k_index: np.ndarray, top_k_weights: np.ndarray,
                get_expert: ExpertGetter, E: int, I: int, G: int = 1,
                N: int = 1) -> Tuple[np.ndarray, Dict[str, np.ndarray]]:
    """Chunked layer: metadata for all chunks once, then per chunk permute ->
    expert FFN -> unpermute/combine into the chunk's token rows.  Returns the
    float64 output [T,H] and the metadata."""
    hidden = np.asarray(hidden, np.float64)
    T, H = hidden.shape
    k = top_k_index.shape[1]
    meta = route_meta(top_k_index, E, G, N)
    out = np.zeros((T, H), np.float64)
    for c, (t0, t1) in enumerate(chunk_bounds(T, N)):
        if t1 == t0:
            continue
        rows = int(meta["offsets"][c, E])
        if rows == 0:  # every slot of the chunk was dropped: its rows stay zero
            continue
        xp = permute(hidden, meta["src_row"][t0 * k:t1 * k], k, rows)
        y = expert_ffn(xp, meta["offsets"][c], get_expert, I)
        out[t0:t1] = unpermute_combine(y, meta["dst_row"][t0 * k:t1 * k],
                                       top_k_weights[t0:t1])
    return out, meta


def moe_tokens(tokens: Sequence[int], hidden: np.ndarray, top_k_index: np.ndarray,
               top_k_weights: np.ndarray, get_expert: ExpertGetter, E: int,
               I: int) -> np.ndarray:
    """The plain definition, token by token, with no permute or metadata:
    out[t] = sum_j w[t,j] FFN_{idx[t,j]}(x[t]).  Used for sampled parity at sizes
    the chunked oracle cannot finish."""
    tokens = list(tokens)
    H = hidden.shape[1]
    out = np.zeros((len(tokens), H), np.float64)
    need: Dict[int, List[Tuple[int, int]]] = {}
    for n, t in enumerate(tokens):
        for j in range(top_k_index.shape[1]):
            e = int(top_k_index[t, j])
            if 0 <= e < E:
                need.setdefault(e, []).append((n, j))
    # one pass per expert so each expert's weights are fetched once
    partial = np.zeros((len(tokens), top_k_index.shape[1], H), np.float64)
    for e in sorted(need):
        wgu, wd = get_expert(e)
        for n, j in need[e]:
            x = np.asarray(hidden[tokens[n]], np.float64)
            act = silu(wgu[:I] @ x) * (wgu[I:2 * I] @ x)
            partial[n, j] = float(top_k_weights[tokens[n], j]) * (wd @ act)
    for j in range(top_k_index.shape[1]):  # ascending slot order
        out += partial[:, j]
    return out


# --------------------------------------------------------------------------
# backward of the whole layer, chunk by chunk with the forward recomputed
# --------------------------------------------------------------------------
def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = s + z s (1 - s) with s = 1 / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s + z * s * (1.0 - s)


def moe_backward(hidden: np.ndarray, top_k_index: np.ndarray, top_k_weights: np.ndarray,
                 get_expert: ExpertGetter, E: int, I: int, grad_out: np.ndarray, G: int = 1,
                 N: int = 1) -> Dict[str, object]:
    """Gradient of L = sum(grad_out * out) with respect to hidden_states,
    top_k_weights and every expert's weights, for the chunked layer of
    ``moe_forward``.  Per chunk: permute again, recompute each expert's g, u, act
    and y, then

    * combine backward: grad_w[t,j] = grad_out[t] . y[r] and
      grad_y[r] = w[t,j] grad_out[t] for r = dst_row[t*k+j] (dropped slots: 0);
    * down: grad_act = grad_y W_d[e];  grad_W_d[e] += grad_y^T act;
    * SwiGLU: grad_g = grad_act * u * silu'(g);  grad_u = grad_act * silu(g);
    * gate/up: grad_W_g[e] += grad_g^T x;  grad_W_u[e] += grad_u^T x;
      grad_x = grad_g W_g[e] + grad_u W_u[e];
    * permute backward: grad_hidden[t] = sum_j grad_x[dst_row[t*k+j]].

    Returns grad_hidden [T,H], grad_w [T,k] and grad_wgu / grad_wd: dicts
    expert -> [2I,H] / [H,I] arrays for the experts that received rows."""
    hidden = np.asarray(hidden, np.float64)
    grad_out = np.asarray(grad_out, np.float64)
    T, H = hidden.shape
    k = top_k_index.shape[1]
    meta = route_meta(top_k_index, E, G, N)
    grad_hidden = np.zeros((T, H), np.float64)
    grad_w = np.zeros((T, k), np.float64)
    gwgu: Dict[int, np.ndarray] = {}
    gwd: Dict[int, np.ndarray] = {}
    for c, (t0, t1) in enumerate(chunk_bounds(T, N)):
        rows = int(meta["offsets"][c, E]) if t1 > t0 else 0
        if rows == 0:
            continue
        off = meta["offsets"][c]
        xp = permute(hidden, meta["src_row"][t0 * k:t1 * k], k, rows)
        dst = np.asarray(meta["dst_row"][t0 * k:t1 * k]).reshape(t1 - t0, k)
        # recompute y, then the combine backward
        y = expert_ffn(xp, off, get_expert, I)
        grad_y = np.zeros((rows, H), np.float64)
        for j in range(k):
            keep = np.nonzero(dst[:, j] >= 0)[0]
            r = dst[keep, j]
            grad_w[t0 + keep, j] = np.sum(grad_out[t0 + keep] * y[r], axis=1)
            grad_y[r] = np.asarray(top_k_weights, np.float64)[t0 + keep, j, None] * grad_out[t0 + keep]
        grad_xp = np.zeros((rows, H), np.float64)
        for e in range(E):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi == lo:
                continue
            wgu, wd = get_expert(e)
            xs = xp[lo:hi]
            g = xs @ wgu[:I].T
            u = xs @ wgu[I:2 * I].T
            act = silu(g) * u
            gy = grad_y[lo:hi]
            grad_act = gy @ wd
            gwd[e] = gwd.get(e, 0.0) + gy.T @ act
            grad_g = grad_act * u * silu_grad(g)
            grad_u = grad_act * silu(g)
            gwgu[e] = gwgu.get(e, 0.0) + np.concatenate([grad_g.T @ xs, grad_u.T @ xs], axis=0)
            grad_xp[lo:hi] = grad_g @ wgu[:I] + grad_u @ wgu[I:2 * I]
        for j in range(k):  # ascending slot order
            keep = np.nonzero(dst[:, j] >= 0)[0]
            grad_hidden[t0 + keep] += grad_xp[dst[keep, j]]
    return {"grad_hidden": grad_hidden, "grad_w": grad_w, "grad_wgu": gwgu, "grad_wd": gwd,
            "meta": meta}


def moe_tokens_backward(tokens: Sequence[int], hidden: np.ndarray, top_k_index: np.ndarray,
                        top_k_weights: np.ndarray, get_expert: ExpertGetter, E: int, I: int,
                        grad_out: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """grad_hidden and grad_w of single tokens from the plain definition (no
    permute): grad_w[t,j] = grad_out[t] . FFN_e(x_t) and grad_hidden[t] =
    sum_j w[t,j] J_e(x_t)^T grad_out[t], with J_e the Jacobian of FFN_e."""
    tokens = list(tokens)
    H = hidden.shape[1]
    k = top_k_index.shape[1]
    gh = np.zeros((len(tokens), H), np.float64)
    gw = np.zeros((len(tokens), k), np.float64)
    for n, t in enumerate(tokens):
        x = np.asarray(hidden[t], np.float64)
        go = np.asarray(grad_out[t], np.float64)
        for j in range(k):
            e = int(top_k_index[t, j])
            if not 0 <= e < E:
                continue
            wgu, wd = get_expert(e)
            g = wgu[:I] @ x
            u = wgu[I:2 * I] @ x
            gw[n, j] = go @ (wd @ (silu(g) * u))
            ga = float(top_k_weights[t, j]) * (wd.T @ go)
            gh[n] += wgu[:I].T @ (ga * u * silu_grad(g)) + wgu[I:2 * I].T @ (ga * silu(g))
    return gh, gw


def expert_weight_grads(e: int, hidden: np.ndarray, top_k_index: np.ndarray,
                        top_k_weights: np.ndarray, get_expert: ExpertGetter, I: int,
                        grad_out: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """grad of L with respect to expert e's weights from the plain definition:
    the sum over every (token, slot) routed to e of the outer products."""
    wgu, wd = get_expert(e)
    t_idx, j_idx = np.nonzero(np.asarray(top_k_index) == e)
    xs = np.asarray(hidden, np.float64)[t_idx]
    gy = np.asarray(top_k_weights, np.float64)[t_idx, j_idx, None] * \
        np.asarray(grad_out, np.float64)[t_idx]
    g = xs @ wgu[:I].T
    u = xs @ wgu[I:2 * I].T
    act = silu(g) * u
    ga = gy @ wd
    gwd = gy.T @ act
    gwgu = np.concatenate([(ga * u * silu_grad(g)).T @ xs, (ga * silu(g)).T @ xs], axis=0)
    return gwgu, gwd


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """The comparison metric for floating-point outputs (the pages give a
    tolerance's size but not its norm; the reading taken is row-wise):
    max over rows t of ||got_t - ref_t||_inf / max(||ref_t||_inf, 1e-30).

    Both arrays must be 2-D with the same shape (no broadcasting: a wrong row
    count is an error, not a comparison of other rows).  A NaN or infinity in
    either array gives +inf, so no tolerance accepts it.  No rows gives 0."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.ndim != 2 or got.shape != ref.shape:
        raise ValueError(f"row_rel_err: shapes {got.shape} and {ref.shape} differ or are not 2-D")
    if got.shape[0] == 0:
        return 0.0
    if not (np.isfinite(got).all() and np.isfinite(ref).all()):
        return float("inf")
    if got.shape[1] == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())

