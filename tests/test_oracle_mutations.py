"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  Each mutant replaces one oracle function for the
duration of the test."""
import numpy as np
import pytest

import oracle.moe_oracle as om
import oracle_checks

_orig_route_meta = om.route_meta
_orig_expert_ffn = om.expert_ffn
_orig_moe_backward = om.moe_backward
_orig_row_rel_err = om.row_rel_err


def _silu_as_sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _silu_wrong_sign(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _ffn_gate_up_swapped(x_perm, offsets_c, get_expert, I):
    def get(e):
        wgu, wd = get_expert(e)
        return np.concatenate([wgu[I:2 * I], wgu[:I]], axis=0), wd
    return _orig_expert_ffn(x_perm, offsets_c, get, I)


def _ffn_down_transposed(x_perm, offsets_c, get_expert, I):
    def get(e):
        wgu, wd = get_expert(e)
        return wgu, (wd.T if wd.shape[0] == wd.shape[1] else wd[::-1])
    return _orig_expert_ffn(x_perm, offsets_c, get, I)


def _combine_reversed_slots(y, dst_row_chunk, weights_chunk):
    w = np.asarray(weights_chunk, np.float64)[:, ::-1]
    tc, k = w.shape
    d = np.asarray(dst_row_chunk).reshape(tc, k)
    out = np.zeros((tc, y.shape[1] if y.ndim == 2 and y.shape[0] else 0))
    for j in range(k):
        keep = d[:, j] >= 0
        out[keep] += w[keep, j, None] * y[d[keep, j]]
    return out


def _route_meta_unstable(top_k_index, E, G, N):
    m = _orig_route_meta(top_k_index, E, G, N)
    # reverse the order inside each expert's block of rows (a non-stable sort)
    T, k = np.asarray(top_k_index).shape
    tc = -(-T // N)
    for c in range(N):
        f0 = min(T, c * tc) * k
        for e in range(E):
            lo, hi = int(m["offsets"][c][e]), int(m["offsets"][c][e + 1])
            if hi - lo > 1:
                blk = m["src_row"][f0 + lo:f0 + hi][::-1].copy()
                m["src_row"][f0 + lo:f0 + hi] = blk
                for r, f in enumerate(blk):
                    m["dst_row"][f] = lo + r
    return m


def _route_meta_offsets_inclusive(top_k_index, E, G, N):
    m = _orig_route_meta(top_k_index, E, G, N)
    m["offsets"][:, :E] = m["offsets"][:, 1:]
    return m


def _chunk_bounds_floor(T, N):
    tc = max(1, T // N)
    return [(min(T, c * tc), min(T, (c + 1) * tc) if c < N - 1 else T) for c in range(N)]


def _resolve_size_wins(T, num_chunks, chunk_size):
    if chunk_size > 0:
        return max(1, -(-T // chunk_size)), num_chunks > 0
    return (num_chunks if num_chunks > 0 else 1), False


def _w_pair_no_min(T, N, k):
    return 2 * (-(-T // N)) * k


def _silu_grad_no_z_term(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _backward_unweighted(hidden, top_k_index, top_k_weights, *a, **kw):
    return _orig_moe_backward(hidden, top_k_index, np.ones_like(top_k_weights), *a, **kw)


def _backward_gate_up_grads_swapped(*a, **kw):
    b = _orig_moe_backward(*a, **kw)
    for e, g in b["grad_wgu"].items():
        half = g.shape[0] // 2
        b["grad_wgu"][e] = np.concatenate([g[half:], g[:half]], axis=0)
    return b


def _backward_grad_w_slots_reversed(*a, **kw):
    b = _orig_moe_backward(*a, **kw)
    b["grad_w"] = b["grad_w"][:, ::-1].copy()
    return b


def _row_rel_err_whole_array(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def _row_rel_err_signed(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    num = (got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def _row_rel_err_elementwise(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    return float((np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)).max())


def _row_rel_err_broadcasts(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float(np.max(num / den))


MUTANTS = {
    "silu_grad_no_z_term": ("silu_grad", _silu_grad_no_z_term),
    "backward_unweighted": ("moe_backward", _backward_unweighted),
    "backward_gate_up_grads_swapped": ("moe_backward", _backward_gate_up_grads_swapped),
    "backward_grad_w_slots_reversed": ("moe_backward", _backward_grad_w_slots_reversed),
    "silu_as_sigmoid": ("silu", _silu_as_sigmoid),
    "silu_wrong_sign": ("silu", _silu_wrong_sign),
    "ffn_gate_up_swapped": ("expert_ffn", _ffn_gate_up_swapped),
    "ffn_down_transposed": ("expert_ffn", _ffn_down_transposed),
    "combine_reversed_slots": ("unpermute_combine", _combine_reversed_slots),
    "route_meta_unstable": ("route_meta", _route_meta_unstable),
    "route_meta_offsets_inclusive": ("route_meta", _route_meta_offsets_inclusive),
    "chunk_bounds_floor": ("chunk_bounds", _chunk_bounds_floor),
    "resolve_chunk_size_wins": ("resolve_num_chunks", _resolve_size_wins),
    "w_pair_no_min": ("w_pair_rows", _w_pair_no_min),
    "row_rel_err_whole_array": ("row_rel_err", _row_rel_err_whole_array),
    "row_rel_err_signed": ("row_rel_err", _row_rel_err_signed),
    "row_rel_err_elementwise": ("row_rel_err", _row_rel_err_elementwise),
    "row_rel_err_broadcasts": ("row_rel_err", _row_rel_err_broadcasts),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(om, attr, fn)
    failed = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the mutant {name}"
