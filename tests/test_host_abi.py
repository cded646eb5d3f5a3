"""The C-ABI library on the host (no GPU): it loads, exports every symbol the
public header declares, and its host-side logic (chunk rule, chunk ranges,
workspace planner, argument checks) matches the oracle and the page figures.
Every call here returns before any HIP call is made."""
import ctypes
import json
import os
import re

import pytest

import combine_top_route_expert_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

lib = moe.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))


def test_exports_match_header():
    declared = header_functions()
    assert declared == set(moe.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    # the binding has a function of the same name for each entry point
    for name in declared:
        assert callable(getattr(moe, name)), name


def test_status_strings():
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED"),
                       (3, "MOE_ERR_WORKSPACE_TOO_SMALL"), (4, "MOE_ERR_HIP")]:
        assert moe.moe_status_string(code) == name


def test_resolve_num_chunks_matches_oracle():
    for T in (0, 1, 3, 100, 16384):
        for n in (-1, 0, 1, 2, 4, 7):
            for cs in (-5, 0, 1, 3, 1000, 4096):
                assert moe.moe_resolve_num_chunks(T, n, cs) == oracle.resolve_num_chunks(T, n, cs)


def test_chunk_range_matches_oracle():
    for T in (0, 1, 2, 3, 10, 97, 4096, 16384):
        for N in (1, 2, 3, 4, 7, 8, 50):
            shape = moe.make_shape(T, 128, 8, 2, 256, 1, N, "f32")
            got = [moe.moe_chunk_range(shape, c) for c in range(N)]
            assert got == oracle.chunk_bounds(T, N), (T, N)
    shape = moe.make_shape(10, 128, 8, 2, 256, 1, 4, "f32")
    for bad in (-1, 4, 100):
        with pytest.raises(moe.MoeError):
            moe.moe_chunk_range(shape, bad)


def test_workspace_follows_pair_model():
    """moe_workspace_size = metadata + min(N,2) slots of ceil(T/N)*k rows of (H+I)
    elements; against the page's figures (no drop at N=2, half at N=4)."""
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "chunk_moe_page_facts.json")))
    frac = facts["facts"]["pair_resident_fraction_of_unchunked"]
    T, H, E, k, I = 16384, 2048, 128, 8, 768
    sizes = {}
    for N in (1, 2, 4, 8):
        shape = moe.make_shape(T, H, E, k, I, 1, N, "bf16")
        ws = moe.moe_workspace_size(shape)
        slots = oracle.w_pair_rows(T, N, k) * (H + I) * 2
        meta = ws - slots
        assert 0 < meta < 8 * T * k + 16 * 1024 * 1024, (N, meta)
        sizes[N] = slots
    for n, f in frac.items():
        assert sizes[int(n)] / sizes[1] == f
    assert sizes[8] / sizes[1] == 0.25
    # backward: the same pair residency, slots of (2H + 3I) elements per row
    bsizes = {}
    for N in (1, 2, 4, 8):
        shape = moe.make_shape(T, H, E, k, I, 1, N, "bf16")
        ws = moe.moe_backward_workspace_size(shape)
        slots = oracle.w_pair_rows(T, N, k) * (2 * H + 3 * I) * 2
        assert 0 < ws - slots < 8 * T * k + 16 * 1024 * 1024, (N, ws - slots)
        bsizes[N] = slots
    for n, f in frac.items():
        assert bsizes[int(n)] / bsizes[1] == f


def test_route_meta_workspace_positive():
    shape = moe.make_shape(4096, 7168, 256, 8, 2048, 16, 1, "bf16")
    assert moe.moe_route_meta_workspace_size(shape) >= 256 * 4


def _raw(fn, *args):
    return getattr(lib, fn)(*args)


@pytest.mark.parametrize("fields,code", [
    (dict(num_tokens=-1), 1), (dict(hidden=0), 1), (dict(num_experts=0), 1),
    (dict(top_k=0), 1), (dict(top_k=65), 2), (dict(num_experts=2048), 2),
    (dict(num_groups=3), 1), (dict(dtype=7), 1), (dict(hidden=96), 2),
    (dict(intermediate=100), 2), (dict(num_chunks=5000), 2),
    (dict(num_tokens=2**30, top_k=8), 2),
])
def test_shape_checks(fields, code):
    base = dict(num_tokens=64, hidden=7168, num_experts=256, top_k=8, intermediate=2048,
                num_groups=16, num_chunks=1, dtype=moe.MOE_BF16)
    base.update(fields)
    shape = moe.moe_shape(**base)
    b = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(shape), ctypes.byref(b)) == code


def test_fp32_shape_limits():
    ok = moe.make_shape(256, 128, 8, 2, 256, 1, 1, "f32")
    b = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(ok), ctypes.byref(b)) == 0
    bad = moe.make_shape(256, 130, 8, 2, 256, 1, 1, "f32")
    assert lib.moe_workspace_size(ctypes.byref(bad), ctypes.byref(b)) == 2


def test_entry_points_reject_bad_arguments_before_any_launch():
    """Null / misaligned pointers, a too-small workspace and a bad chunk index are
    refused by host checks; none of these calls reaches the device."""
    shape = moe.make_shape(64, 7168, 256, 8, 2048, 16, 2, "bf16")
    sp = ctypes.byref(shape)
    fake = 0x10000000  # never dereferenced: every call below fails its checks first
    need = moe.moe_workspace_size(shape)
    # null counts
    assert _raw("moe_route_meta", sp, fake, None, fake, fake, fake, fake, None, fake, 1 << 30,
                None) == 1
    # misaligned workspace
    assert _raw("moe_route_meta", sp, fake, fake, fake, fake, fake, fake, None, fake + 8,
                1 << 30, None) == 1
    # too-small workspace
    assert _raw("moe_route_meta", sp, fake, fake, fake, fake, fake, fake, None, fake, 16,
                None) == 3
    assert _raw("moe_chunked_forward", sp, fake, fake, fake, fake, fake, fake, None, fake,
                need - 1, None, None) == 3
    # misaligned hidden_states
    assert _raw("moe_chunked_forward", sp, fake + 2, fake, fake, fake, fake, fake, None, fake,
                need, None, None) == 1
    # chunk index out of range
    for fn in ("moe_permute",):
        assert _raw(fn, sp, 2, fake, fake, fake, None) == 1
        assert _raw(fn, sp, -1, fake, fake, fake, None) == 1
    assert _raw("moe_expert_gate_up", sp, 5, fake, fake, fake, fake, None) == 1
    assert _raw("moe_expert_down", sp, 0, None, fake, fake, fake, None) == 1
    assert _raw("moe_unpermute_combine", sp, 0, fake, fake, fake, fake + 4, None) == 1
    assert _raw("moe_expert_ffn", sp, 0, fake, None, fake, fake, fake, fake, None) == 1
    # pair FFN: null second-chunk buffers while chunk 1 has rows, misaligned act, bad chunk
    assert _raw("moe_expert_ffn_pair", sp, 0, fake, None, fake, fake, fake, fake, fake, fake,
                None) == 1
    assert _raw("moe_expert_ffn_pair", sp, 0, fake, fake, fake, fake, fake, fake + 2, fake,
                fake, None) == 1
    assert _raw("moe_expert_ffn_pair", sp, 2, fake, fake, fake, fake, fake, fake, fake, fake,
                None) == 1
    # gate/up with rows gathered from hidden_states: null src_row, misaligned
    # hidden_states or src_row, bad chunk
    assert _raw("moe_expert_gate_up_gather_pair", sp, 0, fake, None, fake, fake, fake,
                None) == 1
    assert _raw("moe_expert_gate_up_gather_pair", sp, 0, fake + 2, fake, fake, fake, fake,
                None) == 1
    assert _raw("moe_expert_gate_up_gather_pair", sp, 0, fake, fake + 2, fake, fake, fake,
                None) == 1
    assert _raw("moe_expert_gate_up_gather_pair", sp, 2, fake, fake, fake, fake, fake,
                None) == 1
    # backward: too-small workspace, misaligned grad_out, null weight gradients
    need_b = moe.moe_backward_workspace_size(shape)
    args = [fake] * 10  # hidden .. grad_w_down
    assert _raw("moe_chunked_backward", sp, *args, None, fake, need_b - 1, None, None) == 3
    bad = list(args)
    bad[5] = fake + 2
    assert _raw("moe_chunked_backward", sp, *bad, None, fake, need_b, None, None) == 1
    bad = list(args)
    bad[8] = None
    assert _raw("moe_chunked_backward", sp, *bad, None, fake, need_b, None, None) == 1
    assert _raw("moe_unpermute_combine_backward", sp, 2, fake, fake, fake, fake, fake, fake,
                None) == 1
    assert _raw("moe_unpermute_combine_backward", sp, 0, fake, fake, fake, fake, None, fake,
                None) == 1
    assert _raw("moe_permute_backward", sp, 0, fake + 4, fake, fake, None) == 1
    # unknown schedule
    for sched in (-1, 4):
        assert _raw("moe_chunked_forward_schedule", sp, fake, fake, fake, fake, fake, fake, None,
                    fake, need, None, None, sched) == 1


def test_empty_chunk_calls_are_noops():
    """T=3, N=4: chunk 3 is empty, so its step calls return OK without launching."""
    shape = moe.make_shape(3, 7168, 256, 8, 2048, 16, 4, "bf16")
    assert moe.moe_chunk_range(shape, 3) == (3, 3)
    sp = ctypes.byref(shape)
    assert _raw("moe_permute", sp, 3, None, None, None, None) == 0
    assert _raw("moe_expert_ffn", sp, 3, None, None, None, None, None, None, None) == 0
    assert _raw("moe_unpermute_combine", sp, 3, None, None, None, None, None) == 0
    assert _raw("moe_unpermute_combine_backward", sp, 3, None, None, None, None, None, None,
                None) == 0
    assert _raw("moe_permute_backward", sp, 3, None, None, None, None) == 0
    # a pair whose chunks are both empty; none of its pointers is needed
    assert _raw("moe_expert_ffn_pair", sp, 3, None, None, None, None, None, None, None, None,
                None) == 0
    assert _raw("moe_expert_gate_up_gather_pair", sp, 3, None, None, None, None, None,
                None) == 0


def test_binding_refuses_host_tensors():
    import torch
    shape = moe.make_shape(4, 128, 8, 2, 256, 1, 1, "f32")
    with pytest.raises(ValueError):
        moe.moe_permute(shape, 0, torch.zeros(4, 128), torch.zeros(8, dtype=torch.int32),
                        torch.zeros(8, 128))


def test_noalloc_refuses_oversized_shapes_before_any_hip_call():
    """moe_chunked_forward_noalloc checks the shape's workspace against its 64 MiB
    static scratch on the host, before looking the scratch up on a device or
    enqueuing anything, so the refusal needs no GPU; a bad shape is refused as
    by the other entry points."""
    fake = 0x10000000  # never dereferenced
    big = moe.make_shape(65536, 64, 4, 8, 64, 1, 1, "bf16")  # about 138 MB of workspace
    assert moe.moe_workspace_size(big) > 64 << 20
    assert _raw("moe_chunked_forward_noalloc", ctypes.byref(big), fake, fake, fake, fake, fake,
                fake, None, None) == 3  # MOE_ERR_WORKSPACE_TOO_SMALL
    dsv3 = moe.make_shape(4096, 7168, 256, 8, 2048, 16, 1, "bf16")  # 604 MB
    assert _raw("moe_chunked_forward_noalloc", ctypes.byref(dsv3), fake, fake, fake, fake, fake,
                fake, None, None) == 3
    bad = moe.make_shape(64, 96, 256, 8, 2048, 16, 1, "bf16")  # H not a multiple of 64
    assert _raw("moe_chunked_forward_noalloc", ctypes.byref(bad), fake, fake, fake, fake, fake,
                fake, None, None) == 2  # MOE_ERR_UNSUPPORTED
    # a decode-sized batch fits the scratch
    assert moe.moe_workspace_size(moe.make_shape(64, 7168, 256, 8, 2048, 16, 1, "bf16")) <= 64 << 20
