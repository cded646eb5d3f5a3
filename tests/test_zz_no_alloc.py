"""moe_chunked_forward_noalloc (the forward layer with the library's own static
device scratch as its workspace, for callers that cannot allocate) against
moe_chunked_forward with a caller workspace: the same bits, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents); shapes whose workspace exceeds the 64 MiB scratch are refused before
any work is enqueued."""
import pytest
import torch

import combine_top_route_expert_amd as moe
import synth
from gpu_layer import build_layer, run_forward, say

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def _noalloc(L, shape, out):
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    moe.moe_chunked_forward_noalloc(shape, L.hidden, L.idx, L.w, L.wgu, L.wd, out, err,
                                    stream=torch.cuda.current_stream())
    return err


# (workload, (T, N) of the first call, (T, N) of the second, smaller call)
CASES = [
    ("decode_t64", (64, 1), (20, 1)),      # decode batch on the DeepSeek-V3-shaped experts
    ("t3_n4", (3, 4), (2, 4)),             # an empty chunk in both calls
    ("bf16_e64_zipf", (512, 2), (96, 1)),  # a chunk pair, then one chunk
    ("tiny_f32", (256, 2), (37, 3)),       # fp32, ragged chunks
]


@pytest.mark.parametrize("name,first,second", CASES)
def test_noalloc_equals_workspace_forward(name, first, second):
    cfg = synth.CONFIGS[name]
    layers, refs, outs = [], [], []
    for T, N in (first, second):
        L = build_layer(cfg.with_tokens(T))
        shape = L.shape(N)
        assert moe.moe_workspace_size(shape) <= SCRATCH_BYTES
        say(f"noalloc reference {name} T={T} N={N} (caller workspace)")
        ref, err_ref = run_forward(L, shape, two_streams=False)
        layers.append((L, shape))
        refs.append((ref, err_ref))
    # the two no-allocation calls back to back, the second smaller
    errs = []
    for (L, shape), (ref, _) in zip(layers, refs):
        out = torch.full_like(ref, float("nan"))
        say(f"noalloc call {name} T={shape.T} N={shape.N}")
        errs.append(_noalloc(L, shape, out))
        outs.append(out)
    torch.cuda.synchronize()
    for out, err, (ref, err_ref) in zip(outs, errs, refs):
        assert torch.equal(out, ref)
        assert int(err.item()) == err_ref == 0


def test_noalloc_dropped_ids_counted():
    cfg = synth.CONFIGS["tiny_f32"]
    idx, w = synth.routing(cfg)
    idx = idx.copy()
    idx[3, :] = -1
    idx[7, 1] = cfg.E
    L = build_layer(cfg, idx, w)
    shape = L.shape(3)
    ref, err_ref = run_forward(L, shape, two_streams=False)
    out = torch.full_like(ref, float("nan"))
    say("noalloc dropped ids")
    err = _noalloc(L, shape, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert int(err.item()) == err_ref == cfg.k + 1


def test_noalloc_refuses_shapes_past_the_scratch():
    # 65536 tokens of top-8: 524288 rows of H + I = 128 bf16 elements, about 138 MB
    T, H, E, k, I = 65536, 64, 4, 8, 64
    shape = moe.make_shape(T, H, E, k, I, 1, 1, "bf16")
    assert moe.moe_workspace_size(shape) > SCRATCH_BYTES
    dev = dict(device="cuda")
    hidden = torch.zeros((T, H), dtype=torch.bfloat16, **dev)
    idx = torch.zeros((T, k), dtype=torch.int32, **dev)
    w = torch.zeros((T, k), dtype=torch.float32, **dev)
    wgu = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, **dev)
    wd = torch.zeros((E, H, I), dtype=torch.bfloat16, **dev)
    out = torch.full((T, H), 3.0, dtype=torch.bfloat16, **dev)
    say("noalloc refuses a shape past the scratch")
    with pytest.raises(moe.MoeError) as exc:
        moe.moe_chunked_forward_noalloc(shape, hidden, idx, w, wgu, wd, out)
    assert exc.value.code == 3  # MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())  # nothing was enqueued
