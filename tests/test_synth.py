"""The seeded input generator (host side): bit-identical numpy and torch paths,
prefix stability, and the routing recipe's invariants."""
import numpy as np
import torch

import synth


def test_numpy_and_torch_paths_agree():
    key = synth.stream_key(4, synth.S_W_GATE_UP, 17)
    for n, start in [(1, 0), (1000, 0), (70000, 12345), (300000, 1 << 20)]:
        a = synth._splitmix64_torch(key, n, "cpu", start)
        b = synth.splitmix64(key, n, "cpu", start)
        assert torch.equal(a, b)
        z1 = synth.normal(key, n, 0.02, "cpu", start)
        h = a
        s = (h & 0xFFFF) + (synth._srl(h, 16) & 0xFFFF) + (synth._srl(h, 32) & 0xFFFF) + \
            synth._srl(h, 48)
        z2 = (s - synth._IH_MEAN).to(torch.float32) * torch.tensor(
            np.float32(0.02 / synth._IH_STD))
        assert torch.equal(z1, z2)


def test_splitmix64_reference_value():
    # SplitMix64 seeded with 0: the first output is 0xE220A8397B1DCDAF
    assert int(synth.splitmix64(0, 1).numpy().view(np.uint64)[0]) == 0xE220A8397B1DCDAF


def test_normal_moments_and_prefix():
    x = synth.normal(synth.stream_key(1, 0), 1 << 20, 1.0).numpy().astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert np.abs(x).max() <= 3.47
    cfg = synth.CONFIGS["tiny_f32"]
    full = synth.hidden_states(cfg)
    part = synth.hidden_states(cfg.with_tokens(64))
    assert torch.equal(full[:64], part)


def test_routing_recipe():
    for name, cfg in synth.CONFIGS.items():
        if cfg.T > 4096:
            continue
        idx, w = synth.routing(cfg)
        assert idx.shape == (cfg.T, cfg.k) and idx.dtype == np.int32
        assert w.dtype == np.float32
        assert np.allclose(w.sum(1), 1.0, atol=1e-6)
        assert (w > 0).all()
        if cfg.router == "two_experts":
            assert set(np.unique(idx)) <= {0, 1}
        else:
            assert idx.min() >= 0 and idx.max() < cfg.E
            # top-k picks k distinct experts, weights in descending order
            assert all(len(set(r)) == cfg.k for r in idx.tolist())
            assert (np.diff(w, axis=1) <= 0).all()
