"""Seeded synthetic inputs for the MoE-layer workloads.

This module only *draws* the tensors a caller hands to the MoE layer
(``hidden_states``, ``top_k_index``, ``top_k_weights`` and the expert weights).
It contains no step of the layer itself (no metadata, permute, expert FFN or
combine), so the GPU path and the CPU oracle can both be fed from it without
sharing any of the method's arithmetic.

Random numbers
--------------
Every value is a pure function of (config seed, stream, sub-stream, element
index), computed with the SplitMix64 generator (Steele, Lea & Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014): the i-th output of a
stream with key ``K`` is ``mix64(K + (i + 1) * 0x9E3779B97F4A7C15)``.  It is
evaluated with wrapping 64-bit integer arithmetic (blocked numpy uint64 on the
host, torch int64 on a device), so it gives identical bits on the CPU and on a
GPU, and a prefix of a tensor does not depend on the tensor's length
(``hidden_states`` for T=64 is the first 64 rows of the T=4096 draw).

* "normal(std)": Irwin-Hall sum of the four 16-bit fields of one 64-bit output,
  centred and scaled to ``std`` with a single fp32 multiply.  It has the mean and
  variance of N(0, std^2) and a bounded support of +/- 3.46 std.
* "uniform": the top 24 bits of one output times 2^-24, exact in fp32, in [0, 1).
* bf16 tensors are the fp32 draw rounded to nearest-even once.

Routing (top-k choice and its weights) is drawn on the CPU in float64 and only
then handed to a device, so the integer top-k choice never depends on which
device evaluated the softmax.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1
# standard deviation of the sum of four independent uniform 16-bit integers
_IH_STD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
_IH_MEAN = 2 * 65535

# stream ids
S_HIDDEN, S_LOGITS, S_BIAS_RANK, S_W_GATE_UP, S_W_DOWN, S_TWO_IDX, S_TWO_W = range(7)


def _signed(u: int) -> int:
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int, sub: int = 0) -> int:
    """64-bit key of one stream: the mix of (seed, stream, sub) packed into one word."""
    word = ((seed & 0xFFFF) << 48) | ((stream & 0xFF) << 40) | (sub & 0xFFFFFFFFFF)
    return _mix64_int(word)


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of an int64 tensor (torch's >> is arithmetic)."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def _splitmix64_torch(key: int, n: int, device, start: int) -> torch.Tensor:
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = i * _signed(_GAMMA) + _signed(key)
    z = (z ^ _srl(z, 30)) * _signed(_M1)
    z = (z ^ _srl(z, 27)) * _signed(_M2)
    return z ^ _srl(z, 31)


_BLOCK = 1 << 18
_U64 = np.uint64


def _np_block(key: int, st: int, m: int, base, z, t):
    """SplitMix64 outputs st..st+m-1 into z[:m] (uint64), t is scratch."""
    zz, tt = z[:m], t[:m]
    np.add(base[:m], _U64(st), out=zz)
    zz *= _U64(_GAMMA)
    zz += _U64(key)
    np.right_shift(zz, _U64(30), out=tt); zz ^= tt; zz *= _U64(_M1)
    np.right_shift(zz, _U64(27), out=tt); zz ^= tt; zz *= _U64(_M2)
    np.right_shift(zz, _U64(31), out=tt); zz ^= tt
    return zz, tt


def _np_fill(n: int, fn) -> None:
    """Run fn(st, m, base, z, t, s) over blocks of the range [0, n), on a few threads."""
    import concurrent.futures as cf
    import os
    starts = list(range(0, n, _BLOCK))
    base = np.arange(1, _BLOCK + 1, dtype=np.uint64)

    def work(chunk):
        z = np.empty(_BLOCK, np.uint64)
        t = np.empty(_BLOCK, np.uint64)
        s = np.empty(_BLOCK, np.uint64)
        for st in chunk:
            fn(st, min(_BLOCK, n - st), base, z, t, s)

    nthr = max(1, min(len(starts), os.cpu_count() or 1, 16))
    if nthr == 1:
        work(starts)
        return
    parts = [starts[i::nthr] for i in range(nthr)]
    with cf.ThreadPoolExecutor(nthr) as ex:
        list(ex.map(work, parts))


def splitmix64(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """Outputs start..start+n-1 of the SplitMix64 stream with the given key, as int64 bits."""
    if torch.device(device).type != "cpu":
        return _splitmix64_torch(key, n, device, start)
    out = np.empty(n, np.uint64)

    def fn(st, m, base, z, t, s):
        zz, _ = _np_block(key, start + st, m, base, z, t)
        out[st:st + m] = zz

    _np_fill(n, fn)
    return torch.from_numpy(out.view(np.int64))


def normal(key: int, n: int, std: float, device="cpu", start: int = 0) -> torch.Tensor:
    scale32 = np.float32(std / _IH_STD)
    if torch.device(device).type != "cpu":
        h = _splitmix64_torch(key, n, device, start)
        s = (h & 0xFFFF) + (_srl(h, 16) & 0xFFFF) + (_srl(h, 32) & 0xFFFF) + _srl(h, 48)
        del h
        z = (s - _IH_MEAN).to(torch.float32)
        return z * torch.tensor(scale32, dtype=torch.float32, device=device)
    out = np.empty(n, np.float32)

    def fn(st, m, base, z, t, s):
        zz, tt = _np_block(key, start + st, m, base, z, t)
        ss = s[:m]
        np.bitwise_and(zz, _U64(0xFFFF), out=ss)
        for sh in (16, 32):
            np.right_shift(zz, _U64(sh), out=tt); tt &= _U64(0xFFFF); ss += tt
        np.right_shift(zz, _U64(48), out=tt); ss += tt
        o = out[st:st + m]
        o[:] = ss.view(np.int64) - _IH_MEAN
        o *= scale32

    _np_fill(n, fn)
    return torch.from_numpy(out)


def uniform(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    h = splitmix64(key, n, device, start)
    return _srl(h, 40).to(torch.float32) * (2.0 ** -24)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int          # seed of hidden_states and routing
    weight_seed: int   # seed of the expert weights (shared by workloads with the same experts)
    T: int
    H: int
    E: int
    k: int
    I: int
    dtype: str         # "f32" | "bf16"
    router: str        # "normal" | "uniform" | "two_experts"
    zipf_s: Optional[float]
    groups: int
    num_chunks: Tuple[int, ...]
    hidden_std: float = 1.0
    weight_std: float = 0.02

    def with_tokens(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T)

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    # tiny fp32 layer
    "tiny_f32": MoEConfig("tiny_f32", 1, 1, 256, 128, 8, 2, 256, "f32", "normal", None, 1, (1,)),
    # bf16, 64 experts, top-4, Zipf(1.1)-skewed expert popularity; N=1 and N=2 compared
    "bf16_e64_zipf": MoEConfig("bf16_e64_zipf", 2, 2, 4096, 2048, 64, 4, 1024, "bf16", "normal",
                               1.1, 1, (1, 2)),
    # DeepSeek-V3-shaped layer, all 256 routed experts on one GPU, 16 destination groups
    "dsv3_e256": MoEConfig("dsv3_e256", 3, 3, 4096, 7168, 256, 8, 2048, "bf16", "uniform", None,
                           16, (1,)),
    # long packed sequence, Chunk-MoE sweep
    "packed16k_e128": MoEConfig("packed16k_e128", 4, 4, 16384, 2048, 128, 8, 768, "bf16",
                                "normal", 0.8, 1, (1, 2, 4, 8)),
    # decode-sized batch on the DeepSeek-V3-shaped experts
    "decode_t64": MoEConfig("decode_t64", 5, 3, 64, 7168, 256, 8, 2048, "bf16", "uniform", None,
                            16, (1,)),
    # three tokens in four chunks: the last chunk is empty
    "t3_n4": MoEConfig("t3_n4", 6, 3, 3, 7168, 256, 8, 2048, "bf16", "uniform", None, 16, (4, 1)),
    # every slot routed to expert 0 or 1 (maximal skew)
    "skew_two_experts": MoEConfig("skew_two_experts", 7, 3, 1000, 7168, 256, 8, 2048, "bf16",
                                  "two_experts", None, 16, (1,)),
    # sizes off the tile grids: H = 5*64, I = 3*64 (partial column tiles everywhere)
    "odd_dims_bf16": MoEConfig("odd_dims_bf16", 8, 8, 1536, 320, 8, 4, 192, "bf16", "normal",
                               0.5, 2, (1, 3)),
    # fp32 sizes that are multiples of 4 only, with a ragged token count
    "odd_dims_f32": MoEConfig("odd_dims_f32", 9, 9, 203, 36, 5, 3, 20, "f32", "normal", None, 1,
                              (1, 4)),
}


def hidden_states(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    x = normal(stream_key(cfg.seed, S_HIDDEN), cfg.T * cfg.H, cfg.hidden_std, device)
    return x.view(cfg.T, cfg.H).to(cfg.torch_dtype)


def _zipf_bias(cfg: MoEConfig) -> np.ndarray:
    """Per-expert Zipf-law logit bias -s*ln(rank), ranks a seeded permutation of 1..E."""
    h = splitmix64(stream_key(cfg.seed, S_BIAS_RANK), cfg.E).numpy().view(np.uint64)
    order = np.argsort(h, kind="stable")
    rank = np.empty(cfg.E, dtype=np.float64)
    rank[order] = np.arange(1, cfg.E + 1, dtype=np.float64)
    return -float(cfg.zipf_s) * np.log(rank)


def routing(cfg: MoEConfig) -> Tuple[np.ndarray, np.ndarray]:
    """(top_k_index int32 [T,k], top_k_weights float32 [T,k]) drawn on the CPU.

    Router logits [T,E] -> top-k (descending, ties to the lower expert id) ->
    softmax over the chosen k logits (the renormalised top-k probabilities)."""
    T, E, k = cfg.T, cfg.E, cfg.k
    if cfg.router == "two_experts":
        u = uniform(stream_key(cfg.seed, S_TWO_IDX), T * k).numpy().reshape(T, k)
        idx = (u >= 0.5).astype(np.int32)
        z = normal(stream_key(cfg.seed, S_TWO_W), T * k, 1.0).numpy().astype(np.float64)
        z = z.reshape(T, k)
    else:
        if cfg.router == "normal":
            logits = normal(stream_key(cfg.seed, S_LOGITS), T * E, 1.0).numpy()
        elif cfg.router == "uniform":
            logits = uniform(stream_key(cfg.seed, S_LOGITS), T * E).numpy()
        else:
            raise ValueError(cfg.router)
        logits = logits.astype(np.float64).reshape(T, E)
        if cfg.zipf_s:
            logits = logits + _zipf_bias(cfg)[None, :]
        idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
        z = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    w = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def expert_gate_up(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    """w_gate_up[e]: [2I, H]; rows 0..I-1 are the gate projection, rows I..2I-1 the up projection."""
    w = normal(stream_key(cfg.weight_seed, S_W_GATE_UP, e), 2 * cfg.I * cfg.H, cfg.weight_std,
               device)
    return w.view(2 * cfg.I, cfg.H).to(cfg.torch_dtype)


def expert_down(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    """w_down[e]: [H, I]."""
    w = normal(stream_key(cfg.weight_seed, S_W_DOWN, e), cfg.H * cfg.I, cfg.weight_std, device)
    return w.view(cfg.H, cfg.I).to(cfg.torch_dtype)


def all_expert_weights(cfg: MoEConfig, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """[E,2I,H] and [E,H,I] tensors, generated expert by expert to bound temporaries."""
    wgu = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=cfg.torch_dtype, device=device)
    wd = torch.empty((cfg.E, cfg.H, cfg.I), dtype=cfg.torch_dtype, device=device)
    for e in range(cfg.E):
        wgu[e] = expert_gate_up(cfg, e, device)
        wd[e] = expert_down(cfg, e, device)
    return wgu, wd


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (bf16 or fp32) tensor, on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()
