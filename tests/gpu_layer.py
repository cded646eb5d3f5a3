"""Device-side test workloads: seeded inputs on the GPU plus float64 host views
for the oracle.  Inputs come only from `synth`; nothing here computes any step
of the layer."""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, Optional

import numpy as np
import torch

import combine_top_route_expert_amd as moe
import synth


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says what it ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Layer:
    cfg: synth.MoEConfig
    hidden: torch.Tensor          # [T,H] device
    idx: torch.Tensor             # [T,k] int32 device
    w: torch.Tensor               # [T,k] fp32 device
    wgu: torch.Tensor             # [E,2I,H] device
    wd: torch.Tensor              # [E,H,I] device
    idx_np: np.ndarray
    w_np: np.ndarray
    _f64: Dict[int, tuple] = dataclasses.field(default_factory=dict)
    _n64: int = 0

    def shape(self, N: int = 1, G: Optional[int] = None) -> moe.moe_shape:
        c = self.cfg
        return moe.make_shape(c.T, c.H, c.E, c.k, c.I, c.groups if G is None else G, N, c.dtype)

    def hidden64(self) -> np.ndarray:
        return synth.to_f64(self.hidden)

    def expert64(self, e: int):
        """float64 host copy of expert e's weights (an exact copy of the input:
        widened to float64 on the device, then copied).  At most about 6 GiB of
        experts are kept, so a pass over all 256 DeepSeek-V3-shaped experts
        streams them."""
        if e not in self._f64:
            per = 8 * (self.wgu[e].numel() + self.wd[e].numel())
            if per * (len(self._f64) + 1) > (6 << 30):
                self._f64.clear()
            self._f64[e] = (self.wgu[e].to(torch.float64).cpu().numpy(),
                            self.wd[e].to(torch.float64).cpu().numpy())
            self._n64 += 1
            if self._n64 % 64 == 0:
                say(f"  {self._n64} expert weight sets widened to float64 for the oracle")
        return self._f64[e]


_weight_cache: Dict[tuple, tuple] = {}


def expert_weights(cfg: synth.MoEConfig, device="cuda"):
    key = (cfg.weight_seed, cfg.E, cfg.H, cfg.I, cfg.dtype)
    if key not in _weight_cache:
        _weight_cache.clear()
        torch.cuda.empty_cache()
        say(f"generate expert weights {key}")
        _weight_cache[key] = synth.all_expert_weights(cfg, device)
        torch.cuda.synchronize()
    return _weight_cache[key]


def build_layer(cfg: synth.MoEConfig, idx_np: Optional[np.ndarray] = None,
                w_np: Optional[np.ndarray] = None) -> Layer:
    say(f"inputs {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} {cfg.dtype}")
    if idx_np is None:
        idx_np, w_np = synth.routing(cfg)
    hidden = synth.hidden_states(cfg, "cuda")
    wgu, wd = expert_weights(cfg)
    return Layer(cfg, hidden, torch.from_numpy(np.ascontiguousarray(idx_np)).cuda(),
                 torch.from_numpy(np.ascontiguousarray(w_np)).cuda(), wgu, wd, idx_np, w_np)


def run_route_meta(idx: torch.Tensor, shape: moe.moe_shape):
    T, k, E, N, G = shape.T, shape.k, shape.E, shape.N, shape.G
    i32 = dict(dtype=torch.int32, device="cuda")
    out = {
        "counts": torch.full((N, E), -7, **i32),
        "offsets": torch.full((N, E + 1), -7, **i32),
        "group_splits": torch.full((N, G), -7, **i32),
        "src_row": torch.full((T * k,), -7, **i32),
        "dst_row": torch.full((T * k,), -7, **i32),
        "dev_error": torch.full((1,), -7, **i32),
    }
    ws = torch.empty(moe.moe_route_meta_workspace_size(shape), dtype=torch.uint8, device="cuda")
    moe.moe_route_meta(shape, idx, out["counts"], out["offsets"], out["group_splits"],
                       out["src_row"], out["dst_row"], out["dev_error"], ws)
    torch.cuda.synchronize()
    return {kk: v.cpu().numpy() for kk, v in out.items()}


def run_forward(layer: Layer, shape: moe.moe_shape, two_streams: bool = True,
                out: Optional[torch.Tensor] = None, schedule: Optional[int] = None):
    c = layer.cfg
    if out is None:
        out = torch.full((c.T, c.H), float("nan"), dtype=c.torch_dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else None
    if schedule is None:
        moe.moe_chunked_forward(shape, layer.hidden, layer.idx, layer.w, layer.wgu, layer.wd, out,
                                ws, err, s0=s0, s1=s1)
    else:
        moe.moe_chunked_forward_schedule(shape, layer.hidden, layer.idx, layer.w, layer.wgu,
                                         layer.wd, out, ws, err, s0=s0, s1=s1, schedule=schedule)
    torch.cuda.synchronize()
    return out, int(err.item())


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()
