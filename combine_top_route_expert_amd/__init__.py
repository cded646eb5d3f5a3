"""Python binding of libmoe.so: MoE token dispatch, expert FFN and combine on
one AMD Instinct MI355X (gfx950).

Argument marshalling only.  Each function has the name of the C entry point it
calls (include/moe.h), takes torch tensors that live in device memory, checks
their dtype, contiguity, device and size against the shape (so that no kernel
is handed a buffer smaller than its grid assumes), and passes raw pointers and
the HIP stream to the library.  A non-OK status raises MoeError.  Every step of
the layer runs in the library's HIP kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MoeError", "moe_shape", "make_shape", "library_path", "load_library", "moe_status_string",
    "moe_resolve_num_chunks", "moe_chunk_range", "moe_route_meta_workspace_size",
    "moe_workspace_size", "moe_route_meta", "moe_permute", "moe_expert_gate_up",
    "moe_expert_down", "moe_expert_ffn", "moe_expert_ffn_pair", "moe_expert_gate_up_pair",
    "moe_expert_gate_up_gather_pair", "moe_expert_down_pair", "moe_unpermute_combine", "moe_chunked_forward",
    "moe_chunked_forward_schedule", "moe_backward_workspace_size", "moe_chunked_backward",
    "moe_unpermute_combine_backward", "moe_permute_backward", "MOE_F32", "MOE_BF16",
    "MOE_SCHEDULE_PAIR_FUSED", "MOE_SCHEDULE_PER_CHUNK", "MOE_SCHEDULE_PAIR_FUSED_PREFETCH",
    "MOE_SCHEDULE_EXPERT_HALVES",
    "EXPORTED_SYMBOLS",
    "moe_chunked_forward_noalloc",
]

MOE_F32, MOE_BF16 = 0, 1
MOE_SCHEDULE_PAIR_FUSED, MOE_SCHEDULE_PER_CHUNK, MOE_SCHEDULE_PAIR_FUSED_PREFETCH = 0, 1, 2
MOE_SCHEDULE_EXPERT_HALVES = 3
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

EXPORTED_SYMBOLS = (
    "moe_status_string", "moe_resolve_num_chunks", "moe_chunk_range",
    "moe_route_meta_workspace_size", "moe_workspace_size", "moe_route_meta", "moe_permute",
    "moe_expert_gate_up", "moe_expert_down", "moe_expert_ffn", "moe_expert_gate_up_pair",
    "moe_expert_gate_up_gather_pair", "moe_expert_down_pair", "moe_expert_ffn_pair", "moe_unpermute_combine",
    "moe_chunked_forward", "moe_chunked_forward_schedule", "moe_chunked_forward_noalloc",
    "moe_backward_workspace_size",
    "moe_chunked_backward", "moe_unpermute_combine_backward", "moe_permute_backward",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {_STATUS.get(code, code)}")
        self.code = code


class moe_shape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("num_chunks", ctypes.c_int32), ("dtype", ctypes.c_int32)]

    @property
    def T(self): return self.num_tokens

    @property
    def H(self): return self.hidden

    @property
    def E(self): return self.num_experts

    @property
    def k(self): return self.top_k

    @property
    def I(self): return self.intermediate  # noqa: E743

    @property
    def N(self): return self.num_chunks if self.num_chunks > 0 else 1

    @property
    def G(self): return self.num_groups if self.num_groups > 0 else 1

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == MOE_BF16 else torch.float32


def make_shape(T: int, H: int, E: int, k: int, I: int, G: int = 1, N: int = 1,  # noqa: E741
               dtype: str = "bf16") -> moe_shape:
    return moe_shape(T, H, E, k, I, G, N, MOE_BF16 if dtype == "bf16" else MOE_F32)


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")


_lib = None
_P = ctypes.c_void_p
_SP = ctypes.POINTER(moe_shape)


def load_library() -> ctypes.CDLL:
    """Load the built libmoe.so; raises if it was not built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m combine_top_route_expert_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_resolve_num_chunks": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32,
                                                    ctypes.POINTER(ctypes.c_int32)]),
        "moe_chunk_range": (ctypes.c_int, [_SP, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]),
        "moe_route_meta_workspace_size": (ctypes.c_int, [_SP, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_workspace_size": (ctypes.c_int, [_SP, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_route_meta": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                          _P]),
        "moe_permute": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P]),
        "moe_expert_gate_up": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P]),
        "moe_expert_down": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P]),
        "moe_expert_ffn": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P]),
        "moe_expert_gate_up_pair": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P,
                                                   _P]),
        "moe_expert_gate_up_gather_pair": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P,
                                                          _P, _P]),
        "moe_expert_down_pair": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
        "moe_expert_ffn_pair": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                               _P, _P, _P]),
        "moe_unpermute_combine": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P, _P]),
        "moe_chunked_forward": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_size_t, _P, _P]),
        "moe_chunked_forward_schedule": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P,
                                                        ctypes.c_size_t, _P, _P,
                                                        ctypes.c_int32]),
        "moe_chunked_forward_noalloc": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P]),
        "moe_backward_workspace_size": (ctypes.c_int, [_SP, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_chunked_backward": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                _P, _P, ctypes.c_size_t, _P, _P]),
        "moe_unpermute_combine_backward": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P,
                                                          _P, _P, _P]),
        "moe_permute_backward": (ctypes.c_int, [_SP, ctypes.c_int32, _P, _P, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise MoeError(fn, code)


def _stream(s) -> int:
    if s is None:
        s = torch.cuda.current_stream()
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype, min_numel: int, name: str) -> Optional[int]:
    if t is None:
        if min_numel > 0:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    return t.data_ptr()


def _ws_ptr(ws: torch.Tensor, need: int, name: str = "ws") -> Tuple[int, int]:
    p = _ptr(ws, torch.uint8, need, name)
    return p, ws.numel()


# ---------------------------------------------------------------- host-only helpers
def moe_status_string(code: int) -> str:
    return load_library().moe_status_string(code).decode()


def moe_resolve_num_chunks(T: int, num_chunks: int, chunk_size: int) -> Tuple[int, bool]:
    w = ctypes.c_int32(0)
    n = load_library().moe_resolve_num_chunks(T, num_chunks, chunk_size, ctypes.byref(w))
    return n, bool(w.value)


def moe_chunk_range(shape: moe_shape, chunk: int) -> Tuple[int, int]:
    t0, t1 = ctypes.c_int32(), ctypes.c_int32()
    _check("moe_chunk_range", load_library().moe_chunk_range(
        ctypes.byref(shape), chunk, ctypes.byref(t0), ctypes.byref(t1)))
    return t0.value, t1.value


def moe_route_meta_workspace_size(shape: moe_shape) -> int:
    b = ctypes.c_size_t()
    _check("moe_route_meta_workspace_size",
           load_library().moe_route_meta_workspace_size(ctypes.byref(shape), ctypes.byref(b)))
    return b.value


def moe_workspace_size(shape: moe_shape) -> int:
    b = ctypes.c_size_t()
    _check("moe_workspace_size",
           load_library().moe_workspace_size(ctypes.byref(shape), ctypes.byref(b)))
    return b.value


# ---------------------------------------------------------------- device entry points
def moe_route_meta(shape: moe_shape, top_k_index, counts, offsets, group_splits, src_row,
                   dst_row, dev_error, ws, stream=None) -> None:
    A, N, E, G = shape.T * shape.k, shape.N, shape.E, shape.G
    i32 = torch.int32
    args = (
        _ptr(top_k_index, i32, A, "top_k_index"), _ptr(counts, i32, N * E, "counts"),
        _ptr(offsets, i32, N * (E + 1), "offsets"), _ptr(group_splits, i32, N * G, "group_splits"),
        _ptr(src_row, i32, A, "src_row"), _ptr(dst_row, i32, A, "dst_row"),
        _ptr(dev_error, i32, 0, "dev_error"),
    )
    wp, wn = _ws_ptr(ws, moe_route_meta_workspace_size(shape))
    _check("moe_route_meta", load_library().moe_route_meta(
        ctypes.byref(shape), *args, wp, wn, _stream(stream)))


def _chunk_rows(shape: moe_shape, chunk: int) -> Tuple[int, int, int]:
    t0, t1 = moe_chunk_range(shape, chunk)
    return t0, t1, (t1 - t0) * shape.k


def moe_permute(shape: moe_shape, chunk: int, hidden_states, dst_row, x_perm,
                stream=None) -> None:
    t0, t1, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_permute", load_library().moe_permute(
        ctypes.byref(shape), chunk, _ptr(hidden_states, dt, shape.T * shape.H, "hidden_states"),
        _ptr(dst_row, torch.int32, shape.T * shape.k, "dst_row"),
        _ptr(x_perm, dt, rows * shape.H, "x_perm"), _stream(stream)))


def moe_expert_gate_up(shape: moe_shape, chunk: int, x_perm, offsets, w_gate_up, act,
                       stream=None) -> None:
    _, _, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_gate_up", load_library().moe_expert_gate_up(
        ctypes.byref(shape), chunk, _ptr(x_perm, dt, rows * shape.H, "x_perm"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_gate_up, dt, shape.E * 2 * shape.I * shape.H, "w_gate_up"),
        _ptr(act, dt, rows * shape.I, "act"), _stream(stream)))


def moe_expert_down(shape: moe_shape, chunk: int, act, offsets, w_down, y, stream=None) -> None:
    _, _, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_down", load_library().moe_expert_down(
        ctypes.byref(shape), chunk, _ptr(act, dt, rows * shape.I, "act"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_down, dt, shape.E * shape.H * shape.I, "w_down"),
        _ptr(y, dt, rows * shape.H, "y"), _stream(stream)))


def moe_expert_ffn(shape: moe_shape, chunk: int, x_perm, offsets, w_gate_up, w_down, act, y,
                   stream=None) -> None:
    _, _, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_ffn", load_library().moe_expert_ffn(
        ctypes.byref(shape), chunk, _ptr(x_perm, dt, rows * shape.H, "x_perm"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_gate_up, dt, shape.E * 2 * shape.I * shape.H, "w_gate_up"),
        _ptr(w_down, dt, shape.E * shape.H * shape.I, "w_down"),
        _ptr(act, dt, rows * shape.I, "act"), _ptr(y, dt, rows * shape.H, "y"),
        _stream(stream)))


def _pair_rows(shape: moe_shape, chunk: int) -> Tuple[int, int]:
    rows0 = _chunk_rows(shape, chunk)[2]
    rows1 = _chunk_rows(shape, chunk + 1)[2] if chunk + 1 < shape.N else 0
    return rows0, rows1


def moe_expert_gate_up_pair(shape: moe_shape, chunk: int, x_perm0, x_perm1, offsets, w_gate_up,
                            act, stream=None) -> None:
    rows0, rows1 = _pair_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_gate_up_pair", load_library().moe_expert_gate_up_pair(
        ctypes.byref(shape), chunk, _ptr(x_perm0, dt, rows0 * shape.H, "x_perm0"),
        _ptr(x_perm1, dt, rows1 * shape.H, "x_perm1"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_gate_up, dt, shape.E * 2 * shape.I * shape.H, "w_gate_up"),
        _ptr(act, dt, (rows0 + rows1) * shape.I, "act"), _stream(stream)))


def moe_expert_gate_up_gather_pair(shape: moe_shape, chunk: int, hidden_states, src_row, offsets,
                                   w_gate_up, act, stream=None) -> None:
    rows0, rows1 = _pair_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_gate_up_gather_pair", load_library().moe_expert_gate_up_gather_pair(
        ctypes.byref(shape), chunk, _ptr(hidden_states, dt, shape.T * shape.H, "hidden_states"),
        _ptr(src_row, torch.int32, shape.T * shape.k, "src_row"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_gate_up, dt, shape.E * 2 * shape.I * shape.H, "w_gate_up"),
        _ptr(act, dt, (rows0 + rows1) * shape.I, "act"), _stream(stream)))


def moe_expert_down_pair(shape: moe_shape, chunk: int, act, offsets, w_down, y0, y1,
                         stream=None) -> None:
    rows0, rows1 = _pair_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_down_pair", load_library().moe_expert_down_pair(
        ctypes.byref(shape), chunk, _ptr(act, dt, (rows0 + rows1) * shape.I, "act"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_down, dt, shape.E * shape.H * shape.I, "w_down"),
        _ptr(y0, dt, rows0 * shape.H, "y0"), _ptr(y1, dt, rows1 * shape.H, "y1"),
        _stream(stream)))


def moe_expert_ffn_pair(shape: moe_shape, chunk: int, x_perm0, x_perm1, offsets, w_gate_up,
                        w_down, act, y0, y1, stream=None) -> None:
    """FFN of chunks `chunk` and `chunk + 1` in one launch pair; `act` holds the
    pair's rows grouped by expert.  x_perm1/y1 may be None when the second chunk
    does not exist or is empty."""
    rows0, rows1 = _pair_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_expert_ffn_pair", load_library().moe_expert_ffn_pair(
        ctypes.byref(shape), chunk, _ptr(x_perm0, dt, rows0 * shape.H, "x_perm0"),
        _ptr(x_perm1, dt, rows1 * shape.H, "x_perm1"),
        _ptr(offsets, torch.int32, shape.N * (shape.E + 1), "offsets"),
        _ptr(w_gate_up, dt, shape.E * 2 * shape.I * shape.H, "w_gate_up"),
        _ptr(w_down, dt, shape.E * shape.H * shape.I, "w_down"),
        _ptr(act, dt, (rows0 + rows1) * shape.I, "act"),
        _ptr(y0, dt, rows0 * shape.H, "y0"), _ptr(y1, dt, rows1 * shape.H, "y1"),
        _stream(stream)))


def moe_unpermute_combine(shape: moe_shape, chunk: int, y, dst_row, top_k_weights, out,
                          stream=None) -> None:
    _, _, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_unpermute_combine", load_library().moe_unpermute_combine(
        ctypes.byref(shape), chunk, _ptr(y, dt, rows * shape.H, "y"),
        _ptr(dst_row, torch.int32, shape.T * shape.k, "dst_row"),
        _ptr(top_k_weights, torch.float32, shape.T * shape.k, "top_k_weights"),
        _ptr(out, dt, shape.T * shape.H, "out"), _stream(stream)))


def moe_chunked_forward_schedule(shape: moe_shape, hidden_states, top_k_index, top_k_weights,
                                 w_gate_up, w_down, out, ws, dev_error=None, s0=None, s1=None,
                                 schedule: int = MOE_SCHEDULE_PAIR_FUSED,
                                 _fn: str = "moe_chunked_forward_schedule") -> None:
    dt = shape.torch_dtype
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I  # noqa: E741
    wp, wn = _ws_ptr(ws, moe_workspace_size(shape))
    s0i = _stream(s0)
    s1i = _stream(s1) if s1 is not None else None
    args = (ctypes.byref(shape), _ptr(hidden_states, dt, T * H, "hidden_states"),
            _ptr(top_k_index, torch.int32, T * k, "top_k_index"),
            _ptr(top_k_weights, torch.float32, T * k, "top_k_weights"),
            _ptr(w_gate_up, dt, E * 2 * I * H, "w_gate_up"), _ptr(w_down, dt, E * H * I, "w_down"),
            _ptr(out, dt, T * H, "out"), _ptr(dev_error, torch.int32, 0, "dev_error"), wp, wn,
            s0i, s1i)
    lib = load_library()
    if _fn == "moe_chunked_forward":
        _check(_fn, lib.moe_chunked_forward(*args))
    else:
        _check(_fn, lib.moe_chunked_forward_schedule(*args, schedule))


def moe_chunked_forward(shape: moe_shape, hidden_states, top_k_index, top_k_weights, w_gate_up,
                        w_down, out, ws, dev_error=None, s0=None, s1=None) -> None:
    moe_chunked_forward_schedule(shape, hidden_states, top_k_index, top_k_weights, w_gate_up,
                                 w_down, out, ws, dev_error, s0, s1, _fn="moe_chunked_forward")


def moe_chunked_forward_noalloc(shape: moe_shape, hidden_states, top_k_index, top_k_weights,
                                w_gate_up, w_down, out, dev_error=None, stream=None) -> None:
    """The forward layer with the library's own static 64 MiB device scratch as
    its workspace (no allocation in the call); calls on one GPU must not
    overlap."""
    dt = shape.torch_dtype
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I  # noqa: E741
    _check("moe_chunked_forward_noalloc", load_library().moe_chunked_forward_noalloc(
        ctypes.byref(shape), _ptr(hidden_states, dt, T * H, "hidden_states"),
        _ptr(top_k_index, torch.int32, T * k, "top_k_index"),
        _ptr(top_k_weights, torch.float32, T * k, "top_k_weights"),
        _ptr(w_gate_up, dt, E * 2 * I * H, "w_gate_up"), _ptr(w_down, dt, E * H * I, "w_down"),
        _ptr(out, dt, T * H, "out"), _ptr(dev_error, torch.int32, 0, "dev_error"),
        _stream(stream)))


# ---------------------------------------------------------------- backward
def moe_backward_workspace_size(shape: moe_shape) -> int:
    b = ctypes.c_size_t()
    _check("moe_backward_workspace_size",
           load_library().moe_backward_workspace_size(ctypes.byref(shape), ctypes.byref(b)))
    return b.value


def moe_chunked_backward(shape: moe_shape, hidden_states, top_k_index, top_k_weights, w_gate_up,
                         w_down, grad_out, grad_hidden, grad_top_k_weights, grad_w_gate_up,
                         grad_w_down, ws, dev_error=None, s0=None, s1=None) -> None:
    dt = shape.torch_dtype
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I  # noqa: E741
    wp, wn = _ws_ptr(ws, moe_backward_workspace_size(shape))
    s1i = _stream(s1) if s1 is not None else None
    _check("moe_chunked_backward", load_library().moe_chunked_backward(
        ctypes.byref(shape), _ptr(hidden_states, dt, T * H, "hidden_states"),
        _ptr(top_k_index, torch.int32, T * k, "top_k_index"),
        _ptr(top_k_weights, torch.float32, T * k, "top_k_weights"),
        _ptr(w_gate_up, dt, E * 2 * I * H, "w_gate_up"), _ptr(w_down, dt, E * H * I, "w_down"),
        _ptr(grad_out, dt, T * H, "grad_out"), _ptr(grad_hidden, dt, T * H, "grad_hidden"),
        _ptr(grad_top_k_weights, torch.float32, T * k, "grad_top_k_weights"),
        _ptr(grad_w_gate_up, torch.float32, E * 2 * I * H, "grad_w_gate_up"),
        _ptr(grad_w_down, torch.float32, E * H * I, "grad_w_down"),
        _ptr(dev_error, torch.int32, 0, "dev_error"), wp, wn, _stream(s0), s1i))


def moe_unpermute_combine_backward(shape: moe_shape, chunk: int, grad_out, y, dst_row,
                                   top_k_weights, grad_y, grad_top_k_weights,
                                   stream=None) -> None:
    _, _, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    T, H, k = shape.T, shape.H, shape.k
    _check("moe_unpermute_combine_backward", load_library().moe_unpermute_combine_backward(
        ctypes.byref(shape), chunk, _ptr(grad_out, dt, T * H, "grad_out"),
        _ptr(y, dt, rows * H, "y"), _ptr(dst_row, torch.int32, T * k, "dst_row"),
        _ptr(top_k_weights, torch.float32, T * k, "top_k_weights"),
        _ptr(grad_y, dt, rows * H, "grad_y"),
        _ptr(grad_top_k_weights, torch.float32, T * k, "grad_top_k_weights"), _stream(stream)))


def moe_permute_backward(shape: moe_shape, chunk: int, grad_x_perm, dst_row, grad_hidden,
                         stream=None) -> None:
    _, _, rows = _chunk_rows(shape, chunk)
    dt = shape.torch_dtype
    _check("moe_permute_backward", load_library().moe_permute_backward(
        ctypes.byref(shape), chunk, _ptr(grad_x_perm, dt, rows * shape.H, "grad_x_perm"),
        _ptr(dst_row, torch.int32, shape.T * shape.k, "dst_row"),
        _ptr(grad_hidden, dt, shape.T * shape.H, "grad_hidden"), _stream(stream)))
