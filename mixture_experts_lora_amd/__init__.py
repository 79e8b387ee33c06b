"""MoE-LoRA expert layer on AMD MI355X (gfx950): Python binding of libmoe_lora.so.

The functions below carry the names of the C ABI (include/moe_lora.h) and do
argument marshalling only: they check that each torch tensor is a contiguous
GPU tensor of the shape and dtype the kernels assume, then pass its address
and torch's current HIP stream to the library. Every step of the layer runs in
the HIP kernels; nothing here computes. PyTorch provides the device memory and
the stream.

Layer (per expert e over its rows X, split LoRA, SwiGLU):
    h = X W_gu^T + s (X A_gu^T) B_gu^T,  act = silu(h[:, :I]) h[:, I:],
    y = act W_d^T + s (act A_d^T) B_d^T,  Y[t] = sum_j w[t, j] y[pos(t, j)]
following Unsloth's "Fine-tune MoE models 12x faster" (faster-moe page),
sections "What is torch._grouped_mm?", "Faster LoRA MoE training" and
"Implementation details".
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import MoeBaseGrads, MoeLoraGrads, MoeSaved, MoeShape, MoeWeights, ROUTER_IDS, check

__all__ = [
    "Shape", "moe_workspace_bytes", "moe_route", "moe_route_bwd", "moe_permute",
    "moe_permute_noalloc", "moe_grouped_lora_combine_bwd", "moe_grouped_lora_fwd_gather",
    "moe_grouped_lora_combine_bwd_gather",
    "moe_grouped_lora_fwd", "moe_unpermute_combine", "moe_unpermute_combine_bwd",
    "moe_grouped_lora_bwd", "moe_grouped_full_bwd", "moe_workspace_bytes_lean",
    "moe_grouped_lora_fwd_lean", "moe_grouped_lora_bwd_recompute", "moe_router_workspace_bytes",
    "moe_router_fwd", "moe_router_bwd", "moe_accumulate", "moe_merge_workspace_bytes",
    "moe_merge_lora", "kernel_timer", "ROUTER_IDS",
    "library_path",
]

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
_ABI_DTYPES = {"f32": _lib.MOE_F32, "bf16": _lib.MOE_BF16, "f16": _lib.MOE_F16}


def library_path() -> str:
    return _lib.LIB_PATH


@dataclass(frozen=True)
class Shape:
    T: int
    H: int
    I: int
    E: int
    k: int
    r: int
    dtype: str = "bf16"       # "bf16", "f16" or "f32"
    lora_scale: float = 1.0

    @property
    def N(self) -> int:
        return self.T * self.k

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    def c(self) -> MoeShape:
        return MoeShape(self.T, self.H, self.I, self.E, self.k, self.r,
                        _ABI_DTYPES[self.dtype], float(self.lora_scale))

    @classmethod
    def of(cls, cfg) -> "Shape":
        return cls(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.r, cfg.dtype, cfg.lora_scale)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, shape, dtype, name, optional=False):
    """Address of a contiguous GPU tensor of exactly `shape` and `dtype`."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(t, need, name):
    if need == 0:
        return ctypes.c_void_p(t.data_ptr()) if t is not None else None, 0
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor of >= {need} bytes")
    nbytes = t.numel() * t.element_size()
    return ctypes.c_void_p(t.data_ptr()), nbytes


def moe_workspace_bytes(shape: Shape):
    """(forward, backward, permute) workspace bytes for `shape`."""
    f, b, p = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    check(_lib.load().moe_workspace_bytes(ctypes.byref(shape.c()), ctypes.byref(f),
                                          ctypes.byref(b), ctypes.byref(p)),
          "moe_workspace_bytes")
    return f.value, b.value, p.value


def moe_route(logits, k, router, topk_ids, topk_w, stream=None):
    T, E = logits.shape
    check(_lib.load().moe_route(
        _ptr(logits, (T, E), torch.float32, "logits"), T, E, k, ROUTER_IDS[router],
        _ptr(topk_ids, (T, k), torch.int32, "topk_ids"),
        _ptr(topk_w, (T, k), torch.float32, "topk_w"), _stream(stream)), "moe_route")


def moe_route_bwd(logits, topk_ids, d_topk_w, k, router, d_logits, stream=None):
    T, E = logits.shape
    check(_lib.load().moe_route_bwd(
        _ptr(logits, (T, E), torch.float32, "logits"),
        _ptr(topk_ids, (T, k), torch.int32, "topk_ids"),
        _ptr(d_topk_w, (T, k), torch.float32, "d_topk_w"), T, E, k, ROUTER_IDS[router],
        _ptr(d_logits, (T, E), torch.float32, "d_logits"), _stream(stream)), "moe_route_bwd")


def moe_permute(shape: Shape, topk_ids, x, counts, offsets, sorted_pair, inv_pos, x_perm, ws,
                stream=None):
    _, _, need = moe_workspace_bytes(shape)
    wsp, wsb = _ws(ws, need, "ws")
    dt = shape.torch_dtype
    check(_lib.load().moe_permute(
        ctypes.byref(shape.c()),
        _ptr(topk_ids, (shape.T, shape.k), torch.int32, "topk_ids"),
        _ptr(x, (shape.T, shape.H), dt, "x", optional=x_perm is None),
        _ptr(counts, (shape.E,), torch.int32, "counts"),
        _ptr(offsets, (shape.E + 1,), torch.int32, "offsets"),
        _ptr(sorted_pair, (shape.N,), torch.int32, "sorted_pair"),
        _ptr(inv_pos, (shape.N,), torch.int32, "inv_pos"),
        _ptr(x_perm, (shape.N, shape.H), dt, "x_perm", optional=True),
        wsp, wsb, _stream(stream)), "moe_permute")


def moe_permute_noalloc(shape: Shape, topk_ids, x, counts, offsets, sorted_pair, inv_pos,
                        x_perm, stream=None):
    """moe_permute with its table in the library's own device array (no workspace)."""
    dt = shape.torch_dtype
    check(_lib.load().moe_permute_noalloc(
        ctypes.byref(shape.c()),
        _ptr(topk_ids, (shape.T, shape.k), torch.int32, "topk_ids"),
        _ptr(x, (shape.T, shape.H), dt, "x", optional=x_perm is None),
        _ptr(counts, (shape.E,), torch.int32, "counts"),
        _ptr(offsets, (shape.E + 1,), torch.int32, "offsets"),
        _ptr(sorted_pair, (shape.N,), torch.int32, "sorted_pair"),
        _ptr(inv_pos, (shape.N,), torch.int32, "inv_pos"),
        _ptr(x_perm, (shape.N, shape.H), dt, "x_perm", optional=True),
        _stream(stream)), "moe_permute_noalloc")


def _weights(shape: Shape, w: dict) -> MoeWeights:
    E, H, I, r, dt = shape.E, shape.H, shape.I, shape.r, shape.torch_dtype
    return MoeWeights(
        _ptr(w["w_gu"], (E, 2 * I, H), dt, "w_gu"), _ptr(w["a_gu"], (E, r, H), dt, "a_gu"),
        _ptr(w["b_gu"], (E, 2 * I, r), dt, "b_gu"), _ptr(w["w_d"], (E, H, I), dt, "w_d"),
        _ptr(w["a_d"], (E, r, I), dt, "a_d"), _ptr(w["b_d"], (E, H, r), dt, "b_d"))


def _saved(shape: Shape, s: dict, need_y=True, lean=False) -> MoeSaved:
    """lean: h and act are not part of `s` (activation-lean mode)."""
    N, H, I, r, dt = shape.N, shape.H, shape.I, shape.r, shape.torch_dtype
    return MoeSaved(
        _ptr(s.get("h"), (N, 2 * I), dt, "h", optional=lean),
        _ptr(s.get("act"), (N, I), dt, "act", optional=lean),
        _ptr(s["u_gu"], (N, r), dt, "u_gu"), _ptr(s["u_d"], (N, r), dt, "u_d"),
        _ptr(s.get("y_exp"), (N, H), dt, "y_exp", optional=not need_y))


def moe_grouped_lora_fwd(shape: Shape, x_perm, offsets, weights: dict, saved: dict, ws,
                         stream=None):
    need, _, _ = moe_workspace_bytes(shape)
    wsp, wsb = _ws(ws, need, "ws")
    w = _weights(shape, weights)
    s = _saved(shape, saved)
    check(_lib.load().moe_grouped_lora_fwd(
        ctypes.byref(shape.c()), _ptr(x_perm, (shape.N, shape.H), shape.torch_dtype, "x_perm"),
        _ptr(offsets, (shape.E + 1,), torch.int32, "offsets"), ctypes.byref(w), ctypes.byref(s),
        wsp, wsb, _stream(stream)), "moe_grouped_lora_fwd")


def moe_workspace_bytes_lean(shape: Shape):
    """(forward, backward) workspace bytes of the activation-lean calls."""
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    check(_lib.load().moe_workspace_bytes_lean(ctypes.byref(shape.c()), ctypes.byref(f),
                                               ctypes.byref(b)), "moe_workspace_bytes_lean")
    return f.value, b.value


def moe_grouped_lora_fwd_lean(shape: Shape, x_perm, offsets, weights: dict, saved: dict, ws,
                              stream=None):
    """moe_grouped_lora_fwd that keeps h and act in `ws`; saved needs u_gu, u_d, y_exp."""
    need, _ = moe_workspace_bytes_lean(shape)
    wsp, wsb = _ws(ws, need, "ws")
    w = _weights(shape, weights)
    s = _saved(shape, saved, lean=True)
    check(_lib.load().moe_grouped_lora_fwd_lean(
        ctypes.byref(shape.c()), _ptr(x_perm, (shape.N, shape.H), shape.torch_dtype, "x_perm"),
        _ptr(offsets, (shape.E + 1,), torch.int32, "offsets"), ctypes.byref(w), ctypes.byref(s),
        wsp, wsb, _stream(stream)), "moe_grouped_lora_fwd_lean")


def moe_grouped_lora_fwd_gather(shape: Shape, x, sorted_pair, offsets, weights: dict,
                                saved: dict, ws, lean=False, stream=None):
    """moe_grouped_lora_fwd (lean: moe_grouped_lora_fwd_lean) reading the rows of
    x [T, H] in token order through sorted_pair instead of x_perm."""
    need = moe_workspace_bytes_lean(shape)[0] if lean else moe_workspace_bytes(shape)[0]
    wsp, wsb = _ws(ws, need, "ws")
    w = _weights(shape, weights)
    s = _saved(shape, saved, lean=lean)
    check(_lib.load().moe_grouped_lora_fwd_gather(
        ctypes.byref(shape.c()), _ptr(x, (shape.T, shape.H), shape.torch_dtype, "x"),
        _ptr(sorted_pair, (shape.N,), torch.int32, "sorted_pair"),
        _ptr(offsets, (shape.E + 1,), torch.int32, "offsets"), ctypes.byref(w), ctypes.byref(s),
        1 if lean else 0, wsp, wsb, _stream(stream)), "moe_grouped_lora_fwd_gather")


def moe_unpermute_combine(shape: Shape, y_perm, inv_pos, topk_w, y, stream=None):
    dt = shape.torch_dtype
    check(_lib.load().moe_unpermute_combine(
        ctypes.byref(shape.c()), _ptr(y_perm, (shape.N, shape.H), dt, "y_perm"),
        _ptr(inv_pos, (shape.N,), torch.int32, "inv_pos"),
        _ptr(topk_w, (shape.T, shape.k), torch.float32, "topk_w", optional=True),
        _ptr(y, (shape.T, shape.H), dt, "y"), _stream(stream)), "moe_unpermute_combine")


def moe_unpermute_combine_bwd(shape: Shape, dy, y_exp, inv_pos, topk_w, dy_perm, d_topk_w,
                              stream=None):
    dt = shape.torch_dtype
    check(_lib.load().moe_unpermute_combine_bwd(
        ctypes.byref(shape.c()), _ptr(dy, (shape.T, shape.H), dt, "dy"),
        _ptr(y_exp, (shape.N, shape.H), dt, "y_exp"),
        _ptr(inv_pos, (shape.N,), torch.int32, "inv_pos"),
        _ptr(topk_w, (shape.T, shape.k), torch.float32, "topk_w"),
        _ptr(dy_perm, (shape.N, shape.H), dt, "dy_perm"),
        _ptr(d_topk_w, (shape.T, shape.k), torch.float32, "d_topk_w"), _stream(stream)),
        "moe_unpermute_combine_bwd")


def _bwd_args(shape: Shape, dy_perm, x_perm, offsets, weights: dict, saved: dict, dx_perm,
              grads: dict, ws, lean=False, x_rows=None, dy_optional=False):
    need = moe_workspace_bytes_lean(shape)[1] if lean else moe_workspace_bytes(shape)[1]
    wsp, wsb = _ws(ws, need, "ws")
    E, H, I, r, dt = shape.E, shape.H, shape.I, shape.r, shape.torch_dtype
    w = _weights(shape, weights)
    s = _saved(shape, saved, need_y=False, lean=lean)
    g = MoeLoraGrads(_ptr(grads["da_gu"], (E, r, H), dt, "da_gu"),
                     _ptr(grads["db_gu"], (E, 2 * I, r), dt, "db_gu"),
                     _ptr(grads["da_d"], (E, r, I), dt, "da_d"),
                     _ptr(grads["db_d"], (E, H, r), dt, "db_d"))
    head = (ctypes.byref(shape.c()),
            _ptr(dy_perm, (shape.N, H), dt, "dy_perm", optional=dy_optional),
            _ptr(x_perm, (x_rows or shape.N, H), dt, "x" if x_rows else "x_perm"),
            _ptr(offsets, (E + 1,), torch.int32, "offsets"), ctypes.byref(w), ctypes.byref(s),
            _ptr(dx_perm, (shape.N, H), dt, "dx_perm"), ctypes.byref(g))
    return head, (w, s, g), wsp, wsb


def moe_grouped_lora_bwd(shape: Shape, dy_perm, x_perm, offsets, weights: dict, saved: dict,
                         dx_perm, grads: dict, ws, stream=None):
    head, keep, wsp, wsb = _bwd_args(shape, dy_perm, x_perm, offsets, weights, saved, dx_perm,
                                     grads, ws)
    check(_lib.load().moe_grouped_lora_bwd(*head, wsp, wsb, _stream(stream)),
          "moe_grouped_lora_bwd")


def moe_grouped_full_bwd(shape: Shape, dy_perm, x_perm, offsets, weights: dict, saved: dict,
                         dx_perm, grads: dict, base_grads: dict, ws, stream=None):
    """moe_grouped_lora_bwd plus the base-weight gradients dw_gu [E, 2I, H], dw_d [E, H, I]."""
    head, keep, wsp, wsb = _bwd_args(shape, dy_perm, x_perm, offsets, weights, saved, dx_perm,
                                     grads, ws)
    E, H, I, dt = shape.E, shape.H, shape.I, shape.torch_dtype
    b = MoeBaseGrads(_ptr(base_grads["dw_gu"], (E, 2 * I, H), dt, "dw_gu"),
                     _ptr(base_grads["dw_d"], (E, H, I), dt, "dw_d"))
    check(_lib.load().moe_grouped_full_bwd(*head, ctypes.byref(b), wsp, wsb, _stream(stream)),
          "moe_grouped_full_bwd")


def moe_grouped_lora_bwd_recompute(shape: Shape, dy_perm, x_perm, offsets, weights: dict,
                                   saved: dict, dx_perm, grads: dict, ws, base_grads=None,
                                   stream=None):
    """Backward of the activation-lean forward: recomputes h and act in `ws`.
    base_grads (dw_gu, dw_d) optional: full fine-tuning."""
    head, keep, wsp, wsb = _bwd_args(shape, dy_perm, x_perm, offsets, weights, saved, dx_perm,
                                     grads, ws, lean=True)
    b = None
    if base_grads is not None:
        E, H, I, dt = shape.E, shape.H, shape.I, shape.torch_dtype
        b = MoeBaseGrads(_ptr(base_grads["dw_gu"], (E, 2 * I, H), dt, "dw_gu"),
                         _ptr(base_grads["dw_d"], (E, H, I), dt, "dw_d"))
    check(_lib.load().moe_grouped_lora_bwd_recompute(
        *head, ctypes.byref(b) if b is not None else None, wsp, wsb, _stream(stream)),
        "moe_grouped_lora_bwd_recompute")


def moe_grouped_lora_combine_bwd(shape: Shape, dy, topk_w, sorted_pair, inv_pos, x_perm,
                                 offsets, weights: dict, saved: dict, dy_perm, dx_perm,
                                 grads: dict, d_topk_w, ws, base_grads=None, recompute=False,
                                 stream=None):
    """The combine backward folded into the experts' backward (G = w dY never
    formed, y_exp not read): writes dx_perm, the LoRA gradients (and
    base_grads when given), d_topk_w, and dy's permuted rows into dy_perm."""
    head, keep, wsp, wsb = _bwd_args(shape, dy_perm, x_perm, offsets, weights, saved, dx_perm,
                                     grads, ws, lean=recompute)
    shp, dyp, xp, off, w, sv, dxp, g = head
    T, k, N, H, E, I, dt = shape.T, shape.k, shape.N, shape.H, shape.E, shape.I, shape.torch_dtype
    b = None
    if base_grads is not None:
        b = MoeBaseGrads(_ptr(base_grads["dw_gu"], (E, 2 * I, H), dt, "dw_gu"),
                         _ptr(base_grads["dw_d"], (E, H, I), dt, "dw_d"))
    check(_lib.load().moe_grouped_lora_combine_bwd(
        shp, _ptr(dy, (T, H), dt, "dy"), _ptr(topk_w, (T, k), torch.float32, "topk_w"),
        _ptr(sorted_pair, (N,), torch.int32, "sorted_pair"),
        _ptr(inv_pos, (N,), torch.int32, "inv_pos"), xp, off, w, sv, 1 if recompute else 0,
        dyp, dxp, g, ctypes.byref(b) if b is not None else None,
        _ptr(d_topk_w, (T, k), torch.float32, "d_topk_w"), wsp, wsb, _stream(stream)),
        "moe_grouped_lora_combine_bwd")


def moe_grouped_lora_combine_bwd_gather(shape: Shape, dy, topk_w, sorted_pair, inv_pos, x,
                                        offsets, weights: dict, saved: dict, dy_perm, dx_perm,
                                        grads: dict, d_topk_w, ws, base_grads=None,
                                        recompute=False, stream=None):
    """moe_grouped_lora_combine_bwd reading the rows of x [T, H] in token order
    through sorted_pair instead of x_perm. dy_perm None: dY's rows are read the
    same way, with no permuted copy (not with base_grads, nor for H <= 32)."""
    head, keep, wsp, wsb = _bwd_args(shape, dy_perm, x, offsets, weights, saved, dx_perm,
                                     grads, ws, lean=recompute, x_rows=shape.T,
                                     dy_optional=True)
    shp, dyp, xp, off, w, sv, dxp, g = head
    T, k, N, H, E, I, dt = shape.T, shape.k, shape.N, shape.H, shape.E, shape.I, shape.torch_dtype
    b = None
    if base_grads is not None:
        b = MoeBaseGrads(_ptr(base_grads["dw_gu"], (E, 2 * I, H), dt, "dw_gu"),
                         _ptr(base_grads["dw_d"], (E, H, I), dt, "dw_d"))
    check(_lib.load().moe_grouped_lora_combine_bwd_gather(
        shp, _ptr(dy, (T, H), dt, "dy"), _ptr(topk_w, (T, k), torch.float32, "topk_w"),
        _ptr(sorted_pair, (N,), torch.int32, "sorted_pair"),
        _ptr(inv_pos, (N,), torch.int32, "inv_pos"), xp, off, w, sv, 1 if recompute else 0,
        dyp, dxp, g, ctypes.byref(b) if b is not None else None,
        _ptr(d_topk_w, (T, k), torch.float32, "d_topk_w"), wsp, wsb, _stream(stream)),
        "moe_grouped_lora_combine_bwd_gather")


def _dtype_of(t, name):
    for key, dt in _TORCH_DTYPES.items():
        if t.dtype == dt:
            return key, dt
    raise ValueError(f"{name} must be float32, bfloat16 or float16, got {t.dtype}")


def moe_router_workspace_bytes(T: int, H: int, E: int, dtype: str) -> int:
    n = ctypes.c_size_t()
    check(_lib.load().moe_router_workspace_bytes(T, H, E, _ABI_DTYPES[dtype], ctypes.byref(n)),
          "moe_router_workspace_bytes")
    return n.value


def moe_router_fwd(x, w_r, logits, ws, stream=None):
    """logits [T, E] float32 = x [T, H] W_r [E, H]^T (frozen router projection)."""
    T, H = x.shape
    E = w_r.shape[0]
    key, dt = _dtype_of(x, "x")
    wsp, wsb = _ws(ws, moe_router_workspace_bytes(T, H, E, key), "ws")
    check(_lib.load().moe_router_fwd(
        _ptr(x, (T, H), dt, "x"), _ptr(w_r, (E, H), dt, "w_r"), T, H, E, _ABI_DTYPES[key],
        _ptr(logits, (T, E), torch.float32, "logits"), wsp, wsb, _stream(stream)),
        "moe_router_fwd")


def moe_router_bwd(d_logits, w_r, dx, ws, stream=None):
    """dx [T, H] += d_logits [T, E] W_r [E, H] (the router projection's input gradient)."""
    T, H = dx.shape
    E = w_r.shape[0]
    key, dt = _dtype_of(dx, "dx")
    wsp, wsb = _ws(ws, moe_router_workspace_bytes(T, H, E, key), "ws")
    check(_lib.load().moe_router_bwd(
        _ptr(d_logits, (T, E), torch.float32, "d_logits"), _ptr(w_r, (E, H), dt, "w_r"),
        T, H, E, _ABI_DTYPES[key], _ptr(dx, (T, H), dt, "dx"), wsp, wsb, _stream(stream)),
        "moe_router_bwd")


def moe_accumulate(src, dst, stream=None):
    """dst += src, element-wise (float32 sum, one rounding)."""
    key, dt = _dtype_of(dst, "dst")
    check(_lib.load().moe_accumulate(
        _ABI_DTYPES[key], dst.numel(), _ptr(src, tuple(dst.shape), dt, "src"),
        _ptr(dst, tuple(dst.shape), dt, "dst"), _stream(stream)), "moe_accumulate")


def moe_merge_workspace_bytes(shape: Shape) -> int:
    n = ctypes.c_size_t()
    check(_lib.load().moe_merge_workspace_bytes(ctypes.byref(shape.c()), ctypes.byref(n)),
          "moe_merge_workspace_bytes")
    return n.value


def moe_merge_lora(shape: Shape, weights: dict, w_gu_merged=None, w_d_merged=None, ws=None,
                   stream=None):
    """Merged export: w_gu_merged = w_gu + s b_gu a_gu, w_d_merged = w_d + s b_d a_d, per
    expert. Either output may be None (skipped) or the base weight itself (in place)."""
    E, H, I, dt = shape.E, shape.H, shape.I, shape.torch_dtype
    wsp, wsb = _ws(ws, moe_merge_workspace_bytes(shape), "ws")
    check(_lib.load().moe_merge_lora(
        ctypes.byref(shape.c()), ctypes.byref(_weights(shape, weights)),
        _ptr(w_gu_merged, (E, 2 * I, H), dt, "w_gu_merged", optional=True),
        _ptr(w_d_merged, (E, H, I), dt, "w_d_merged", optional=True), wsp, wsb,
        _stream(stream)), "moe_merge_lora")


class kernel_timer:
    """Per-kernel HIP-event timer of the library (see moe_kernel_timer_* in the header).

    with kernel_timer() as kt:
        ...launches...
    torch.cuda.synchronize(); kt.read("gate_up_fwd") -> (total_ms, launches)

    only: names of the kernels to time (default: all of them).
    """

    def __init__(self, only=None):
        self.mask = 0xFFFFFFFF if only is None else sum(1 << _lib.KERNEL_IDS[n] for n in only)

    def __enter__(self):
        lib = _lib.load()
        check(lib.moe_kernel_timer_reset(), "moe_kernel_timer_reset")
        check(lib.moe_kernel_timer_select(self.mask), "moe_kernel_timer_select")
        check(lib.moe_kernel_timer_enable(1), "moe_kernel_timer_enable")
        return self

    def __exit__(self, *exc):
        lib = _lib.load()
        check(lib.moe_kernel_timer_enable(0), "moe_kernel_timer_enable")
        check(lib.moe_kernel_timer_select(0xFFFFFFFF), "moe_kernel_timer_select")
        return False

    @staticmethod
    def read(name: str):
        ms, n = ctypes.c_double(), ctypes.c_int32()
        check(_lib.load().moe_kernel_timer_read(_lib.KERNEL_IDS[name], ctypes.byref(ms),
                                                ctypes.byref(n)), "moe_kernel_timer_read")
        return ms.value, n.value

    @staticmethod
    def reset():
        check(_lib.load().moe_kernel_timer_reset(), "moe_kernel_timer_reset")


# Load at import when the library is built; if it is not (for instance while
# `python -m mixture_experts_lora_amd.build` runs), every entry point raises
# on first use: there is no fallback implementation.
try:
    _lib.load()
except RuntimeError:
    pass

from .layer import (LayerScratch, MoELoRABlock, MoELoRAChunkedLayer, MoELoRAFunction,  # noqa: E402
                    MoELoRALayer)

__all__ += ["LayerScratch", "MoELoRABlock", "MoELoRAChunkedLayer", "MoELoRALayer",
            "MoELoRAFunction"]
