"""The whole MoE-LoRA layer as a sequence of C-ABI calls.

MoELoRALayer owns every buffer of one layer shape (allocated once with torch,
so nothing is allocated inside a step) and issues, on torch's current stream:

  forward   moe_route -> moe_permute (+ gather) -> moe_grouped_lora_fwd
            -> moe_unpermute_combine
  backward  moe_unpermute_combine_bwd -> moe_route_bwd -> moe_grouped_lora_bwd
            -> moe_unpermute_combine (weights 1: dX_perm summed back to tokens)

MoELoRAFunction wraps the same calls as a torch.autograd.Function whose
gradients are dX, d logits and the four LoRA gradients (base weights frozen).
"""
from __future__ import annotations

import torch

from . import (Shape, moe_grouped_full_bwd, moe_grouped_lora_bwd, moe_grouped_lora_bwd_recompute,
               moe_grouped_lora_fwd, moe_grouped_lora_fwd_lean, moe_permute, moe_route,
               moe_route_bwd, moe_unpermute_combine, moe_unpermute_combine_bwd,
               moe_workspace_bytes, moe_workspace_bytes_lean)

WEIGHT_NAMES = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")
GRAD_NAMES = ("da_gu", "db_gu", "da_d", "db_d")


class MoELoRALayer:
    """full_ft=True also computes the base-weight gradients (full fine-tuning).
    recompute=True is the activation-lean mode: h and act are not kept between
    forward and backward (they live in the forward workspace and are recomputed
    in the backward's)."""

    def __init__(self, shape: Shape, router: str, device="cuda", full_ft: bool = False,
                 recompute: bool = False):
        self.shape, self.router, self.full_ft, self.recompute = shape, router, full_ft, recompute
        T, H, I, E, k, r, N = shape.T, shape.H, shape.I, shape.E, shape.k, shape.r, shape.N
        dt = shape.torch_dtype
        z = lambda *s, dtype=dt: torch.empty(s, device=device, dtype=dtype)  # noqa: E731
        i32, f32 = torch.int32, torch.float32
        self.topk_ids, self.topk_w = z(T, k, dtype=i32), z(T, k, dtype=f32)
        self.counts, self.offsets = z(E, dtype=i32), z(E + 1, dtype=i32)
        self.sorted_pair, self.inv_pos = z(N, dtype=i32), z(N, dtype=i32)
        self.x_perm = z(N, H)
        self.saved = {"u_gu": z(N, r), "u_d": z(N, r), "y_exp": z(N, H)}
        if not recompute:
            self.saved.update(h=z(N, 2 * I), act=z(N, I))
        self.y = z(T, H)
        self.dy_perm, self.d_topk_w, self.d_logits = z(N, H), z(T, k, dtype=f32), z(T, E, dtype=f32)
        self.dx_perm, self.dx = z(N, H), z(T, H)
        self.grads = {"da_gu": z(E, r, H), "db_gu": z(E, 2 * I, r), "da_d": z(E, r, I),
                      "db_d": z(E, H, r)}
        self.base_grads = ({"dw_gu": z(E, 2 * I, H), "dw_d": z(E, H, I)} if full_ft else None)
        fwd, bwd, perm = moe_workspace_bytes(shape)
        if recompute:
            fwd, bwd = moe_workspace_bytes_lean(shape)
        # one scratch buffer serves both calls: they run one after the other on
        # the stream, and nothing in the forward's scratch is read by the backward
        self.ws_fwd = self.ws_bwd = z(max(fwd, bwd, 1), dtype=torch.uint8)
        self.ws_perm = z(max(perm, 1), dtype=torch.uint8)

    def saved_bytes(self) -> int:
        """Bytes held from forward to backward: the saved activations and x_perm
        (the routing results and indices aside)."""
        t = list(self.saved.values()) + [self.x_perm]
        return sum(v.numel() * v.element_size() for v in t)

    def forward(self, x, logits, weights: dict, stream=None):
        s = self.shape
        moe_route(logits, s.k, self.router, self.topk_ids, self.topk_w, stream)
        moe_permute(s, self.topk_ids, x, self.counts, self.offsets, self.sorted_pair,
                    self.inv_pos, self.x_perm, self.ws_perm, stream)
        fwd = moe_grouped_lora_fwd_lean if self.recompute else moe_grouped_lora_fwd
        fwd(s, self.x_perm, self.offsets, weights, self.saved, self.ws_fwd, stream)
        moe_unpermute_combine(s, self.saved["y_exp"], self.inv_pos, self.topk_w, self.y, stream)
        return self.y

    def backward(self, dy, logits, weights: dict, stream=None):
        s = self.shape
        moe_unpermute_combine_bwd(s, dy, self.saved["y_exp"], self.inv_pos, self.topk_w,
                                  self.dy_perm, self.d_topk_w, stream)
        moe_route_bwd(logits, self.topk_ids, self.d_topk_w, s.k, self.router, self.d_logits,
                      stream)
        if self.recompute:
            moe_grouped_lora_bwd_recompute(s, self.dy_perm, self.x_perm, self.offsets, weights,
                                           self.saved, self.dx_perm, self.grads, self.ws_bwd,
                                           self.base_grads, stream)
        elif self.full_ft:
            moe_grouped_full_bwd(s, self.dy_perm, self.x_perm, self.offsets, weights, self.saved,
                                 self.dx_perm, self.grads, self.base_grads, self.ws_bwd, stream)
        else:
            moe_grouped_lora_bwd(s, self.dy_perm, self.x_perm, self.offsets, weights, self.saved,
                                 self.dx_perm, self.grads, self.ws_bwd, stream)
        moe_unpermute_combine(s, self.dx_perm, self.inv_pos, None, self.dx, stream)
        return self.dx, self.d_logits, self.grads

    def step(self, x, logits, dy, weights: dict, stream=None):
        """One forward and backward pass."""
        self.forward(x, logits, weights, stream)
        return self.backward(dy, logits, weights, stream)


class MoELoRAFunction(torch.autograd.Function):
    """Y = layer(x, logits); gradients for x, logits and the LoRA A/B. The base
    weights are frozen unless w_gu or w_d requires grad (full fine-tuning), in
    which case their gradients are computed too."""

    @staticmethod
    def forward(ctx, x, logits, w_gu, a_gu, b_gu, w_d, a_d, b_d, router, k, lora_scale=1.0):
        T, H = x.shape
        E, r = logits.shape[1], a_gu.shape[1]
        I = w_gu.shape[1] // 2
        dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[x.dtype]
        shape = Shape(T, H, I, E, k, r, dtype, lora_scale)
        full = bool(ctx.needs_input_grad[2] or ctx.needs_input_grad[5])
        layer = MoELoRALayer(shape, router, device=x.device, full_ft=full)
        weights = dict(zip(WEIGHT_NAMES, (w_gu, a_gu, b_gu, w_d, a_d, b_d)))
        y = layer.forward(x.contiguous(), logits.contiguous(), weights).clone()
        ctx.layer, ctx.weights, ctx.logits = layer, weights, logits.contiguous()
        return y

    @staticmethod
    def backward(ctx, dy):
        layer = ctx.layer
        dx, dl, g = layer.backward(dy.contiguous(), ctx.logits, ctx.weights)
        bg = layer.base_grads
        dw_gu = bg["dw_gu"].clone() if bg is not None and ctx.needs_input_grad[2] else None
        dw_d = bg["dw_d"].clone() if bg is not None and ctx.needs_input_grad[5] else None
        return (dx.clone(), dl.clone(), dw_gu, g["da_gu"].clone(), g["db_gu"].clone(), dw_d,
                g["da_d"].clone(), g["db_d"].clone(), None, None, None)
