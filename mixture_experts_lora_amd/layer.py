"""The whole MoE-LoRA layer as a sequence of C-ABI calls.

MoELoRALayer owns every buffer of one layer shape (allocated once with torch,
so nothing is allocated inside a step) and issues, on torch's current stream:

  forward   moe_route -> moe_permute (indices only) -> moe_grouped_lora_fwd_gather
            (the GEMMs read x's rows through sorted_pair) -> moe_unpermute_combine
  backward  moe_grouped_lora_combine_bwd_gather (the combine backward folded
            into the experts' backward: d_topk_w from the down backward, no G;
            the GEMMs read dY's rows through sorted_pair as well)
            -> moe_route_bwd -> moe_unpermute_combine (weights 1: dX_perm
            summed back to tokens)
  With gather_x=False, moe_permute also gathers x_perm and the calls without
  _gather read it. With fold_combine_bwd=False the backward runs the separate
  calls moe_unpermute_combine_bwd -> moe_route_bwd -> moe_grouped_lora_bwd
  (on x_perm), which read the expert outputs y_exp, so those are then kept
  from the forward.

MoELoRAFunction wraps the same calls as a torch.autograd.Function whose
gradients are dX, d logits and the four LoRA gradients (base weights frozen).

MoELoRAChunkedLayer runs the layer over its tokens in chunks that share one
set of workspaces (long contexts: the peak is one chunk's transients plus
every chunk's saved activations).

MoELoRABlock is the block a model sees: it starts from hidden states, makes the
logits with the frozen router projection (moe_router_fwd), runs the routed
layer, and adds an optional always-on shared expert (a dense LoRA SwiGLU MLP
over every token: the grouped calls with one expert, k = 1 and the tokens in
their own order); its backward adds the router's and the shared expert's input
gradients to dX (moe_router_bwd, moe_accumulate).
"""
from __future__ import annotations

import torch

from . import (Shape, moe_accumulate, moe_grouped_full_bwd, moe_grouped_lora_bwd,
               moe_grouped_lora_combine_bwd, moe_grouped_lora_combine_bwd_gather,
               moe_grouped_lora_fwd_gather,
               moe_grouped_lora_bwd_recompute, moe_grouped_lora_fwd, moe_grouped_lora_fwd_lean,
               moe_permute, moe_route, moe_route_bwd, moe_router_bwd, moe_router_fwd,
               moe_router_workspace_bytes, moe_unpermute_combine, moe_unpermute_combine_bwd,
               moe_workspace_bytes, moe_workspace_bytes_lean)

WEIGHT_NAMES = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")
GRAD_NAMES = ("da_gu", "db_gu", "da_d", "db_d")


class LayerScratch:
    """Buffers a layer needs only while one of its calls runs: the workspace
    shared by forward and backward, the permute workspace, the permuted
    gradient rows (G and dX_perm), d_topk_w and, in the activation-lean mode
    with x_perm (x_perm_rows), x_perm (the backward gathers it again). Several
    layers or chunks that run
    one after another can share one LayerScratch; it is sized for the largest
    shape passed in and handed out as views."""

    def __init__(self, shapes, recompute: bool, device="cuda", x_perm_rows: bool = True):
        shapes = list(shapes)
        es = max(s.torch_dtype.itemsize for s in shapes)
        ws = perm = rows = tk = 0
        for sh in shapes:
            f, b, pm = moe_workspace_bytes(sh)
            if recompute:
                f, b = moe_workspace_bytes_lean(sh)
            ws, perm = max(ws, f, b), max(perm, pm)
            rows, tk = max(rows, sh.N * sh.H), max(tk, sh.T * sh.k)
        self.recompute = recompute
        u8 = dict(device=device, dtype=torch.uint8)
        self.ws = torch.empty(max(ws, 1), **u8)
        self.ws_perm = torch.empty(max(perm, 1), **u8)
        nrow = 3 if recompute and x_perm_rows else 2          # G, dX_perm (+ x_perm)
        self.rows = torch.empty(max(nrow * rows * es, 1), **u8)
        self.rows_each = rows * es
        self.d_topk_w = torch.empty(max(tk, 1), device=device, dtype=torch.float32)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.ws, self.ws_perm, self.rows, self.d_topk_w))

    def row_view(self, i: int, shape: Shape):
        n = shape.N * shape.H * shape.torch_dtype.itemsize
        b = self.rows[i * self.rows_each: i * self.rows_each + n]
        return b.view(shape.torch_dtype).view(shape.N, shape.H)


def _gatherable(shape: Shape) -> bool:
    """The GEMMs read x's rows through sorted_pair when x is below 2 GiB."""
    return shape.T * shape.H * shape.torch_dtype.itemsize < (1 << 31)


class MoELoRALayer:
    """full_ft=True also computes the base-weight gradients (full fine-tuning).
    recompute=True is the activation-lean mode: h and act are not kept between
    forward and backward (they live in the forward workspace and are recomputed
    in the backward's), and neither is x_perm (the backward gathers it again
    from x, so backward() needs x).

    fold_combine_bwd=True (the default) runs the combine backward inside the
    experts' backward, so the expert outputs y_exp are a forward transient
    (held in the scratch rows the backward later uses for dY's rows) rather
    than a saved activation.

    gather_x=True (with fold_combine_bwd, for x below 2 GiB): the expert GEMMs
    read x's rows in token order through sorted_pair, so x_perm is never
    formed (no gather pass, nothing of it held); backward() needs x. None (the
    default) is True without full_ft: the base-weight gradient dW_gu = dH^T X
    runs faster on x_perm (gpt-oss-20b shape on MI355X: 6.06 against 6.25 ms
    per full fine-tuning step).
    gather_dy=True (the default; with gather_x, not with full_ft, for H > 32):
    the backward's GEMMs read dY's rows the same way instead of a copy of them
    in expert order.

    scratch: a LayerScratch to share with other layers or chunks (one is made
    when None). out: optional views {"y", "dx", "d_logits"} to write the
    outputs into (a chunk writes its rows of the whole layer's outputs).
    grads, base_grads: optional gradient buffers to write into."""

    def __init__(self, shape: Shape, router: str, device="cuda", full_ft: bool = False,
                 recompute: bool = False, scratch: LayerScratch | None = None,
                 out: dict | None = None, grads: dict | None = None,
                 base_grads: dict | None = None, fold_combine_bwd: bool = True,
                 gather_x: bool | None = None, gather_dy: bool = True):
        self.shape, self.router, self.full_ft, self.recompute = shape, router, full_ft, recompute
        self.fold = fold_combine_bwd
        if gather_x is None:
            gather_x = not full_ft
        self.gather = gather_x and fold_combine_bwd and _gatherable(shape)
        T, H, I, E, k, r, N = shape.T, shape.H, shape.I, shape.E, shape.k, shape.r, shape.N
        dt = shape.torch_dtype
        z = lambda *s, dtype=dt: torch.empty(s, device=device, dtype=dtype)  # noqa: E731
        i32, f32 = torch.int32, torch.float32
        if scratch is None:
            scratch = LayerScratch([shape], recompute, device, x_perm_rows=not self.gather)
        assert scratch.recompute == recompute
        self.scratch = scratch
        self.topk_ids, self.topk_w = z(T, k, dtype=i32), z(T, k, dtype=f32)
        self.counts, self.offsets = z(E, dtype=i32), z(E + 1, dtype=i32)
        self.sorted_pair, self.inv_pos = z(N, dtype=i32), z(N, dtype=i32)
        if self.gather:
            self.x_perm = None
        else:
            self.x_perm = scratch.row_view(2, shape) if recompute else z(N, H)
        self.saved = {"u_gu": z(N, r), "u_d": z(N, r)}
        if not recompute:
            self.saved.update(h=z(N, 2 * I), act=z(N, I))
        if self.fold:
            # forward transient: consumed by the combine, then the rows hold dY's
            self.y_exp = scratch.row_view(0, shape)
        else:
            self.y_exp = self.saved["y_exp"] = z(N, H)
        out = out or {}
        self.y = out["y"] if "y" in out else z(T, H)
        self.dx = out["dx"] if "dx" in out else z(T, H)
        self.d_logits = out["d_logits"] if "d_logits" in out else z(T, E, dtype=f32)
        # dY's rows in expert order (not formed when the GEMMs read dY in place)
        self.gather_dy = self.gather and gather_dy and not full_ft and shape.H > 32
        self.dy_perm = None if self.gather_dy else scratch.row_view(0, shape)
        self.dx_perm = scratch.row_view(1, shape)
        self.d_topk_w = scratch.d_topk_w[:T * k].view(T, k)
        self.grads = grads if grads is not None else {
            "da_gu": z(E, r, H), "db_gu": z(E, 2 * I, r), "da_d": z(E, r, I), "db_d": z(E, H, r)}
        self.base_grads = None
        if full_ft:
            self.base_grads = base_grads if base_grads is not None else {
                "dw_gu": z(E, 2 * I, H), "dw_d": z(E, H, I)}
        self.ws_fwd = self.ws_bwd = scratch.ws
        self.ws_perm = scratch.ws_perm

    def saved_bytes(self) -> int:
        """Bytes held from forward to backward: the saved activations and, unless
        the backward gathers it again, x_perm (the routing results and indices
        aside)."""
        t = list(self.saved.values()) + ([] if self.recompute or self.gather else [self.x_perm])
        return sum(v.numel() * v.element_size() for v in t)

    def _permute(self, x, stream):
        s = self.shape
        moe_permute(s, self.topk_ids, x, self.counts, self.offsets, self.sorted_pair,
                    self.inv_pos, self.x_perm, self.ws_perm, stream)

    def forward(self, x, logits, weights: dict, stream=None):
        s = self.shape
        moe_route(logits, s.k, self.router, self.topk_ids, self.topk_w, stream)
        self._permute(x, stream)
        saved = {**self.saved, "y_exp": self.y_exp}
        if self.gather:
            moe_grouped_lora_fwd_gather(s, x, self.sorted_pair, self.offsets, weights, saved,
                                        self.ws_fwd, lean=self.recompute, stream=stream)
        else:
            fwd = moe_grouped_lora_fwd_lean if self.recompute else moe_grouped_lora_fwd
            fwd(s, self.x_perm, self.offsets, weights, saved, self.ws_fwd, stream)
        moe_unpermute_combine(s, self.y_exp, self.inv_pos, self.topk_w, self.y, stream)
        return self.y

    def backward(self, dy, logits, weights: dict, stream=None, x=None):
        s = self.shape
        if self.gather:
            if x is None:
                raise ValueError("the backward reads x's rows through sorted_pair: pass x")
        elif self.recompute:
            if x is None:
                raise ValueError("the activation-lean backward gathers x_perm again: pass x")
            self._permute(x, stream)   # same routing, so the same permutation and rows
        if self.fold:
            bwd = moe_grouped_lora_combine_bwd_gather if self.gather else moe_grouped_lora_combine_bwd
            bwd(s, dy, self.topk_w, self.sorted_pair, self.inv_pos,
                x if self.gather else self.x_perm, self.offsets, weights, self.saved,
                self.dy_perm, self.dx_perm, self.grads, self.d_topk_w, self.ws_bwd,
                base_grads=self.base_grads, recompute=self.recompute, stream=stream)
            moe_route_bwd(logits, self.topk_ids, self.d_topk_w, s.k, self.router, self.d_logits,
                          stream)
            moe_unpermute_combine(s, self.dx_perm, self.inv_pos, None, self.dx, stream)
            return self.dx, self.d_logits, self.grads
        moe_unpermute_combine_bwd(s, dy, self.y_exp, self.inv_pos, self.topk_w,
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
        return self.backward(dy, logits, weights, stream, x=x)


class MoELoRAChunkedLayer:
    """The layer over its T tokens in `chunks` consecutive chunks, for long
    contexts: every output row depends only on its own token, so each chunk
    runs the same calls on its rows (writing its rows of Y, dX and d logits,
    which are bit-identical to the unchunked layer's), and only the weight
    gradients, sums over all rows, are added up across chunks (float32 sum,
    one rounding per chunk). Saved activations stay per chunk; the workspaces
    and the permuted gradient rows are sized for one chunk and shared, which
    is what lowers the peak."""

    def __init__(self, shape: Shape, router: str, chunks: int, device="cuda",
                 full_ft: bool = False, recompute: bool = False, gather_x: bool | None = None,
                 gather_dy: bool = True):
        if chunks < 1 or chunks > shape.T:
            raise ValueError(f"chunks must be in [1, T], got {chunks}")
        self.shape, self.router, self.chunks = shape, router, chunks
        self.full_ft, self.recompute = full_ft, recompute
        T, H, E = shape.T, shape.H, shape.E
        dt = shape.torch_dtype
        bounds = [T * i // chunks for i in range(chunks + 1)]
        self.bounds = list(zip(bounds[:-1], bounds[1:]))
        shapes = [Shape(hi - lo, shape.H, shape.I, shape.E, shape.k, shape.r, shape.dtype,
                        shape.lora_scale) for lo, hi in self.bounds]
        if gather_x is None:
            gather_x = not full_ft
        gather = gather_x and all(_gatherable(sh) for sh in shapes)
        self.scratch = LayerScratch(shapes, recompute, device, x_perm_rows=not gather)
        self.y = torch.empty(T, H, device=device, dtype=dt)
        self.dx = torch.empty(T, H, device=device, dtype=dt)
        self.d_logits = torch.empty(T, E, device=device, dtype=torch.float32)
        # chunk 0 writes the gradients; every other chunk writes into one
        # shared spare set, which is then added in
        self.parts = []
        spare = None
        for i, ((lo, hi), sh) in enumerate(zip(self.bounds, shapes)):
            out = {"y": self.y[lo:hi], "dx": self.dx[lo:hi], "d_logits": self.d_logits[lo:hi]}
            g = None if i < 2 else spare
            part = MoELoRALayer(sh, router, device, full_ft, recompute, self.scratch, out,
                                grads=None if g is None else g[0],
                                base_grads=None if g is None else g[1], gather_x=gather,
                                gather_dy=gather_dy)
            if i == 1:
                spare = (part.grads, part.base_grads)
            self.parts.append(part)
        self.grads = self.parts[0].grads
        self.base_grads = self.parts[0].base_grads

    def saved_bytes(self) -> int:
        return sum(p.saved_bytes() for p in self.parts)

    def forward(self, x, logits, weights: dict, stream=None):
        for (lo, hi), p in zip(self.bounds, self.parts):
            p.forward(x[lo:hi], logits[lo:hi], weights, stream)
        return self.y

    def backward(self, dy, logits, weights: dict, stream=None, x=None):
        for i, ((lo, hi), p) in enumerate(zip(self.bounds, self.parts)):
            p.backward(dy[lo:hi], logits[lo:hi], weights, stream,
                       x=None if x is None else x[lo:hi])
            if i > 0:
                for n, g in p.grads.items():
                    moe_accumulate(g, self.grads[n], stream)
                if p.base_grads is not None:
                    for n, g in p.base_grads.items():
                        moe_accumulate(g, self.base_grads[n], stream)
        return self.dx, self.d_logits, self.grads

    def step(self, x, logits, dy, weights: dict, stream=None):
        self.forward(x, logits, weights, stream)
        return self.backward(dy, logits, weights, stream, x=x)


def _one_expert(w: dict) -> dict:
    """A single expert's weights as the stacked [1, ...] tensors the grouped calls take."""
    return {n: v.unsqueeze(0) for n, v in w.items()}


class _DenseExpertBuffers:
    """Saved activations, gradients and workspace of one expert run over all
    tokens (the grouped calls with E = 1, k = 1)."""

    def __init__(self, shape: Shape, device, full_ft: bool, recompute: bool):
        T, H, I, r = shape.T, shape.H, shape.I, shape.r
        z = lambda *s: torch.empty(s, device=device, dtype=shape.torch_dtype)  # noqa: E731
        self.full_ft, self.recompute = full_ft, recompute
        self.saved = {"u_gu": z(T, r), "u_d": z(T, r), "y_exp": z(T, H)}
        if not recompute:
            self.saved.update(h=z(T, 2 * I), act=z(T, I))
        self.grads = {"da_gu": z(1, r, H), "db_gu": z(1, 2 * I, r), "da_d": z(1, r, I),
                      "db_d": z(1, H, r)}
        self.base_grads = {"dw_gu": z(1, 2 * I, H), "dw_d": z(1, H, I)} if full_ft else None
        fwd, bwd, _ = moe_workspace_bytes(shape)
        if recompute:
            fwd, bwd = moe_workspace_bytes_lean(shape)
        self.ws_fwd = self.ws_bwd = torch.empty(max(fwd, bwd, 1), device=device,
                                                dtype=torch.uint8)


class MoELoRABlock:
    """Router projection + routed MoE-LoRA layer + optional shared expert.

    shared_I: intermediate width of the shared expert (None: no shared expert).
    The shared expert carries its own LoRA adapters of rank shape.r and the
    same scale; its weights are passed as a dict of w_gu [2 shared_I, H],
    a_gu, b_gu, w_d [H, shared_I], a_d, b_d. full_ft and recompute apply to
    the routed and the shared experts alike."""

    def __init__(self, shape: Shape, router: str, shared_I: int | None = None, device="cuda",
                 full_ft: bool = False, recompute: bool = False):
        self.shape, self.shared_I = shape, shared_I
        self.routed = MoELoRALayer(shape, router, device, full_ft, recompute)
        T, H, E = shape.T, shape.H, shape.E
        self.logits = torch.empty(T, E, device=device, dtype=torch.float32)
        self.ws_router = torch.empty(max(moe_router_workspace_bytes(T, H, E, shape.dtype), 1),
                                     device=device, dtype=torch.uint8)
        self.shared = None
        if shared_I:
            # one expert over all T tokens in token order: x is its own x_perm
            self.shared_shape = Shape(T, H, int(shared_I), 1, 1, shape.r, shape.dtype,
                                      shape.lora_scale)
            self.shared = _DenseExpertBuffers(self.shared_shape, device, full_ft, recompute)
            self.shared_offsets = torch.tensor([0, T], device=device, dtype=torch.int32)
            self.shared_dx = torch.empty(T, H, device=device, dtype=shape.torch_dtype)

    def forward(self, x, w_r, weights: dict, shared_weights: dict | None = None, stream=None):
        moe_router_fwd(x, w_r, self.logits, self.ws_router, stream)
        y = self.routed.forward(x, self.logits, weights, stream)
        if self.shared is not None:
            L, sh = self.shared, self.shared_shape
            fwd = moe_grouped_lora_fwd_lean if L.recompute else moe_grouped_lora_fwd
            fwd(sh, x, self.shared_offsets, _one_expert(shared_weights), L.saved, L.ws_fwd,
                stream)
            moe_accumulate(L.saved["y_exp"], y, stream)
        return y

    def backward(self, dy, x, w_r, weights: dict, shared_weights: dict | None = None,
                 stream=None):
        """Returns (dx, d_logits, routed LoRA grads, shared LoRA grads or None)."""
        dx, dl, g = self.routed.backward(dy, self.logits, weights, stream, x=x)
        moe_router_bwd(dl, w_r, dx, self.ws_router, stream)
        if self.shared is None:
            return dx, dl, g, None
        L, sh = self.shared, self.shared_shape
        shared_weights = _one_expert(shared_weights)
        if L.recompute:
            moe_grouped_lora_bwd_recompute(sh, dy, x, self.shared_offsets, shared_weights,
                                           L.saved, self.shared_dx, L.grads, L.ws_bwd,
                                           L.base_grads, stream)
        elif L.full_ft:
            moe_grouped_full_bwd(sh, dy, x, self.shared_offsets, shared_weights, L.saved,
                                 self.shared_dx, L.grads, L.base_grads, L.ws_bwd, stream)
        else:
            moe_grouped_lora_bwd(sh, dy, x, self.shared_offsets, shared_weights, L.saved,
                                 self.shared_dx, L.grads, L.ws_bwd, stream)
        moe_accumulate(self.shared_dx, dx, stream)
        return dx, dl, g, {n: v[0] for n, v in L.grads.items()}

    def step(self, x, w_r, dy, weights: dict, shared_weights: dict | None = None, stream=None):
        self.forward(x, w_r, weights, shared_weights, stream)
        return self.backward(dy, x, w_r, weights, shared_weights, stream)


class MoELoRAFunction(torch.autograd.Function):
    """Y = layer(x, logits); gradients for x, logits and the LoRA A/B. The base
    weights are frozen unless w_gu or w_d requires grad (full fine-tuning), in
    which case their gradients are computed too."""

    @staticmethod
    def forward(ctx, x, logits, w_gu, a_gu, b_gu, w_d, a_d, b_d, router, k, lora_scale=1.0):
        T, H = x.shape
        E, r = logits.shape[1], a_gu.shape[1]
        I = w_gu.shape[1] // 2
        dtype = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[x.dtype]
        shape = Shape(T, H, I, E, k, r, dtype, lora_scale)
        full = bool(ctx.needs_input_grad[2] or ctx.needs_input_grad[5])
        layer = MoELoRALayer(shape, router, device=x.device, full_ft=full)
        weights = dict(zip(WEIGHT_NAMES, (w_gu, a_gu, b_gu, w_d, a_d, b_d)))
        x = x.contiguous()
        y = layer.forward(x, logits.contiguous(), weights).clone()
        ctx.layer, ctx.weights, ctx.logits, ctx.x = layer, weights, logits.contiguous(), x
        return y

    @staticmethod
    def backward(ctx, dy):
        layer = ctx.layer
        dx, dl, g = layer.backward(dy.contiguous(), ctx.logits, ctx.weights, x=ctx.x)
        bg = layer.base_grads
        dw_gu = bg["dw_gu"].clone() if bg is not None and ctx.needs_input_grad[2] else None
        dw_d = bg["dw_d"].clone() if bg is not None and ctx.needs_input_grad[5] else None
        return (dx.clone(), dl.clone(), dw_gu, g["da_gu"].clone(), g["db_gu"].clone(), dw_d,
                g["da_d"].clone(), g["db_d"].clone(), None, None, None)
