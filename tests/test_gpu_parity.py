"""GPU parity of the HIP layer against the CPU oracle, element by element.

The small layers (tests/../workloads PARITY_CONFIGS) span several tiles with
ragged tails in every dimension, zero-token experts, k = 1, k = E, r = 1,
r = 64, T = 1, lora_scale != 1 and all four router modes. Every output and
every saved activation is compared with the oracle run on host copies of the
same inputs; indices bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import PARITY_CONFIGS
from workloads.synth import to_numpy

from gpu_util import TOL, WEIGHTS, close, gpu_inputs, run_gpu, say

pytestmark = pytest.mark.gpu


def _mel():
    import mixture_experts_lora_amd as mel
    return mel


def _check_layer(name, seed, fold, gather=True, gather_dy=True):
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[parity] {name} seed={seed} fold={fold} gather={gather} gather_dy={gather_dy} "
        f"T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} r={cfg.r} {cfg.dtype} {cfg.router}")
    inp = gpu_inputs(cfg, seed)
    layer = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, fold_combine_bwd=fold,
                             gather_x=gather, gather_dy=gather_dy)
    # the GEMMs read x's rows through sorted_pair exactly when folded and
    # gathering, and dY's rows too when asked (H > 32)
    assert (layer.x_perm is None) == (fold and gather)
    assert (layer.dy_perm is None) == (fold and gather and gather_dy and cfg.H > 32)
    w = {n: inp[n] for n in WEIGHTS}
    layer.forward(inp["x"], inp["logits"], w)
    torch.cuda.synchronize()
    # the expert outputs before the backward reuses their rows (folded mode)
    y_exp = to_numpy(layer.y_exp)
    layer.backward(inp["dy"], inp["logits"], w, x=inp["x"])
    torch.cuda.synchronize()
    h = {n: to_numpy(v) for n, v in inp.items()}
    Y, g, c = oracle.layer_forward_backward(h["x"], h["logits"], h["dy"], h, cfg.k, cfg.router,
                                            cfg.lora_scale)
    tol = TOL[cfg.dtype]
    s = cfg.lora_scale
    # routing and permutation: exact
    np.testing.assert_array_equal(to_numpy(layer.topk_ids), c["ids"])
    np.testing.assert_array_equal(to_numpy(layer.counts), c["counts"])
    np.testing.assert_array_equal(to_numpy(layer.offsets), c["offsets"])
    np.testing.assert_array_equal(to_numpy(layer.sorted_pair), c["sorted_pair"])
    np.testing.assert_array_equal(to_numpy(layer.inv_pos), c["inv_pos"])
    if layer.x_perm is not None:
        np.testing.assert_array_equal(to_numpy(layer.x_perm),
                                      oracle.gather_rows(h["x"], c["sorted_pair"], cfg.k))
    close("topk_w", to_numpy(layer.topk_w), c["w"], 1e-5)
    # saved activations, rows in permuted order
    N = cfg.N
    ref = {n: np.zeros((N,) + v.shape[1:], np.float32)
           for n, v in next(iter(c["per_expert"].values())).items()}
    for e, f in c["per_expert"].items():
        lo, hi = c["offsets"][e], c["offsets"][e + 1]
        for n in ref:
            ref[n][lo:hi] = f[n]
    close("h", to_numpy(layer.saved["h"]), ref["h"], tol)
    close("act", to_numpy(layer.saved["act"]), ref["a"], tol)
    close("u_gu", to_numpy(layer.saved["u_gu"]), s * ref["u_gu"], tol)
    close("u_d", to_numpy(layer.saved["u_d"]), s * ref["u_d"], tol)
    close("y_exp", y_exp, ref["y"], tol)
    close("Y", to_numpy(layer.y), Y, tol)
    # backward
    close("d_topk_w", to_numpy(layer.d_topk_w), g["dw"], tol)
    close("d_logits", to_numpy(layer.d_logits), g["dlogits"], tol)
    close("dX", to_numpy(layer.dx), g["dx"], tol)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        close(n, to_numpy(layer.grads[n]), g[n], tol)
        dead = np.where(c["counts"] == 0)[0]
        assert (to_numpy(layer.grads[n])[dead] == 0).all()
    if fold:
        assert "y_exp" not in layer.saved


@pytest.mark.parametrize("name", list(PARITY_CONFIGS))
@pytest.mark.parametrize("seed", [0, 3407])
def test_layer_matches_oracle(name, seed):
    """The layer with the combine backward folded into the experts' backward
    and the GEMMs reading x's and dY's rows through sorted_pair
    (moe_grouped_lora_fwd_gather, moe_grouped_lora_combine_bwd_gather)."""
    _check_layer(name, seed, fold=True)


@pytest.mark.parametrize("name", list(PARITY_CONFIGS))
def test_layer_with_dy_copy_matches_oracle(name):
    """x's rows read through sorted_pair, dY's rows copied into expert order
    first (the gathered backward given dy_perm)."""
    _check_layer(name, 0, fold=True, gather_dy=False)


@pytest.mark.parametrize("name", ["tiny", "mini-bf16", "mini-skew", "mini-r1", "mini-f16",
                                  "mini-split", "mini-f32-split", "max-E-k"])
def test_layer_with_x_perm_matches_oracle(name):
    """The folded backward with x gathered into x_perm first
    (moe_grouped_lora_fwd / moe_grouped_lora_combine_bwd on x_perm)."""
    _check_layer(name, 0, fold=True, gather=False)


@pytest.mark.parametrize("name", list(PARITY_CONFIGS))
def test_layer_with_separate_combine_backward_matches_oracle(name):
    """The separate calls moe_unpermute_combine_bwd and moe_grouped_lora_bwd
    (G formed, y_exp kept from the forward)."""
    _check_layer(name, 0, fold=False)


@pytest.mark.parametrize("name", ["tiny", "mini-bf16", "mini-skew", "mini-f32", "mini-k1",
                                  "mini-renorm", "mini-f16", "mini-split", "mini-f32-split"])
@pytest.mark.parametrize("gather_x", [None, True])
def test_full_fine_tuning_base_grads(name, gather_x):
    """Full fine-tuning: dW_gu and dW_d against the oracle; every other output
    bit-identical to the LoRA-only backward (which reads x's and dY's rows
    through sorted_pair). gather_x None: x_perm (the default with full_ft);
    True: dW_gu reads x's rows through sorted_pair too."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[full-ft] {name} gather_x={gather_x}")
    inp = gpu_inputs(cfg, 5)
    full = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, full_ft=True, gather_x=gather_x)
    assert (full.x_perm is None) == bool(gather_x)
    full.step(inp["x"], inp["logits"], inp["dy"], {n: inp[n] for n in WEIGHTS})
    torch.cuda.synchronize()
    h = {n: to_numpy(v) for n, v in inp.items()}
    _, g, c = oracle.layer_forward_backward(h["x"], h["logits"], h["dy"], h, cfg.k, cfg.router,
                                            cfg.lora_scale, base_grads=True)
    tol = TOL[cfg.dtype]
    dead = np.where(c["counts"] == 0)[0]
    for n in ("dw_gu", "dw_d"):
        close(n, to_numpy(full.base_grads[n]), g[n], tol)
        assert (to_numpy(full.base_grads[n])[dead] == 0).all()
    lora = run_gpu(mel.MoELoRALayer, mel.Shape.of(cfg), cfg, inp)
    for a, b in [(full.dx, lora.dx), (full.d_logits, lora.d_logits)] + \
            [(full.grads[n], lora.grads[n]) for n in lora.grads]:
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["tiny", "mini-bf16", "mini-skew", "mini-r1", "mini-f32",
                                  "mini-f16-skew"])
@pytest.mark.parametrize("full_ft", [False, True])
@pytest.mark.parametrize("gather", ["x+dy", "x", "none"])
def test_recompute_mode_is_bit_identical(name, full_ft, gather):
    """Activation-lean mode (h and act recomputed in the backward by the same
    kernel): every output and gradient equals the saving mode's bit for bit,
    with x's (and dY's) rows read through sorted_pair or gathered into x_perm
    (the lean backward then gathers it again)."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[recompute] {name} full_ft={full_ft} gather={gather}")
    inp = gpu_inputs(cfg, 7)
    w = {n: inp[n] for n in WEIGHTS}
    gx, gdy = gather != "none", gather == "x+dy"
    a = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, full_ft=full_ft, gather_x=gx,
                         gather_dy=gdy)
    b = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, full_ft=full_ft, recompute=True,
                         gather_x=gx, gather_dy=gdy)
    a.step(inp["x"], inp["logits"], inp["dy"], w)
    b.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    assert "h" not in b.saved and "act" not in b.saved
    assert b.saved_bytes() < a.saved_bytes()
    pairs = [(a.y, b.y), (a.dx, b.dx), (a.d_logits, b.d_logits),
             (a.saved["u_gu"], b.saved["u_gu"]), (a.saved["u_d"], b.saved["u_d"])]
    pairs += [(a.grads[n], b.grads[n]) for n in a.grads]
    if full_ft:
        pairs += [(a.base_grads[n], b.base_grads[n]) for n in a.base_grads]
    for t1, t2 in pairs:
        assert torch.equal(t1, t2)


@pytest.mark.parametrize("name,chunks", [("tiny", 3), ("mini-bf16", 2), ("mini-skew", 4),
                                         ("mini-f32", 3), ("mini-T1", 1), ("mini-split", 5),
                                         ("mini-f16", 2)])
@pytest.mark.parametrize("recompute", [False, True])
def test_chunked_layer(name, chunks, recompute):
    """The layer in token chunks: Y, dX and d logits (per token) bit-identical
    to the unchunked layer; the LoRA gradients, summed over chunks, against
    the oracle."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[chunked] {name} chunks={chunks} recompute={recompute}")
    inp = gpu_inputs(cfg, 9)
    w = {n: inp[n] for n in WEIGHTS}
    a = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, recompute=recompute)
    b = mel.MoELoRAChunkedLayer(mel.Shape.of(cfg), cfg.router, chunks, recompute=recompute)
    a.step(inp["x"], inp["logits"], inp["dy"], w)
    b.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    for t1, t2 in [(a.y, b.y), (a.dx, b.dx), (a.d_logits, b.d_logits)]:
        assert torch.equal(t1, t2)
    h = {n: to_numpy(v) for n, v in inp.items()}
    _, g, _ = oracle.layer_forward_backward(h["x"], h["logits"], h["dy"], h, cfg.k, cfg.router,
                                            cfg.lora_scale)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        close(n, to_numpy(b.grads[n]), g[n], TOL[cfg.dtype])
    assert b.saved_bytes() == a.saved_bytes()


def test_chunked_full_fine_tuning():
    mel = _mel()
    cfg = PARITY_CONFIGS["mini-skew"]
    say("[chunked full-ft] mini-skew")
    inp = gpu_inputs(cfg, 10)
    b = mel.MoELoRAChunkedLayer(mel.Shape.of(cfg), cfg.router, 3, full_ft=True, recompute=True)
    b.step(inp["x"], inp["logits"], inp["dy"], {n: inp[n] for n in WEIGHTS})
    torch.cuda.synchronize()
    h = {n: to_numpy(v) for n, v in inp.items()}
    _, g, _ = oracle.layer_forward_backward(h["x"], h["logits"], h["dy"], h, cfg.k, cfg.router,
                                            cfg.lora_scale, base_grads=True)
    for n in ("dw_gu", "dw_d"):
        close(n, to_numpy(b.base_grads[n]), g[n], TOL[cfg.dtype])


def test_lean_backward_needs_x():
    mel = _mel()
    cfg = PARITY_CONFIGS["mini-bf16"]
    inp = gpu_inputs(cfg, 11)
    w = {n: inp[n] for n in WEIGHTS}
    layer = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, recompute=True)
    layer.forward(inp["x"], inp["logits"], w)
    with pytest.raises(ValueError):
        layer.backward(inp["dy"], inp["logits"], w)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["mini-bf16", "mini-skew", "tiny"])
def test_layer_is_deterministic(name):
    """Atomic-free kernels: two runs give bit-identical outputs."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[determinism] {name}")
    inp = gpu_inputs(cfg, 1)
    a = run_gpu(mel.MoELoRALayer, mel.Shape.of(cfg), cfg, inp)
    b = run_gpu(mel.MoELoRALayer, mel.Shape.of(cfg), cfg, inp)
    for t1, t2 in [(a.y, b.y), (a.dx, b.dx), (a.d_logits, b.d_logits)] + \
            [(a.grads[n], b.grads[n]) for n in a.grads]:
        assert torch.equal(t1, t2)


def test_autograd_function_matches_layer():
    mel = _mel()
    cfg = PARITY_CONFIGS["mini-bf16"]
    say("[autograd] mini-bf16")
    inp = gpu_inputs(cfg, 2)
    layer = run_gpu(mel.MoELoRALayer, mel.Shape.of(cfg), cfg, inp)
    x = inp["x"].clone().requires_grad_(True)
    lg = inp["logits"].clone().requires_grad_(True)
    ps = {n: inp[n].clone().requires_grad_(n[0] in "ab") for n in WEIGHTS}
    y = mel.MoELoRAFunction.apply(x, lg, *[ps[n] for n in WEIGHTS], cfg.router, cfg.k,
                                  cfg.lora_scale)
    y.backward(inp["dy"])
    assert torch.equal(y, layer.y)
    assert torch.equal(x.grad, layer.dx)
    assert torch.equal(lg.grad, layer.d_logits)
    for n in ("a_gu", "b_gu", "a_d", "b_d"):
        assert torch.equal(ps[n].grad, layer.grads["d" + n])
    assert ps["w_gu"].grad is None and ps["w_d"].grad is None  # frozen: no base gradients


def test_autograd_function_full_fine_tuning():
    """With the base weights requiring grad, the autograd wrapper returns dW too."""
    mel = _mel()
    cfg = PARITY_CONFIGS["mini-bf16"]
    say("[autograd full-ft] mini-bf16")
    inp = gpu_inputs(cfg, 2)
    full = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, full_ft=True)
    full.step(inp["x"], inp["logits"], inp["dy"], {n: inp[n] for n in WEIGHTS})
    torch.cuda.synchronize()
    x = inp["x"].clone().requires_grad_(True)
    lg = inp["logits"].clone().requires_grad_(True)
    ps = {n: inp[n].clone().requires_grad_(True) for n in WEIGHTS}
    y = mel.MoELoRAFunction.apply(x, lg, *[ps[n] for n in WEIGHTS], cfg.router, cfg.k,
                                  cfg.lora_scale)
    y.backward(inp["dy"])
    assert torch.equal(x.grad, full.dx)
    assert torch.equal(ps["w_gu"].grad, full.base_grads["dw_gu"])
    assert torch.equal(ps["w_d"].grad, full.base_grads["dw_d"])


@pytest.mark.parametrize("name", ["mini-bf16", "mini-f16"])
def test_unaligned_weights(name):
    """Weights and x handed over as views that start 2 bytes past a 16-byte
    boundary. The 256-row expert GEMMs cannot read them in 16-byte pieces and
    take the buffer->LDS kernel with element-wise fills (the LoRA side
    products and gradients likewise fall back to element-wise fills and to
    their unfused kernels, and x's rows are fetched element by element through
    sorted_pair); every result against the oracle."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[unaligned] {name}")
    inp = gpu_inputs(cfg, 4)
    w = {}
    for n in WEIGHTS:
        t = inp[n]
        buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 16 != 0
        w[n] = v
    # x too: the GEMMs read its rows through sorted_pair (element-wise fills)
    xb = torch.empty(inp["x"].numel() + 8, dtype=inp["x"].dtype, device="cuda")
    x = xb[1:1 + inp["x"].numel()].view(inp["x"].shape)
    x.copy_(inp["x"])
    layer = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router)
    assert layer.x_perm is None
    layer.step(x, inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    h = {n: to_numpy(v) for n, v in inp.items()}
    Y, g, c = oracle.layer_forward_backward(h["x"], h["logits"], h["dy"], h, cfg.k, cfg.router,
                                            cfg.lora_scale)
    tol = TOL[cfg.dtype]
    np.testing.assert_array_equal(to_numpy(layer.sorted_pair), c["sorted_pair"])
    close("Y", to_numpy(layer.y), Y, tol)
    close("dX", to_numpy(layer.dx), g["dx"], tol)
    close("d_logits", to_numpy(layer.d_logits), g["dlogits"], tol)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        close(n, to_numpy(layer.grads[n]), g[n], tol)
    # and close to the aligned layer, whose kernels read the same values
    ref = run_gpu(mel.MoELoRALayer, mel.Shape.of(cfg), cfg, inp)
    close("Y vs aligned", to_numpy(layer.y), to_numpy(ref.y), tol)
