"""GPU parity of the router projection, the accumulate call and the whole MoE
block (router projection -> routed experts + shared expert) against the oracle.

- logits = x W_r^T: float32 accumulation on both sides; compared normwise at
  1e-5 (the products of bf16 inputs are exact in float32, so only the
  summation order differs).
- dx += d_logits W_r: checked on its own (dx starting at zero) at the layer
  tolerance, and as an update of a nonzero dx.
- accumulate: bit-exact (one float32 sum, one rounding, on both sides).
- block: the oracle routes on the GPU's float32 logits, so both sides take
  the same top-k decisions (the logits themselves are checked first); every
  output and gradient at the layer tolerances.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, PARITY_CONFIGS, make_block_inputs
from workloads.synth import to_numpy

from gpu_util import TOL, WEIGHTS, ExpertSlices, close, say

pytestmark = pytest.mark.gpu

ROUTER_SHAPES = [  # (T, H, E, dtype)
    (300, 584, 6, "bf16"), (129, 256, 8, "bf16"), (1, 64, 3, "bf16"), (640, 512, 64, "bf16"),
    (8192, 2880, 32, "bf16"), (16384, 2048, 128, "bf16"), (333, 200, 5, "f32"),
    (256, 256, 8, "f32"), (70, 136, 130, "f32"), (300, 584, 6, "f16"), (8192, 2880, 32, "f16"),
]


def _mel():
    import mixture_experts_lora_amd as mel
    return mel


@pytest.mark.parametrize("T,H,E,dtype", ROUTER_SHAPES)
def test_router_projection_and_its_input_gradient(T, H, E, dtype):
    mel = _mel()
    say(f"[router] T={T} H={H} E={E} {dtype}")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    g = torch.Generator(device="cuda")
    g.manual_seed(T * 7919 + H * 31 + E)
    x = torch.randn(T, H, device="cuda", generator=g).to(tdt)
    w_r = (torch.randn(E, H, device="cuda", generator=g) * 0.02).to(tdt)
    dl = torch.randn(T, E, device="cuda", generator=g)
    ws = torch.empty(max(mel.moe_router_workspace_bytes(T, H, E, dtype), 1), device="cuda",
                     dtype=torch.uint8)
    logits = torch.full((T, E), float("nan"), device="cuda")
    mel.moe_router_fwd(x, w_r, logits, ws)
    dx = torch.zeros(T, H, device="cuda", dtype=tdt)
    mel.moe_router_bwd(dl, w_r, dx, ws)
    dx0 = torch.randn(T, H, device="cuda", generator=g).to(tdt)
    dx1 = dx0.clone()
    mel.moe_router_bwd(dl, w_r, dx1, ws)
    torch.cuda.synchronize()
    xh, wh, dlh = to_numpy(x), to_numpy(w_r), to_numpy(dl)
    close("logits", to_numpy(logits), oracle.router_logits(xh, wh, np.float64), 1e-5)
    # 16-bit layers feed d_logits to the MFMA rounded to the layer dtype
    ref = oracle.router_input_grad(dlh, wh, np.float64)
    close("dx (router term)", to_numpy(dx), ref, {"f32": 1e-4, "bf16": 1e-2, "f16": 2e-3}[dtype])
    close("dx (updated)", to_numpy(dx1), to_numpy(dx0) + ref, TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n", [1, 255, 256, 1000003])
def test_accumulate_is_one_rounded_sum(dtype, n):
    mel = _mel()
    say(f"[accumulate] n={n} {dtype}")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    g = torch.Generator(device="cuda")
    g.manual_seed(n)
    src = torch.randn(n, device="cuda", generator=g).to(tdt)
    dst = torch.randn(n, device="cuda", generator=g).to(tdt)
    want = (src.cpu().float() + dst.cpu().float()).to(tdt)
    mel.moe_accumulate(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), want)


BLOCK_CASES = [  # (parity config, shared expert width)
    ("tiny", 96), ("mini-bf16", 200), ("mini-renorm", 128), ("mini-f32", 72), ("mini-k1", None),
    ("mini-T1", 64), ("mini-f16", 104),
]


def _block_run(mel, cfg, inp, shared_I, **kw):
    blk = mel.MoELoRABlock(mel.Shape.of(cfg), cfg.router, shared_I, **kw)
    sw = {n: inp["shared_" + n] for n in WEIGHTS} if shared_I else None
    blk.step(inp["x"], inp["w_r"], inp["dy"], {n: inp[n] for n in WEIGHTS}, sw)
    torch.cuda.synchronize()
    return blk


@pytest.mark.parametrize("name,shared_I", BLOCK_CASES)
def test_block_matches_oracle(name, shared_I):
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[block] {name} shared_I={shared_I}")
    inp = make_block_inputs(cfg, 11, device="cuda", shared_I=shared_I)
    blk = _block_run(mel, cfg, inp, shared_I)
    h = {n: to_numpy(v) for n, v in inp.items()}
    gl = to_numpy(blk.logits)
    close("logits", gl, oracle.router_logits(h["x"], h["w_r"], np.float64), 1e-5)
    shared = {n: h["shared_" + n] for n in WEIGHTS} if shared_I else None
    Y, g = oracle.layer_with_router_and_shared(h["x"], h["w_r"], h["dy"], h, shared, cfg.k,
                                               cfg.router, cfg.lora_scale, logits=gl)
    tol = TOL[cfg.dtype]
    ids, _ = oracle.route(gl, cfg.k, cfg.router)
    np.testing.assert_array_equal(to_numpy(blk.routed.topk_ids), ids)
    close("Y", to_numpy(blk.routed.y), Y, tol)
    close("d_logits", to_numpy(blk.routed.d_logits), g["dlogits"], tol)
    close("dX", to_numpy(blk.routed.dx), g["dx"], tol)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        close(n, to_numpy(blk.routed.grads[n]), g[n], tol)
        if shared_I:
            close("shared " + n, to_numpy(blk.shared.grads[n][0]), g["shared_" + n], tol)


@pytest.mark.parametrize("full_ft", [False, True])
def test_block_recompute_is_bit_identical(full_ft):
    mel = _mel()
    cfg = PARITY_CONFIGS["mini-bf16"]
    say(f"[block recompute] full_ft={full_ft}")
    inp = make_block_inputs(cfg, 12, device="cuda", shared_I=136)
    a = _block_run(mel, cfg, inp, 136, full_ft=full_ft)
    b = _block_run(mel, cfg, inp, 136, full_ft=full_ft, recompute=True)
    pairs = [(a.routed.y, b.routed.y), (a.routed.dx, b.routed.dx), (a.logits, b.logits)]
    pairs += [(a.shared.grads[n], b.shared.grads[n]) for n in a.shared.grads]
    if full_ft:
        pairs += [(a.shared.base_grads[n], b.shared.base_grads[n]) for n in a.shared.base_grads]
    for t1, t2 in pairs:
        assert torch.equal(t1, t2)


def test_full_size_block_with_shared_expert():
    """gpt-oss-20b-shaped block with the router projection and one shared
    expert of width I: routing exact against the oracle's own routing of the
    GPU logits, sampled tokens for Y and dX, the shared expert's LoRA
    gradients over all tokens on a column slice."""
    mel = _mel()
    cfg = CONFIGS["gpt-oss-20b"]
    say("[fullsize block] gpt-oss-20b + shared expert")
    inp = make_block_inputs(cfg, 3407, device="cuda", shared_I=cfg.I)
    blk = _block_run(mel, cfg, inp, cfg.I)
    tol = TOL[cfg.dtype]
    gl = to_numpy(blk.logits)
    xh, wrh = to_numpy(inp["x"]), to_numpy(inp["w_r"])
    rows = np.random.default_rng(1).choice(cfg.T, 64, replace=False)
    close("logits[rows]", gl[rows], oracle.router_logits(xh[rows], wrh, np.float64), 1e-5)
    ids, _ = oracle.route(gl, cfg.k, cfg.router)
    np.testing.assert_array_equal(to_numpy(blk.routed.topk_ids), ids)
    wts = {n: ExpertSlices(inp[n]) for n in WEIGHTS}
    shared = {n: to_numpy(inp["shared_" + n]) for n in WEIGHTS}
    S = np.array([0, 1234, 5000, cfg.T - 1])
    Ys, gs = oracle.layer_with_router_and_shared(xh[S], wrh, to_numpy(inp["dy"][S]), wts, shared,
                                                 cfg.k, cfg.router, cfg.lora_scale, logits=gl[S])
    close("Y[sample]", to_numpy(blk.routed.y[S]), Ys, tol)
    close("dX[sample]", to_numpy(blk.routed.dx[S]), gs["dx"], tol)
    say("  sampled tokens ok")
    # shared expert LoRA gradients: per-token sums, so the oracle runs all T
    # tokens through the dense expert once
    f = oracle.expert_forward(xh, **shared, s=cfg.lora_scale)
    b = oracle.expert_backward(xh, to_numpy(inp["dy"]), f, **shared, s=cfg.lora_scale)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        close("shared " + n, to_numpy(blk.shared.grads[n][0]), b[n], tol)
    say("  shared expert gradients ok")
