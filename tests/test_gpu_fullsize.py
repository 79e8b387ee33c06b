"""GPU parity at the full layer sizes, in the launch configuration the bench times.

At these sizes the oracle cannot redo the whole layer in seconds, so:
  - routing ids and the permutation are checked bit for bit over all tokens;
  - Y, dX, d logits and the routing weights are checked on sampled tokens
    (the layer is per token, so the oracle runs on just those tokens);
  - the saved activations and the LoRA gradients are checked for sampled
    experts (the oracle runs that expert's full row group);
  - every zero-token expert must get exactly zero LoRA gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS
from workloads.synth import to_numpy

from gpu_util import TOL, WEIGHTS, ExpertSlices, close, gpu_inputs, say

pytestmark = pytest.mark.gpu

SEED = 3407


@pytest.mark.parametrize("name", ["gpt-oss-20b", "qwen3-30b-a3b", "deepseek-v3",
                                  "gpt-oss-20b-long", "gpt-oss-20b-f16"])
def test_full_size_layer(name):
    import mixture_experts_lora_amd as mel
    cfg = CONFIGS[name]
    say(f"[fullsize] {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} r={cfg.r}")
    inp = gpu_inputs(cfg, SEED)
    tol = TOL[cfg.dtype]
    logits = to_numpy(inp["logits"])
    ids, w = oracle.route(logits, cfg.k, cfg.router)
    counts, offsets, sp, inv = oracle.permute(ids, cfg.E)
    nz = np.where(counts > 0)[0]
    experts = sorted({int(nz[np.argmax(counts[nz])]), int(nz[len(nz) // 2])})
    layer = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router)
    wd = {n: inp[n] for n in WEIGHTS}
    layer.forward(inp["x"], inp["logits"], wd)
    torch.cuda.synchronize()
    # expert outputs of the sampled experts, before the backward reuses their rows
    y_exp = {e: to_numpy(layer.y_exp[int(offsets[e]):int(offsets[e + 1])]) for e in experts}
    layer.backward(inp["dy"], inp["logits"], wd, x=inp["x"])
    torch.cuda.synchronize()
    say("  gpu layer done")
    np.testing.assert_array_equal(to_numpy(layer.topk_ids), ids)
    np.testing.assert_array_equal(to_numpy(layer.counts), counts)
    np.testing.assert_array_equal(to_numpy(layer.offsets), offsets)
    np.testing.assert_array_equal(to_numpy(layer.sorted_pair), sp)
    np.testing.assert_array_equal(to_numpy(layer.inv_pos), inv)
    close("topk_w", to_numpy(layer.topk_w), w, 1e-5)
    say(f"  routing exact; experts with no rows: {int((counts == 0).sum())}, "
        f"max rows {int(counts.max())}")

    wts = {n: ExpertSlices(inp[n]) for n in WEIGHTS}
    x, dy = inp["x"], inp["dy"]
    rng = np.random.default_rng(0)
    nsamp = 4 if cfg.H * cfg.I > 8_000_000 else 6
    S = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, nsamp - 2, replace=False)]))
    xs, dys = to_numpy(x[S]), to_numpy(dy[S])
    Ys, gs, _ = oracle.layer_forward_backward(xs, logits[S], dys, wts, cfg.k, cfg.router,
                                              cfg.lora_scale)
    close("Y[sample]", to_numpy(layer.y[S]), Ys, tol)
    close("dX[sample]", to_numpy(layer.dx[S]), gs["dx"], tol)
    close("d_topk_w[sample]", to_numpy(layer.d_topk_w[S]), gs["dw"], tol)
    close("d_logits[sample]", to_numpy(layer.d_logits[S]), gs["dlogits"], tol)
    say(f"  sampled tokens {S.tolist()} ok")

    # the experts' inputs come from the oracle's routing, never from the GPU's
    wn = w
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pairs = sp[lo:hi]
        toks = pairs // cfg.k
        X_e = to_numpy(x[torch.from_numpy(toks).cuda()])
        G_e = wn.reshape(-1)[pairs][:, None] * to_numpy(dy[torch.from_numpy(toks).cuda()])
        we = {n: wts[n][e] for n in WEIGHTS}
        f = oracle.expert_forward(X_e, **we, s=cfg.lora_scale)
        b = oracle.expert_backward(X_e, G_e, f, **we, s=cfg.lora_scale)
        close(f"h[e={e}]", to_numpy(layer.saved["h"][lo:hi]), f["h"], tol)
        close(f"act[e={e}]", to_numpy(layer.saved["act"][lo:hi]), f["a"], tol)
        close(f"y_exp[e={e}]", y_exp[e], f["y"], tol)
        close(f"dx_perm[e={e}]", to_numpy(layer.dx_perm[lo:hi]), b["dx"], tol)
        for n in ("da_gu", "db_gu", "da_d", "db_d"):
            close(f"{n}[e={e}]", to_numpy(layer.grads[n][e]), b[n], tol)
        say(f"  expert {e} ({hi - lo} rows) ok")
    dead = np.where(counts == 0)[0]
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        if dead.size:
            assert float(layer.grads[n][torch.from_numpy(dead).cuda()].abs().max()) == 0.0


@pytest.mark.parametrize("name", ["gpt-oss-20b", "qwen3-30b-a3b"])
def test_full_size_full_fine_tuning(name):
    """Base-weight gradients of full fine-tuning at full size, on sampled experts."""
    import mixture_experts_lora_amd as mel
    cfg = CONFIGS[name]
    say(f"[fullsize full-ft] {name}")
    inp = gpu_inputs(cfg, SEED)
    layer = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, full_ft=True)
    layer.step(inp["x"], inp["logits"], inp["dy"], {n: inp[n] for n in WEIGHTS})
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    # routing and permutation from the oracle (and the GPU's checked against them)
    ids, wn = oracle.route(to_numpy(inp["logits"]), cfg.k, cfg.router)
    counts, offsets, sp, inv = oracle.permute(ids, cfg.E)
    np.testing.assert_array_equal(to_numpy(layer.topk_ids), ids)
    np.testing.assert_array_equal(to_numpy(layer.offsets), offsets)
    np.testing.assert_array_equal(to_numpy(layer.sorted_pair), sp)
    close("topk_w", to_numpy(layer.topk_w), wn, 1e-5)
    wts = {n: ExpertSlices(inp[n]) for n in WEIGHTS}
    nz = np.where(counts > 0)[0]
    for e in sorted({int(nz[0]), int(nz[-1])}):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pairs = sp[lo:hi]
        toks = torch.from_numpy(pairs // cfg.k).cuda()
        X_e = to_numpy(inp["x"][toks])
        G_e = wn.reshape(-1)[pairs][:, None] * to_numpy(inp["dy"][toks])
        we = {n: wts[n][e] for n in WEIGHTS}
        f = oracle.expert_forward(X_e, **we, s=cfg.lora_scale)
        b = oracle.expert_backward(X_e, G_e, f, **we, s=cfg.lora_scale, base_grads=True)
        close(f"dw_gu[e={e}]", to_numpy(layer.base_grads["dw_gu"][e]), b["dw_gu"], tol)
        close(f"dw_d[e={e}]", to_numpy(layer.base_grads["dw_d"][e]), b["dw_d"], tol)
        say(f"  expert {e} ({hi - lo} rows) ok")


def test_full_size_recompute_long_context():
    """Activation-lean mode at the long-context size: bit-identical to the
    saving mode, with h and act no longer held between forward and backward
    (x_perm is never formed: the GEMMs read x's rows through sorted_pair)."""
    import mixture_experts_lora_amd as mel
    cfg = CONFIGS["gpt-oss-20b-long"]
    say(f"[fullsize recompute] {cfg.name} T={cfg.T}")
    inp = gpu_inputs(cfg, SEED)
    w = {n: inp[n] for n in WEIGHTS}
    b = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, recompute=True)
    b.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    a = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router)
    a.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    saved_a, saved_b = a.saved_bytes(), b.saved_bytes()
    say(f"  saved bytes: {saved_a / 1e9:.2f} GB -> {saved_b / 1e9:.2f} GB")
    # h [N, 2I] and act [N, I]
    assert a.x_perm is None and b.x_perm is None
    assert saved_a - saved_b == cfg.N * 3 * cfg.I * 2
    # with the combine backward folded in, the expert outputs y_exp [N, H] are
    # not held either: the lean layer keeps only u_gu and u_d [N, r]
    assert saved_b == 2 * cfg.N * cfg.r * 2
    for t1, t2 in [(a.y, b.y), (a.dx, b.dx), (a.d_logits, b.d_logits)] + \
            [(a.grads[n], b.grads[n]) for n in a.grads]:
        assert torch.equal(t1, t2)


def test_full_size_chunked_long_context():
    """Long context in 4 token chunks, activation-lean: Y, dX and d logits
    bit-identical to the unchunked lean layer, gradients close to its, and a
    lower peak allocation (one chunk's workspaces instead of the whole
    layer's)."""
    import mixture_experts_lora_amd as mel
    cfg = CONFIGS["gpt-oss-20b-long"]
    say("[fullsize chunked] gpt-oss-20b-long, 4 chunks, lean")
    inp = gpu_inputs(cfg, SEED)
    w = {n: inp[n] for n in WEIGHTS}
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    b = mel.MoELoRAChunkedLayer(mel.Shape.of(cfg), cfg.router, 4, recompute=True)
    b.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    peak_chunked = torch.cuda.max_memory_allocated() - base
    ys, dxs, dls = b.y.clone(), b.dx.clone(), b.d_logits.clone()
    gs = {n: v.clone() for n, v in b.grads.items()}
    del b
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    a = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router, recompute=True)
    a.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    peak_whole = torch.cuda.max_memory_allocated() - base
    say(f"  peak above inputs: whole {peak_whole / 1e9:.2f} GB, 4 chunks {peak_chunked / 1e9:.2f} GB")
    assert torch.equal(a.y, ys) and torch.equal(a.dx, dxs) and torch.equal(a.d_logits, dls)
    for n, v in gs.items():
        close(n, to_numpy(v), to_numpy(a.grads[n]), 1e-2)
    assert peak_chunked < 0.6 * peak_whole
