"""Pins for the oracle's expert layer, forward and backward (CPU only).

- split LoRA equals the PEFT merge W + s B A (the faster-moe page: the order of
  the products changes, not losses, gradients or outputs), in float64;
- a hand-worked example with a closed-form answer (gate is the first half,
  SwiGLU is silu(gate) * up, the adapter enters as (X A^T) B^T);
- E = 1, k = 1 reduces to the dense LoRA SwiGLU MLP in the fast_lora tutorial's
  notation (separate gate, up, down weights each with its merged adapter);
- B = 0 gives zero dA; y is linear in B_d;
- central finite differences of a scalar loss for x, logits, A and B;
- an independent float64 torch.autograd differentiation of the same layer.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import LayerConfig, make_inputs
from workloads.synth import to_numpy

WNAMES = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")


def rand_layer(T, H, I, E, k, r, router, seed, s=1.0, b_scale=0.3):
    rng = np.random.default_rng(seed)
    d = {
        "x": rng.normal(size=(T, H)),
        "w_gu": rng.normal(size=(E, 2 * I, H)) * 0.3,
        "a_gu": rng.normal(size=(E, r, H)) * 0.3,
        "b_gu": rng.normal(size=(E, 2 * I, r)) * b_scale,
        "w_d": rng.normal(size=(E, H, I)) * 0.3,
        "a_d": rng.normal(size=(E, r, I)) * 0.3,
        "b_d": rng.normal(size=(E, H, r)) * b_scale,
        "dy": rng.normal(size=(T, H)),
    }
    # well separated float32 logits: small perturbations never flip a choice
    d["logits"] = (rng.permutation(T * E).reshape(T, E) * (4.0 / (T * E)) - 2.0).astype(np.float32)
    return d


@pytest.mark.parametrize("router", oracle.ROUTERS)
@pytest.mark.parametrize("s", [1.0, 2.0])
def test_split_equals_merged(router, s):
    d = rand_layer(T=40, H=24, I=12, E=5, k=2, r=3, router=router, seed=1)
    Y, _ = oracle.layer_forward(d["x"], d["logits"], d, 2, router, s, np.float64)
    Ym = oracle.merged_forward(d["x"], d["logits"], d, 2, router, s, np.float64)
    assert np.abs(Y - Ym).max() <= 1e-12 * np.abs(Y).max()


def test_merge_of_zero_b_is_the_base_weight_and_rank_one_is_an_outer_product():
    d = rand_layer(T=4, H=24, I=12, E=3, k=2, r=1, router="softmax_topk", seed=6)
    m0 = oracle.merge_lora({**d, "b_gu": 0 * d["b_gu"], "b_d": 0 * d["b_d"]}, 1.7, np.float64)
    np.testing.assert_array_equal(m0["w_gu"], d["w_gu"])
    np.testing.assert_array_equal(m0["w_d"], d["w_d"])
    m = oracle.merge_lora(d, 1.7, np.float64)
    for e in range(3):
        np.testing.assert_allclose(
            m["w_gu"][e], d["w_gu"][e] + 1.7 * np.outer(d["b_gu"][e][:, 0], d["a_gu"][e][0]),
            rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(
            m["w_d"][e], d["w_d"][e] + 1.7 * np.outer(d["b_d"][e][:, 0], d["a_d"][e][0]),
            rtol=1e-14, atol=1e-15)
    assert m["w_gu"].shape == d["w_gu"].shape and m["w_d"].shape == d["w_d"].shape


def test_split_equals_merged_on_tiny_config():
    cfg = LayerConfig("t", T=256, H=256, I=128, E=8, k=2, r=8, dtype="f32", router="softmax_topk")
    d = {n: to_numpy(v) for n, v in make_inputs(cfg, 3).items()}
    Y, _ = oracle.layer_forward(d["x"], d["logits"], d, cfg.k, cfg.router, 1.0, np.float64)
    Ym = oracle.merged_forward(d["x"], d["logits"], d, cfg.k, cfg.router, 1.0, np.float64)
    assert np.abs(Y - Ym).max() <= 1e-12 * np.abs(Y).max()


def worked_example():
    """H=2, I=1, E=2, k=1, r=1, s=1, softmax_topk router; one token.

    Expert 1 is chosen (logit 1 > 0), w = e/(1+e). Its values are picked so the
    gate pre-activation is ln 3, where sigmoid = 3/4:
      u_gu = x A^T = 1,  h = [0.5, 1] + u [ln3 - 0.5, 1] = [ln3, 2]
      a = ln3 * 3/4 * 2 = 1.5 ln3,  u_d = 2a = 3 ln3
      y = a [1, 0] + u_d [0, 1] = [1.5 ln3, 3 ln3]
    """
    L3 = math.log(3.0)
    d = {
        "x": np.array([[1.0, 0.0]]),
        "logits": np.array([[0.0, 1.0]], np.float32),
        "w_gu": np.array([np.zeros((2, 2)), [[0.5, 0.0], [1.0, 0.0]]]),
        "a_gu": np.array([np.zeros((1, 2)), [[1.0, 0.0]]]),
        "b_gu": np.array([np.zeros((2, 1)), [[L3 - 0.5], [1.0]]]),
        "w_d": np.array([np.zeros((2, 1)), [[1.0], [0.0]]]),
        "a_d": np.array([np.zeros((1, 1)), [[2.0]]]),
        "b_d": np.array([np.zeros((2, 1)), [[0.0], [1.0]]]),
        "dy": np.array([[1.0, 1.0]]),
    }
    return d, L3


def test_worked_example_forward_and_backward():
    d, L3 = worked_example()
    Y, g, c = oracle.layer_forward_backward(d["x"], d["logits"], d["dy"], d, 1,
                                            "softmax_topk", 1.0, np.float64)
    e = math.e
    w = e / (1 + e)
    p0, p1 = 1 / (1 + e), e / (1 + e)
    y = np.array([1.5 * L3, 3 * L3])
    np.testing.assert_allclose(Y[0], w * y, rtol=1e-14)
    assert list(c["ids"][0]) == [1]
    # backward, by hand: G = w dY
    dw = y.sum()                                   # <dY, y>
    np.testing.assert_allclose(g["dw"][0, 0], dw, rtol=1e-14)
    np.testing.assert_allclose(g["dlogits"][0], [-p0 * p1 * dw, p0 * p1 * dw], rtol=1e-13)
    gb = w                                          # G B_d = [w, w].[0, 1]
    da = w + 2 * gb                                 # G W_d + s gb A_d
    np.testing.assert_allclose(g["db_d"][1], [[3 * w * L3], [3 * w * L3]], rtol=1e-14)
    np.testing.assert_allclose(g["da_d"][1], [[gb * 1.5 * L3]], rtol=1e-14)
    sg = 0.75
    dg = da * 2 * sg * (1 + L3 * (1 - sg))
    dv = da * L3 * sg
    dhb = dg * (L3 - 0.5) + dv
    np.testing.assert_allclose(g["dx"][0], [0.5 * dg + dv + dhb, 0.0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g["db_gu"][1], [[dg], [dv]], rtol=1e-13)
    np.testing.assert_allclose(g["da_gu"][1], [[dhb, 0.0]], rtol=1e-13, atol=1e-15)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        assert (g[n][0] == 0).all()                  # expert 0 got no rows


def test_single_expert_is_the_dense_lora_swiglu_mlp():
    """E=1, k=1: the fast_lora tutorial's LoRA MLP, e = X G, f = e sigmoid(e),
    g = X U, h = f g, i = h W, each weight with its own merged adapter."""
    rng = np.random.default_rng(3)
    T, H, I, r, s = 17, 20, 9, 4, 2.0
    X = torch.tensor(rng.normal(size=(T, H)), dtype=torch.float64)
    # column-major "x @ G" weights of the dense MLP, each with an adapter A @ B
    G = torch.tensor(rng.normal(size=(H, I)) * 0.3)
    U = torch.tensor(rng.normal(size=(H, I)) * 0.3)
    W = torch.tensor(rng.normal(size=(I, H)) * 0.3)
    Ag, Bg = torch.tensor(rng.normal(size=(H, r)) * 0.3), torch.tensor(rng.normal(size=(r, I)) * 0.3)
    Au, Bu = torch.tensor(rng.normal(size=(H, r)) * 0.3), torch.tensor(rng.normal(size=(r, I)) * 0.3)
    Aw, Bw = torch.tensor(rng.normal(size=(I, r)) * 0.3), torch.tensor(rng.normal(size=(r, H)) * 0.3)
    Gm, Um, Wm = G + s * Ag @ Bg, U + s * Au @ Bu, W + s * Aw @ Bw
    e = X @ Gm
    f = e * torch.sigmoid(e)
    g = X @ Um
    i = (f * g) @ Wm
    # the same MLP as one stacked expert: gate_up rows = [G^T; U^T]. A single
    # rank-2r adapter over the stacked projection reproduces both adapters:
    # A = [Ag^T; Au^T] (2r x H), B = blockdiag(Bg^T, Bu^T) (2I x 2r).
    w_gu = torch.cat([G.T, U.T], 0)[None]
    a_gu = torch.cat([Ag.T, Au.T], 0)[None]
    b_gu = torch.zeros(2 * I, 2 * r, dtype=torch.float64)
    b_gu[:I, :r] = Bg.T
    b_gu[I:, r:] = Bu.T
    w_d = W.T[None]
    a_d = Aw.T[None]
    b_d = Bw.T[None]
    d = {"w_gu": w_gu.numpy(), "a_gu": a_gu.numpy(), "b_gu": b_gu[None].numpy(),
         "w_d": w_d.numpy(), "a_d": a_d.numpy(), "b_d": b_d.numpy()}
    logits = np.zeros((T, 1), np.float32)
    for router in oracle.ROUTERS:
        Y, _ = oracle.layer_forward(X.numpy(), logits, d, 1, router, s, np.float64)
        np.testing.assert_allclose(Y, i.numpy(), rtol=1e-11, atol=1e-12)   # w = 1 for E = k = 1


def test_zero_b_gives_zero_da_and_base_output():
    d = rand_layer(T=30, H=16, I=8, E=4, k=2, r=3, router="topk_softmax", seed=7)
    for n in ("b_gu", "b_d"):
        d[n] = np.zeros_like(d[n])
    Y, g, _ = oracle.layer_forward_backward(d["x"], d["logits"], d["dy"], d, 2, "topk_softmax",
                                            1.0, np.float64)
    assert (g["da_gu"] == 0).all() and (g["da_d"] == 0).all()
    d2 = dict(d)
    d2["a_gu"] = d["a_gu"] * 5 + 1.0
    d2["a_d"] = d["a_d"] * -3
    Y2, _ = oracle.layer_forward(d2["x"], d2["logits"], d2, 2, "topk_softmax", 1.0, np.float64)
    np.testing.assert_array_equal(Y, Y2)          # A is irrelevant when B = 0


def test_output_linear_in_down_adapter_b():
    d = rand_layer(T=30, H=16, I=8, E=4, k=2, r=3, router="softmax_topk", seed=8)
    f = lambda bd: oracle.layer_forward(d["x"], d["logits"], {**d, "b_d": bd}, 2,
                                        "softmax_topk", 1.0, np.float64)[0]
    Y0, Y1, Y2 = f(0 * d["b_d"]), f(d["b_d"]), f(2 * d["b_d"])
    np.testing.assert_allclose(Y2 - Y1, Y1 - Y0, rtol=1e-10, atol=1e-12)


def _loss(d, router, k, s):
    Y, _ = oracle.layer_forward(d["x"], d["logits"], d, k, router, s, np.float64)
    return float((Y * d["dy"]).sum())


@pytest.mark.parametrize("router", oracle.ROUTERS)
def test_backward_central_finite_differences(router):
    T, H, I, E, k, r, s = 8, 16, 8, 4, 2, 4, 1.5
    d = rand_layer(T, H, I, E, k, r, router, seed=13)
    _, g, _ = oracle.layer_forward_backward(d["x"], d["logits"], d["dy"], d, k, router, s,
                                            np.float64, base_grads=True)
    rng = np.random.default_rng(0)
    h = 1e-6
    for name, gname in (("x", "dx"), ("a_gu", "da_gu"), ("b_gu", "db_gu"),
                        ("a_d", "da_d"), ("b_d", "db_d"), ("w_gu", "dw_gu"), ("w_d", "dw_d")):
        # full element-wise FD on a few random coordinates plus one random direction
        base = d[name]
        flat_idx = rng.choice(base.size, size=min(12, base.size), replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, base.shape)
            dp, dm = base.copy(), base.copy()
            dp[idx] += h
            dm[idx] -= h
            num = (_loss({**d, name: dp}, router, k, s) - _loss({**d, name: dm}, router, k, s)) / (2 * h)
            assert abs(num - g[gname][idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, g[gname][idx])
        V = rng.normal(size=base.shape)
        num = (_loss({**d, name: base + h * V}, router, k, s)
               - _loss({**d, name: base - h * V}, router, k, s)) / (2 * h)
        ana = float((g[gname] * V).sum())
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(num)), (name, num, ana)
    # logits: float32 inputs, perturb on a float32-exact grid
    eps = 2.0 ** -14
    L = d["logits"].astype(np.float64)
    for t in range(T):
        for e in range(E):
            lp, lm = L.copy(), L.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            num = (_loss({**d, "logits": lp.astype(np.float32)}, router, k, s)
                   - _loss({**d, "logits": lm.astype(np.float32)}, router, k, s)) / (2 * eps)
            assert abs(num - g["dlogits"][t, e]) <= 1e-5 * max(1.0, abs(num)), (t, e, num)


def torch_layer(x, logits, p, k, router, s):
    """Differentiable float64 torch form of the layer, written from the pages'
    description independently of the oracle's NumPy code (selection fixed
    from the logits by torch.topk ordering with ties to the lower index)."""
    T, E = logits.shape
    # stable descending order: sort (-logit, index)
    order = torch.argsort(-logits.detach() * 1.0, dim=1, stable=True)
    S = order[:, :k]
    if router in ("softmax_topk", "softmax_topk_renorm"):
        pr = torch.softmax(logits, 1).gather(1, S)
        w = pr / pr.sum(1, keepdim=True) if router.endswith("renorm") else pr
    elif router == "topk_softmax":
        w = torch.softmax(logits.gather(1, S), 1)
    else:
        sg = torch.sigmoid(logits.gather(1, S))
        w = sg / sg.sum(1, keepdim=True)
    I = p["w_gu"].shape[1] // 2
    Y = torch.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = int(S[t, j])
            xe = x[t:t + 1]
            h = xe @ p["w_gu"][e].T + s * (xe @ p["a_gu"][e].T) @ p["b_gu"][e].T
            a = torch.nn.functional.silu(h[:, :I]) * h[:, I:]
            y = a @ p["w_d"][e].T + s * (a @ p["a_d"][e].T) @ p["b_d"][e].T
            Y[t] = Y[t] + w[t, j] * y[0]
    return Y


@pytest.mark.parametrize("router", oracle.ROUTERS)
def test_backward_matches_torch_autograd(router):
    T, H, I, E, k, r, s = 24, 32, 16, 6, 3, 5, 2.0
    d = rand_layer(T, H, I, E, k, r, router, seed=29)
    _, g, _ = oracle.layer_forward_backward(d["x"], d["logits"], d["dy"], d, k, router, s,
                                            np.float64, base_grads=True)
    tp = {n: torch.tensor(d[n], dtype=torch.float64, requires_grad=True) for n in WNAMES}
    x = torch.tensor(d["x"], requires_grad=True)
    lg = torch.tensor(d["logits"].astype(np.float64), requires_grad=True)
    Y = torch_layer(x, lg, tp, k, router, s)
    (Y * torch.tensor(d["dy"])).sum().backward()
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dlogits"], lg.grad.numpy(), rtol=1e-9, atol=1e-12)
    for n in ("a_gu", "b_gu", "a_d", "b_d", "w_gu", "w_d"):
        np.testing.assert_allclose(g["d" + n], tp[n].grad.numpy(), rtol=1e-10, atol=1e-12)
