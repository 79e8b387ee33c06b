"""Pins of the oracle's router projection and shared expert.

The router projection (logits = x W_r^T, and its input gradient) and the
always-on shared expert (a dense LoRA SwiGLU MLP added to the routed output,
the DeepSeek-style layout of GLM-4.7-Flash on the faster-moe page, section
"GLM 4.7 benchmark") are pinned by:
- special inputs with known images: identity rows give W_r^T, identity
  gradients give W_r;
- reduction to the routed layer: the shared expert is exactly a one-expert,
  one-slot routed layer;
- an independent float64 torch.autograd form of the whole block (router
  projection -> routed experts + shared expert), forward and every gradient.
"""
import numpy as np
import pytest
import torch

import oracle

WNAMES = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")


def rand_block(T, H, I, E, k, r, seed, b_scale=0.3):
    rng = np.random.default_rng(seed)
    d = {"x": rng.normal(size=(T, H)), "w_r": rng.normal(size=(E, H)) * 0.5,
         "dy": rng.normal(size=(T, H))}
    for n, shp in (("w_gu", (2 * I, H)), ("a_gu", (r, H)), ("b_gu", (2 * I, r)),
                   ("w_d", (H, I)), ("a_d", (r, I)), ("b_d", (H, r))):
        sc = b_scale if n.startswith("b") else 0.3
        d[n] = rng.normal(size=(E,) + shp) * sc
        d["shared_" + n] = rng.normal(size=shp) * sc
    return d


def shared_of(d):
    return {n: d["shared_" + n] for n in WNAMES}


def test_router_logits_of_identity_rows_are_the_router_columns():
    rng = np.random.default_rng(3)
    E, H = 5, 7
    w_r = rng.normal(size=(E, H))
    L = oracle.router_logits(np.eye(H), w_r, np.float64)
    assert L.shape == (H, E)
    np.testing.assert_array_equal(L, w_r.T)
    x = rng.normal(size=(4, H))
    # linear in x, and each logit the projection on one expert's row
    np.testing.assert_allclose(oracle.router_logits(2 * x, w_r, np.float64),
                               2 * oracle.router_logits(x, w_r, np.float64), rtol=1e-14)
    for e in range(E):
        for t in range(4):
            assert abs(oracle.router_logits(x, w_r, np.float64)[t, e]
                       - float(np.dot(x[t], w_r[e]))) < 1e-12


def test_router_input_grad_of_identity_is_the_router_weight():
    rng = np.random.default_rng(4)
    E, H = 6, 9
    w_r = rng.normal(size=(E, H))
    np.testing.assert_array_equal(oracle.router_input_grad(np.eye(E), w_r, np.float64), w_r)
    # adjoint of the projection: <L(x), g> = <x, L^T(g)>
    x, g = rng.normal(size=(3, H)), rng.normal(size=(3, E))
    lhs = float((oracle.router_logits(x, w_r, np.float64) * g).sum())
    rhs = float((x * oracle.router_input_grad(g, w_r, np.float64)).sum())
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_shared_expert_is_a_one_expert_one_slot_routed_layer():
    T, H, I, E, k, r, s = 12, 16, 8, 4, 2, 3, 1.5
    d = rand_block(T, H, I, E, k, r, seed=5)
    routed = {n: d[n] for n in WNAMES}
    Y0, g0 = oracle.layer_with_router_and_shared(d["x"], d["w_r"], d["dy"], routed, None, k,
                                                 "softmax_topk", s, np.float64)
    Y1, g1 = oracle.layer_with_router_and_shared(d["x"], d["w_r"], d["dy"], routed, shared_of(d),
                                                 k, "softmax_topk", s, np.float64)
    one = {n: d["shared_" + n][None] for n in WNAMES}
    Ys, gs, _ = oracle.layer_forward_backward(d["x"], np.zeros((T, 1), np.float32), d["dy"], one,
                                              1, "softmax_topk", s, np.float64)
    np.testing.assert_allclose(Y1 - Y0, Ys, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g1["dx"] - g0["dx"], gs["dx"], rtol=1e-10, atol=1e-12)
    for n in ("da_gu", "db_gu", "da_d", "db_d"):
        np.testing.assert_allclose(g1["shared_" + n], gs[n][0], rtol=1e-10, atol=1e-12)
    # the routed part is unchanged by the shared expert
    for n in ("dlogits", "da_gu", "db_gu", "da_d", "db_d"):
        np.testing.assert_array_equal(g1[n], g0[n])


def torch_block(x, w_r, p, sp, k, router, s):
    """float64 torch form: logits from the router projection, the top-k routed
    LoRA SwiGLU experts, plus the shared expert on every token."""
    logits = x @ w_r.T
    T, E = logits.shape
    S = torch.argsort(-logits.detach(), dim=1, stable=True)[:, :k]
    if router == "softmax_topk":
        w = torch.softmax(logits, 1).gather(1, S)
    elif router == "softmax_topk_renorm":
        pr = torch.softmax(logits, 1).gather(1, S)
        w = pr / pr.sum(1, keepdim=True)
    elif router == "topk_softmax":
        w = torch.softmax(logits.gather(1, S), 1)
    else:
        sg = torch.sigmoid(logits.gather(1, S))
        w = sg / sg.sum(1, keepdim=True)
    I = p["w_gu"].shape[1] // 2

    def mlp(xe, q):
        h = xe @ q["w_gu"].T + s * (xe @ q["a_gu"].T) @ q["b_gu"].T
        a = torch.nn.functional.silu(h[:, :I]) * h[:, I:]
        return a @ q["w_d"].T + s * (a @ q["a_d"].T) @ q["b_d"].T

    rows = []
    for t in range(T):
        yt = mlp(x[t:t + 1], sp)[0]
        for j in range(k):
            e = int(S[t, j])
            yt = yt + w[t, j] * mlp(x[t:t + 1], {n: p[n][e] for n in WNAMES})[0]
        rows.append(yt)
    return torch.stack(rows), S


@pytest.mark.parametrize("router", oracle.ROUTERS)
def test_block_matches_torch_autograd(router):
    T, H, I, E, k, r, s = 20, 24, 12, 6, 2, 4, 2.0
    d = rand_block(T, H, I, E, k, r, seed=31)
    routed = {n: d[n] for n in WNAMES}
    Y, g = oracle.layer_with_router_and_shared(d["x"], d["w_r"], d["dy"], routed, shared_of(d),
                                               k, router, s, np.float64)
    x = torch.tensor(d["x"], requires_grad=True)
    w_r = torch.tensor(d["w_r"])
    p = {n: torch.tensor(d[n], requires_grad=True) for n in WNAMES}
    sp = {n: torch.tensor(d["shared_" + n], requires_grad=True) for n in WNAMES}
    Yt, S = torch_block(x, w_r, p, sp, k, router, s)
    # same experts chosen (the oracle selects on float32-rounded logits)
    ids, _ = oracle.route(g["logits"], k, router)
    assert np.array_equal(np.sort(ids, 1), np.sort(S.numpy(), 1))
    (Yt * torch.tensor(d["dy"])).sum().backward()
    # the oracle's logits are float32 (as the kernels'), the torch form's float64:
    # agreement to ~1e-6 relative, far below any wrong term's effect
    tol = dict(rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(Y, Yt.detach().numpy(), **tol)
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), **tol)
    for n in ("a_gu", "b_gu", "a_d", "b_d"):
        np.testing.assert_allclose(g["d" + n], p[n].grad.numpy(), **tol)
        np.testing.assert_allclose(g["shared_d" + n], sp[n].grad.numpy(), **tol)
