"""Pins for the oracle's routing and permutation (CPU only).

Routing is checked against a brute-force per-token sort, closed forms for
all-equal logits and k = E, a library softmax, and central finite differences
for the backward. The permutation is checked against a brute-force loop and its
defining invariants (every (token, slot) pair exactly once, counts summing to
T*k, experts non-decreasing along the order, stable within an expert).
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import softmax as sp_softmax, expit

import oracle

ROUTERS = oracle.ROUTERS


def brute_topk(row, k):
    return [i for _, i in sorted((-float(v), i) for i, v in enumerate(row))][:k]


@pytest.mark.parametrize("router", ROUTERS)
def test_route_matches_brute_force_with_ties(router):
    rng = np.random.default_rng(11)
    T, E, k = 200, 12, 3
    # quarter-integer logits: many exact ties
    logits = (rng.integers(-6, 7, size=(T, E)) / 4.0).astype(np.float32)
    ids, w = oracle.route(logits, k, router, np.float64)
    for t in range(T):
        assert list(ids[t]) == brute_topk(logits[t], k)
    assert ids.dtype == np.int32


@pytest.mark.parametrize("router", ROUTERS)
def test_route_weights_closed_forms(router):
    rng = np.random.default_rng(5)
    T, E, k = 64, 10, 4
    logits = rng.normal(size=(T, E)).astype(np.float32)
    ids, w = oracle.route(logits, k, router, np.float64)
    l64 = logits.astype(np.float64)
    sel = np.take_along_axis(l64, ids, 1)
    if router == "softmax_topk":
        ref = np.take_along_axis(sp_softmax(l64, axis=1), ids, 1)
    elif router == "softmax_topk_renorm":
        p = np.take_along_axis(sp_softmax(l64, axis=1), ids, 1)
        ref = p / p.sum(1, keepdims=True)
    elif router == "topk_softmax":
        ref = sp_softmax(sel, axis=1)
    else:
        s = expit(sel)
        ref = s / s.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-12, atol=0)
    if router != "softmax_topk":
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("router", ROUTERS)
def test_route_all_equal_logits(router):
    T, E, k = 5, 7, 3
    logits = np.full((T, E), 0.25, np.float32)
    ids, w = oracle.route(logits, k, router, np.float64)
    assert (ids == np.arange(k)).all()
    want = 1.0 / E if router == "softmax_topk" else 1.0 / k
    np.testing.assert_allclose(w, want, rtol=1e-14)


@pytest.mark.parametrize("router", ROUTERS)
def test_route_k_equals_E_selects_everything(router):
    rng = np.random.default_rng(2)
    logits = rng.normal(size=(30, 6)).astype(np.float32)
    ids, w = oracle.route(logits, 6, router, np.float64)
    assert (np.sort(ids, axis=1) == np.arange(6)).all()
    if router in ("softmax_topk", "softmax_topk_renorm", "topk_softmax"):
        np.testing.assert_allclose(np.sort(w, 1), np.sort(sp_softmax(logits.astype(np.float64), 1), 1),
                                   rtol=1e-12)


def test_renorm_equals_topk_softmax():
    rng = np.random.default_rng(9)
    logits = (3 * rng.normal(size=(100, 16))).astype(np.float32)
    _, w1 = oracle.route(logits, 5, "softmax_topk_renorm", np.float64)
    _, w2 = oracle.route(logits, 5, "topk_softmax", np.float64)
    np.testing.assert_allclose(w1, w2, rtol=1e-12)


def test_route_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((2, 3), np.float32), 4, "topk_softmax")


@pytest.mark.parametrize("router", ROUTERS)
def test_route_backward_finite_differences(router):
    rng = np.random.default_rng(21)
    T, E, k = 12, 9, 3
    # well separated logits so that +-eps never changes the selection
    logits = (rng.permutation(T * E).reshape(T, E) * 0.05 - 2.0).astype(np.float64)
    dw = rng.normal(size=(T, k))
    ids, _ = oracle.route(logits.astype(np.float32), k, router, np.float64)
    got = oracle.route_backward(logits.astype(np.float32), ids, dw, router, np.float64)

    def loss(L):
        # weights as a function of logits with the selection held fixed
        L32 = L.astype(np.float32)
        i2, w2 = oracle.route(L32, k, router, np.float64)
        assert (i2 == ids).all()
        return (w2 * dw).sum()

    # logits are fed as float32: FD in float64 on values exactly representable
    base = logits.astype(np.float32).astype(np.float64)
    eps = 2.0 ** -12
    num = np.zeros_like(base)
    for t in range(T):
        for e in range(E):
            lp, lm = base.copy(), base.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            num[t, e] = (loss(lp) - loss(lm)) / (2 * eps)
    np.testing.assert_allclose(got, num, rtol=1e-5, atol=1e-7)
    if router != "softmax_topk":
        mask = np.ones((T, E), bool)
        mask[np.arange(T)[:, None], ids] = False
        assert (got[mask] == 0).all()


def brute_permute(ids, E):
    T, k = ids.shape
    sorted_pair = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    sorted_pair.append(t * k + j)
    return np.array(sorted_pair, dtype=np.int32)


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 40), E=st.integers(1, 12), data=st.data())
def test_permute_against_brute_force(T, E, data):
    k = data.draw(st.integers(1, E))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    # distinct experts per token, as routing produces
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_pair, inv_pos = oracle.permute(ids, E)
    N = T * k
    assert counts.sum() == N
    assert offsets[0] == 0 and offsets[-1] == N
    assert (np.diff(offsets) == counts).all()
    assert sorted(sorted_pair.tolist()) == list(range(N))          # each pair exactly once
    assert (inv_pos[sorted_pair] == np.arange(N)).all()
    e_along = ids.ravel()[sorted_pair]
    assert (np.diff(e_along) >= 0).all()                           # grouped by expert
    for e in range(E):
        seg = sorted_pair[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()                             # stable
        assert (ids.ravel()[seg] == e).all()
    assert (sorted_pair == brute_permute(ids, E)).all()


def test_gather_then_unpermute_is_identity_for_k1():
    rng = np.random.default_rng(4)
    T, E, H = 50, 7, 5
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    x = rng.normal(size=(T, H))
    _, _, sp, inv = oracle.permute(ids, E)
    xp = oracle.gather_rows(x, sp, 1)
    back = oracle.combine(xp, inv, None, T, 1, np.float64)
    assert (back == x).all()


def test_gather_rows_are_the_routed_tokens():
    # Distinct token rows identify tokens: expert e's rows are exactly the
    # tokens that chose e, in token order, and every token appears k times.
    rng = np.random.default_rng(5)
    T, E, k, H = 40, 6, 3, 4
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = rng.normal(size=(T, H))
    _, off, sp, _ = oracle.permute(ids, E)
    xp = oracle.gather_rows(x, sp, k)
    tok = [int(np.flatnonzero((x == row).all(axis=1))[0]) for row in xp]
    for e in range(E):
        assert tok[off[e]:off[e + 1]] == [t for t in range(T) if e in ids[t]]
    assert np.bincount(tok, minlength=T).tolist() == [k] * T


def test_combine_one_hot_selects_expert_output():
    rng = np.random.default_rng(6)
    T, k, H = 20, 3, 4
    y = rng.normal(size=(T * k, H))
    inv = rng.permutation(T * k).astype(np.int32)
    j = rng.integers(0, k, size=T)
    w = np.zeros((T, k))
    w[np.arange(T), j] = 1.0
    Y = oracle.combine(y, inv, w, T, k, np.float64)
    want = y[inv.reshape(T, k)[np.arange(T), j]]
    assert (Y == want).all()
    # linear in w
    w2 = rng.normal(size=(T, k))
    Y2 = oracle.combine(y, inv, w2, T, k, np.float64)
    Y3 = oracle.combine(y, inv, 2 * w2 + w, T, k, np.float64)
    np.testing.assert_allclose(Y3, 2 * Y2 + Y, rtol=1e-12, atol=1e-12)
    assert math.isfinite(float(Y.sum()))
