"""Pins for the accounting the faster-moe page prints (CPU only).

The numbers come from tests/golden/pages_numbers.json, each with its citation.
The layer FLOP count used by the bench is tied to the page's split-LoRA FLOP
equation, and the equation itself to a direct count of the oracle's products.
"""
import json
import os

import numpy as np

import oracle
from oracle import accounting as acc
from workloads import CONFIGS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_lora_params_per_expert_projection():
    g = GOLD["moe_lora_params_per_expert_projection"]
    assert acc.lora_params(g["m"], g["n"], g["r"]) == g["value"]
    f = GOLD["moe_lora_fraction_of_projection"]
    assert abs(acc.lora_params(f["m"], f["n"], f["r"]) / (f["m"] * f["n"]) - f["value"]) < f["tol"]


def test_dense_lora_fraction():
    g = GOLD["dense_lora_fraction"]
    n = acc.lora_params(g["m"], g["n"], g["r"])
    assert abs(n - g["lora_values_about"]) / g["lora_values_about"] < 0.05
    assert abs(n / (g["m"] * g["n"]) - g["value"]) < g["tol"]


def test_fast_lora_example():
    g = GOLD["fast_lora_example"]
    assert g["m"] * g["n"] == g["full"]
    assert g["m"] * g["r"] == g["a_values"] and g["r"] * g["n"] == g["b_values"]
    assert acc.lora_params(g["m"], g["n"], g["r"]) == g["total"]
    assert round(g["total"] / g["full"], 4) == g["fraction"]


def test_split_memory_threshold():
    g = GOLD["split_memory_threshold_qwen3"]
    assert acc.split_memory_threshold(g["E"], g["m"], g["k"]) == g["value"]
    # below the threshold the split form keeps fewer values than the merge (r << n)
    s = g["value"] // 2
    assert acc.split_lora_values(g["k"], s, 0, g["n"]) < acc.peft_delta_values(g["E"], g["m"], g["n"])


def test_flop_crossover_is_where_counts_meet():
    E, m, n, r, k = 128, 2048, 768, 64, 8
    s = acc.flop_crossover(E, m, n, r, k)
    # at the crossover, the LoRA-specific terms of the two counts are equal:
    # 2 k s r (m + n)  ==  E (2 m n r + m n)
    lhs = 2 * k * s * r * (m + n)
    rhs = E * (2 * m * n * r + m * n)
    assert abs(lhs - rhs) / rhs < 1e-12
    assert acc.peft_flops(E, m, n, r, k, int(s) + 1) - acc.split_flops(m, n, r, k, int(s) + 1) < 0


def count_oracle_forward_flops(T, H, I, E, k, r):
    """Count 2*m*n*p for every matrix product the oracle's expert_forward performs."""
    calls = []

    class Rec(np.ndarray):
        def __matmul__(self, other):
            a, b = self.view(np.ndarray), np.asarray(other).view(np.ndarray)
            calls.append(2 * a.shape[0] * a.shape[1] * b.shape[1])
            return (a @ b).view(Rec)

    class NumpyProxy:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def asarray(a, dtype=None):
            out = np.asarray(a, dtype=dtype)
            return out.view(Rec) if out.ndim == 2 else out

    rng = np.random.default_rng(0)
    X = rng.normal(size=(T * k, H))
    ws = [rng.normal(size=s) for s in ((2 * I, H), (r, H), (2 * I, r), (H, I), (r, I), (H, r))]
    mod = oracle.moe_oracle
    mod.np = NumpyProxy()
    try:
        mod.expert_forward(X, *ws, s=1.0, dtype=np.float64)
    finally:
        mod.np = np
    return sum(calls)


def test_layer_flops_follow_split_equation():
    for cfg in CONFIGS.values():
        fwd = acc.layer_flops_fwd(cfg.T, cfg.H, cfg.I, cfg.r, cfg.k)
        # forward is half of the dX-side work; LoRA grads add 2 N r (m + n) per projection
        wgrad = 2 * cfg.N * cfg.r * ((cfg.H + 2 * cfg.I) + (cfg.I + cfg.H))
        assert cfg.flops_fwd_bwd() == 2 * fwd + wgrad
    # and the equation matches what the oracle actually multiplies
    T, H, I, E, k, r = 7, 12, 5, 3, 2, 3
    assert count_oracle_forward_flops(T, H, I, E, k, r) == acc.layer_flops_fwd(T, H, I, r, k)
