"""Helpers shared by the GPU parity tests: run the HIP layer, run the oracle on
host copies of the very same inputs, and compare to the stated tolerances.

Tolerances (per tensor, normwise): max |gpu - ref| <= tol * max |ref|, with
tol = 1e-4 for float32 layers, 2e-2 for bfloat16 layers and 5e-3 for float16
layers (ten units of half's rounding, 2^-11, as 2e-2 is about five of
bfloat16's 2^-8). The routing-weight gradients (d_topk_w, d logits) are
float32 arithmetic on both sides but consume 16-bit activations (the expert
output, or the SwiGLU output recomputed from the stored h), so they take the
layer dtype's tolerance like every other gradient. The routing weights
themselves use 1e-5. Indices are compared bit for bit.

Where the tolerance is 1e-4 or tighter (float32 results), every element is
also held to a relative bound: |gpu - ref| <= tol * |ref| + tol / 10 * max|ref|.
The absolute term, a tenth of the normwise bound, admits the rounding of
elements that cancel to near zero (a float32 sum of K products carries about
sqrt(K) * 2^-24 of the products' magnitudes), while a small element with a
large relative error (a rare expert's gradient row, a small routing-weight
gradient) no longer hides under a tensor's largest values.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from workloads import make_inputs
from workloads.synth import to_numpy

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}
WEIGHTS = ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def close(name, got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    err = float(diff.max()) if got.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol} * max|ref| {scale:.3e}"
    if tol <= 1e-4 and got.size:
        bound = tol * np.abs(ref) + 0.1 * tol * scale
        bad = diff > bound
        if bad.any():
            i = np.unravel_index(int(np.argmax(diff - bound)), diff.shape)
            raise AssertionError(
                f"{name}: {int(bad.sum())} of {diff.size} elements outside {tol}|ref| + "
                f"{0.1 * tol * scale:.3e}; worst at {i}: gpu {got[i]:.6e} ref {ref[i]:.6e}")
    return err, scale


class ExpertSlices:
    """Indexable by expert: a float32 host copy of one expert's slice (cached)."""

    def __init__(self, t: torch.Tensor):
        self.t, self.cache = t, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = to_numpy(self.t[e])
        return self.cache[e]


def run_gpu(layer_cls, shape, cfg, inp):
    layer = layer_cls(shape, cfg.router)
    w = {n: inp[n] for n in WEIGHTS}
    layer.step(inp["x"], inp["logits"], inp["dy"], w)
    torch.cuda.synchronize()
    return layer


def gpu_inputs(cfg, seed):
    return make_inputs(cfg, seed, device="cuda")
