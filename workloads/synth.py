"""Seeded synthetic inputs for the MoE-LoRA expert layer.

Distributions (second argument of N(0, s) is the standard deviation, the usual
0.02-initialiser convention):

  x ~ N(0, 1) [T, H]                  dY ~ N(0, 1) [T, H]
  W_r ~ N(0, 0.02) [E, H]             (router weights; only used to make logits)
  W_gu ~ N(0, 0.02) [E, 2I, H]        W_d ~ N(0, 0.02) [E, H, I]
  A_gu ~ N(0, 1/r) [E, r, H]          A_d ~ N(0, 1/r) [E, r, I]
  B_gu ~ N(0, 0.02) [E, 2I, r]        B_d ~ N(0, 0.02) [E, H, r]

LoRA B is drawn nonzero on purpose (a fresh adapter starts at B = 0, which
would make every LoRA gradient but dB vanish). bf16 layers round each fp32
draw to bfloat16 (round to nearest even, torch's conversion); f16 layers likewise
round to IEEE half.

Router logits are the frozen router projection x W_r^T, computed in float64
from the (already rounded) x and W_r and rounded once to float32. Layers with
zipf_s > 0 add -zipf_s * ln(rank_e) to every token's logit of expert e, with
rank a seeded permutation of 1..E, so expert popularity is Zipf-skewed; the
n_dead least popular experts also get -30, so they receive no tokens.

Every tensor gets its own sub-seed from numpy's SeedSequence over
(seed, tensor id[, expert]). Values come from torch's generator on the device
asked for: a CPU draw and a GPU draw of the same seed differ, so any test that
compares the two sides hands the oracle a host copy of the very tensors the
GPU consumed.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import LayerConfig

TENSOR_IDS = {"x": 0, "w_r": 1, "w_gu": 2, "w_d": 3, "a_gu": 4, "b_gu": 5,
              "a_d": 6, "b_d": 7, "dy": 8, "zipf": 9,
              "shared_w_gu": 10, "shared_w_d": 11, "shared_a_gu": 12, "shared_b_gu": 13,
              "shared_a_d": 14, "shared_b_d": 15}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def seed_for(seed: int, name: str, expert: int | None = None) -> int:
    """63-bit sub-seed for one tensor (or one expert's slice of it)."""
    key = [int(seed), TENSOR_IDS[name]] + ([] if expert is None else [int(expert)])
    st = np.random.SeedSequence(key).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _normal(shape, std, seed, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def _stacked(name, E, shape, std, seed, device, dtype):
    """[E, *shape], drawn one expert at a time (bounded temporaries)."""
    out = torch.empty((E,) + tuple(shape), device=device, dtype=dtype)
    for e in range(E):
        out[e].copy_(_normal(shape, std, seed_for(seed, name, e), device, dtype))
    return out


def zipf_offsets(cfg: LayerConfig, seed: int) -> np.ndarray:
    """Per-expert logit offsets (float64); zeros when the layer is not skewed."""
    b = np.zeros(cfg.E, dtype=np.float64)
    if cfg.zipf_s <= 0 and cfg.n_dead == 0:
        return b
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), TENSOR_IDS["zipf"]])))
    rank = rng.permutation(cfg.E) + 1          # rank_e in 1..E
    if cfg.zipf_s > 0:
        b -= cfg.zipf_s * np.log(rank.astype(np.float64))
    if cfg.n_dead > 0:
        b[rank > cfg.E - cfg.n_dead] = -30.0
    return b


def make_inputs(cfg: LayerConfig, seed: int, device="cpu", with_dy=True) -> dict:
    """All layer inputs for `cfg` as torch tensors on `device`."""
    dev = torch.device(device)
    dt = TORCH_DTYPE[cfg.dtype]
    T, H, I, E, r = cfg.T, cfg.H, cfg.I, cfg.E, cfg.r
    out = {}
    out["x"] = _normal((T, H), 1.0, seed_for(seed, "x"), dev, dt)
    w_r = _normal((E, H), 0.02, seed_for(seed, "w_r"), dev, dt)
    logits = out["x"].double() @ w_r.double().t()
    off = zipf_offsets(cfg, seed)
    if np.any(off != 0):
        logits = logits + torch.from_numpy(off).to(dev)[None, :]
    out["logits"] = logits.float().contiguous()
    del w_r, logits
    out["w_gu"] = _stacked("w_gu", E, (2 * I, H), 0.02, seed, dev, dt)
    out["w_d"] = _stacked("w_d", E, (H, I), 0.02, seed, dev, dt)
    out["a_gu"] = _stacked("a_gu", E, (r, H), 1.0 / r, seed, dev, dt)
    out["b_gu"] = _stacked("b_gu", E, (2 * I, r), 0.02, seed, dev, dt)
    out["a_d"] = _stacked("a_d", E, (r, I), 1.0 / r, seed, dev, dt)
    out["b_d"] = _stacked("b_d", E, (H, r), 0.02, seed, dev, dt)
    if with_dy:
        out["dy"] = _normal((T, H), 1.0, seed_for(seed, "dy"), dev, dt)
    return out


def make_block_inputs(cfg: LayerConfig, seed: int, device="cpu", shared_I: int | None = None,
                      with_dy=True) -> dict:
    """make_inputs plus what a whole MoE block starts from: the router weight
    w_r [E, H] (the very draw the logits were made from) and, when shared_I is
    given, one always-on shared expert with intermediate width shared_I:
    shared_w_gu [2 shared_I, H], shared_a_gu [r, H], shared_b_gu [2 shared_I, r],
    shared_w_d [H, shared_I], shared_a_d [r, shared_I], shared_b_d [H, r], drawn
    with the routed experts' distributions."""
    dev = torch.device(device)
    dt = TORCH_DTYPE[cfg.dtype]
    out = make_inputs(cfg, seed, device, with_dy)
    H, r = cfg.H, cfg.r
    out["w_r"] = _normal((cfg.E, H), 0.02, seed_for(seed, "w_r"), dev, dt)
    if shared_I:
        Is = int(shared_I)
        for n, shp, std in (("w_gu", (2 * Is, H), 0.02), ("w_d", (H, Is), 0.02),
                            ("a_gu", (r, H), 1.0 / r), ("b_gu", (2 * Is, r), 0.02),
                            ("a_d", (r, Is), 1.0 / r), ("b_d", (H, r), 0.02)):
            out["shared_" + n] = _normal(shp, std, seed_for(seed, "shared_" + n), dev, dt)
    return out


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host float32 (or integer) copy of a tensor; bf16 values are exact in float32."""
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def expert_histogram(topk_ids: np.ndarray, E: int) -> np.ndarray:
    """Rows per expert for a given routing (a plain count, used for reporting)."""
    return np.bincount(np.asarray(topk_ids).ravel(), minlength=E)


__all__ = ["make_inputs", "make_block_inputs", "seed_for", "zipf_offsets", "to_numpy", "expert_histogram",
           "TENSOR_IDS", "TORCH_DTYPE"]
