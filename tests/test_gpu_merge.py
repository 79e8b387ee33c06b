"""GPU parity of the merged export W' = W + s B A (moe_merge_lora).

Each merged element is one float32 sum of the base weight and the rank-r
product, rounded once to the layer dtype, so against the float32 oracle the
error is at most half an ulp of the dtype plus the float32 summation-order
difference of the r-term product: checked element-wise at one ulp (2^-8 of
the element for bf16, 2^-11 for float16, 1e-5 of the tensor's largest value
for float32) and
normwise at the layer tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, PARITY_CONFIGS, make_inputs
from workloads.synth import to_numpy

from gpu_util import TOL, WEIGHTS, close, say

pytestmark = pytest.mark.gpu


def _mel():
    import mixture_experts_lora_amd as mel
    return mel


# float16 layers with ranks above 16, so every (dtype, k-step count) pair of
# the merge kernel runs (ranks up to 16, 32 and 64 take one, two and four
# k steps)
EXTRA = {
    "mini-f16-r32": PARITY_CONFIGS["mini-f16"].with_(name="mini-f16-r32", r=32),
    "mini-f16-r64": PARITY_CONFIGS["mini-f16"].with_(name="mini-f16-r64", r=64, lora_scale=0.5),
}


def _cfg(name):
    return EXTRA[name] if name in EXTRA else PARITY_CONFIGS[name]


def _check(name, got, ref, dtype):
    close(name, got, ref, TOL[dtype])
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ulp = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}.get(dtype)
    bound = ulp * np.abs(ref) + 1e-6 * np.abs(ref).max() if ulp else 1e-5 * np.abs(ref).max()
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond one ulp"


def _merge(mel, cfg, inp, **kw):
    shape = mel.Shape.of(cfg)
    ws = torch.empty(max(mel.moe_merge_workspace_bytes(shape), 1), device="cuda",
                     dtype=torch.uint8)
    out = {"w_gu": torch.full_like(inp["w_gu"], float("nan")),
           "w_d": torch.full_like(inp["w_d"], float("nan"))}
    mel.moe_merge_lora(shape, {n: inp[n] for n in WEIGHTS}, out["w_gu"], out["w_d"], ws, **kw)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("name", list(PARITY_CONFIGS) + list(EXTRA))
def test_merge_matches_oracle(name):
    mel = _mel()
    cfg = _cfg(name)
    say(f"[merge] {name} H={cfg.H} I={cfg.I} E={cfg.E} r={cfg.r} {cfg.dtype} s={cfg.lora_scale}")
    inp = make_inputs(cfg, 21, device="cuda", with_dy=False)
    out, _ = _merge(mel, cfg, inp)
    h = {n: to_numpy(inp[n]) for n in WEIGHTS}
    ref = oracle.merge_lora(h, cfg.lora_scale)
    for n in ("w_gu", "w_d"):
        _check(n, to_numpy(out[n]), ref[n], cfg.dtype)


@pytest.mark.parametrize("name", ["mini-bf16", "mini-f32", "mini-r1", "mini-f16"])
def test_merge_in_place_and_one_projection(name):
    """Merging into the base weight itself equals the out-of-place merge bit for
    bit; a NULL output skips that projection."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[merge in place] {name}")
    inp = make_inputs(cfg, 22, device="cuda", with_dy=False)
    out, ws = _merge(mel, cfg, inp)
    shape = mel.Shape.of(cfg)
    w = {n: inp[n].clone() for n in WEIGHTS}
    mel.moe_merge_lora(shape, w, w["w_gu"], None, ws)
    torch.cuda.synchronize()
    assert torch.equal(w["w_gu"], out["w_gu"])
    assert torch.equal(w["w_d"], inp["w_d"])           # untouched
    mel.moe_merge_lora(shape, w, None, w["w_d"], ws)
    torch.cuda.synchronize()
    assert torch.equal(w["w_d"], out["w_d"])


@pytest.mark.parametrize("name", ["mini-bf16", "mini-renorm", "tiny", "mini-f16"])
def test_merged_weights_reproduce_the_layer(name):
    """The exported weights with the adapters zeroed give the trained layer's
    output (split order with the adapters) up to the dtype's rounding."""
    mel = _mel()
    cfg = PARITY_CONFIGS[name]
    say(f"[merge reproduces layer] {name}")
    inp = make_inputs(cfg, 23, device="cuda")
    out, _ = _merge(mel, cfg, inp)
    w = {n: inp[n] for n in WEIGHTS}
    a = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router)
    ya = a.forward(inp["x"], inp["logits"], w).clone()
    wm = dict(w, w_gu=out["w_gu"], w_d=out["w_d"], b_gu=torch.zeros_like(w["b_gu"]),
              b_d=torch.zeros_like(w["b_d"]))
    b = mel.MoELoRALayer(mel.Shape.of(cfg), cfg.router)
    yb = b.forward(inp["x"], inp["logits"], wm)
    torch.cuda.synchronize()
    close("Y merged vs split", to_numpy(yb), to_numpy(ya), TOL[cfg.dtype])


def _unaligned(t):
    """A contiguous copy of t whose data starts 2 bytes past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 8, device=t.device, dtype=t.dtype)
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 2
    return v


@pytest.mark.parametrize("which", ["base", "all"])
@pytest.mark.parametrize("name", ["mini-bf16", "mini-skew", "mini-r64", "mini-f16", "mini-r1",
                                  "mini-f16-r32", "mini-f16-r64"])
def test_merge_unaligned_weights(name, which):
    """Base weights and outputs (and with "all" the LoRA factors too) that
    cannot be read in 16-byte pieces take the element-wise paths: same results
    bit for bit, and within one ulp of the oracle."""
    mel = _mel()
    cfg = _cfg(name)
    say(f"[merge unaligned] {name} {which}")
    inp = make_inputs(cfg, 24, device="cuda", with_dy=False)
    ref_out, ws = _merge(mel, cfg, inp)
    moved = ("w_gu", "w_d") if which == "base" else WEIGHTS
    w = {n: _unaligned(inp[n]) if n in moved else inp[n] for n in WEIGHTS}
    out = {n: _unaligned(torch.full_like(inp[n], float("nan"))) for n in ("w_gu", "w_d")}
    mel.moe_merge_lora(mel.Shape.of(cfg), w, out["w_gu"], out["w_d"], ws)
    torch.cuda.synchronize()
    h = {n: to_numpy(inp[n]) for n in WEIGHTS}
    ref = oracle.merge_lora(h, cfg.lora_scale)
    for n in ("w_gu", "w_d"):
        assert torch.equal(out[n], ref_out[n]), n
        _check(n, to_numpy(out[n]), ref[n], cfg.dtype)


def test_full_size_merge():
    """gpt-oss-20b-shaped weights: merged on the GPU, sampled experts against the oracle."""
    mel = _mel()
    cfg = CONFIGS["gpt-oss-20b"]
    say("[fullsize merge] gpt-oss-20b")
    inp = make_inputs(cfg, 3407, device="cuda", with_dy=False)
    out, _ = _merge(mel, cfg, inp)
    for e in (0, 17, cfg.E - 1):
        h = {n: to_numpy(inp[n][e:e + 1]) for n in WEIGHTS}
        ref = oracle.merge_lora(h, cfg.lora_scale)
        for n in ("w_gu", "w_d"):
            _check(f"{n}[{e}]", to_numpy(out[n][e:e + 1]), ref[n], cfg.dtype)
    say("  sampled experts ok")
