"""Layer shapes for the MoE-LoRA expert layer.

Symbols follow the faster-moe page (Unsloth, "Fine-tune MoE models 12x faster",
section "Implementation details"): T tokens, H hidden size, I intermediate size
(the per-expert MLP width), E experts, k experts chosen per token, r LoRA rank.
The stacked expert weights are gate_up_proj [E, 2I, H] and down_proj [E, H, I]
(same page, section "What is torch._grouped_mm?").

The five named layers are shaped like the models the pages fine-tune
(gpt-oss-20b, Qwen3-30B-A3B, DeepSeek-V3) plus a tiny fp32 layer and a
long-context gpt-oss layer. The PARITY_CONFIGS are small layers whose sizes are
chosen so the oracle finishes in seconds while the GPU kernels still see
several tiles, ragged tails, zero-token experts and the degenerate cases
(k = 1, k = E, r = 1, T = 1).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

ROUTERS = ("softmax_topk", "softmax_topk_renorm", "topk_softmax", "sigmoid_topk_renorm")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    r: int
    dtype: str            # "f32", "bf16" or "f16": x, weights, LoRA params, activations, outputs
    router: str           # one of ROUTERS
    zipf_s: float = 0.0   # >0: add -zipf_s*ln(rank_e) to every token's logit of expert e
    n_dead: int = 0       # experts (lowest popularity ranks) whose logits get -30
    lora_scale: float = 1.0

    @property
    def N(self) -> int:
        """Routed (token, slot) pairs."""
        return self.T * self.k

    def flops_fwd_bwd(self) -> int:
        """Algorithmic FLOPs of one forward + backward with frozen base weights.

        Forward, per projection with (in, out) = (m, n) over N routed rows:
        2N(mn + mr + rn) (the split-LoRA count of the faster-moe page, section
        "Implementation details", split-LoRA FLOP equation, with k*s = N).
        The backward's dX costs the same again; the LoRA gradients dA, dB add
        2N r (m + n) per projection. Summed over gate_up (H, 2I) and down (I, H):
        12 N H I + 6 N r (2H + 3I).
        """
        N, H, I, r = self.N, self.H, self.I, self.r
        return 12 * N * H * I + 6 * N * r * (2 * H + 3 * I)

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, H=256, I=128, E=8, k=2, r=8,
                        dtype="f32", router="softmax_topk"),
    "gpt-oss-20b": LayerConfig("gpt-oss-20b", T=8192, H=2880, I=2880, E=32, k=4, r=16,
                               dtype="bf16", router="topk_softmax"),
    "qwen3-30b-a3b": LayerConfig("qwen3-30b-a3b", T=16384, H=2048, I=768, E=128, k=8, r=16,
                                 dtype="bf16", router="softmax_topk_renorm"),
    "deepseek-v3": LayerConfig("deepseek-v3", T=8192, H=7168, I=2048, E=256, k=8, r=32,
                               dtype="bf16", router="sigmoid_topk_renorm",
                               zipf_s=1.2, n_dead=8),
    "gpt-oss-20b-long": LayerConfig("gpt-oss-20b-long", T=65536, H=2880, I=2880, E=32, k=4,
                                    r=16, dtype="bf16", router="topk_softmax"),
    # the gpt-oss layer in IEEE half (float16 MFMA)
    "gpt-oss-20b-f16": LayerConfig("gpt-oss-20b-f16", T=8192, H=2880, I=2880, E=32, k=4, r=16,
                                   dtype="f16", router="topk_softmax"),
}

# The layer the throughput figure is quoted on (fits one GPU).
BENCH_CONFIG = "gpt-oss-20b"

# Small layers for element-by-element parity. Sizes are picked against the
# kernels' tiles (rows in blocks of 128, columns in blocks of 128/256, K in
# blocks of 64): every one has a ragged tail somewhere.
PARITY_CONFIGS = {
    "tiny": CONFIGS["tiny"],
    "tiny-s2": CONFIGS["tiny"].with_(name="tiny-s2", lora_scale=2.0, router="topk_softmax"),
    "tiny-sigmoid": CONFIGS["tiny"].with_(name="tiny-sigmoid", router="sigmoid_topk_renorm",
                                          zipf_s=1.2, n_dead=2),
    "mini-bf16": LayerConfig("mini-bf16", T=300, H=584, I=200, E=6, k=3, r=16,
                             dtype="bf16", router="topk_softmax"),
    "mini-renorm": LayerConfig("mini-renorm", T=640, H=512, I=384, E=8, k=2, r=16,
                               dtype="bf16", router="softmax_topk_renorm"),
    "mini-skew": LayerConfig("mini-skew", T=257, H=264, I=136, E=16, k=4, r=32,
                             dtype="bf16", router="sigmoid_topk_renorm", zipf_s=1.2, n_dead=4),
    "mini-k1": LayerConfig("mini-k1", T=100, H=128, I=64, E=4, k=1, r=8,
                           dtype="bf16", router="softmax_topk"),
    "mini-kE": LayerConfig("mini-kE", T=64, H=256, I=96, E=4, k=4, r=4,
                           dtype="bf16", router="softmax_topk_renorm", lora_scale=2.0),
    "mini-r1": LayerConfig("mini-r1", T=200, H=136, I=72, E=5, k=2, r=1,
                           dtype="bf16", router="topk_softmax"),
    "mini-T1": LayerConfig("mini-T1", T=1, H=256, I=128, E=8, k=2, r=16,
                           dtype="bf16", router="topk_softmax"),
    "mini-r64": LayerConfig("mini-r64", T=160, H=192, I=160, E=3, k=2, r=64,
                            dtype="bf16", router="softmax_topk"),
    "mini-f32": LayerConfig("mini-f32", T=333, H=200, I=136, E=5, k=3, r=16,
                            dtype="f32", router="topk_softmax", lora_scale=0.5),
    # few experts with many rows each: the LoRA weight gradients split every
    # expert's rows into chunks (one expert empty, skewed counts)
    "mini-split": LayerConfig("mini-split", T=2000, H=320, I=192, E=4, k=2, r=16,
                              dtype="bf16", router="sigmoid_topk_renorm", zipf_s=1.2, n_dead=1),
    "mini-f32-split": LayerConfig("mini-f32-split", T=1500, H=136, I=72, E=2, k=1, r=8,
                                  dtype="f32", router="softmax_topk"),
    # IEEE half layers (the same kernels with the float16 MFMA)
    "mini-f16": LayerConfig("mini-f16", T=300, H=584, I=200, E=6, k=3, r=16,
                            dtype="f16", router="topk_softmax"),
    "mini-f16-skew": LayerConfig("mini-f16-skew", T=1100, H=264, I=136, E=16, k=4, r=32,
                                 dtype="f16", router="sigmoid_topk_renorm", zipf_s=1.2,
                                 n_dead=4, lora_scale=2.0),
    # half with a rank that is not a multiple of 8 (element-wise side-product rows)
    "mini-f16-r4": LayerConfig("mini-f16-r4", T=200, H=136, I=72, E=5, k=2, r=4,
                               dtype="f16", router="softmax_topk_renorm"),
    # half with the widest rank (r > 32 tile shapes) and with split weight gradients
    "mini-f16-r64": LayerConfig("mini-f16-r64", T=160, H=192, I=160, E=3, k=2, r=64,
                                dtype="f16", router="softmax_topk"),
    "mini-f16-split": LayerConfig("mini-f16-split", T=2000, H=320, I=192, E=4, k=2, r=16,
                                  dtype="f16", router="sigmoid_topk_renorm", zipf_s=1.2,
                                  n_dead=1),
    # split weight gradients of a rank that is not a multiple of 8 (the B
    # gradients without their fused side products)
    "mini-split-r12": LayerConfig("mini-split-r12", T=1800, H=256, I=160, E=3, k=2, r=12,
                                  dtype="bf16", router="softmax_topk_renorm"),
    "mini-f16-split-r12": LayerConfig("mini-f16-split-r12", T=1800, H=256, I=160, E=3, k=2,
                                      r=12, dtype="f16", router="topk_softmax"),
    # 65..128 experts (two logits per lane in the routing kernels), E not a
    # multiple of the wave
    "mini-e96": LayerConfig("mini-e96", T=300, H=136, I=72, E=96, k=6, r=8,
                            dtype="bf16", router="softmax_topk_renorm"),
    # heavily skewed routing at E = 256 (23 live experts, five of more than
    # 4096 rows): the LoRA A gradient over x's gathered rows runs over all of
    # a hot expert's rows in one block, past the 4096 rows whose offsets one
    # pass of its LDS table holds
    "mini-hot": LayerConfig("mini-hot", T=4500, H=264, I=72, E=256, k=8, r=16,
                            dtype="bf16", router="sigmoid_topk_renorm", zipf_s=1.2, n_dead=8),
    # the largest expert count and top-k the library accepts: about two rows per expert
    "max-E-k": LayerConfig("max-E-k", T=64, H=64, I=32, E=1024, k=32, r=8,
                           dtype="bf16", router="softmax_topk"),
    "max-E-k-f32": LayerConfig("max-E-k-f32", T=64, H=64, I=32, E=1024, k=32, r=8,
                               dtype="f32", router="topk_softmax"),
    "max-E-k-f16": LayerConfig("max-E-k-f16", T=64, H=64, I=32, E=1024, k=32, r=8,
                               dtype="f16", router="sigmoid_topk_renorm"),
}


def get_config(name: str) -> LayerConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in PARITY_CONFIGS:
        return PARITY_CONFIGS[name]
    raise KeyError(f"unknown layer config {name!r}; known: "
                   f"{sorted(set(CONFIGS) | set(PARITY_CONFIGS))}")
