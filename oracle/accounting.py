"""Parameter, memory and FLOP accounting the faster-moe page states.

TEST INFRASTRUCTURE (see the package header): used by the pins and by the
bench's work count, never by the HIP library.

Source: Unsloth, "Fine-tune MoE models 12x faster" (unsloth.ai docs, faster-moe
page), section "Implementation details": a LoRA adapter on an (m, n) weight
adds (m, r) and (r, n) matrices; the memory comparison of the PEFT merge
(E m n values) with split LoRA (k s (r + n) values) and its threshold s < E m / k;
the FLOP counts of the merge, E (2 m n r + m n) + 2 k s m n, and of split LoRA,
2 k (s m n + s m r + s r n), with the crossover s ~ E m n / (k (m + n)) (1 + 1/(2r)).
Here s is the number of tokens and k s the routed (token, expert) pairs.
"""
from __future__ import annotations


def lora_params(m: int, n: int, r: int) -> int:
    """Trainable values of one rank-r adapter on an (m, n) weight: m r + r n."""
    return m * r + r * n


def peft_delta_values(E: int, m: int, n: int) -> int:
    """Values materialised by merging every expert's delta: E m n."""
    return E * m * n


def split_lora_values(k: int, s: int, r: int, n: int) -> int:
    """Values split LoRA keeps instead: k s (r + n)."""
    return k * s * (r + n)


def split_memory_threshold(E: int, m: int, k: int) -> float:
    """Split LoRA needs less memory while s < E m / k."""
    return E * m / k


def peft_flops(E: int, m: int, n: int, r: int, k: int, s: int) -> int:
    """Merge then multiply: E (2 m n r + m n) + 2 k s m n."""
    return E * (2 * m * n * r + m * n) + 2 * k * s * m * n


def split_flops(m: int, n: int, r: int, k: int, s: int) -> int:
    """Split LoRA forward of one projection: 2 k (s m n + s m r + s r n)."""
    return 2 * k * (s * m * n + s * m * r + s * r * n)


def flop_crossover(E: int, m: int, n: int, r: int, k: int) -> float:
    """Token count where the two FLOP counts meet: E m n / (k (m + n)) (1 + 1/(2r))."""
    return E * m * n / (k * (m + n)) * (1.0 + 1.0 / (2 * r))


def layer_flops_fwd(T: int, H: int, I: int, r: int, k: int) -> int:
    """Forward of the whole expert layer: split_flops over gate_up (H -> 2I) and down (I -> H)."""
    return split_flops(H, 2 * I, r, k, T) + split_flops(I, H, r, k, T)
