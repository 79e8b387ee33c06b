"""The seeded input generators: same seed, same tensors; sub-seeds per tensor
(and per expert) so that one tensor's draw does not depend on another's size;
the skewed layers leave their dead experts without tokens."""
import numpy as np
import torch

import oracle
from workloads import PARITY_CONFIGS, make_block_inputs, make_inputs, seed_for
from workloads.synth import zipf_offsets


def test_same_seed_same_tensors_other_seed_other_tensors():
    cfg = PARITY_CONFIGS["mini-bf16"]
    a, b, c = make_inputs(cfg, 5), make_inputs(cfg, 5), make_inputs(cfg, 6)
    for n in a:
        assert torch.equal(a[n], b[n]), n
        assert not torch.equal(a[n], c[n]), n


def test_sub_seeds_are_independent_of_other_sizes():
    cfg = PARITY_CONFIGS["mini-bf16"]
    a = make_inputs(cfg, 7)
    b = make_inputs(cfg.with_(T=cfg.T + 37), 7)          # more tokens: weights unchanged
    for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d"):
        assert torch.equal(a[n], b[n]), n
    c = make_inputs(cfg.with_(E=cfg.E + 2), 7)           # more experts: the first ones unchanged
    assert torch.equal(a["w_gu"], c["w_gu"][:cfg.E])
    assert len({seed_for(1, "x"), seed_for(1, "w_gu", 0), seed_for(1, "w_gu", 1),
                seed_for(2, "x")}) == 4


def test_block_inputs_extend_the_layer_inputs():
    cfg = PARITY_CONFIGS["mini-renorm"]
    a, b = make_inputs(cfg, 3), make_block_inputs(cfg, 3, shared_I=96)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    # the logits are the router projection of x by the returned w_r
    ref = (b["x"].double() @ b["w_r"].double().t()).float()
    assert torch.equal(b["logits"], ref)
    assert b["shared_w_gu"].shape == (192, cfg.H) and b["shared_w_d"].shape == (cfg.H, 96)


def test_bf16_and_f16_layers_hold_exact_16_bit_values():
    for name, dt in (("mini-bf16", torch.bfloat16), ("mini-f16", torch.float16)):
        x = make_inputs(PARITY_CONFIGS[name], 1)["x"]
        assert x.dtype == dt


def test_dead_experts_get_no_tokens():
    for name in ("mini-skew", "tiny-sigmoid", "mini-split", "mini-f16-skew"):
        cfg = PARITY_CONFIGS[name]
        off = zipf_offsets(cfg, 3407)
        dead = np.where(off <= -30.0)[0]
        assert dead.size == cfg.n_dead
        inp = make_inputs(cfg, 3407)
        ids, _ = oracle.route(inp["logits"].numpy(), cfg.k, cfg.router)
        assert not np.isin(ids, dead).any()
