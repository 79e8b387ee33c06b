"""moe_permute_noalloc, the permute whose per-chunk expert counts live in the
library's own device array instead of a caller workspace: through the C ABI,
its outputs equal moe_permute's bit for bit (and the oracle's), on two calls
in a row, the second with a smaller input (the array keeps the first call's
contents, which the second must not read)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, PARITY_CONFIGS, make_inputs
from workloads.synth import to_numpy

from gpu_util import say

pytestmark = pytest.mark.gpu


def _run(mel, cfg, seed, noalloc):
    inp = make_inputs(cfg, seed, device="cuda")
    sh = mel.Shape.of(cfg)
    dev = dict(device="cuda", dtype=torch.int32)
    ids = torch.empty(cfg.T, cfg.k, **dev)
    w = torch.empty(cfg.T, cfg.k, device="cuda", dtype=torch.float32)
    mel.moe_route(inp["logits"], cfg.k, cfg.router, ids, w)
    out = {"counts": torch.full((cfg.E,), -7, **dev), "offsets": torch.full((cfg.E + 1,), -7, **dev),
           "sorted_pair": torch.full((cfg.N,), -7, **dev), "inv_pos": torch.full((cfg.N,), -7, **dev),
           "x_perm": torch.zeros(cfg.N, cfg.H, device="cuda", dtype=sh.torch_dtype)}
    args = (sh, ids, inp["x"], out["counts"], out["offsets"], out["sorted_pair"], out["inv_pos"],
            out["x_perm"])
    if noalloc:
        mel.moe_permute_noalloc(*args)
    else:
        _, _, need = mel.moe_workspace_bytes(sh)
        ws = torch.empty(max(need, 1), device="cuda", dtype=torch.uint8)
        mel.moe_permute(*args, ws)
    torch.cuda.synchronize()
    return ids, inp, out


@pytest.mark.parametrize("big,small", [("qwen3-30b-a3b", "mini-skew"),
                                       ("gpt-oss-20b-long", "max-E-k"),
                                       ("gpt-oss-20b", "mini-T1")])
def test_noalloc_permute_matches_workspace_permute(big, small):
    import mixture_experts_lora_amd as mel
    for name in (big, small):
        cfg = CONFIGS.get(name) or PARITY_CONFIGS[name]
        say(f"[noalloc permute] {name} T={cfg.T} E={cfg.E} k={cfg.k}")
        ids, inp, got = _run(mel, cfg, 3, noalloc=True)
        _, _, ref = _run(mel, cfg, 3, noalloc=False)
        for n in got:
            assert torch.equal(got[n], ref[n]), n
        counts, offsets, sp, inv = oracle.permute(to_numpy(ids), cfg.E)
        np.testing.assert_array_equal(to_numpy(got["counts"]), counts)
        np.testing.assert_array_equal(to_numpy(got["offsets"]), offsets)
        np.testing.assert_array_equal(to_numpy(got["sorted_pair"]), sp)
        np.testing.assert_array_equal(to_numpy(got["inv_pos"]), inv)
        rows = torch.from_numpy(sp // cfg.k).cuda().long()
        assert torch.equal(got["x_perm"], inp["x"][rows])
