"""Host-side logic of bench.py (no GPU): kernel-name classification for the
counter runs, the FLOP accounting of every mode, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402

NS = "void moe::(anonymous namespace)::"
ARGS = "(moe::(anonymous namespace)::GemmArgs)"


def name(*t):
    return NS + "gemm16<" + ", ".join(str(x).lower() for x in t) + ">" + ARGS


@pytest.mark.parametrize("f16", [False, True])
def test_classify_gemm(f16):
    big = (f16, 256, 256, 128, 64, 64, 2, 1)
    assert bench.classify_gemm(name(*big, 0, 1, True, True, True, 1)) == "gate_up_fwd"
    assert bench.classify_gemm(name(*big, 0, 0, False, True, True, 1)) == "down_fwd"
    assert bench.classify_gemm(name(*big, 0, 2, False, True, False, 1)) == "down_bwd"
    assert bench.classify_gemm(name(*big, 0, 0, False, True, False, 1)) == "gate_up_bwd"
    # LoRA side products, weight gradients, router projection, merge: not expert GEMMs
    assert bench.classify_gemm(name(f16, 128, 32, 32, 32, 64, 3, 2, 0, 0, False, True, True, 0)) is None
    assert bench.classify_gemm(name(f16, 128, 256, 64, 128, 32, 3, 2, 1, 0, False, False, False, 0)) is None
    assert bench.classify_gemm(name(f16, 128, 256, 64, 128, 32, 3, 2, 0, 4, False, True, False, 0)) is None
    assert bench.classify_gemm(name(f16, 128, 64, 32, 64, 64, 3, 2, 0, 3, False, True, True, 0)) is None
    assert bench.classify_gemm(NS + "combine_kernel<unsigned short>" + ARGS) is None


def test_step_flops_of_every_mode():
    cfg = get_config("gpt-oss-20b")
    N, H, I, r, T, E = cfg.N, cfg.H, cfg.I, cfg.r, cfg.T, cfg.E
    F = 12 * N * H * I + 6 * N * r * (2 * H + 3 * I)
    assert bench.step_flops(cfg, False) == F == cfg.flops_fwd_bwd()
    assert bench.step_flops(cfg, True) == F + 6 * N * H * I
    shared = 12 * T * H * I + 6 * T * r * (2 * H + 3 * I)     # one expert, k = 1, width I
    assert bench.step_flops(cfg, False, I, block=True) == F + 4 * T * E * H + shared
    assert bench.step_flops(cfg, False, None, block=True) == F + 4 * T * E * H


def test_expert_gemm_flops_add_up():
    """The four expert GEMM kernels' FLOPs plus the LoRA side products and
    weight gradients make up the layer's F."""
    cfg = get_config("qwen3-30b-a3b")
    N, H, I, r = cfg.N, cfg.H, cfg.I, cfg.r
    gemms = sum(bench.kernel_flops(k, cfg) for k in ("gate_up_fwd", "down_fwd", "down_bwd",
                                                    "gate_up_bwd"))
    side = 2 * N * r * (H + I) + 2 * N * r * (H + 2 * I)      # X A^T, act A^T, G B_d, dH B_gu
    wgrad = 2 * N * r * (H + I) + 2 * N * r * (2 * I + H)     # dA, dB of both projections
    assert gemms + side + wgrad == cfg.flops_fwd_bwd()


def test_kernel_bytes_cover_the_memory_kernels():
    cfg = get_config("gpt-oss-20b")
    for k in ("route", "permute", "gather", "combine", "combine_bwd", "route_bwd", "unpermute",
              "router_fwd", "router_bwd", "accumulate"):
        assert bench.kernel_bytes(k, cfg) > 0
    assert bench.kernel_bytes("gate_up_fwd", cfg) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
