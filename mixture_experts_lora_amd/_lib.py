"""ctypes declarations of libmoe_lora.so (the C ABI in include/moe_lora.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_lora.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
ROUTER_IDS = {"softmax_topk": 0, "softmax_topk_renorm": 1, "topk_softmax": 2,
              "sigmoid_topk_renorm": 3}
KERNEL_IDS = {"route": 0, "permute": 1, "gather": 2, "gate_up_fwd": 3, "down_fwd": 4,
              "combine": 5, "combine_bwd": 6, "route_bwd": 7, "down_bwd": 8, "gate_up_bwd": 9,
              "lora_side": 10, "lora_wgrad": 11, "unpermute": 12, "base_wgrad": 13,
              "router_fwd": 14, "router_bwd": 15, "accumulate": 16, "merge": 17,
              "dy_gather": 18, "dw_sum": 19, "row_scale": 20}

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_route_bwd", "moe_permute",
           "moe_grouped_lora_fwd", "moe_unpermute_combine", "moe_unpermute_combine_bwd",
           "moe_grouped_lora_bwd", "moe_grouped_full_bwd", "moe_workspace_bytes_lean",
           "moe_grouped_lora_fwd_lean", "moe_grouped_lora_bwd_recompute",
           "moe_router_workspace_bytes", "moe_router_fwd", "moe_router_bwd", "moe_accumulate",
           "moe_merge_workspace_bytes", "moe_merge_lora", "moe_permute_noalloc",
           "moe_grouped_lora_combine_bwd", "moe_grouped_lora_fwd_gather",
           "moe_grouped_lora_combine_bwd_gather",
           "moe_status_str",
           "moe_last_error",
           "moe_kernel_timer_enable", "moe_kernel_timer_select", "moe_kernel_timer_reset",
           "moe_kernel_timer_read")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("r", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("lora_scale", ctypes.c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gu", "a_gu", "b_gu", "w_d", "a_d", "b_d")]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("h", "act", "u_gu", "u_d", "y_exp")]


class MoeLoraGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("da_gu", "db_gu", "da_d", "db_d")]


class MoeBaseGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dw_gu", "dw_d")]


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m mixture_experts_lora_amd.build` "
            "(hipcc, gfx950). There is no non-HIP implementation of this layer.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    st = ctypes.c_int
    sig = {
        "moe_workspace_bytes": (st, [ctypes.POINTER(MoeShape), ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_size_t)]),
        "moe_route": (st, [P, I32, I32, I32, I32, P, P, P]),
        "moe_route_bwd": (st, [P, P, P, I32, I32, I32, I32, P, P]),
        "moe_permute": (st, [ctypes.POINTER(MoeShape), P, P, P, P, P, P, P, P, ctypes.c_size_t,
                             P]),
        "moe_permute_noalloc": (st, [ctypes.POINTER(MoeShape), P, P, P, P, P, P, P, P]),
        "moe_grouped_lora_fwd": (st, [ctypes.POINTER(MoeShape), P, P,
                                      ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeSaved), P,
                                      ctypes.c_size_t, P]),
        "moe_unpermute_combine": (st, [ctypes.POINTER(MoeShape), P, P, P, P, P]),
        "moe_unpermute_combine_bwd": (st, [ctypes.POINTER(MoeShape), P, P, P, P, P, P, P]),
        "moe_grouped_lora_bwd": (st, [ctypes.POINTER(MoeShape), P, P, P,
                                      ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeSaved), P,
                                      ctypes.POINTER(MoeLoraGrads), P, ctypes.c_size_t, P]),
        "moe_grouped_full_bwd": (st, [ctypes.POINTER(MoeShape), P, P, P,
                                      ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeSaved), P,
                                      ctypes.POINTER(MoeLoraGrads), ctypes.POINTER(MoeBaseGrads),
                                      P, ctypes.c_size_t, P]),
        "moe_workspace_bytes_lean": (st, [ctypes.POINTER(MoeShape),
                                          ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)]),
        "moe_grouped_lora_fwd_lean": (st, [ctypes.POINTER(MoeShape), P, P,
                                           ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeSaved),
                                           P, ctypes.c_size_t, P]),
        "moe_grouped_lora_bwd_recompute": (st, [ctypes.POINTER(MoeShape), P, P, P,
                                                ctypes.POINTER(MoeWeights),
                                                ctypes.POINTER(MoeSaved), P,
                                                ctypes.POINTER(MoeLoraGrads),
                                                ctypes.POINTER(MoeBaseGrads), P, ctypes.c_size_t,
                                                P]),
        "moe_grouped_lora_combine_bwd": (st, [ctypes.POINTER(MoeShape), P, P, P, P, P, P,
                                              ctypes.POINTER(MoeWeights),
                                              ctypes.POINTER(MoeSaved), I32, P, P,
                                              ctypes.POINTER(MoeLoraGrads),
                                              ctypes.POINTER(MoeBaseGrads), P, P,
                                              ctypes.c_size_t, P]),
        "moe_grouped_lora_combine_bwd_gather": (st, [ctypes.POINTER(MoeShape), P, P, P, P, P, P,
                                                     ctypes.POINTER(MoeWeights),
                                                     ctypes.POINTER(MoeSaved), I32, P, P,
                                                     ctypes.POINTER(MoeLoraGrads),
                                                     ctypes.POINTER(MoeBaseGrads), P, P,
                                                     ctypes.c_size_t, P]),
        "moe_grouped_lora_fwd_gather": (st, [ctypes.POINTER(MoeShape), P, P, P,
                                             ctypes.POINTER(MoeWeights),
                                             ctypes.POINTER(MoeSaved), I32, P, ctypes.c_size_t,
                                             P]),
        "moe_router_workspace_bytes": (st, [I32, I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_router_fwd": (st, [P, P, I32, I32, I32, I32, P, P, ctypes.c_size_t, P]),
        "moe_router_bwd": (st, [P, P, I32, I32, I32, I32, P, P, ctypes.c_size_t, P]),
        "moe_accumulate": (st, [I32, ctypes.c_int64, P, P, P]),
        "moe_merge_workspace_bytes": (st, [ctypes.POINTER(MoeShape),
                                           ctypes.POINTER(ctypes.c_size_t)]),
        "moe_merge_lora": (st, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), P, P, P,
                                ctypes.c_size_t, P]),
        "moe_status_str": (ctypes.c_char_p, [st]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_kernel_timer_enable": (st, [I32]),
        "moe_kernel_timer_select": (st, [ctypes.c_uint32]),
        "moe_kernel_timer_reset": (st, []),
        "moe_kernel_timer_read": (st, [I32, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int32)]),
    }
    # every export gets an explicit signature (sizes are 64-bit size_t)
    assert set(sig) == set(EXPORTS), sorted(set(EXPORTS) ^ set(sig))
    for name, (res, args) in sig.items():
        try:
            fn = getattr(lib, name)
        except AttributeError:
            # an older build of the library: refuse it (and let the build module import)
            raise RuntimeError(f"{LIB_PATH} lacks {name}: it is out of date, rebuild it with "
                               "`python -m mixture_experts_lora_amd.build`") from None
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        detail = lib.moe_last_error().decode()
        super().__init__(f"{where}: {lib.moe_status_str(status).decode()} ({detail})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)
