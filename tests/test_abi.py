"""The C ABI on the CPU: the library loads, exports every entry point the header
declares, sizes its workspaces, and rejects bad arguments before touching the
GPU (each call here fails validation, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_lora.h")


@pytest.fixture(scope="module")
def lib():
    from mixture_experts_lora_amd import _lib
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_layer_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_lora_fwd", "moe_grouped_lora_bwd",
              "moe_unpermute_combine"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    from mixture_experts_lora_amd import _lib
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(_lib.EXPORTS)


def shape(T=64, H=128, I=64, E=8, k=2, r=16, dtype=1, s=1.0):
    from mixture_experts_lora_amd._lib import MoeShape
    return MoeShape(T, H, I, E, k, r, dtype, s)


def ws(lib, sh):
    f, b, p = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = lib.moe_workspace_bytes(ctypes.byref(sh), ctypes.byref(f), ctypes.byref(b), ctypes.byref(p))
    return st, f.value, b.value, p.value


def test_workspace_never_holds_a_merged_delta(lib):
    from workloads import CONFIGS
    for cfg in CONFIGS.values():
        sh = shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.r,
                   {"f32": 0, "bf16": 1, "f16": 2}[cfg.dtype])
        st, f, b, p = ws(lib, sh)
        assert st == 0
        esz = 4 if cfg.dtype == "f32" else 2
        delta = cfg.E * 2 * cfg.I * cfg.H * esz   # one materialised W + B A for gate_up
        # forward scratch is a tile list only; backward holds dH [N, 2I], four
        # [N, r] (G B_d, dH B_gu, and for the folded combine backward w u_d and
        # w G B_d), for 16-bit layers the float32 partials of the side
        # products fused into the B gradients (one [N, r] per 256 features of
        # the wider of H and 2I), the routing weight per row and the dw
        # partial sums (float32 [slots, N], a slot per 64 columns of I);
        # these layers have experts enough for no split-K partials
        assert f < 1 << 20
        side = -(-max(cfg.H, 2 * cfg.I) // 256) * cfg.N * cfg.r * 4 if cfg.dtype != "f32" else 0
        slots = -(-cfg.I // 64) if cfg.dtype == "f32" else -(-cfg.I // 256) * 4
        assert b <= (cfg.N * (2 * cfg.I + 4 * cfg.r) * esz + side + cfg.N * 4 * (1 + slots)
                     + (1 << 20))
        if cfg.T * cfg.k < cfg.E * cfg.H:            # the regime the pages' memory model favours
            assert b < delta
        assert p > 0


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), 1), (dict(k=0), 1), (dict(k=9), 1), (dict(E=0), 1), (dict(E=2000, k=2), 1),
    (dict(H=100), 2), (dict(I=12), 2), (dict(r=65), 2), (dict(r=0), 1), (dict(dtype=7), 1),
    (dict(k=40, E=64), 2),
    # one activation tensor above 32 GiB: N * 2I * 2 bytes = 2^25 * 2048 * 2 = 2^37
    (dict(T=1 << 22, k=8, E=8, I=1024, H=1024), 1),
    # one expert's weight matrix of 2 GiB (2I * H * 2 bytes = 2^31)
    (dict(H=32768, I=16384), 1),
    (dict(H=32768, I=16384, dtype=0), 1),
])
def test_shape_validation(lib, kw, status):
    st, *_ = ws(lib, shape(**kw))
    assert st == status
    assert lib.moe_last_error()


def test_shape_limits_at_the_edge(lib):
    """The largest accepted sizes: a 32 GiB activation tensor and an expert
    weight matrix just under 2 GiB."""
    # N * 2I * 2 bytes = 2^22 * 2^12 * 2 = 2^35 exactly
    st, *_ = ws(lib, shape(T=1 << 19, k=8, E=8, I=2048, H=1024))
    assert st == 0
    st, *_ = ws(lib, shape(T=1 << 19, k=8, E=8, I=2056, H=1024))
    assert st == 1
    # 2I * H * 2 bytes = 2^31 - 2^16
    st, *_ = ws(lib, shape(T=8, H=32768 - 8, I=16384, k=2, E=8))
    assert st == 0


def test_null_pointers_rejected(lib):
    P = ctypes.c_void_p
    fake = P(0x10000)
    sh = shape()
    assert lib.moe_route(None, 64, 8, 2, 0, fake, fake, None) == 1
    assert lib.moe_route(fake, 64, 8, 2, 9, fake, fake, None) == 1        # unknown router
    assert lib.moe_route(fake, 64, 8, 9, 0, fake, fake, None) == 1        # k > E
    assert lib.moe_route_bwd(fake, fake, fake, 64, 8, 2, 0, None, None) == 1
    assert lib.moe_permute(ctypes.byref(sh), None, fake, fake, fake, fake, fake, fake, fake,
                           1 << 30, None) == 1
    assert lib.moe_unpermute_combine(ctypes.byref(sh), fake, fake, None, None, None) == 1
    assert lib.moe_unpermute_combine_bwd(ctypes.byref(sh), fake, fake, fake, None, fake, fake,
                                         None) == 1
    from mixture_experts_lora_amd._lib import MoeLoraGrads, MoeSaved, MoeWeights
    w = MoeWeights(*(0x10000,) * 6)
    sv = MoeSaved(0x10000, 0x10000, 0x10000, 0x10000, None)
    assert lib.moe_grouped_lora_fwd(ctypes.byref(sh), fake, fake, ctypes.byref(w), ctypes.byref(sv),
                                    fake, 1 << 30, None) == 1           # y_exp missing
    g = MoeLoraGrads(0x10000, None, 0x10000, 0x10000)
    assert lib.moe_grouped_lora_bwd(ctypes.byref(sh), fake, fake, fake, ctypes.byref(w),
                                    ctypes.byref(sv), P(0x20000), ctypes.byref(g), fake, 1 << 30,
                                    None) == 1


def test_token_rows_must_be_16_byte_aligned(lib):
    """The gather and combine kernels move token rows in 16-byte pieces: their
    row buffers off a 16-byte boundary are refused before any launch."""
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x20002)
    sh = shape()
    ws_bytes = 1 << 30
    # moe_permute with a gather: x, x_perm
    assert lib.moe_permute(ctypes.byref(sh), fake, odd, fake, fake, fake, fake, P(0x30000), fake,
                           ws_bytes, None) == 1
    assert b"16-byte" in lib.moe_last_error()
    assert lib.moe_permute(ctypes.byref(sh), fake, P(0x30000), fake, fake, fake, fake, odd, fake,
                           ws_bytes, None) == 1
    assert lib.moe_permute_noalloc(ctypes.byref(sh), fake, odd, fake, fake, fake, fake,
                                   P(0x30000), None) == 1
    # combine (and unpermute): y_perm, y
    assert lib.moe_unpermute_combine(ctypes.byref(sh), odd, fake, None, P(0x30000), None) == 1
    assert lib.moe_unpermute_combine(ctypes.byref(sh), fake, fake, None, odd, None) == 1
    # combine backward: dy, y_exp, dy_perm
    for args in ((odd, fake, P(0x30000)), (fake, odd, P(0x30000)), (fake, P(0x40000), odd)):
        dy, y_exp, dy_perm = args
        assert lib.moe_unpermute_combine_bwd(ctypes.byref(sh), dy, y_exp, fake, fake, dy_perm,
                                             fake, None) == 1
    # the folded combine backward: dy, dy_perm
    from mixture_experts_lora_amd._lib import MoeLoraGrads, MoeSaved, MoeWeights
    w = MoeWeights(*(0x10000,) * 6)
    sv = MoeSaved(*(0x30000 + i * 0x1000 for i in range(5)))
    g = MoeLoraGrads(*(0x50000 + i * 0x1000 for i in range(4)))
    for dy, dy_perm in ((odd, P(0x60000)), (fake, odd)):
        assert lib.moe_grouped_lora_combine_bwd(
            ctypes.byref(sh), dy, fake, fake, fake, P(0x70000), fake, ctypes.byref(w),
            ctypes.byref(sv), 0, dy_perm, P(0x80000), ctypes.byref(g), None, fake, fake,
            ws_bytes, None) == 1
        assert b"16-byte" in lib.moe_last_error()


def test_gather_backward_dy_perm_rules(lib):
    """moe_grouped_lora_combine_bwd_gather with dy_perm = NULL reads dY's rows
    in token order; that is refused before any launch for full fine-tuning
    (dW_d is formed from w dY in expert order) and for H <= 32, and a given
    dy_perm must be 16-byte aligned."""
    P = ctypes.c_void_p
    fake, odd = P(0x10000), P(0x20002)
    sh = shape()
    from mixture_experts_lora_amd._lib import MoeBaseGrads, MoeLoraGrads, MoeSaved, MoeWeights
    w = MoeWeights(*(0x10000,) * 6)
    sv = MoeSaved(*(0x30000 + i * 0x1000 for i in range(5)))
    g = MoeLoraGrads(*(0x50000 + i * 0x1000 for i in range(4)))
    b = MoeBaseGrads(0x90000, 0xa0000)

    def call(dy_perm, base, sh=sh):
        return lib.moe_grouped_lora_combine_bwd_gather(
            ctypes.byref(sh), fake, fake, fake, fake, P(0x70000), fake, ctypes.byref(w),
            ctypes.byref(sv), 0, dy_perm, P(0x80000), ctypes.byref(g), base, fake, fake,
            1 << 30, None)

    assert call(None, ctypes.byref(b)) == 1
    assert b"dy_perm is required with base" in lib.moe_last_error()
    assert call(None, None, shape(H=32)) == 1
    assert b"dy_perm is required for H <= 32" in lib.moe_last_error()
    assert call(odd, None) == 1
    assert b"16-byte" in lib.moe_last_error()


def test_noalloc_permute_rejects_tables_beyond_its_array(lib):
    """moe_permute_noalloc's table (E * ceil(T k / 64) int32) must fit its
    4 MiB device array; a larger one is refused before any GPU call."""
    P = ctypes.c_void_p
    fake = P(0x10000)
    # E = 1024, N = 65600 pairs: 1024 * 1025 * 4 bytes > 4 MiB
    sh = shape(T=65600, k=1, E=1024, H=64, I=32)
    st = lib.moe_permute_noalloc(ctypes.byref(sh), fake, None, fake, fake, fake, fake, None, None)
    assert st == 2
    assert b"4194304" in lib.moe_last_error()
    assert lib.moe_permute_noalloc(ctypes.byref(shape()), None, None, fake, fake, fake, fake,
                                   None, None) == 1


def test_short_workspace_rejected(lib):
    P = ctypes.c_void_p
    fake = P(0x10000)
    sh = shape()
    st, f, b, p = ws(lib, sh)
    from mixture_experts_lora_amd._lib import MoeLoraGrads, MoeSaved, MoeWeights
    w = MoeWeights(*(0x10000,) * 6)
    sv = MoeSaved(*(0x30000 + i * 0x1000 for i in range(5)))
    g = MoeLoraGrads(*(0x50000 + i * 0x1000 for i in range(4)))
    assert lib.moe_permute(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, P(0x20000), fake,
                           p - 1, None) == 3
    assert lib.moe_grouped_lora_fwd(ctypes.byref(sh), fake, fake, ctypes.byref(w), ctypes.byref(sv),
                                    fake, f - 1, None) == 3
    assert lib.moe_grouped_lora_bwd(ctypes.byref(sh), fake, P(0x60000), fake, ctypes.byref(w),
                                    ctypes.byref(sv), P(0x70000), ctypes.byref(g), fake, b - 1,
                                    None) == 3


def test_full_ft_and_lean_entry_points_validate(lib):
    """The full fine-tuning and activation-lean calls check their extra
    arguments (and workspace sizes) before anything is launched."""
    P = ctypes.c_void_p
    fake = P(0x10000)
    sh = shape()
    from mixture_experts_lora_amd._lib import MoeBaseGrads, MoeLoraGrads, MoeSaved, MoeWeights
    w = MoeWeights(*(0x10000,) * 6)
    sv = MoeSaved(*(0x30000 + i * 0x1000 for i in range(5)))
    g = MoeLoraGrads(*(0x50000 + i * 0x1000 for i in range(4)))
    _, f, b, _ = ws(lib, sh)
    fl, bl = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.moe_workspace_bytes_lean(ctypes.byref(sh), ctypes.byref(fl), ctypes.byref(bl)) == 0
    # the lean calls hold h [N, 2I] and act [N, I] in their workspaces
    extra = sh.T * sh.k * 3 * sh.I * 2
    assert fl.value >= f + extra and bl.value >= b + extra
    args = (ctypes.byref(sh), fake, P(0x60000), fake, ctypes.byref(w), ctypes.byref(sv),
            P(0x70000), ctypes.byref(g))
    # full fine-tuning: base grads required, not aliased
    assert lib.moe_grouped_full_bwd(*args, None, fake, 1 << 40, None) == 1
    assert lib.moe_grouped_full_bwd(*args, ctypes.byref(MoeBaseGrads(0x80000, None)), fake,
                                    1 << 40, None) == 1
    assert lib.moe_grouped_full_bwd(*args, ctypes.byref(MoeBaseGrads(0x80000, 0x80000)), fake,
                                    1 << 40, None) == 1
    assert lib.moe_grouped_full_bwd(*args, ctypes.byref(MoeBaseGrads(0x80000, 0x70000)), fake,
                                    1 << 40, None) == 1          # dw_d aliases dx_perm
    assert lib.moe_grouped_full_bwd(*args, ctypes.byref(MoeBaseGrads(0x80000, 0x90000)), fake,
                                    b - 1, None) == 3
    # lean mode: h and act may be NULL; the larger workspace is required
    lean = MoeSaved(None, None, 0x30000, 0x31000, 0x32000)
    assert lib.moe_grouped_lora_fwd_lean(ctypes.byref(sh), fake, fake, ctypes.byref(w),
                                         ctypes.byref(lean), fake, fl.value - 1, None) == 3
    assert lib.moe_grouped_lora_fwd(ctypes.byref(sh), fake, fake, ctypes.byref(w),
                                    ctypes.byref(lean), fake, 1 << 40, None) == 1
    assert lib.moe_grouped_lora_bwd_recompute(ctypes.byref(sh), fake, P(0x60000), fake,
                                              ctypes.byref(w), ctypes.byref(lean), P(0x70000),
                                              ctypes.byref(g), None, fake, bl.value - 1,
                                              None) == 3


def test_router_and_accumulate_validate(lib):
    """Router projection and accumulate: dimensions, dtype, workspace and
    aliasing are checked on the host before any launch."""
    P = ctypes.c_void_p
    fake = P(0x10000)
    n = ctypes.c_size_t()
    assert lib.moe_router_workspace_bytes(4096, 2880, 32, 1, ctypes.byref(n)) == 0
    need_bf16 = n.value
    assert need_bf16 >= 4096 * 32 * 2            # bf16 copy of d_logits for the MFMA
    assert lib.moe_router_workspace_bytes(4096, 2880, 32, 0, ctypes.byref(n)) == 0
    assert n.value < need_bf16
    assert lib.moe_router_workspace_bytes(4096, 2882, 32, 1, ctypes.byref(n)) == 2  # H % 8
    assert lib.moe_router_workspace_bytes(4096, 2880, 1025, 1, ctypes.byref(n)) == 1
    assert lib.moe_router_workspace_bytes(0, 2880, 32, 1, ctypes.byref(n)) == 1
    assert lib.moe_router_workspace_bytes(16, 64, 8, 7, ctypes.byref(n)) == 1       # dtype
    assert lib.moe_router_workspace_bytes(16, 64, 8, 1, None) == 1
    args = (fake, P(0x20000), 4096, 2880, 32, 1)
    assert lib.moe_router_fwd(*args, P(0x30000), P(0x40000), need_bf16 - 1, None) == 3
    assert lib.moe_router_fwd(*args, None, P(0x40000), need_bf16, None) == 1
    assert lib.moe_router_fwd(*args, fake, P(0x40000), need_bf16, None) == 1  # logits is x
    assert lib.moe_router_bwd(*args, P(0x30000), None, need_bf16, None) == 1
    assert lib.moe_router_bwd(*args, P(0x30000), P(0x40000), need_bf16 - 1, None) == 3
    assert lib.moe_router_bwd(*args, fake, P(0x40000), need_bf16, None) == 1  # dx is d_logits
    assert lib.moe_accumulate(1, 0, None, None, None) == 0                 # empty: nothing to do
    assert lib.moe_accumulate(1, -1, fake, P(0x20000), None) == 1
    assert lib.moe_accumulate(3, 16, fake, P(0x20000), None) == 1            # no such dtype
    assert lib.moe_accumulate(1, 16, fake, fake, None) == 1
    assert lib.moe_accumulate(1, 16, fake, P(0x10000 + 30), None) == 1   # partial overlap
    assert lib.moe_accumulate(0, 16, P(0x10000 + 60), fake, None) == 1    # f32: 64 bytes


def test_merge_validates(lib):
    """Merged export: shape, outputs, aliasing and workspace checked on the host."""
    P = ctypes.c_void_p
    from mixture_experts_lora_amd._lib import MoeShape, MoeWeights
    sh = MoeShape(0, 2880, 2880, 32, 0, 16, 1, 1.0)      # T and k are not read
    n = ctypes.c_size_t()
    assert lib.moe_merge_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)) == 0
    need = n.value
    assert 0 < need < (1 << 20)
    w = MoeWeights(*(0x10000 + i * 0x1000 for i in range(6)))   # w_gu a_gu b_gu w_d a_d b_d
    ws = P(0x90000)
    args = (ctypes.byref(sh), ctypes.byref(w))
    assert lib.moe_merge_lora(*args, None, None, ws, need, None) == 1          # nothing to do
    assert lib.moe_merge_lora(*args, P(0x80000), None, ws, need - 1, None) == 3
    assert lib.moe_merge_lora(*args, P(0x11000), None, ws, need, None) == 1    # a_gu
    assert lib.moe_merge_lora(*args, None, P(0x15000), ws, need, None) == 1    # b_d
    assert lib.moe_merge_lora(*args, P(0x13000), None, ws, need, None) == 1    # w_d
    assert lib.moe_merge_lora(*args, P(0x80000), P(0x80000), ws, need, None) == 1
    assert lib.moe_merge_lora(*args, None, P(0x10000), ws, need, None) == 1    # w_gu
    assert lib.moe_merge_lora(*args, P(0x80000), None, None, need, None) == 1
    bad = MoeShape(0, 2882, 2880, 32, 0, 16, 1, 1.0)
    assert lib.moe_merge_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == 2
    bad = MoeShape(0, 2880, 2880, 32, 0, 65, 1, 1.0)
    assert lib.moe_merge_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == 2
    bad = MoeShape(0, 2880, 2880, 0, 0, 16, 1, 1.0)
    assert lib.moe_merge_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == 1


def test_aliasing_rejected(lib):
    P = ctypes.c_void_p
    fake = P(0x10000)
    sh = shape()
    assert lib.moe_unpermute_combine(ctypes.byref(sh), fake, P(0x20000), None, fake, None) == 1
    assert lib.moe_route_bwd(fake, P(0x20000), P(0x30000), 64, 8, 2, 0, fake, None) == 1


def test_status_strings(lib):
    for st in range(5):
        assert lib.moe_status_str(st)


def test_python_binding_checks_shapes_on_host():
    import torch
    import mixture_experts_lora_amd as mel
    with pytest.raises(ValueError):
        mel.moe_route(torch.zeros(4, 8), 2, "topk_softmax", torch.zeros(4, 2, dtype=torch.int32),
                      torch.zeros(4, 2))          # CPU tensors are refused before any call



def test_kernel_timer_selection(lib):
    """The timer can be restricted to chosen kernels (host-side state only)."""
    import mixture_experts_lora_amd as mel
    from mixture_experts_lora_amd import _lib
    assert mel.kernel_timer(only=["gate_up_fwd"]).mask == 1 << _lib.KERNEL_IDS["gate_up_fwd"]
    assert mel.kernel_timer(only=["route", "merge"]).mask == (1 << 0) | (1 << 17)
    assert mel.kernel_timer().mask == 0xFFFFFFFF
    assert lib.moe_kernel_timer_select(0) == 0
    assert lib.moe_kernel_timer_select(0xFFFFFFFF) == 0
