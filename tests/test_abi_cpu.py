"""Host-side checks of the C-ABI library that need no GPU.

The library loads, exports every function include/moe.h declares, sizes its
workspaces consistently, and rejects bad arguments on the host before it
would launch anything (so none of these calls reaches the GPU).
"""
import ctypes
import os
import re

import pytest

import routed_mixture_experts_amd as moe
from routed_mixture_experts_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\*?\s+\*?(moe_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m routed_mixture_experts_amd.build)")
    return L.load()


def test_header_declares_the_five_calls():
    names = _declared_functions()
    for n in ["moe_route", "moe_permute", "moe_experts", "moe_combine", "moe_forward"]:
        assert n in names
    assert sorted(L.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(5):
        assert lib.moe_status_string(st)
    assert b"unknown" in lib.moe_status_string(99)


def _cfg(**kw):
    base = dict(num_experts=16, top_k=4)
    base.update(kw)
    return moe.RouteConfig(**base).c()


@pytest.mark.parametrize("kw,code", [
    (dict(num_experts=0), L.MOE_EINVAL),
    (dict(top_k=0), L.MOE_EINVAL),
    (dict(top_k=17), L.MOE_EINVAL),               # k > E
    (dict(num_experts=2048, top_k=4), L.MOE_ENOTSUP),
    (dict(top_k=33, num_experts=64), L.MOE_ENOTSUP),
    (dict(num_groups=3), L.MOE_EINVAL),           # E % G != 0
    (dict(num_groups=4, topk_group=5), L.MOE_EINVAL),
    (dict(num_groups=8, topk_group=1), L.MOE_EINVAL),   # 1 group of 2 < k
    (dict(num_groups=16, topk_group=16, group_score="top2sum"), L.MOE_EINVAL),
])
def test_route_rejects_bad_config(lib, kw, code):
    c = _cfg(**kw)
    st = lib.moe_route(ctypes.byref(c), 8, ctypes.c_void_p(16), None, ctypes.c_void_p(16),
                       ctypes.c_void_p(16), None)
    assert st == code


def test_route_null_pointers_and_empty(lib):
    c = _cfg()
    assert lib.moe_route(ctypes.byref(c), 8, None, None, None, None, None) == L.MOE_EINVAL
    assert lib.moe_route(ctypes.byref(c), -1, None, None, None, None, None) == L.MOE_EINVAL
    assert lib.moe_route(None, 8, None, None, None, None, None) == L.MOE_EINVAL
    # T == 0 launches nothing and succeeds
    assert lib.moe_route(ctypes.byref(c), 0, None, None, None, None, None) == L.MOE_OK


def test_workspace_sizes_grow_with_capacity(lib):
    a = lib.moe_permute_workspace(128, 8, 384)
    b = lib.moe_permute_workspace(8192, 8, 384)
    assert 0 < a < b
    e1 = lib.moe_experts_workspace(L.MOE_DTYPE_BF16, 128, 8, 384, 7168, 2048)
    e2 = lib.moe_experts_workspace(L.MOE_DTYPE_BF16, 8192, 8, 384, 7168, 2048)
    # the intermediate h alone is P * I bf16 values
    assert e1 >= 128 * 8 * 2048 * 2 and e2 >= 8192 * 8 * 2048 * 2 and e2 > e1
    c = _cfg(num_experts=384, top_k=8)
    f = lib.moe_forward_workspace(ctypes.byref(c), L.MOE_DTYPE_BF16, 8192, 7168, 2048, None,
                                  None)
    # the expert rows dominate: P * D fp16 values in a bf16 layer, fp32 in an
    # fp32 one
    assert f >= 8192 * 8 * 7168 * 2
    f32 = lib.moe_forward_workspace(ctypes.byref(c), L.MOE_DTYPE_F32, 8192, 7168, 2048, None,
                                    None)
    assert f32 >= 8192 * 8 * 7168 * 4
    assert lib.moe_forward_workspace(ctypes.byref(c), 7, 128, 7168, 2048, None, None) == 0


@pytest.mark.parametrize("E,H,latent", [(384, 7168, None), (256, 4096, None), (16, 1024, 320),
                                         (256, 7168, 2048), (1000, 512, None)])
def test_forward_workspace_never_shrinks_with_capacity(lib, E, H, latent):
    # A workspace sized for max_T must be accepted for every T <= max_T: the
    # forward checks ws_bytes against the size for its own T.  The partial
    # sums of the K-sliced router and latent products peak at different
    # batch sizes, so the size is checked at every batch size up to 2100 and
    # at the band edges of larger ones.
    c = _cfg(num_experts=E, top_k=8)
    lat = None
    if latent:
        # the size query checks the description but reads no weights
        lat = L.moe_latent_t(w_down=256, gamma=256, w_up=256, latent=latent, rms_eps=1e-6)
    sizes = []
    Ts = list(range(1, 2101)) + [4095, 4096, 4097, 8191, 8192, 8193, 16384, 32768, 40000]
    for T in Ts:
        n = lib.moe_forward_workspace(ctypes.byref(c), L.MOE_DTYPE_BF16, T, H, 256,
                                      ctypes.byref(lat) if lat else None, None)
        assert n > 0, T
        sizes.append(n)
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))


def test_forward_rejects_unaligned_and_missing(lib):
    c = _cfg(num_experts=8, top_k=2)
    # H not a multiple of 64
    st = lib.moe_forward(ctypes.byref(c), L.MOE_DTYPE_BF16, 4, 100, 64, *([None] * 15), None, 0,
                         None)
    assert st == L.MOE_ENOTSUP
    # missing weights
    st = lib.moe_forward(ctypes.byref(c), L.MOE_DTYPE_BF16, 4, 128, 64, *([None] * 15), None, 0,
                         None)
    assert st == L.MOE_EINVAL
    # workspace too small (pointers only need to be non-null for the check)
    p = ctypes.c_void_p(256)
    st = lib.moe_forward(ctypes.byref(c), L.MOE_DTYPE_BF16, 4, 128, 64, p, p, None, None, None,
                         p, p, None, None, p, None, None, None, None, None, p, 16, None)
    assert st == L.MOE_ENOSPACE
    lat = L.moe_latent_t(p, p, p, 100, 1e-6)
    st = lib.moe_forward(ctypes.byref(c), L.MOE_DTYPE_BF16, 4, 128, 64, p, p, None, None, None,
                         p, p, ctypes.byref(lat), None, p, None, None, None, None, None, p,
                         1 << 30, None)
    assert st == L.MOE_ENOTSUP


def test_experts_and_combine_validation(lib):
    p = ctypes.c_void_p(256)
    assert lib.moe_experts(L.MOE_DTYPE_BF16, 4, 2, 8, 100, 64, p, p, p, p, p, p, p, 1 << 20,
                           None) == L.MOE_ENOTSUP
    assert lib.moe_experts(L.MOE_DTYPE_BF16, 4, 2, 8, 128, 64, p, p, p, p, p, p, p, 16,
                           None) == L.MOE_ENOSPACE
    assert lib.moe_experts(L.MOE_DTYPE_BF16, 0, 2, 8, 128, 64, None, None, None, None, None,
                           None, None, 0, None) == L.MOE_OK
    assert lib.moe_combine(L.MOE_DTYPE_BF16, 4, 2, 6, p, p, p, p, None) == L.MOE_ENOTSUP
    assert lib.moe_combine(L.MOE_DTYPE_BF16, 4, 40, 8, p, p, p, p, None) == L.MOE_ENOTSUP
    assert lib.moe_combine(L.MOE_DTYPE_BF16, 0, 2, 8, None, None, None, None, None) == L.MOE_OK
    assert lib.moe_permute(4, 9, 8, p, p, p, p, p, p, 1 << 20, None) == L.MOE_EINVAL
    assert lib.moe_permute(4, 2, 8, p, p, p, p, p, p, 0, None) == L.MOE_ENOSPACE


# ---------------------------------------------------- widened entry points ---
# Host-side validation only: every case below returns before anything is
# launched (T = 0 is valid and launches nothing), so no GPU is needed.

def _ew(fmt=L.MOE_WEIGHT_DTYPE, scales=True, act=0, alpha=1.702, limit=7.0):
    p = ctypes.c_void_p(256)
    s = p if scales else None
    return L.moe_expert_weights_t(fmt, p, p, s, s, act, alpha, limit)


def _experts_ex(lib, desc, dtype=L.MOE_DTYPE_BF16, T=4, D=128, I=128):
    p = ctypes.c_void_p(256)
    return lib.moe_experts_ex(dtype, T, 2, 8, D, I, p, p, p,
                              ctypes.byref(desc) if desc is not None else None, p, p, 16, None)


def test_experts_ex_rejects_bad_descriptions(lib):
    assert _experts_ex(lib, None) == L.MOE_EINVAL
    assert _experts_ex(lib, _ew(fmt=9)) == L.MOE_EINVAL
    assert _experts_ex(lib, _ew(act=4)) == L.MOE_EINVAL
    assert _experts_ex(lib, _ew(act=-1)) == L.MOE_EINVAL
    clip = L.ACTIVATIONS["swiglu_clip"]
    assert _experts_ex(lib, _ew(act=clip, alpha=0.0)) == L.MOE_EINVAL
    assert _experts_ex(lib, _ew(act=clip, limit=-1.0)) == L.MOE_EINVAL
    # quantised weights need a bf16 layer
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_FP8_E4M3), L.MOE_DTYPE_F32) == L.MOE_ENOTSUP
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_MXFP4), L.MOE_DTYPE_F32) == L.MOE_ENOTSUP
    # MXFP4 reads 128 elements per load unit along both reduction widths
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_MXFP4), D=192) == L.MOE_ENOTSUP
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_MXFP4), I=192) == L.MOE_ENOTSUP
    # missing scales of a quantised format
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_FP8_E4M3, scales=False)) == L.MOE_EINVAL
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_MXFP4, scales=False)) == L.MOE_EINVAL
    # workspace too small, after the description passed
    assert _experts_ex(lib, _ew(L.MOE_WEIGHT_MXFP4)) == L.MOE_ENOSPACE


def test_experts_ex_accepts_valid_descriptions_with_no_tokens(lib):
    for fmt in (L.MOE_WEIGHT_DTYPE, L.MOE_WEIGHT_FP8_E4M3, L.MOE_WEIGHT_MXFP4):
        for act in L.ACTIVATIONS.values():
            assert _experts_ex(lib, _ew(fmt, act=act), T=0) == L.MOE_OK, (fmt, act)


def test_placement_validation_and_workspace(lib):
    c = _cfg(num_experts=8, top_k=2)
    table = ctypes.c_void_p(256)
    base = lib.moe_forward_workspace_ex(ctypes.byref(c), L.MOE_DTYPE_BF16, 64, 128, 64, None,
                                        None, None)
    more = L.moe_placement_t(12, table, None)
    with_pl = lib.moe_forward_workspace_ex(ctypes.byref(c), L.MOE_DTYPE_BF16, 64, 128, 64, None,
                                           None, ctypes.byref(more))
    assert base > 0 and with_pl > base   # slot ids, and per-slot buffers for 12 slots
    plain = lib.moe_forward_workspace(ctypes.byref(c), L.MOE_DTYPE_BF16, 64, 128, 64, None, None)
    assert plain == base
    p = ctypes.c_void_p(256)
    ew = _ew()

    def fwd(pl):
        return lib.moe_forward_ex(ctypes.byref(c), L.MOE_DTYPE_BF16, 4, 128, 64, p, p, None,
                                  None, None, ctypes.byref(ew), ctypes.byref(pl), None, None, p,
                                  None, None, None, None, None, p, 1 << 30, None)

    assert fwd(L.moe_placement_t(0, table, None)) == L.MOE_EINVAL       # no slots
    assert fwd(L.moe_placement_t(12, None, None)) == L.MOE_EINVAL       # no table
    assert fwd(L.moe_placement_t(2000, table, None)) == L.MOE_ENOTSUP   # > 1024 slots


def test_log2phy_and_load_accumulate_validation(lib):
    p = ctypes.c_void_p(256)
    assert lib.moe_log2phy(0, 2, 8, 8, None, None, None, None) == L.MOE_OK
    assert lib.moe_log2phy(4, 2, 8, 8, None, p, p, None) == L.MOE_EINVAL
    assert lib.moe_log2phy(4, 0, 8, 8, p, p, p, None) == L.MOE_EINVAL
    assert lib.moe_log2phy(4, 2, 8, 0, p, p, p, None) == L.MOE_EINVAL
    assert lib.moe_log2phy(4, 2, 2000, 8, p, p, p, None) == L.MOE_ENOTSUP
    assert lib.moe_load_accumulate(0, None, None, None) == L.MOE_OK
    assert lib.moe_load_accumulate(-1, p, p, None) == L.MOE_EINVAL
    assert lib.moe_load_accumulate(4, None, p, None) == L.MOE_EINVAL


def test_noalloc_rejects_a_need_beyond_its_scratch(lib):
    """moe_forward_noalloc checks the layer's scratch need against its fixed
    array before any device call: the decode layer at 377 tokens needs more
    than 64 MiB, so the call returns MOE_ENOSPACE (the pointers are never
    touched); invalid shapes are rejected as by moe_forward_ex."""
    assert L.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20
    c = L.RouteConfig(384, 8).c()
    need = lib.moe_forward_workspace_ex(ctypes.byref(c), L.MOE_DTYPE_BF16, 377, 7168, 2048,
                                        None, None, None)
    assert need > L.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_workspace_ex(ctypes.byref(c), L.MOE_DTYPE_BF16, 376, 7168, 2048,
                                        None, None, None) <= L.MOE_NOALLOC_SCRATCH_BYTES
    wc = L.moe_expert_weights_t(L.MOE_WEIGHT_DTYPE, 16, 16, None, None, 0, 0.0, 0.0)

    def call(T, H=7168, cfg=c, w=wc):
        return lib.moe_forward_noalloc(ctypes.byref(cfg), L.MOE_DTYPE_BF16, T, H, 2048, 16, 16,
                                       None, None, None, ctypes.byref(w), None, None, None, 16,
                                       None, None, None, None, None)
    assert call(377) == L.MOE_ENOSPACE
    assert call(100000) == L.MOE_ENOSPACE
    assert call(0) == L.MOE_OK                          # T == 0 launches nothing
    assert call(8, H=7000) == L.MOE_ENOTSUP             # width not a multiple of 64
    bad = L.RouteConfig(384, 8).c()
    bad.top_k = 0
    assert call(8, cfg=bad) == L.MOE_EINVAL
    badw = L.moe_expert_weights_t(7, 16, 16, None, None, 0, 0.0, 0.0)
    assert call(8, w=badw) == L.MOE_EINVAL
