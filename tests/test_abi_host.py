"""Host-side checks of the C ABI (no GPU needed): every symbol declared in
include/moe.h is exported, and argument validation rejects bad calls before
anything is launched."""
import ctypes
import os
import re

import pytest

from fine_grained_mixture_top_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("HIP library not built: run python -m fine_grained_mixture_top_amd.build")
    return B.lib()


def test_header_functions_exported(lib):
    names = declared_functions()
    assert set(names) == {"moe_row_capacity", "moe_workspace_bytes", "moe_workspace_offset",
                          "moe_route", "moe_route_noalloc", "moe_fwd", "moe_bwd", "moe_strerror",
                          "moe_unfused_cache_bytes", "moe_fwd_unfused", "moe_bwd_unfused", "moe_fwd_mxfp8",
                          "moe_bwd_mxfp8"}
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(MOE_[A-Z0-9_]+)\s+(-?\d+)u?", text))
    for k, v in consts.items():
        assert getattr(B, k) == int(v), k


def test_capacity_and_workspace():
    d = B.make_desc(256, 128, 8, 64, 2, "f32")
    assert B.moe_row_capacity(d) == 512
    dn = B.make_desc(1000, 128, 16, 64, 2, "bf16", round_mode=1)
    assert B.moe_row_capacity(dn) == 2000 + 16 * 64
    ds = B.make_desc(1000, 128, 16, 64, 2, "bf16", round_mode=2)
    assert B.moe_row_capacity(ds) == 2000 + 16 * 127
    dcap = B.make_desc(10, 128, 16, 64, 2, "bf16", round_mode=2)
    assert B.moe_row_capacity(dcap) == 10 * 16
    for which in (0, 1, 2, 3):
        assert B.moe_workspace_bytes(d, which) > 0
        assert B.moe_workspace_bytes(d, which) % 256 == 0
    assert B.moe_workspace_bytes(d, 7) == 0
    for item in range(7):
        off = B.moe_workspace_offset(d, item)
        assert off >= 0 and off % 256 == 0
    assert B.moe_workspace_offset(d, 99) == -1


def test_mx_weight_grad_workspace():
    """MOE_FLAG_MXFP8_WGRAD grows the MXFP8 backward workspace by the padded
    segment operands and gives their items offsets; without it they have none."""
    T, d, E, n, K = 1000, 512, 16, 256, 2
    plain = B.make_desc(T, d, E, n, K, "bf16")
    flagged = B.make_desc(T, d, E, n, K, "bf16", flags=B.MOE_FLAG_MXFP8_WGRAD)
    a = B.moe_workspace_bytes(plain, B.MOE_WS_BWD_MXFP8)
    b = B.moe_workspace_bytes(flagged, B.MOE_WS_BWD_MXFP8)
    rows = B.moe_row_capacity(plain) + 127 * E
    assert a > 0 and b >= a + (d + 2 * n + n + d) * rows * (1 + 1 / 32)
    assert B.moe_workspace_bytes(flagged, B.MOE_WS_BWD) == B.moe_workspace_bytes(plain, B.MOE_WS_BWD)
    offs = [B.moe_workspace_offset(flagged, i)
            for i in range(B.MOE_ITEM_MX_WG_PADOFF, B.MOE_ITEM_MX_WG_OS + 1)]
    assert all(o >= a and o % 256 == 0 for o in offs) and offs == sorted(offs) and offs[-1] < b
    assert all(B.moe_workspace_offset(plain, i) == -1
               for i in range(B.MOE_ITEM_MX_WG_PADOFF, B.MOE_ITEM_MX_WG_OS + 1))
    # the flag asks nothing of the other workspaces' shapes, but its own
    # byte-range limit: (cap + 127 E) * max(d, 2n) below 2^31
    big = B.make_desc(125000, 2048, 1024, 256, 8, "bf16", flags=B.MOE_FLAG_MXFP8_WGRAD)
    assert B.moe_workspace_bytes(big, B.MOE_WS_BWD_MXFP8) == 0
    assert B.moe_workspace_bytes(big, B.MOE_WS_FWD_MXFP8) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), B.MOE_EINVAL), (dict(K=0), B.MOE_EINVAL), (dict(K=9), B.MOE_EINVAL),
    (dict(dtype=7), B.MOE_EDTYPE), (dict(round_mode=3), B.MOE_EINVAL), (dict(tile=64), B.MOE_ESHAPE), (dict(tile=512), B.MOE_ESHAPE),
    (dict(d=100), B.MOE_ESHAPE), (dict(n=48), B.MOE_ESHAPE), (dict(E=12, K=2), B.MOE_ESHAPE),
    (dict(flags=8), B.MOE_EINVAL),
])
def test_invalid_descriptors_rejected(lib, kw, code):
    a = dict(T=256, d=128, E=8, n=64, K=2, dtype="f32")
    a.update(kw)
    d = B.make_desc(**a)
    assert B.moe_row_capacity(d) == 0
    assert B.moe_workspace_bytes(d, 0) == 0
    st = lib.moe_route(ctypes.byref(d), None, None, None, None, None, 0, None)
    assert st == code
    st = lib.moe_fwd(ctypes.byref(d), None, None, None, None, None, None, None, 0, None)
    assert st == code


def test_null_pointers_and_workspace_rejected_before_launch(lib):
    d = B.make_desc(256, 128, 8, 64, 2, "f32")
    # null routing
    assert lib.moe_route(ctypes.byref(d), 16, 16, None, None, None, 0, None) == B.MOE_EINVAL
    # fake (never dereferenced) device pointers: validation fails on the workspace first
    r = B.MoeRouting(*([4096] * len(B.ROUTING_FIELDS)))
    need = B.moe_workspace_bytes(d, B.MOE_WS_ROUTE)
    assert lib.moe_route(ctypes.byref(d), 4096, 4096, None, ctypes.byref(r), 4096, need - 1,
                         None) == B.MOE_EWORKSPACE
    assert lib.moe_route(ctypes.byref(d), 4096, 4096, None, ctypes.byref(r), 4097, need,
                         None) == B.MOE_EINVAL  # misaligned
    assert lib.moe_route(ctypes.byref(d), None, 4096, None, ctypes.byref(r), 4096, need,
                         None) == B.MOE_EINVAL  # x missing without given scores
    r2 = B.MoeRouting(*([4096] * (len(B.ROUTING_FIELDS) - 1) + [0]))
    assert lib.moe_fwd(ctypes.byref(d), 4096, 4096, 4096, ctypes.byref(r2), 4096, 4096, 4096,
                       1 << 30, None) == B.MOE_EINVAL
    need_b = B.moe_workspace_bytes(d, B.MOE_WS_BWD)
    assert lib.moe_bwd(ctypes.byref(d), *([4096] * 4), ctypes.byref(r), *([4096] * 6), None, None,
                       4096, need_b - 256, None) == B.MOE_EWORKSPACE


def test_unfused_cache_and_validation(lib):
    d = B.make_desc(256, 128, 8, 64, 2, "bf16")
    cap = B.moe_row_capacity(d)
    up = lambda v: (v + 255) // 256 * 256
    # rows of X_g [d], H [2n], A [n], Y [d], each block 256-byte aligned
    assert B.moe_unfused_cache_bytes(d) == up(cap * 128 * 2) + up(cap * 128 * 2) + up(cap * 64 * 2) + \
        up(cap * 128 * 2)
    bad = B.make_desc(256, 100, 8, 64, 2, "bf16")
    assert B.moe_unfused_cache_bytes(bad) == 0
    assert lib.moe_fwd_unfused(ctypes.byref(bad), None, None, None, None, None, None, 0, None) == B.MOE_ESHAPE
    r = B.MoeRouting(*([4096] * len(B.ROUTING_FIELDS)))
    need_c = B.moe_unfused_cache_bytes(d)
    assert lib.moe_fwd_unfused(ctypes.byref(d), 4096, 4096, 4096, ctypes.byref(r), 4096, 4096, need_c - 1,
                               None) == B.MOE_EWORKSPACE
    assert lib.moe_fwd_unfused(ctypes.byref(d), 4096, 4096, 4096, ctypes.byref(r), 4096, 4097, need_c,
                               None) == B.MOE_EINVAL  # misaligned cache
    assert lib.moe_fwd_unfused(ctypes.byref(d), 4096, None, 4096, ctypes.byref(r), 4096, 4096, need_c,
                               None) == B.MOE_EINVAL
    need_b = B.moe_workspace_bytes(d, B.MOE_WS_BWD_UNFUSED)
    assert need_b > 0
    assert lib.moe_bwd_unfused(ctypes.byref(d), *([4096] * 4), ctypes.byref(r), *([4096] * 6), None, None,
                               4096, need_b - 256, None) == B.MOE_EWORKSPACE
    assert lib.moe_bwd_unfused(ctypes.byref(d), *([4096] * 4), ctypes.byref(r), None, *([4096] * 5), None,
                               None, 4096, need_b, None) == B.MOE_EINVAL  # no cache


def test_mxfp8_shapes_and_validation(lib):
    ok = B.make_desc(256, 512, 8, 256, 2, "bf16")
    assert B.moe_workspace_bytes(ok, B.MOE_WS_FWD_MXFP8) > 0
    assert B.moe_workspace_offset(ok, B.MOE_ITEM_MX_Y) % 256 == 0
    r = B.MoeRouting(*([4096] * len(B.ROUTING_FIELDS)))
    for kw, code in ((dict(n=128), B.MOE_ESHAPE), (dict(d=2304), B.MOE_ESHAPE), (dict(n=2304), B.MOE_ESHAPE),
                     (dict(dtype="f32"), B.MOE_EDTYPE)):
        a = dict(T=256, d=512, E=8, n=256, K=2, dtype="bf16")
        a.update(kw)
        d = B.make_desc(**a)
        assert B.moe_workspace_bytes(d, B.MOE_WS_FWD_MXFP8) == 0
        assert B.moe_workspace_offset(d, B.MOE_ITEM_MX_XQ) == -1
        assert lib.moe_fwd_mxfp8(ctypes.byref(d), 4096, 4096, 4096, ctypes.byref(r), 4096, 4096, 4096, 1 << 40,
                                 None) == code
    assert B.moe_workspace_bytes(ok, B.MOE_WS_BWD_MXFP8) > B.moe_workspace_bytes(ok, B.MOE_WS_BWD)
    big_n = B.make_desc(256, 512, 8, 1280, 2, "bf16")  # 2n = 2560 > 2048: backward only
    assert B.moe_workspace_bytes(big_n, B.MOE_WS_BWD_MXFP8) == 0
    assert lib.moe_bwd_mxfp8(ctypes.byref(big_n), *([4096] * 4), ctypes.byref(r), *([4096] * 6), None, None,
                             4096, 1 << 40, None) == B.MOE_ESHAPE
    nb = B.moe_workspace_bytes(ok, B.MOE_WS_BWD_MXFP8)
    assert lib.moe_bwd_mxfp8(ctypes.byref(ok), *([4096] * 4), ctypes.byref(r), *([4096] * 6), None, None,
                             4096, nb - 256, None) == B.MOE_EWORKSPACE
    need = B.moe_workspace_bytes(ok, B.MOE_WS_FWD_MXFP8)
    assert lib.moe_fwd_mxfp8(ctypes.byref(ok), 4096, 4096, 4096, ctypes.byref(r), 4096, 4096, 4096, need - 1,
                             None) == B.MOE_EWORKSPACE
    assert lib.moe_fwd_mxfp8(ctypes.byref(ok), 4096, None, 4096, ctypes.byref(r), 4096, 4096, 4096, need,
                             None) == B.MOE_EINVAL


def test_strerror():
    assert B.moe_strerror(0) == "ok"
    assert "workspace" in B.moe_strerror(B.MOE_EWORKSPACE)
    assert B.moe_strerror(12345) == "unknown status"
