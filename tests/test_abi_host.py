"""CPU checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments on the host before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("qi4.h", "qi4_probe.h")]


def _declared():
    """Functions declared in include/*.h, in header order."""
    assert sorted(HEADERS) == sorted(os.path.join(ROOT, "include", h)
                                     for h in os.listdir(os.path.join(ROOT, "include")))
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)
    kw = {"if", "sizeof", "defined"}
    return [n for n in dict.fromkeys(names) if n not in kw]


@pytest.fixture(scope="module")
def q():
    import ffn_int4_g128_amd as q
    if not os.path.exists(q.LIB_PATH):
        q.build()
    q.lib()
    return q


def test_header_and_binding_agree(q):
    assert _declared() == q.EXPORTED


def test_every_declared_symbol_is_exported(q):
    L = ctypes.CDLL(q.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def test_version_and_status_strings(q):
    L = q.lib()
    assert L.qi4_abi_version() == 1
    for s in range(-8, 1):
        assert L.qi4_status_string(s)
    assert L.qi4_status_string(-99) == b"unknown status"


def test_packed_bytes(q):
    L = q.lib()
    # 16-row tiles x 128-wide groups: 1024 B of codes each; per group, the
    # scales (128 B) and zeros (32 B) of each quad of 4 tiles (the last quad
    # padded); the total rounded up to 256 B
    def size(nt, G, h=1):
        return ((nt * G * 1024 + -(-nt // 4) * G * 160 * h + 255) // 256) * 256
    assert L.qi4_packed_bytes(16, 128, 128, 0) == 1280 == size(1, 1)  # 1184 rounded up
    assert L.qi4_packed_bytes(4096, 4096, 128, 0) == 256 * 32 * 1064 == size(256, 32)
    assert L.qi4_packed_bytes(17, 256, 128, 0) == 4608 == size(2, 2)
    # gate/up: each half padded to whole tiles
    assert L.qi4_packed_bytes(48, 128, 128, 1) == size(4, 1)
    assert L.qi4_packed_bytes(16, 100, 128, 0) == -2
    # group sizes: 64 (two halves per block record), multiples of 128 dividing K
    # and 0 (one group per row) share the g128 size
    assert L.qi4_packed_bytes(17, 256, 64, 0) == size(2, 2, 2)
    assert L.qi4_packed_bytes(17, 256, 256, 0) == size(2, 2)
    assert L.qi4_packed_bytes(17, 768, 384, 0) == size(2, 6)
    assert L.qi4_packed_bytes(17, 256, 0, 0) == size(2, 2)
    assert L.qi4_packed_bytes(16, 128, 256, 0) == -2   # does not divide K
    assert L.qi4_packed_bytes(16, 128, 100, 0) == -4
    assert L.qi4_packed_bytes(16, 128, 32, 0) == -4
    assert L.qi4_packed_bytes(16, 128, -128, 0) == -4
    assert L.qi4_packed_bytes(17, 128, 128, 1) == -2
    assert L.qi4_packed_bytes(0, 128, 128, 0) == -2
    assert L.qi4_packed_bytes(16, 128, 128, 4) == -7


def test_argument_errors_return_before_any_launch(q):
    L = q.lib()
    p = ctypes.c_void_p(0x1000)
    # K not a multiple of 128, group size, dtype, epilogue/flags combination, NULL, alias
    assert L.qlinear_int4_g128(p, 1, 1, 100, p, 16, 0, p, 1, 0, None) == -2
    assert L.qlinear_int4_g128(p, 7, 1, 128, p, 16, 0, p, 1, 0, None) == -3
    assert L.qlinear_int4_g128(p, 1, 1, 128, p, 16, 0, p, 9, 0, None) == -3
    assert L.qlinear_int4_g128(p, 1, 1, 128, p, 16, 0, p, 1, 1, None) == -7
    assert L.qlinear_int4_g128(None, 1, 1, 128, p, 16, 0, p, 1, 0, None) == -1
    assert L.qlinear_int4_g128(p, 1, -1, 128, p, 16, 0, p, 1, 0, None) == -2
    assert L.qlinear_int4_g128(p, 1, 0, 128, p, 16, 0, p, 1, 0, None) == 0   # T == 0: no-op
    x = ctypes.c_void_p(0x100000)
    assert L.qlinear_int4_g128(x, 1, 4, 128, ctypes.c_void_p(0x200000), 16, 0,
                               ctypes.c_void_p(0x100000 + 64), 1, 0, None) == -6
    assert L.qlinear_int4_g128(ctypes.c_void_p(0x1004), 1, 1, 128, p, 16, 0, p, 1, 0, None) == -2
    assert L.qi4_pack(p, p, p, 16, 128, 96, 0, p, None) == -4
    assert L.qi4_pack(p, p, p, 16, 128, 256, 0, p, None) == -2   # group does not divide K
    assert L.qlinear_int4(p, 1, 1, 128, p, 16, 192, 0, p, 1, 0, None) == -4
    assert L.qlinear_int4(p, 1, 1, 384, p, 16, 256, 0, p, 1, 0, None) == -2
    assert L.qi4_pack(None, p, p, 16, 128, 128, 0, p, None) == -1
    assert L.qi4_dequant_f32(p, 16, 96, 128, 0, p, None) == -2
    assert L.moe_route_topk(p, 4, 8, 9, p, p, None) == -2
    assert L.moe_route_topk(p, 4, 2000, 8, p, p, None) == -2
    # router: H not a multiple of 32, NULL, overlapping logits
    assert L.moe_router_topk(p, 4, 100, p, 256, 8, p, p, p, None) == -2
    assert L.moe_router_topk(None, 4, 128, p, 256, 8, p, p, p, None) == -1
    assert L.moe_router_topk(ctypes.c_void_p(0x100000), 4, 128, ctypes.c_void_p(0x200000), 256, 8,
                             ctypes.c_void_p(0x100000 + 512), ctypes.c_void_p(0x300000),
                             ctypes.c_void_p(0x400000), None) == -6
    assert L.moe_sort_tokens(None, 4, 8, 256, p, p, p, None, None) == -1
    # 8-bit format: packed size is that of the 4-bit matrix of twice the width;
    # unknown flag bits; qlinear_int4 refuses an 8-bit matrix; quantizer alignment
    assert L.qi4_packed_bytes(48, 512, 128, 2) == L.qi4_packed_bytes(48, 1024, 128, 0)
    assert L.qi4_packed_bytes(48, 512, 64, 3) == L.qi4_packed_bytes(48, 1024, 64, 1)
    assert L.qi4_packed_bytes(48, 512, 0, 2) > L.qi4_packed_bytes(48, 512, 0, 0)
    assert L.qi4_packed_bytes(48, 512, 128, 4) == -7
    assert L.qlinear_int4(p, 1, 1, 128, p, 16, 128, 2, p, 1, 0, None) == -7
    assert L.qlinear_int8(p, 1, 1, 100, p, 16, 128, 0, p, 1, 0, None) == -2
    assert L.qlinear_int8(None, 1, 1, 128, p, 16, 128, 0, p, 1, 0, None) == -1
    assert L.qlinear_int8(p, 1, 0, 128, p, 16, 128, 0, p, 1, 0, None) == 0
    assert L.qi4_quantize_int8(p, 1, 16, 128, 128, ctypes.c_void_p(0x1004), p, p, None) == -2
    assert L.qi4_quantize_int8(None, 1, 16, 128, 128, p, p, p, None) == -1
    assert L.qi4_pack(p, p, p, 16, 128, 128, 2, ctypes.c_void_p(0x2004), None) == -2
    # W4A8: scale, workspace, 8-bit weights refused
    inf, nan = float("inf"), float("nan")
    assert L.qlinear_w4a8_workspace_bytes(3, 256) == 768
    assert L.qlinear_w4a8_workspace_bytes(3, 100) == -2
    xs, ys, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    for bad in (0.0, -1.0, inf, nan, 1e-39):
        assert L.qlinear_w4a8(xs, 1, bad, 1, 128, p, 16, 128, 0, ys, 1, 0, ws, 128, None) == -2
    assert L.qlinear_w4a8(p, 1, 0.1, 2, 128, p, 16, 128, 0, ctypes.c_void_p(0x200000), 1, 0,
                          ctypes.c_void_p(0x300000), 255, None) == -5
    assert L.qlinear_w4a8(p, 1, 0.1, 2, 128, p, 16, 128, 0, ctypes.c_void_p(0x200000), 1, 0,
                          None, 256, None) == -1
    assert L.qlinear_w4a8(xs, 1, 0.1, 1, 128, p, 16, 128, 2, ys, 1, 0, ws, 128, None) == -7
    assert L.qlinear_w4a8(p, 1, 0.1, 0, 128, p, 16, 128, 0, p, 1, 0, None, 0, None) == 0
    # fused routing + permutation: shape, NULL, aliasing, T == 0
    assert L.moe_route_sort(p, 4, 8, 9, p, p, p, p, p, p, None) == -2
    assert L.moe_route_sort(p, 4, 2000, 8, p, p, p, p, p, p, None) == -2
    assert L.moe_route_sort(p, 4, 256, 8, p, p, p, p, p, None, None) == -1
    assert L.moe_route_sort(p, 0, 256, 8, p, p, p, p, p, p, None) == 0
    a = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(7)]
    assert L.moe_route_sort(a[0], 4, 256, 8, a[1], a[2], a[3], a[4], ctypes.c_void_p(0x500000 + 16),
                            a[6], None) == -6
    # quantizer: NULL, dtype, group size, K, alignment, overlapping outputs
    assert L.qi4_quantize(None, 1, 16, 128, 128, p, p, p, None) == -1
    assert L.qi4_quantize(p, 5, 16, 128, 128, p, p, p, None) == -3
    assert L.qi4_quantize(p, 1, 16, 128, 32, p, p, p, None) == -4
    assert L.qi4_quantize(p, 1, 16, 100, 128, p, p, p, None) == -2
    assert L.qi4_quantize(ctypes.c_void_p(0x1008), 1, 16, 128, 128, p, p, p, None) == -2
    w = ctypes.c_void_p(0x100000)
    assert L.qi4_quantize(w, 1, 16, 128, 128, ctypes.c_void_p(0x100000 + 256), p, p, None) == -6


def test_moe_descriptor_errors(q):
    L = q.lib()
    D = q._MoeDesc
    ok = D(256, 7168, 2048, 8, 128, 1, 0)
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(ok), 32) > 0
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 64, 1, 0)), 1) > 0
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 0, 1, 0)), 1) > 0
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 96, 1, 0)), 1) == -4
    # 896 (7 x 128) divides hidden (7168) but not inter (2048)
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 896, 1, 0)), 1) == -2
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7000, 2048, 8, 128, 1, 0)), 1) == -2
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(4, 7168, 2048, 8, 128, 1, 0)), 1) == -2
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 128, 2, 0)), 1) == -7
    # W4A8 MoE: workspace size, scales, 8-bit experts refused
    p = ctypes.c_void_p(0x1000)
    assert L.moe_ffn_w4a8_workspace_bytes(ctypes.byref(ok), 32) > 0
    assert L.moe_ffn_w4a8_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 96, 1, 0)), 1) == -4
    xw, ow, ww = (ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000),
                  ctypes.c_void_p(0x30000000))
    for sx, sh_ in ((0.0, 0.1), (0.1, -1.0), (float("nan"), 0.1), (0.1, float("inf"))):
        assert L.moe_ffn_w4a8(ctypes.byref(ok), xw, sx, sh_, 4, p, None, None, p, p, p, p, ow, ww,
                              1 << 40, None) == -2
    assert L.moe_ffn_w4a8(ctypes.byref(D(256, 7168, 2048, 8, 128, 1, 2)), xw, 0.1, 0.1, 4, p, None,
                          None, p, p, p, p, ow, ww, 1 << 40, None) == -7
    assert L.moe_ffn_w4a8(ctypes.byref(ok), xw, 0.1, 0.1, 4, p, None, None, p, p, p, p, ow, ww,
                          256, None) == -5
    # flags: QI4_INT8 (8-bit experts) is accepted, other bits are not
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 128, 1, 2)), 32) > 0
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 128, 1, 1)), 1) == -7
    assert L.moe_ffn_int4_workspace_bytes(ctypes.byref(D(256, 7168, 2048, 8, 128, 1, 4)), 1) == -7
    p = ctypes.c_void_p(0x1000)
    small = ctypes.c_void_p(0x10000000)
    # workspace too small
    assert L.moe_ffn_int4(ctypes.byref(ok), ctypes.c_void_p(0x20000000), 4, p, None, None, p, p,
                          p, p, ctypes.c_void_p(0x30000000), small, 256, None) == -5
    # shared pointers must match has_shared
    assert L.moe_ffn_int4(ctypes.byref(ok), p, 4, p, None, None, p, p, None, p, p, small,
                          1 << 40, None) == -1
