"""CPU tests of the C ABI: the library loads and exports every symbol include/wq.h declares,
the host helpers reproduce the pages' values, and invalid arguments are rejected on the host
before anything is launched (none of these calls reaches the GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def wq():
    import weight_only_bit_amd as wq

    if not os.path.exists(wq.LIB_PATH):
        from weight_only_bit_amd import build

        build.build()
    wq.lib()
    return wq


def _declared():
    with open(os.path.join(ROOT, "include", "wq.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(wq):
    names = _declared()
    assert len(names) >= 10
    L = wq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(wq.EXPORTS) == names


def test_pack_helpers_match_printed_values(wq):
    assert wq.wq_pack_int4([1, -2]).tolist() == [225]
    assert wq.wq_pack_int4([7, -8]).tolist() == [135]
    assert wq.wq_pack_int4([3, -1, 5]).tolist() == [0xF3, 0x05]
    data = np.arange(256, dtype=np.uint8)
    codes = wq.wq_unpack_int4(data, 512)
    assert np.array_equal(wq.wq_pack_int4(codes), data)
    assert wq.wq_packed_size(7_000_000_000, 4) == 3_500_000_000
    assert wq.wq_packed_size(7_000_000_000, 16) == 14_000_000_000
    assert wq.wq_packed_size(3, 4) == 2
    assert wq.wq_packed_size(-1, 4) == -1
    big = (2**63 - 1 - 7) // 32  # the largest count whose bit count fits int64 at 32 bits
    assert wq.wq_packed_size(big, 32) == (big * 32 + 7) // 8
    assert wq.wq_packed_size(big + 1, 32) == -1
    assert wq.wq_packed_size(2**62, 4) == -1
    for bad in ([8], [-9]):
        with pytest.raises(ValueError, match="WQ_ERR_RANGE"):
            wq.wq_pack_int4(bad)


def test_pack_helpers_agree_with_oracle(wq, orc):
    codes = np.random.default_rng(0).integers(-8, 8, 1001).astype(np.int32)
    assert np.array_equal(wq.wq_pack_int4(codes), orc.pack_int4(codes))
    packed = orc.pack_int4(codes)
    assert np.array_equal(wq.wq_unpack_int4(packed, 1001), orc.unpack_int4(packed, 1001))


def test_status_strings(wq):
    L = wq.lib()
    assert L.wq_status_string(0) == b"WQ_OK"
    assert L.wq_status_string(-5) == b"WQ_ERR_WORKSPACE"
    assert L.wq_status_string(99) == b"WQ_ERR_UNKNOWN"


def _weight(wq, **kw):
    base = dict(format=3, group=64, experts=1, n=64, k=256, codes=0x1000, scales=None,
                zeros=None, qscale=0x2000, super_scale=0x3000, code_scale=0x4000,
                code_zero=0x5000, zp=32)
    base.update(kw)
    return wq._CWeight(*[base[f] for f, _ in wq._CWeight._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(k=100), -2),                 # k not a multiple of 64
    (dict(format=9), -2),              # unknown format
    (dict(group=32), -2),              # CCQ needs group 64
    (dict(codes=None), -1),            # null codes
    (dict(codes=0x1001), -3),          # misaligned
    (dict(qscale=None), -1),
    (dict(zp=200), -2),
    (dict(zp=33), -2),                 # products need a power-of-two CCQ zero point
    (dict(n=0), -1),
    (dict(format=1, group=128, scales=0x6000), -2),
    (dict(format=2, scales=0x6000, zeros=None), -1),
    (dict(format=4, super_scale=None), -1),   # (4,3,2) needs its super scale
    (dict(format=5, super_scale=0x3004), -3),  # misaligned super scale
    (dict(format=5, zp=6), -2),               # hybrid zero point not a power of two
    (dict(format=4, group=0), -2),
    (dict(format=6, scales=None), -1),        # INT8 needs scales
    (dict(format=6, group=32, scales=0x6000), -2),
    (dict(format=7), -2),
    (dict(n=1, k=1 << 30), -2),               # products address an activation row in 32 bits
])
def test_gemm_rejects_bad_descriptors_without_launch(wq, kw, status):
    L = wq.lib()
    w = _weight(wq, **kw)
    st = L.wq_gemm(ctypes.c_void_p(0x7000), 4, ctypes.byref(w), ctypes.c_void_p(0x8000), None)
    assert st == status, L.wq_last_error()
    assert L.wq_last_error()


def test_gemm_argument_checks(wq):
    L = wq.lib()
    w = _weight(wq)
    assert L.wq_gemm(ctypes.c_void_p(0x7000), -1, ctypes.byref(w), ctypes.c_void_p(0x8000), None) == -1
    assert L.wq_gemm(None, 0, ctypes.byref(w), None, None) == 0  # m == 0 is a no-op
    assert L.wq_gemm(None, 2, ctypes.byref(w), ctypes.c_void_p(0x8000), None) == -1
    assert L.wq_gemm(ctypes.c_void_p(0x7008), 2, ctypes.byref(w), ctypes.c_void_p(0x8000), None) == -3
    w2 = _weight(wq, experts=3)
    assert L.wq_gemm(ctypes.c_void_p(0x7000), 2, ctypes.byref(w2), ctypes.c_void_p(0x8000), None) == -1
    assert L.wq_dequantize(ctypes.byref(w), None, None) == -1


def test_moe_argument_checks(wq):
    L = wq.lib()
    E, H, I, T, K = 4, 256, 128, 8, 2
    g = _weight(wq, experts=E, n=I, k=H)
    u = _weight(wq, experts=E, n=I, k=H)
    d = _weight(wq, experts=E, n=H, k=I)
    need = L.wq_moe_workspace_bytes(T, K, E, H, I)
    assert need >= T * K * (I * 2 + H * 4)
    x, ids, wts, y, ws = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))
    call = lambda gg, uu, dd, wsb, hidden=H: L.wq_moe_ffn(x, T, hidden, ids, wts, K, ctypes.byref(gg),
                                                          ctypes.byref(uu), ctypes.byref(dd), y, ws,
                                                          wsb, None)
    assert call(g, u, d, need - 1) == -5          # workspace too small
    bad_d = _weight(wq, experts=E, n=H, k=256)    # down's k must equal inter
    assert call(g, u, bad_d, need) == -1
    bad_u = _weight(wq, experts=E + 1, n=I, k=H)
    assert call(g, bad_u, d, need) == -1
    mixed = _weight(wq, experts=E, n=I, k=H, format=1, scales=0x6000, qscale=None)
    assert call(g, mixed, d, need) == -2          # gate and up must share a format
    big = _weight(wq, experts=1000, n=I, k=H)
    assert call(big, big, _weight(wq, experts=1000, n=H, k=I), need) == -2
    assert L.wq_moe_route(ids, T, K, 0, ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000), None, 0, None) == -1


def test_quantize_ccq_argument_checks(wq):
    L = wq.lib()
    p = [ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000)]
    call = lambda n, k, zp, w=p[0]: L.wq_quantize_ccq(w, n, k, zp, 1, *p[1:], None)
    assert call(4, 100, 32) == -2                  # k not a multiple of 64
    assert call(4, 131072 + 64, 32) == -2          # a row's codes must fit the LDS
    assert call(0, 256, 32) == -1
    assert call(4, 256, 200) == -2
    assert call(4, 256, 32, w=None) == -1
    assert call(4, 256, 32, w=ctypes.c_void_p(0x10008)) == -3
    for bad in (-1, 4, 7):                         # refine is a mask of 1 (re-pick) and 2 (scale update)
        assert L.wq_quantize_ccq(p[0], 4, 256, 32, bad, *p[1:], None) == -1


def test_route_workspace_sizes_and_checks(wq):
    L = wq.lib()
    # no table at most 4096 pairs; above, chunks of max(2048, ceil(pairs / 512)) pairs, one
    # int32 per chunk and expert
    assert L.wq_moe_route_workspace_bytes(32, 8, 64) == 0
    assert L.wq_moe_route_workspace_bytes(512, 8, 64) == 0
    assert L.wq_moe_route_workspace_bytes(513, 8, 64) == 3 * 64 * 4
    assert L.wq_moe_route_workspace_bytes(4096, 8, 64) == 16 * 64 * 4
    assert L.wq_moe_route_workspace_bytes(1 << 27, 8, 512) == 512 * 512 * 4
    for bad in ((-1, 8, 64), (4, 0, 64), (4, 8, 0), (4, 8, 513), ((1 << 27) + 1, 8, 64)):
        assert L.wq_moe_route_workspace_bytes(*bad) == 0, bad
    # the FFN workspace holds the table above 4096 pairs
    base = L.wq_moe_workspace_bytes(4096, 8, 64, 256, 128)
    assert base >= 16 * 64 * 4 + 4096 * 8 * (4 + 2 * 128 + 4 * 256)
    ids = ctypes.c_void_p(0x50000)
    off, pairs = ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000)
    assert L.wq_moe_route(ids, 4, 2, 8, off, pairs, None, 256, None) == -1
    assert b"without a workspace" in L.wq_last_error()
    need = L.wq_moe_route_workspace_bytes(4096, 8, 64)
    assert L.wq_moe_route(ids, 4096, 8, 64, off, pairs, ctypes.c_void_p(0x80000), need - 4, None) == -5
    assert L.wq_moe_route(ids, 4096, 8, 64, off, pairs, ctypes.c_void_p(0x80008), need, None) == -3


def test_last_error_detail_is_the_last_failure_under_both_names(wq):
    L = wq.lib()
    assert L.wq_pack_int4((ctypes.c_int32 * 2)(3, 9), 2, (ctypes.c_uint8 * 1)()) == -4
    assert b"outside -8..7" in L.wq_last_error_detail()
    assert L.wq_last_error_detail() == L.wq_last_error()
    assert L.wq_moe_route(None, 1, 1, 1, None, None, None, 0, None) == -1
    assert L.wq_last_error_detail() == L.wq_last_error() != b""
    assert b"outside -8..7" not in L.wq_last_error_detail()


def test_products_reject_experts_beyond_the_32bit_buffer_range(wq):
    """One expert's codes are addressed through 32-bit buffer resources whose range the
    kernels cap at 0x7FFFFFF0 bytes (plus up to 6 bytes of dword alignment for the (4,3,2) and
    hybrid views): a larger expert is rejected before any launch instead of reading zeros."""
    L = wq.lib()
    x, y = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    limit = 0x7FFFFFF0 - 8
    # hybrid, k = 64: 20 bytes per row
    n_ok, n_bad = limit // 20, limit // 20 + 1
    for n, want in ((n_bad, -2), (107374182, -2)):  # 107374182 * 20 = 2^31 - 8
        w = _weight(wq, experts=1, n=n, k=64, format=5, qscale=None, code_scale=None, code_zero=None)
        assert L.wq_gemm(x, 1, ctypes.byref(w), y, None) == want, n
        assert b"codes must not exceed" in L.wq_last_error()
    assert n_ok * 20 <= limit
    # INT8 per channel: k bytes per row
    w = _weight(wq, experts=1, n=(limit // 4096) + 1, k=4096, format=6, group=0, scales=0x6000,
                qscale=None, super_scale=None, code_scale=None, code_zero=None)
    assert L.wq_gemm(x, 1, ctypes.byref(w), y, None) == -2


def test_binding_rejects_host_tensors(wq):
    import torch

    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    w = wq.PackedWeight(wq.FMT_INT4, 8, 64, 1, 64, torch.zeros(8 * 32, dtype=torch.uint8),
                        torch.zeros(8, dtype=torch.int16))
    with pytest.raises(ValueError, match="GPU tensor"):
        wq.wq_gemm(x, w, y=torch.zeros((2, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        w.cstruct()
    assert wq._layout(wq.FMT_CCQ2, 2, 8, 128, 64)["qscale"] == (2 * 8 * 1, 1)
    assert wq._layout(wq.FMT_INT4, 1, 8, 128, 0)["scales"] == (8, 2)
    assert wq._layout(wq.FMT_CCQ432, 1, 8, 128, 64)["codes"] == (8 * 2 * 22, 1)
    assert wq._layout(wq.FMT_INT4, 1, 8, 100, 64) is None
