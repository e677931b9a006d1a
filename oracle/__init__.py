"""CPU oracle for the weight-only low-bit dequantize-and-multiply path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg are the only callers.  The product package never imports this module, and this module
imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain C, fp64 sums, one rounding per output); this file
builds it with the host C compiler and marshals numpy arrays through ctypes.  Each wrapper
names the passage of the pages it follows:

* [CCQ]   "CCQ: Convolutional Code for Extreme Low-bit Quantization in LLMs"
* [WINT2] FastDeploy "WINT2 Quantization"
* [E6.4]  coursefy lesson E6.4 "GPTQ and AWQ"

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``.  The first
stage of the code-cluster decode (``ccq_expand``) has no numeric example in the pages; it is
pinned by the code cluster's round trip (Eq. 1 of [CCQ]: on encoder rows with alpha != 1 every
expanded code lies within alpha / 2 + 1/2 of the code it stands for, which fixes the direction
C' * alpha + beta and the roles of alpha and beta) and by invariants (identity, clamps,
monotonicity).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_SANITIZE=1 builds and loads an AddressSanitizer / UndefinedBehaviorSanitizer build
# instead (the process must preload the ASan runtime; tests/test_oracle_sanitized.py does so).
_SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined"]

INT4, AFFINE2, CCQ, CCQ432, CCQ_HYBRID, INT8 = 1, 2, 3, 4, 5, 6
CCQ_ZP = 32  # reading: weight zero point 2^(L-1) for L = 6
CCQ432_ZP = 8  # reading: 2^(L-1) for the 4-bit states of (4,3,2)
CCQ_HYBRID_ZP = 4  # reading: 2^(L-1) for the 3-bit states of (3,3,2)(3,4,2)
ALG2_GROUP_BYTES = {CCQ432: 22, CCQ_HYBRID: 20}  # code bytes per 64-weight group


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with the host compiler (no fused multiply-adds)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", *(_SAN_FLAGS if _SANITIZE else []),
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Weight(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("experts", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("qscale", ctypes.c_void_p),
        ("super_scale", ctypes.c_void_p),
        ("code_scale", ctypes.c_void_p),
        ("code_zero", ctypes.c_void_p),
        ("zp", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        sig = {
            "orc_f32_to_bf16": (None, [vp, i64, vp]),
            "orc_f64_to_bf16": (None, [vp, i64, vp]),
            "orc_pack_int4": (i32, [vp, i64, vp]),
            "orc_unpack_int4": (None, [vp, i64, vp]),
            "orc_packed_size": (i64, [i64, i32]),
            "orc_rtn": (None, [vp, i64, ctypes.c_double, vp]),
            "orc_affine_quant": (None, [vp, i64, ctypes.c_double, i32, i32, i32, vp]),
            "orc_affine_dequant": (None, [vp, i64, ctypes.c_double, i32, vp]),
            "orc_ccq_total_bits": (i32, [i32, i32, i32]),
            "orc_ccq_shifts": (None, [i32, i32, i32, vp]),
            "orc_ccq_states": (None, [ctypes.c_uint32, i32, i32, i32, vp]),
            "orc_ccq_bpw": (ctypes.c_double, [i32, i32, i32, i32]),
            "orc_ccq_expand": (ctypes.c_uint32, [ctypes.c_uint32, ctypes.c_float, ctypes.c_float]),
            "orc_dequantize": (i32, [ctypes.POINTER(_Weight), i64, i64, i64, vp]),
            "orc_gemm_bf16": (None, [vp, i64, i64, vp, i64, vp, vp]),
            "orc_moe_route": (i32, [vp, i64, i32, i32, vp, vp]),
            "orc_moe_ffn": (i32, [vp, i64, i64, vp, vp, i32, i32, ctypes.POINTER(_Weight),
                                  ctypes.POINTER(_Weight), ctypes.POINTER(_Weight), i64, vp, i64,
                                  vp]),
            "orc_quant_int4": (i32, [vp, i64, i64, i32, vp, vp]),
            "orc_quant_affine2": (i32, [vp, i64, i64, vp, vp, vp]),
            "orc_ccq_search": (ctypes.c_uint32, [vp, ctypes.c_double, i32, vp]),
            "orc_quant_ccq": (i32, [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp]),
            "orc_ccq_encode_group": (ctypes.c_double, [vp, ctypes.c_float, ctypes.c_uint32, i32,
                                                       i32, vp, vp]),
            "orc_quant_alg2": (i32, [vp, i64, i64, i32, i32, i32, vp, vp]),
            "orc_quant_int8": (i32, [vp, i64, i64, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------------------------

def f32_to_bf16(a) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round half to even, NaN -> 0x7FC0."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f32_to_bf16(_p(a), a.size, _p(out))
    return out


def f64_to_bf16(a) -> np.ndarray:
    """fp64 -> bf16 bits with a single rounding (half to even), NaN -> 0x7FC0."""
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f64_to_bf16(_p(a), a.size, _p(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# [E6.4] packing, size, RTN and affine formulas
# ---------------------------------------------------------------------------------------------

def pack_int4(codes) -> np.ndarray:
    """[E6.4] pack_int4: two signed codes per byte, first code in the low nibble, odd count
    padded with 0.  Raises ValueError for a code outside -8..7."""
    c = _c(codes, np.int32).ravel()
    out = np.zeros((c.size + 1) // 2, np.uint8)
    if lib().orc_pack_int4(_p(c), c.size, _p(out)) != 0:
        raise ValueError("INT4 code out of range -8..7")
    return out


def unpack_int4(data, n: int) -> np.ndarray:
    """[E6.4] unpack_int4: the first n signed codes, each 4-bit field sign-extended."""
    d = _c(data, np.uint8).ravel()
    if n > 2 * d.size:
        raise ValueError("not enough bytes")
    out = np.empty(n, np.int32)
    lib().orc_unpack_int4(_p(d), n, _p(out))
    return out


def packed_size(n_codes: int, bits: int = 4) -> int:
    """[E6.4] nominal packed size M = N*b/8 bytes, scales excluded."""
    return int(lib().orc_packed_size(int(n_codes), int(bits)))


def rtn(w, scale: float) -> np.ndarray:
    """[E6.4] rtn: clip(round(w/scale), -8, 7) * scale, round half to even."""
    a = _c(w, np.float64)
    out = np.empty(a.shape, np.float64)
    lib().orc_rtn(_p(a), a.size, float(scale), _p(out))
    return out


def affine_quant(x, s: float, z: int, qmin: int, qmax: int) -> np.ndarray:
    """[E6.4] q = clip(round(x/s) + z) over [qmin, qmax]."""
    a = _c(x, np.float64)
    q = np.empty(a.shape, np.int32)
    lib().orc_affine_quant(_p(a), a.size, float(s), int(z), int(qmin), int(qmax), _p(q))
    return q


def affine_dequant(q, s: float, z: int) -> np.ndarray:
    """[E6.4] x_hat = s (q - z)."""
    a = _c(q, np.int32)
    out = np.empty(a.shape, np.float64)
    lib().orc_affine_dequant(_p(a), a.size, float(s), int(z), _p(out))
    return out


# ---------------------------------------------------------------------------------------------
# [CCQ] codebook arithmetic
# ---------------------------------------------------------------------------------------------

def ccq_total_bits(L: int, N: int, S: int) -> int:
    """[CCQ] section 3.1: T = L + (N-1) S."""
    return int(lib().orc_ccq_total_bits(L, N, S))


def ccq_shifts(L: int, N: int, S: int) -> list[int]:
    out = np.empty(N, np.int32)
    lib().orc_ccq_shifts(L, N, S, _p(out))
    return out.tolist()


def ccq_states(code: int, L: int, N: int, S: int) -> list[int]:
    """[CCQ] section 3.1 bit-shift decoding: the N states of one code."""
    out = np.empty(N, np.int32)
    lib().orc_ccq_states(int(code), L, N, S, _p(out))
    return out.tolist()


def ccq_bpw(T: int, g: int, N: int, scale_bits: int) -> float:
    """[CCQ] section 3.4, bits-per-weight equation."""
    return float(lib().orc_ccq_bpw(T, g, N, scale_bits))


def ccq_expand(cprime: int, code_scale: float, code_zero: float) -> int:
    """[CCQ] section 3.5 stage 1: C = clamp(round(fma(C', alpha, beta)), 0, 2^15 - 1)."""
    return int(lib().orc_ccq_expand(int(cprime), float(code_scale), float(code_zero)))


def ccq_search(v, scale: float, zp: int = CCQ_ZP):
    """[CCQ] Algorithm 'Convolutional Code Quantization' for one 4-vector: (code, cost)."""
    a = _c(v, np.float64)
    assert a.size == 4
    cost = np.zeros(1, np.float64)
    code = lib().orc_ccq_search(_p(a), float(scale), int(zp), _p(cost))
    return int(code), float(cost[0])


def ccq_encode_group(wg, super_scale: float, sq: int, zp: int = CCQ_ZP, update: bool = True):
    """One 64-weight group of the (6,4,3) encoder: trellis search at fl(sq * super), then
    (update) the [CCQ] section 3.4 least-squares scale update, kept only when the group error
    drops.  Returns (codes [16] of 15 bits, final 4-bit scale, group squared error)."""
    a = _c(wg, np.float32)
    assert a.size == 64
    codes = np.zeros(16, np.uint32)
    sq_out = np.zeros(1, np.uint32)
    err = lib().orc_ccq_encode_group(_p(a), float(super_scale), int(sq), int(zp), int(bool(update)),
                                     _p(codes), _p(sq_out))
    return codes.astype(np.int64), int(sq_out[0]), float(err)


# Encoder refinements of the (6,4,3) code-cluster quantizer (bit mask):
CCQ_REPICK = 1        # re-pick each C' among the row's 256 decodable codes (reading R11)
CCQ_SCALE_UPDATE = 2  # [CCQ] section 3.4 least-squares group scale update


def _ccq_refine_bits(refine) -> int:
    if isinstance(refine, bool):
        return CCQ_REPICK | CCQ_SCALE_UPDATE if refine else 0
    return int(refine)


# ---------------------------------------------------------------------------------------------
# Packed weights
# ---------------------------------------------------------------------------------------------

@dataclass
class Packed:
    """A packed low-bit weight tensor [experts, n, k] in the oracle's layout."""
    format: int
    n: int
    k: int
    experts: int = 1
    group: int = 64
    codes: np.ndarray = None
    scales: np.ndarray = None       # bf16 bits (INT4, affine)
    zeros: np.ndarray = None        # u8 (affine)
    qscale: np.ndarray = None       # u8, two 4-bit group scales per byte (CCQ)
    super_scale: np.ndarray = None  # f32 per row (all CCQ formats)
    code_scale: np.ndarray = None   # f32 per row (CCQ)
    code_zero: np.ndarray = None    # f32 per row (CCQ)
    zp: int = CCQ_ZP
    _keep: list = field(default_factory=list, repr=False)

    def _struct(self) -> _Weight:
        arrs = {}
        for name, dt in (("codes", np.uint8), ("scales", np.uint16), ("zeros", np.uint8),
                         ("qscale", np.uint8), ("super_scale", np.float32),
                         ("code_scale", np.float32), ("code_zero", np.float32)):
            a = getattr(self, name)
            arrs[name] = None if a is None else _c(a, dt)
        self._keep = list(arrs.values())
        return _Weight(self.format, self.group, self.experts, self.n, self.k,
                       *[None if arrs[nm] is None else arrs[nm].ctypes.data for nm in
                         ("codes", "scales", "zeros", "qscale", "super_scale", "code_scale",
                          "code_zero")],
                       self.zp)

    def nbytes(self) -> int:
        tot = 0
        for name in ("codes", "scales", "zeros", "qscale", "super_scale", "code_scale",
                     "code_zero"):
            a = getattr(self, name)
            if a is not None:
                tot += a.nbytes
        return tot


def default_zp(fmt: int) -> int:
    return {CCQ: CCQ_ZP, CCQ432: CCQ432_ZP, CCQ_HYBRID: CCQ_HYBRID_ZP}.get(fmt, CCQ_ZP)


def quantize(w, fmt: int, group: int = 64, refine=True, zp: int | None = None,
             return_full: bool = False):
    """Quantize fp32 weights [n, k] or [E, n, k] with the oracle's quantizers.

    CCQ: ``refine`` is True (re-pick and scale update), False, or a mask of CCQ_REPICK |
    CCQ_SCALE_UPDATE; with ``return_full`` the result is (Packed, codes before the cluster
    u16 [E, n, k/4])."""
    zp = default_zp(fmt) if zp is None else zp
    w = _c(w, np.float32)
    if w.ndim == 2:
        w = w[None]
    E, n, k = w.shape
    flat = w.reshape(E * n, k)
    G = k // 64
    if fmt == INT4:
        codes = np.zeros((E * n, k // 2), np.uint8)
        scales = np.zeros((E * n, G if group else 1), np.uint16)
        rc = lib().orc_quant_int4(_p(flat), E * n, k, group, _p(codes), _p(scales))
        if rc:
            raise ValueError("bad INT4 shape/group")
        return Packed(INT4, n, k, E, group, codes.reshape(E, n, -1),
                      scales.reshape(E, n, -1) if group else scales.reshape(E, n))
    if fmt == INT8:
        codes = np.zeros((E * n, k), np.int8)
        scales = np.zeros((E * n, G if group else 1), np.uint16)
        rc = lib().orc_quant_int8(_p(flat), E * n, k, group, _p(codes), _p(scales))
        if rc:
            raise ValueError("bad INT8 shape/group")
        return Packed(INT8, n, k, E, group, codes.view(np.uint8).reshape(E, n, k),
                      scales.reshape(E, n, -1) if group else scales.reshape(E, n))
    if fmt == AFFINE2:
        codes = np.zeros((E * n, k // 4), np.uint8)
        scales = np.zeros((E * n, G), np.uint16)
        zeros = np.zeros((E * n, G), np.uint8)
        rc = lib().orc_quant_affine2(_p(flat), E * n, k, _p(codes), _p(scales), _p(zeros))
        if rc:
            raise ValueError("bad affine shape")
        return Packed(AFFINE2, n, k, E, 64, codes.reshape(E, n, -1), scales.reshape(E, n, -1),
                      zeros.reshape(E, n, -1))
    if fmt == CCQ:
        codes = np.zeros((E * n, k // 4), np.uint8)
        qscale = np.zeros((E * n, (G + 1) // 2), np.uint8)
        sup = np.zeros(E * n, np.float32)
        cs = np.zeros(E * n, np.float32)
        cz = np.zeros(E * n, np.float32)
        full = np.zeros((E * n, k // 4), np.uint16) if return_full else None
        rc = lib().orc_quant_ccq(_p(flat), E * n, k, zp, _ccq_refine_bits(refine), _p(codes),
                                 _p(qscale), _p(sup), _p(cs), _p(cz), _p(full))
        if rc:
            raise ValueError("bad CCQ shape")
        p = Packed(CCQ, n, k, E, 64, codes.reshape(E, n, -1), qscale=qscale.reshape(E, n, -1),
                   super_scale=sup.reshape(E, n), code_scale=cs.reshape(E, n),
                   code_zero=cz.reshape(E, n), zp=zp)
        return (p, full.reshape(E, n, -1)) if return_full else p
    if fmt in ALG2_GROUP_BYTES:
        codes = np.zeros((E * n, G * ALG2_GROUP_BYTES[fmt]), np.uint8)
        sup = np.zeros(E * n, np.float32)
        rc = lib().orc_quant_alg2(_p(flat), E * n, k, fmt, zp, int(bool(refine)), _p(codes),
                                  _p(sup))
        if rc:
            raise ValueError("bad CCQ (4,3,2) / hybrid shape")
        return Packed(fmt, n, k, E, 64, codes.reshape(E, n, -1), super_scale=sup.reshape(E, n),
                      zp=zp)
    raise ValueError(f"unknown format {fmt}")


def alg2_pack(fmt: int, words, super_scale, zp: int | None = None) -> Packed:
    """Packed (4,3,2) / hybrid weight from raw code words [E, n, G, P] (u8 values for
    (4,3,2), P = 22; u16 values for the hybrid, P = 10, stored little endian)."""
    words = np.asarray(words)
    E, n, G, P = words.shape
    if fmt == CCQ432:
        assert P == 22
        codes = words.astype(np.uint8).reshape(E, n, G * 22)
    elif fmt == CCQ_HYBRID:
        assert P == 10
        codes = words.astype("<u2").reshape(E, n, G * 10).view(np.uint8)
    else:
        raise ValueError(f"not an Algorithm-2 format: {fmt}")
    return Packed(fmt, n, 64 * G, E, 64, np.ascontiguousarray(codes),
                  super_scale=_c(super_scale, np.float32).reshape(E, n),
                  zp=default_zp(fmt) if zp is None else zp)


def dequantize(p: Packed, expert: int = 0, n0: int = 0, n1: int | None = None) -> np.ndarray:
    """Decode rows [n0, n1) of one expert to bf16 bits ([CCQ] section 3.5; [E6.4])."""
    n1 = p.n if n1 is None else n1
    out = np.empty((n1 - n0, p.k), np.uint16)
    st = p._struct()
    if lib().orc_dequantize(ctypes.byref(st), expert, n0, n1, _p(out)) != 0:
        raise ValueError("bad dequantize arguments")
    return out


def gemm_bf16(x, w, want_f64: bool = False):
    """y = bf16(x @ w^T) with bf16 operands and an fp64 sum per output."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    m, k = x.shape
    n, k2 = w.shape
    assert k == k2
    y = np.empty((m, n), np.uint16)
    y64 = np.empty((m, n), np.float64) if want_f64 else None
    lib().orc_gemm_bf16(_p(x), m, k, _p(w), n, _p(y), _p(y64))
    return (y, y64) if want_f64 else y


def gemm(x, p: Packed, expert: int = 0):
    """Dense weight-only product: y = bf16(x @ dequantize(W)^T)."""
    return gemm_bf16(x, dequantize(p, expert))


def moe_route(ids, experts: int):
    """Stable counting sort of pair indices p = t*topk + j by expert id."""
    ids = _c(ids, np.int32)
    t, topk = ids.shape
    offsets = np.empty(experts + 1, np.int32)
    pairs = np.empty(t * topk, np.int32)
    if lib().orc_moe_route(_p(ids), t, topk, experts, _p(offsets), _p(pairs)) != 0:
        raise ValueError("expert id out of range")
    return offsets, pairs


def moe_ffn(x, ids, weights, gate: Packed, up: Packed, down: Packed, tokens=None):
    """Expert FFN y_t = bf16(sum_j w_tj * W_down[e] bf16(SiLU(W_gate[e] x_t) * W_up[e] x_t)).

    Returns y for the listed tokens (all tokens if ``tokens`` is None)."""
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    weights = _c(weights, np.float32)
    t, hidden = x.shape
    topk = ids.shape[1]
    experts = gate.experts
    tok = None if tokens is None else _c(tokens, np.int32)
    n_tok = t if tok is None else tok.size
    y = np.empty((n_tok, hidden), np.uint16)
    sg, su, sd = gate._struct(), up._struct(), down._struct()
    rc = lib().orc_moe_ffn(_p(x), t, hidden, _p(ids), _p(weights), topk, experts,
                           ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), gate.n,
                           _p(tok), n_tok, _p(y))
    if rc != 0:
        raise ValueError(f"orc_moe_ffn failed ({rc})")
    return y
