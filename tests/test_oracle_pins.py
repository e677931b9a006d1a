"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them re-types an oracle formula: each compares the
oracle with a printed value of the pages (fixtures under tests/golden/), a library routine
(torch, numpy), a brute-force enumeration, or an invariant that a plausible mistake (a
dropped term, a wrong sign, index or shift, a swapped nibble) would break.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------------------------------------
# bf16 conversions
# ---------------------------------------------------------------------------------------------

def test_f32_to_bf16_matches_torch_on_every_exponent_and_rounding_case(orc):
    # Every high half (sign, exponent, 7 mantissa bits) combined with the low halves that
    # decide rounding (exact, just below/at/above the tie, maximum) plus random low halves.
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000]
    lows += list(np.random.default_rng(1).integers(0, 1 << 16, 8))
    bits = (hi[:, None] | np.array(lows, np.uint32)[None, :]).ravel()
    f = bits.view(np.float32)
    ours = orc.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_f32_to_bf16_matches_torch_on_every_fp32_pattern(orc):
    # all 2^32 fp32 bit patterns, 2^24 at a time: round half to even on the high 16 bits, every
    # NaN to the canonical 0x7FC0
    low = np.arange(1 << 24, dtype=np.uint32)
    for hi in range(256):
        bits = low | np.uint32(hi << 24)
        f = bits.view(np.float32)
        ours = orc.f32_to_bf16(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(ours[~nan], ref[~nan]), hex(hi << 24)
        assert np.all(ours[nan] == 0x7FC0), hex(hi << 24)


def _bf16_val(b):
    return Fraction(float(orc_bits_to_f32(b)))


def orc_bits_to_f32(b):
    return np.array([b], np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)[0]


def test_f64_to_bf16_is_nearest_even_by_exhaustive_neighbour_check(orc):
    # Property of the definition: the result r is a bf16 value no farther from d than either
    # bf16 neighbour of r, and on an exact tie r has an even mantissa.
    g = np.random.default_rng(7)
    d = np.concatenate([
        g.standard_normal(3000) * np.exp(g.uniform(-85, 85, 3000)),
        g.standard_normal(200) * 1e-39,  # bf16 subnormal range
    ])
    r = orc.f64_to_bf16(d)
    for di, ri in zip(d, r):
        ri = int(ri)
        dv = Fraction(float(di))
        rv = Fraction(float(orc_bits_to_f32(ri)))
        for nb in (ri - 1, ri + 1):
            if (nb & 0x7F80) == 0x7F80 or nb < 0 or nb > 0xFFFF:
                continue
            if (nb ^ ri) & 0x8000:
                continue
            nv = Fraction(float(orc_bits_to_f32(nb)))
            assert abs(dv - rv) <= abs(dv - nv)
            if abs(dv - rv) == abs(dv - nv):
                assert ri % 2 == 0


def test_f64_to_bf16_avoids_double_rounding(orc):
    # 1 + 2^-8 is a bf16 tie (even -> 1.0); a double just above it must round up even though
    # its fp32 rounding lands exactly on the tie.
    d = np.array([1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40, -(1.0 + 2.0 ** -8 + 2.0 ** -40)])
    r = orc.f64_to_bf16(d)
    assert r[0] == 0x3F80
    assert r[1] == 0x3F81
    assert r[2] == 0xBF81
    # whereas going through fp32 first would give the tie's even value
    via32 = torch.tensor(d[1:2], dtype=torch.float64).float().to(torch.bfloat16)
    assert via32.view(torch.int16).item() == 0x3F80


# ---------------------------------------------------------------------------------------------
# [E6.4] packing, sizes, RTN, affine worked example
# ---------------------------------------------------------------------------------------------

def test_pack_int4_printed_bytes(orc):
    for first, second, byte in _rows("int4_pack_table.txt"):
        out = orc.pack_int4([int(first), int(second)])
        assert out.tolist() == [int(byte)]
        assert orc.unpack_int4(out, 2).tolist() == [int(first), int(second)]


def test_unpack_every_byte_roundtrips(orc):
    data = np.arange(256, dtype=np.uint8)
    codes = orc.unpack_int4(data, 512)
    assert codes.min() == -8 and codes.max() == 7
    assert np.array_equal(orc.pack_int4(codes), data)
    # low nibble is the first code: byte 0x0F -> (-1, 0), byte 0xF0 -> (0, -1)
    assert orc.unpack_int4(np.array([0x0F, 0xF0], np.uint8), 4).tolist() == [-1, 0, 0, -1]


def test_pack_odd_count_pads_with_zero_and_rejects_out_of_range(orc):
    assert orc.pack_int4([3, -1, 5]).tolist() == [0xF3, 0x05]
    assert orc.unpack_int4(orc.pack_int4([3, -1, 5]), 3).tolist() == [3, -1, 5]
    for bad in ([8], [-9], [0, 100]):
        with pytest.raises(ValueError):
            orc.pack_int4(bad)


def test_packed_size_printed_counts(orc):
    for n, bits, nbytes in _rows("byte_counts.txt"):
        assert orc.packed_size(int(n), int(bits)) == int(nbytes)
    assert orc.packed_size(3, 4) == 2  # odd count padded
    assert orc.packed_size(8, 2) == 2


def test_rtn_ties_to_even_and_clip_like_numpy(orc):
    w = np.array([0.5, 1.5, 2.5, -2.5, -0.5, 3.49, 100.0, -100.0, 7.5, -8.5])
    got = orc.rtn(w, 1.0)
    ref = np.clip(np.round(w), -8, 7)  # numpy's round is the exercise's stated rounding
    assert np.array_equal(got, ref)
    assert got[:4].tolist() == [0.0, 2.0, 2.0, -2.0]
    g = np.random.default_rng(3).standard_normal(1000) * 0.05
    assert np.array_equal(orc.rtn(g, 0.01), np.clip(np.round(g / 0.01), -8, 7) * 0.01)


def test_affine_worked_example(orc):
    (x, s, z, q, xhat, err), = _rows("affine_worked_example.txt")
    qv = orc.affine_quant([float(x)], float(s), int(z), -8, 7)
    assert qv.tolist() == [int(q)]
    xv = orc.affine_dequant(qv, float(s), int(z))
    assert math.isclose(xv[0], float(xhat), rel_tol=1e-12)
    assert math.isclose(abs(float(x) - xv[0]), float(err), rel_tol=1e-9)


def test_affine_zero_point_and_clip(orc):
    # q = clip(round(x/s) + z): with z = 2 the value -0.2/0.1 = -2 maps to code 0; beyond the
    # range codes clip; x_hat = s(q - z) undoes z.
    q = orc.affine_quant([-0.2, 0.0, 0.1, 5.0, -5.0], 0.1, 2, 0, 3)
    assert q.tolist() == [0, 2, 3, 3, 0]
    assert np.allclose(orc.affine_dequant(q, 0.1, 2), [-0.2, 0.0, 0.1, 0.1, -0.2])


# ---------------------------------------------------------------------------------------------
# [CCQ] codebook, bit-shift decode, bpw, configuration table
# ---------------------------------------------------------------------------------------------

def test_codebook_example(orc):
    (L, N, S, code, states), = _rows("codebook_example.txt")
    L, N, S, code = int(L), int(N), int(S), int(code)
    assert orc.ccq_total_bits(L, N, S) == 4  # a 4-bit code 0010
    assert orc.ccq_states(code, L, N, S) == [int(s) for s in states.split(",")]


def test_dequant_config_table(orc):
    for configs, bpw, wmask, smask, shifts, cluster in _rows("dequant_config_table.txt"):
        parts = [tuple(int(v) for v in c.split(",")) for c in configs.split("+")]
        shifts = [int(v) for v in shifts.split(",")]
        # masks are 2^L - 1
        assert all((1 << L) - 1 == int(wmask, 16) for L, _, _ in parts)
        # closed form (N-1-i)*S, a hybrid word holding its parts top to bottom
        total = sum(orc.ccq_total_bits(*p) for p in parts)
        got, base = [], total
        for p in parts:
            base -= orc.ccq_total_bits(*p)
            got += [base + s for s in orc.ccq_shifts(*p)]
        assert got == shifts
        if cluster == "yes":
            assert abs(orc.ccq_bpw(8, 64, parts[0][1], 4) - float(bpw)) < 0.005
            assert int(smask, 16) == 0xF


def test_scale_bits_and_bpw_equation(orc):
    for name, g, per_code, code_bits, codes, spare, bpw in _rows("scale_bits_example.txt"):
        g, per_code, code_bits, codes, spare = int(g), int(per_code), int(code_bits), int(codes), int(spare)
        assert -(-g // per_code) == codes
        if name == "432":
            L = 4
            assert code_bits - L == spare  # only the first state of the last code is used
            assert orc.ccq_bpw(8, g, 3, 0) == float(bpw)
        elif name == "hybrid":
            assert code_bits == orc.ccq_total_bits(3, 3, 2) + orc.ccq_total_bits(3, 4, 2)
            assert code_bits - 3 == spare
            assert orc.ccq_bpw(16, g, 7, 0) == float(bpw)
        else:
            assert orc.ccq_bpw(code_bits, g, per_code, 4) == float(bpw)


def test_state_overlap_invariant_all_codes(orc):
    # adjacent (6,4,3) states share L - S = 3 bits: low 3 bits of state j = high 3 of j+1
    for code in range(0, 1 << 15, 37):
        u = orc.ccq_states(code, 6, 4, 3)
        for j in range(3):
            assert (u[j] & 7) == (u[j + 1] >> 3)
        # and the states determine the code (T = 15 bits carried without loss)
        assert ((u[0] << 9) | (u[1] & 7) << 6 | (u[2] & 7) << 3 | (u[3] & 7)) == code


# ---------------------------------------------------------------------------------------------
# [CCQ] stage 1 of the code-cluster decode (parity unpinned by the pages: invariants and an
# exact-rational re-statement only)
# ---------------------------------------------------------------------------------------------

def _round_to_f32(fr: Fraction) -> Fraction:
    """Correctly rounded fp32 value of an exact rational (nearest, ties to even)."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        cv = Fraction(float(cand))
        key = (abs(cv - fr), int(np.array([cand]).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, cv)
    return best[1]


def test_ccq_expand_exact_rational(orc):
    g = np.random.default_rng(11)
    cases = [(1.0, 0.0), (128.0, 5.0), (127.37, 0.25)]
    cases += [(float(np.float32(g.uniform(1, 130))), float(np.float32(g.uniform(0, 200))))
              for _ in range(4)]
    cases += [(float(np.float32(128.5)), float(np.float32(0.5)))]  # exact .5 ties
    for a, b in cases:
        for cp in range(256):
            t = _round_to_f32(Fraction(cp) * Fraction(a) + Fraction(b))
            ref = round(t)  # Fraction rounds half to even
            ref = min(max(ref, 0), 32767)
            assert orc.ccq_expand(cp, a, b) == ref, (a, b, cp)


def test_ccq_expand_identity_clamp_monotone(orc):
    assert [orc.ccq_expand(c, 1.0, 0.0) for c in range(256)] == list(range(256))
    assert orc.ccq_expand(255, 200.0, 0.0) == 32767
    assert orc.ccq_expand(0, 1.0, -10.0) == 0
    vals = [orc.ccq_expand(c, 97.3, 11.0) for c in range(256)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


# ---------------------------------------------------------------------------------------------
# Full decode functions
# ---------------------------------------------------------------------------------------------

def _bf16_of(x):
    return torch.tensor(x, dtype=torch.float64).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_int4_decode_matches_unpack_times_scale(orc):
    g = np.random.default_rng(5)
    n, k = 3, 256
    codes = g.integers(0, 256, (1, n, k // 2), dtype=np.uint8)
    scales = _bf16_of(g.uniform(0.001, 0.01, (1, n, k // 64)))
    p = orc.Packed(orc.INT4, n, k, 1, 64, codes, scales)
    got = orc.dequantize(p)
    for r in range(n):
        q = orc.unpack_int4(codes[0, r], k)
        s = orc.bf16_to_f32(np.repeat(scales[0, r], 64))
        assert np.array_equal(got[r], _bf16_of(q.astype(np.float64) * s.astype(np.float64)))
    # per-channel scale
    sc = _bf16_of(g.uniform(0.001, 0.01, (1, n)))
    p2 = orc.Packed(orc.INT4, n, k, 1, 0, codes, sc)
    got2 = orc.dequantize(p2)
    for r in range(n):
        q = orc.unpack_int4(codes[0, r], k)
        assert np.array_equal(got2[r], _bf16_of(q * float(orc.bf16_to_f32(sc[0, r:r + 1])[0])))


def test_affine2_decode_matches_affine_formula(orc):
    g = np.random.default_rng(6)
    n, k = 2, 128
    q = g.integers(0, 4, (n, k))
    codes = np.zeros((1, n, k // 4), np.uint8)
    for j in range(4):  # the first of each 4 weights in the lowest two bits
        codes[0] |= (q[:, j::4] << (2 * j)).astype(np.uint8)
    scales = _bf16_of(g.uniform(0.01, 0.05, (1, n, k // 64)))
    zeros = g.integers(0, 4, (1, n, k // 64), dtype=np.uint8)
    p = orc.Packed(orc.AFFINE2, n, k, 1, 64, codes, scales, zeros)
    got = orc.dequantize(p)
    for r in range(n):
        for gi in range(k // 64):
            s = float(orc.bf16_to_f32(scales[0, r, gi:gi + 1])[0])
            ref = orc.affine_dequant(q[r, gi * 64:(gi + 1) * 64], s, int(zeros[0, r, gi]))
            assert np.array_equal(got[r, gi * 64:(gi + 1) * 64], _bf16_of(ref))


def test_ccq_decode_every_code_reduces_to_states_and_affine(orc):
    # 128 rows with code scale 1 and code zero 256*r cover all 2^15 codes; the decode must give
    # the bit-shift states of each code in order, mapped by x_hat = s (u - zp).
    rows, k = 128, 1024
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))  # k/4 = 256 bytes per row
    g = np.random.default_rng(8)
    sq = g.integers(0, 16, (rows, k // 64), dtype=np.uint8)
    qscale = (sq[:, 0::2] | (sq[:, 1::2] << 4)).astype(np.uint8)
    sup = g.uniform(1e-4, 1e-3, rows).astype(np.float32)
    p = orc.Packed(orc.CCQ, rows, k, 1, 64, codes[None], qscale=qscale[None],
                   super_scale=sup[None], code_scale=np.ones((1, rows), np.float32),
                   code_zero=(256.0 * np.arange(rows, dtype=np.float32))[None], zp=32)
    got = orc.dequantize(p)
    for r in range(0, rows, 9):
        for c in range(256):
            code = 256 * r + c
            u = orc.ccq_states(code, 6, 4, 3)
            for j in range(4):
                kk = 4 * c + j
                gi = kk // 64
                s = np.float32(np.float32(sq[r, gi]) * sup[r])  # group scale x super scale
                ref = orc.affine_dequant([u[j]], float(s), 32)
                assert got[r, kk] == _bf16_of(ref)[0], (r, c, j)


# ---------------------------------------------------------------------------------------------
# Quantizers
# ---------------------------------------------------------------------------------------------

def test_int4_quantizer_rtn_properties(orc):
    w = np.random.default_rng(9).standard_normal((4, 256)).astype(np.float32) * 0.02
    p = orc.quantize(w, orc.INT4, 64)
    for r in range(4):
        q = orc.unpack_int4(p.codes[0, r], 256)
        for gi in range(4):
            seg = w[r, gi * 64:(gi + 1) * 64]
            s = orc.bf16_to_f32(p.scales[0, r, gi:gi + 1])[0]
            assert s == orc.bf16_to_f32(_bf16_of(np.float32(np.abs(seg).max()) / np.float32(7)))[0]
            qq = q[gi * 64:(gi + 1) * 64]
            exact = seg.astype(np.float64) / float(s)
            inside = (exact > -8.5) & (exact < 7.5)
            assert np.all(np.abs(qq[inside] - exact[inside]) <= 0.5 + 1e-6)
            assert np.all(qq >= -8) and np.all(qq <= 7)
    # dequantized values equal the exercise's rtn with the stored scale (up to bf16)
    dq = orc.bf16_to_f32(orc.dequantize(p))
    ref = np.concatenate([orc.rtn(w[0, gi * 64:(gi + 1) * 64],
                                  float(orc.bf16_to_f32(p.scales[0, 0, gi:gi + 1])[0]))
                          for gi in range(4)])
    assert np.allclose(dq[0], ref, rtol=2 ** -8, atol=0)


def test_affine2_quantizer_properties(orc):
    w = np.random.default_rng(10).standard_normal((3, 128)).astype(np.float32) * 0.02
    p = orc.quantize(w, orc.AFFINE2)
    dq = orc.bf16_to_f32(orc.dequantize(p)).astype(np.float64)
    for r in range(3):
        for gi in range(2):
            seg = w[r, gi * 64:(gi + 1) * 64]
            s = float(orc.bf16_to_f32(p.scales[0, r, gi:gi + 1])[0])
            err = np.abs(dq[r, gi * 64:(gi + 1) * 64] - seg)
            # within the representable range the error is at most half a step (+ bf16)
            assert err.max() <= 0.5 * s * 1.01 + 1e-6 or err.max() <= s * 1.01


def test_ccq_search_equals_brute_force(orc):
    # brute force over all 2^15 codes using the generic bit-shift decoder
    codes = np.arange(1 << 15)
    states = np.stack([(codes >> (9 - 3 * j)) & 0x3F for j in range(4)], axis=1)
    g = np.random.default_rng(12)
    for trial in range(40):
        s = float(g.uniform(0.0005, 0.002))
        v = g.standard_normal(4) * 0.02
        if trial % 10 == 0:
            v = np.zeros(4)
        cost = (((v[None, :] - (states - 32) * s) ** 2)).sum(axis=1)
        best = int(np.argmin(cost))  # argmin returns the first (smallest) code on ties
        code, c = orc.ccq_search(v, s)
        assert abs(c - cost[best]) <= 1e-12 * max(1.0, cost[best])
        if code != best:  # only an exact-to-rounding tie may pick another code
            assert abs(cost[code] - cost[best]) <= 1e-15
        if trial % 10 == 0:
            assert code == best


def test_ccq_quantizer_reconstructs_gaussian(orc):
    w = np.random.default_rng(13).standard_normal((8, 512)).astype(np.float32) * 0.02
    p = orc.quantize(w, orc.CCQ, refine=True)
    dq = orc.bf16_to_f32(orc.dequantize(p)).astype(np.float64)
    rel = np.sqrt(((dq - w) ** 2).mean() / (w.astype(np.float64) ** 2).mean())
    # The code cluster keeps 256 of the 2^15 codes per row (about 2 bits per weight of
    # freedom); on i.i.d. Gaussian rows that costs far more than the 6-bit states would.  The
    # bound only guards against a broken encoder (a sign or scale slip gives rel >= 1).
    assert rel < 0.5, rel
    raw = orc.quantize(w, orc.CCQ, refine=False)
    dq_raw = orc.bf16_to_f32(orc.dequantize(raw)).astype(np.float64)
    rel_raw = np.sqrt(((dq_raw - w) ** 2).mean() / (w.astype(np.float64) ** 2).mean())
    assert rel <= rel_raw + 1e-12  # re-picking among decodable codes never hurts
    sq = np.stack([p.qscale & 0xF, p.qscale >> 4], axis=-1).reshape(1, 8, -1)
    assert sq.min() >= 1 and sq.max() <= 15
    assert p.code_zero.min() >= 0 and p.code_scale.min() > 0


# ---------------------------------------------------------------------------------------------
# GEMM, routing, MoE
# ---------------------------------------------------------------------------------------------

def test_gemm_matches_torch_fp64_and_one_hot(orc):
    g = np.random.default_rng(14)
    x = _bf16_of(g.standard_normal((5, 192)))
    w = _bf16_of(g.standard_normal((7, 192)) * 0.02)
    y, y64 = orc.gemm_bf16(x, w, want_f64=True)
    xt = torch.from_numpy(orc.bf16_to_f32(x).astype(np.float64))
    wt = torch.from_numpy(orc.bf16_to_f32(w).astype(np.float64))
    ref = (xt @ wt.T).numpy()
    bound = 192 * 2 ** -52 * (np.abs(xt.numpy()) @ np.abs(wt.numpy()).T)
    assert np.all(np.abs(y64 - ref) <= bound + 1e-300)
    assert np.array_equal(y, torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)) or \
        np.abs(orc.bf16_to_f32(y) - ref).max() <= np.abs(ref).max() * 2 ** -8
    onehot = np.zeros((1, 192), np.uint16)
    onehot[0, 17] = 0x3F80  # 1.0
    assert np.array_equal(orc.gemm_bf16(onehot, w)[0], w[:, 17])


def test_route_matches_sorted_and_bincount(orc):
    g = np.random.default_rng(15)
    ids = g.integers(0, 16, (40, 4)).astype(np.int32)
    off, pairs = orc.moe_route(ids, 16)
    flat = ids.ravel()
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=16))
    assert pairs.tolist() == sorted(range(flat.size), key=lambda p: (flat[p], p))
    with pytest.raises(ValueError):
        orc.moe_route(np.array([[0, 16]], np.int32), 16)


def _dense_ffn_f64(orc, x, wg, wu, wd):
    """h = bf16(SiLU(g) u) from unrounded g, u; d unrounded -- via the oracle's GEMM sums."""
    _, g64 = orc.gemm_bf16(x, wg, want_f64=True)
    _, u64 = orc.gemm_bf16(x, wu, want_f64=True)
    h = orc.f64_to_bf16(torch.nn.functional.silu(torch.from_numpy(g64)).numpy() * u64)
    _, d64 = orc.gemm_bf16(h, wd, want_f64=True)
    return d64


def test_moe_reduces_to_dense_ffn(orc):
    g = np.random.default_rng(16)
    E, H, I, T = 4, 128, 64, 6
    wg = g.standard_normal((E, I, H)).astype(np.float32) * 0.05
    wu = g.standard_normal((E, I, H)).astype(np.float32) * 0.05
    wd = g.standard_normal((E, H, I)).astype(np.float32) * 0.05
    pg, pu, pd = (orc.quantize(a, orc.INT4, 64) for a in (wg, wu, wd))
    x = _bf16_of(g.standard_normal((T, H)))
    # k = 1, weight 1: every token is the dense FFN of its expert
    ids = g.integers(0, E, (T, 1)).astype(np.int32)
    y = orc.moe_ffn(x, ids, np.ones((T, 1), np.float32), pg, pu, pd)
    for t in range(T):
        e = int(ids[t, 0])
        d = _dense_ffn_f64(orc, x[t:t + 1], orc.dequantize(pg, e), orc.dequantize(pu, e),
                           orc.dequantize(pd, e))
        assert np.array_equal(y[t], orc.f64_to_bf16(d[0]))
    # k = 2 with weights: the weighted sum of two dense FFNs, slot order 0 then 1
    ids2 = np.stack([np.zeros(T, np.int32), np.full(T, 3, np.int32)], axis=1)
    w2 = g.uniform(0.1, 0.9, (T, 2)).astype(np.float32)
    y2 = orc.moe_ffn(x, ids2, w2, pg, pu, pd, tokens=np.array([1, 4], np.int32))
    for i, t in enumerate((1, 4)):
        d0 = _dense_ffn_f64(orc, x[t:t + 1], orc.dequantize(pg, 0), orc.dequantize(pu, 0), orc.dequantize(pd, 0))
        d3 = _dense_ffn_f64(orc, x[t:t + 1], orc.dequantize(pg, 3), orc.dequantize(pu, 3), orc.dequantize(pd, 3))
        ref = orc.f64_to_bf16(float(w2[t, 0]) * d0[0] + float(w2[t, 1]) * d3[0])
        assert np.array_equal(y2[i], ref)
    # permuting slots changes at most the last bit of some outputs
    y3 = orc.moe_ffn(x, ids2[:, ::-1].copy(), w2[:, ::-1].copy(), pg, pu, pd, tokens=np.array([1, 4], np.int32))
    diff = np.abs(y3.astype(np.int32) - y2.astype(np.int32))
    assert diff.max() <= 1
