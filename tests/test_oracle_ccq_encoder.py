"""Pins of the oracle's (6,4,3) code-cluster encoder and of stage 1 of its decode.

"CCQ: Convolutional Code for Extreme Low-bit Quantization in LLMs":
  * section 3.3 "Code Cluster", Eq. 1: C' = round((C - beta) / alpha), C in [0, 2^T - 1],
    C' in [0, 255], alpha the code scale and beta the code zero point of an asymmetric
    quantization of the row's codes;
  * section 3.5, "Dequantization with Code Cluster": stage 1 widens C' back to a code,
    round(C' * alpha + beta);
  * section 3.4 "Scale Optimization", Eq. 2-4: with the searched codes fixed, the group error
    sum (W_i - W^q_i S)^2 is least at S = sum W_i W^q_i / sum (W^q_i)^2.

Nothing here re-types the oracle's arithmetic: Eq. 1 is evaluated in exact rationals, the codes
it maps are checked against the brute-force-pinned trellis search, the round trip is a bound
that follows from Eq. 1 alone, and the scale update is checked against numpy's least-squares
solver.  A slip in any of these steps (alpha over 256 levels instead of 255, floor for round,
alpha and beta exchanged, the least-squares ratio inverted or its denominator taken over the
weights) fails at least one test below.  The rule that keeps the updated scale only when the
group error drops cannot be told apart from always keeping it except on exact ties: the error
with the codes fixed is a parabola in S, the re-quantized S* is the feasible grid point nearest
its minimum, and the search at that point can only lower the error further.
"""
from fractions import Fraction

import numpy as np
import pytest


def _nibbles(qscale_row, groups):
    q = np.asarray(qscale_row).astype(np.int64)
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(-1)[:groups]


def _states(orc, code):
    return orc.ccq_states(int(code), 6, 4, 3)


def _rows_for_cluster():
    g = np.random.default_rng(2101)
    rows = [g.standard_normal(512) * 0.02 for _ in range(5)]
    # heavy outliers widen one group's scale and spread the row's codes
    r = g.standard_normal(512) * 0.02
    r[[3, 200, 411]] = [0.5, -0.4, 0.3]
    rows.append(r)
    # a smooth ramp: neighbouring codes close together
    rows.append(np.linspace(-0.03, 0.05, 512))
    return np.stack(rows).astype(np.float32)


@pytest.fixture(scope="module")
def cluster_case(orc):
    w = _rows_for_cluster()
    p, full = orc.quantize(w, orc.CCQ, refine=0, return_full=True)
    return w, p, full[0].astype(np.int64)


def test_cluster_maps_the_searched_codes(orc, cluster_case):
    """The codes Eq. 1 maps are the trellis-search codes of each vector at its group's decode
    scale f32(s_q) * super (the search itself is pinned against brute force)."""
    w, p, full = cluster_case
    n, k = w.shape
    for r in range(n):
        sq = _nibbles(p.qscale[0, r], k // 64)
        for c in range(k // 4):
            s = float(np.float32(np.float32(sq[c // 16]) * p.super_scale[0, r]))
            code, _ = orc.ccq_search(w[r, 4 * c:4 * c + 4].astype(np.float64), s)
            assert full[r, c] == code, (r, c)


def test_eq1_code_cluster_exact(orc, cluster_case):
    """Eq. 1 on every code of every row: C' = round_half_even((C - beta) / alpha) in exact
    rationals, already inside [0, 255] (no clipping), the row's smallest code at 0 and its
    largest at 255; beta is the smallest code (the asymmetric zero point)."""
    w, p, full = cluster_case
    for r in range(w.shape[0]):
        C = full[r]
        alpha = Fraction(float(p.code_scale[0, r]))
        beta = Fraction(float(p.code_zero[0, r]))
        assert beta == int(C.min())
        assert alpha > 1  # every row here has distinct codes spread over more than 255
        cp = p.codes[0, r].astype(np.int64)
        for c in range(C.size):
            exact = round((Fraction(int(C[c])) - beta) / alpha)  # Fraction rounds half to even
            assert 0 <= exact <= 255, (r, c, exact)
            assert cp[c] == exact, (r, c, cp[c], exact)
        assert cp[np.argmin(C)] == 0
        assert cp[np.argmax(C)] == 255


def test_eq1_ties_round_to_even(orc):
    """Exact half-way codes go to the even neighbour.  The row's weights are the decoded states
    (u - 32) of chosen codes at a decode scale of exactly 1 (every group's absmax is 31, so
    s_g = 1, s_q = 15 and f32(15 * f32(1/15)) = 1), so the search returns those codes at zero
    error.  Its codes span 4681 .. 5191, so alpha = 510 / 255 = 2 and beta = 4681; the codes
    4682, 4684, 4686 and 5112 sit at (C - beta) / alpha = 0.5, 1.5, 2.5 and 215.5."""
    # no state is 0 (value -32) and code 5112 carries a state 63 (value +31) in both groups
    group0 = [4681, 5191, 4682, 4684, 4686, 5112] + [4681] * 10
    group1 = [5112] + [4681] * 15
    w = np.array([[u - 32 for code in group0 + group1 for u in _states(orc, code)]], np.float32)
    assert np.abs(w).max() == 31
    p, full = orc.quantize(w, orc.CCQ, refine=0, return_full=True)
    assert full[0, 0].tolist() == group0 + group1
    assert float(p.code_scale[0, 0]) == 2.0 and float(p.code_zero[0, 0]) == 4681.0
    assert p.codes[0, 0, :6].tolist() == [0, 255, 0, 2, 2, 216]
    assert p.codes[0, 0, 16] == 216


def test_stage1_round_trip_bound(orc, cluster_case):
    """Stage 1 inverts Eq. 1 to within the cluster's resolution: expanding C' gives back every
    code to within alpha / 2 + 1/2 (the Eq. 1 rounding, the fp32 evaluation and the rounding
    to an integer).  This fixes the direction of stage 1 (C' * alpha + beta) and the roles of
    alpha and beta for alpha != 1."""
    w, p, full = cluster_case
    for r in range(w.shape[0]):
        a = float(p.code_scale[0, r])
        b = float(p.code_zero[0, r])
        bound = a / 2 + 0.5 + 2.0 ** -8
        for c in range(full.shape[1]):
            back = orc.ccq_expand(int(p.codes[0, 0 + r, c]), a, b)
            assert abs(back - int(full[r, c])) <= bound, (r, c, back, full[r, c], a)


def test_constant_row_cluster(orc):
    """A row whose codes are all equal has alpha = 1 (the reading for a zero range), beta = C
    and C' = 0 everywhere, and stage 1 returns C itself."""
    w = np.zeros((1, 256), np.float32)
    p, full = orc.quantize(w, orc.CCQ, refine=0, return_full=True)
    C = full[0, 0]
    assert np.all(C == C[0])
    assert float(p.code_scale[0, 0]) == 1.0 and float(p.code_zero[0, 0]) == float(C[0])
    assert np.all(p.codes == 0)
    assert orc.ccq_expand(0, 1.0, float(C[0])) == int(C[0])


# ---------------------------------------------------------------------------------------------
# Section 3.4 Eq. 2-4: scale optimization
# ---------------------------------------------------------------------------------------------

def _group_error(orc, wg, codes, s, zp=32):
    q = np.array([[u - zp for u in _states(orc, c)] for c in codes], np.float64).reshape(-1)
    r = wg.astype(np.float64) - q * s
    return float(np.dot(r, r)), q


def test_scale_update_is_least_squares(orc):
    g = np.random.default_rng(2102)
    accepted = rejected = unchanged = 0
    for trial in range(60):
        wg = (g.standard_normal(64) * 0.02).astype(np.float32)
        if trial % 3 == 0:
            wg[g.integers(0, 64)] *= 8  # an outlier: absmax scale far above least squares
        s_g = float(np.abs(wg.astype(np.float64)).max()) / 31.0
        sup = np.float32(s_g / float(g.uniform(6, 15)))
        sq = int(np.clip(np.rint(s_g / float(sup)), 1, 15))
        codes0, sq0, err0 = orc.ccq_encode_group(wg, sup, sq, update=False)
        assert sq0 == sq
        s = float(np.float32(np.float32(sq) * sup))
        e0, q = _group_error(orc, wg, codes0, s)
        assert abs(e0 - err0) <= 1e-12 * max(e0, 1e-30)
        # S* with the codes fixed: the least-squares solution of q * S ~ w
        S = float(np.linalg.lstsq(q[:, None], wg.astype(np.float64), rcond=None)[0][0])
        sq2 = int(np.clip(np.rint(S / float(sup)), 1, 15))
        codes1, sq1, err1 = orc.ccq_encode_group(wg, sup, sq, update=True)
        if sq2 == sq or S <= 0:
            assert sq1 == sq and list(codes1) == list(codes0) and err1 == err0
            unchanged += 1
            continue
        s2 = float(np.float32(np.float32(sq2) * sup))
        codes2 = [orc.ccq_search(wg[4 * c:4 * c + 4].astype(np.float64), s2)[0] for c in range(16)]
        e2, _ = _group_error(orc, wg, codes2, s2)
        if abs(e2 - e0) <= 1e-12 * e0:
            continue  # too close to call in a different summation order
        if e2 < e0:
            assert sq1 == sq2 and list(codes1) == codes2, trial
            assert abs(err1 - e2) <= 1e-12 * e2
            accepted += 1
        else:
            assert sq1 == sq and list(codes1) == list(codes0), trial
            rejected += 1
    # the cases exercise every branch of the update
    assert accepted > 0 and rejected + unchanged > 0, (accepted, rejected, unchanged)


def test_scale_update_never_increases_error(orc):
    """The property the update rests on: the re-quantized least-squares scale never loses to the
    first scale (the pinned search minimizes each vector's error at the new scale)."""
    g = np.random.default_rng(2103)
    for _ in range(40):
        wg = (g.standard_normal(64) * g.uniform(0.005, 0.05)).astype(np.float32)
        sup = np.float32(float(np.abs(wg).max()) / 31.0 / 15.0)
        sq = int(g.integers(1, 16))
        _, _, e0 = orc.ccq_encode_group(wg, sup, sq, update=False)
        _, _, e1 = orc.ccq_encode_group(wg, sup, sq, update=True)
        assert e1 <= e0


def test_quantizer_applies_the_update_group_by_group(orc):
    """With the scale update on, every group's 4-bit scale and codes are what the group
    update gives from the scale the plain quantizer chose for it."""
    w = (np.random.default_rng(2104).standard_normal((6, 1024)) * 0.02).astype(np.float32)
    w[2, 77] = 0.3
    p0, full0 = orc.quantize(w, orc.CCQ, refine=0, return_full=True)
    p2, full2 = orc.quantize(w, orc.CCQ, refine=orc.CCQ_SCALE_UPDATE, return_full=True)
    assert np.array_equal(p0.super_scale, p2.super_scale)
    changed = 0
    for r in range(w.shape[0]):
        sq0 = _nibbles(p0.qscale[0, r], 16)
        sq2 = _nibbles(p2.qscale[0, r], 16)
        for gi in range(16):
            codes, sq, _ = orc.ccq_encode_group(w[r, 64 * gi:64 * gi + 64], p0.super_scale[0, r],
                                                int(sq0[gi]), update=True)
            assert sq2[gi] == sq
            assert np.array_equal(full2[0, r, 16 * gi:16 * gi + 16], codes)
            changed += int(sq != sq0[gi])
    assert changed > 0
    # the update lowers the reconstruction error before the cluster
    dq0 = orc.bf16_to_f32(orc.dequantize(orc.quantize(w, orc.CCQ, refine=orc.CCQ_REPICK)))
    dq3 = orc.bf16_to_f32(orc.dequantize(orc.quantize(w, orc.CCQ, refine=True)))
    e0 = float(((dq0 - w) ** 2).sum())
    e3 = float(((dq3 - w) ** 2).sum())
    assert e3 < e0 * 1.05, (e3, e0)
