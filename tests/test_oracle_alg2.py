"""Pins of the oracle's CCQ formats without code cluster: (4,3,2) at 2.75 bpw and the hybrid
(3,3,2)+(3,4,2) at 2.5 bpw ("CCQ: Convolutional Code for Extreme Low-bit Quantization in
LLMs", section 3.5, algorithm "Dequantization without Code Cluster" and the table of
dequantization configurations; section 3.4, scale compression).

The decode is checked against the generic bit-shift state decoder (itself pinned by the
pages' codebook example and the configuration table), the table's scale masks read from the
golden fixture, and the byte counts the pages state; the quantizer against exhaustive search
and an exact round trip.  Runs on the CPU.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table():
    rows = {}
    with open(os.path.join(GOLDEN, "dequant_config_table.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                configs, bpw, wmask, smask, shifts, cluster = ln.split()
                rows[configs] = dict(bpw=float(bpw), wmask=int(wmask, 16), smask=int(smask, 16),
                                     shifts=[int(v) for v in shifts.split(",")])
    return rows


def _bf16_of(x):
    return (torch.tensor(np.asarray(x, np.float64), dtype=torch.float64).float()
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def _state_tables(orc, fmt):
    """Per stored word value: the states it carries, in weight order (generic decoder)."""
    if fmt == orc.CCQ432:
        return np.array([orc.ccq_states(c, 4, 3, 2) for c in range(256)], np.int64)
    s1 = np.array([orc.ccq_states(c, 3, 3, 2) for c in range(128)], np.int64)
    s2 = np.array([orc.ccq_states(c, 3, 4, 2) for c in range(512)], np.int64)
    w = np.arange(1 << 16)
    return np.concatenate([s1[w >> 9], s2[w & 0x1FF]], axis=1)  # (3,3,2) part on top


def _reference_decode(orc, fmt, words, sup, zp):
    """words [n, G, P] -> fp64 values [n, 64 G]: weight 7i+j (hybrid) or 3i+j ((4,3,2)) is
    state j of word i; weight 63 is the first state of the last word; the group scale is the
    last word masked with the table's scale mask, times the row's super scale (fp32)."""
    tab = _table()["4,3,2" if fmt == orc.CCQ432 else "3,3,2+3,4,2"]
    st = _state_tables(orc, fmt)
    n, G, P = words.shape
    per = st.shape[1]
    vals = st[words]                       # [n, G, P, per]
    u = vals.reshape(n, G, P * per)[:, :, :64]
    sq = (words[:, :, -1] & tab["smask"]).astype(np.float32)
    s = (sq * sup[:, None].astype(np.float32)).astype(np.float32)  # fp32 product
    out = (u - zp).astype(np.float64) * s[:, :, None].astype(np.float64)
    return out.reshape(n, 64 * G)


@pytest.mark.parametrize("name", ["432", "hybrid"])
def test_alg2_decode_every_word_value(orc, name):
    fmt = orc.CCQ432 if name == "432" else orc.CCQ_HYBRID
    P = 22 if name == "432" else 10
    nvals = 256 if name == "432" else 65536
    g = np.random.default_rng(21 if name == "432" else 22)
    # every word value appears in a non-last position at least once
    n = 16
    G = -(-nvals // (n * (P - 1)))
    body = np.resize(np.arange(nvals), n * G * (P - 1)).reshape(n, G, P - 1)
    last = g.integers(0, nvals, (n, G, 1))
    words = np.concatenate([body, last], axis=2)
    sup = g.uniform(1e-5, 1e-3, n).astype(np.float32)
    zp = orc.default_zp(fmt)
    p = orc.alg2_pack(fmt, words[None], sup[None])
    got = orc.dequantize(p)
    ref = _bf16_of(_reference_decode(orc, fmt, words, sup, zp))
    assert np.array_equal(got, ref)


def test_alg2_weight_63_and_scale_share_the_last_word(orc):
    # the last word's high state is weight 63; its low bits are the scale and decode to no
    # weight: changing them rescales the group, changing weight 63's bits moves only it.
    for fmt, P, top, L in ((orc.CCQ432, 22, 4, 4), (orc.CCQ_HYBRID, 10, 13, 3)):
        zp = orc.default_zp(fmt)
        words = np.full((1, 1, 1, P), 0, np.int64)
        words[..., -1] = ((zp + 1) << top) | 1      # weight 63 = +1, scale field 1
        sup = np.array([[0.5]], np.float32)
        a = orc.bf16_to_f32(orc.dequantize(orc.alg2_pack(fmt, words, sup)))[0]
        assert a[63] == 0.5 and np.all(a[:63] == -zp * 0.5)
        words[..., -1] = ((zp + 1) << top) | 3      # scale field 3
        b = orc.bf16_to_f32(orc.dequantize(orc.alg2_pack(fmt, words, sup)))[0]
        assert np.array_equal(b, 3 * a)
        words[..., -1] = ((zp + 3) << top) | 1
        c = orc.bf16_to_f32(orc.dequantize(orc.alg2_pack(fmt, words, sup)))[0]
        assert c[63] == 1.5 and np.array_equal(c[:63], a[:63])
        assert (1 << L) - 1 == (0xF if fmt == orc.CCQ432 else 0x7)


def test_alg2_storage_matches_the_stated_bpw(orc):
    # section 3.4: the scale lives in the codes, so a group's bytes are its whole storage
    tab = _table()
    for fmt, key in ((orc.CCQ432, "4,3,2"), (orc.CCQ_HYBRID, "3,3,2+3,4,2")):
        w = np.random.default_rng(23).standard_normal((3, 256)).astype(np.float32)
        p = orc.quantize(w, fmt)
        bits_per_weight = 8 * p.codes.nbytes / w.size
        assert bits_per_weight == tab[key]["bpw"]
        # the super scale is one f32 per output channel (not counted by the pages' bpw)
        assert p.super_scale.shape == (1, 3)


@pytest.mark.parametrize("fmt_name", ["CCQ432", "CCQ_HYBRID"])
def test_alg2_quantizer_round_trips_representable_weights(orc, fmt_name):
    # Weights on the format's grid (scale = s_q * 2^-10 with the largest s_q the full range,
    # every group reaching +max state and avoiding the lowest state so its absmax fixes the
    # scale) must come back exactly: the search has a zero-cost code for every vector.
    fmt = getattr(orc, fmt_name)
    g = np.random.default_rng(24)
    n, G = 6, 5
    P = 22 if fmt == orc.CCQ432 else 10
    smask = 0xF if fmt == orc.CCQ432 else 0x1FFF
    top = 4 if fmt == orc.CCQ432 else 13
    st = _state_tables(orc, fmt)
    ok = np.where((st > 0).all(axis=1))[0]         # words with no lowest state
    full = int(np.where((st == st.max()).all(axis=1))[0][0])  # every state at its maximum
    words = g.choice(ok, (n, G, P))
    words[:, :, 3] = full
    hi = st.max()
    sq = g.integers(1, smask + 1, (n, G))
    sq[:, 0] = smask
    words[:, :, -1] = (g.integers(1, hi + 1, (n, G)) << top) | sq
    sup = np.full(n, 2.0 ** -10, np.float32)
    zp = orc.default_zp(fmt)
    w = _reference_decode(orc, fmt, words, sup, zp).astype(np.float32)
    for refine in (False, True):
        p = orc.quantize(w, fmt, refine=refine)
        assert np.array_equal(p.super_scale[0], sup)
        # the grid values are exact in fp32; the decode rounds them to bf16 once
        assert np.array_equal(orc.dequantize(p), _bf16_of(w))
        got_words = (p.codes.reshape(n, G, P) if fmt == orc.CCQ432 else
                     p.codes.reshape(n, G, 2 * P).view("<u2"))
        assert np.array_equal(got_words[:, :, :-1], words[:, :, :-1])
        assert np.array_equal(got_words[:, :, -1] & smask, sq)


@pytest.mark.parametrize("fmt_name", ["CCQ432", "CCQ_HYBRID"])
def test_alg2_quantizer_search_is_exhaustive_argmin(orc, fmt_name):
    # Every non-last word is the cheapest codebook entry for its weights at the group's scale
    # (ties to the smallest code); the last word's weight 63 is the nearest single state.
    fmt = getattr(orc, fmt_name)
    g = np.random.default_rng(25)
    n, G = 4, 3
    w = (g.standard_normal((n, 64 * G)) * 0.02).astype(np.float32)
    w[1, :64] = 0.0  # a zero group
    p = orc.quantize(w, fmt, refine=False)
    zp = orc.default_zp(fmt)
    P, per = (22, 3) if fmt == orc.CCQ432 else (10, 7)
    smask = 0xF if fmt == orc.CCQ432 else 0x1FFF
    top, L = (4, 4) if fmt == orc.CCQ432 else (13, 3)
    words = (p.codes.reshape(n, G, P) if fmt == orc.CCQ432 else
             p.codes.reshape(n, G, 2 * P).view("<u2")).astype(np.int64)
    if fmt == orc.CCQ432:
        parts = [(_state_tables(orc, fmt), 0, 8)]
    else:
        parts = [(np.array([orc.ccq_states(c, 3, 3, 2) for c in range(128)]), 9, 7),
                 (np.array([orc.ccq_states(c, 3, 4, 2) for c in range(512)]), 0, 9)]
    for r in range(n):
        sup = np.float32(p.super_scale[0, r])
        for gi in range(G):
            sq = int(words[r, gi, -1] & smask)
            s = float(np.float32(np.float32(sq) * sup))
            grp = w[r, gi * 64:(gi + 1) * 64].astype(np.float64)
            for i in range(P - 1):
                pos = i * per
                for states, base, T in parts:
                    N = states.shape[1]
                    v = grp[pos:pos + N]
                    cost = ((v[None, :] - (states - zp) * s) ** 2).sum(axis=1)
                    code = (int(words[r, gi, i]) >> base) & ((1 << T) - 1)
                    assert code == int(np.argmin(cost)), (r, gi, i)
                    pos += N
            u63 = int(words[r, gi, -1]) >> top
            c63 = (grp[63] - (np.arange(1 << L) - zp) * s) ** 2
            assert u63 == int(np.argmin(c63))


@pytest.mark.parametrize("fmt_name,bound", [("CCQ432", 0.4), ("CCQ_HYBRID", 0.5)])
def test_alg2_quantizer_reconstructs_gaussian(orc, fmt_name, bound):
    fmt = getattr(orc, fmt_name)
    w = np.random.default_rng(26).standard_normal((8, 512)).astype(np.float32) * 0.02
    p = orc.quantize(w, fmt, refine=True)
    dq = orc.bf16_to_f32(orc.dequantize(p)).astype(np.float64)
    rel = np.sqrt(((dq - w) ** 2).mean() / (w.astype(np.float64) ** 2).mean())
    raw = orc.quantize(w, fmt, refine=False)
    dq_raw = orc.bf16_to_f32(orc.dequantize(raw)).astype(np.float64)
    rel_raw = np.sqrt(((dq_raw - w) ** 2).mean() / (w.astype(np.float64) ** 2).mean())
    # guards against a broken encoder (a sign, shift or scale slip gives rel >= 1); the
    # scale update is kept only where it lowers a group's error
    assert rel < bound, rel
    assert rel <= rel_raw + 1e-12
