"""Evidence for the reading that the products multiply the bf16-rounded decoded weights.

FastDeploy "WINT2 Quantization" states that the low-bit weights are decoded to BF16 and the
arithmetic is carried out on BF16 values; the CCQ paper's dequantization algorithms likewise
end each weight as a BF16 value.  The kernels therefore decode every weight exactly to the
bf16 bits the dequantize entry point returns.  A cheaper product would keep the states in the
integer domain and apply (u - zp) * s per group after the sum, i.e. it would multiply the
activations by the unrounded values (u - zp) * s.  This CPU emulation measures what that
shortcut costs against the oracle on an MoE layer: the outputs leave the 1e-2 tolerance
(|y - y_ref| <= 1e-2 (|y_ref| + rms(y_ref))) at a number of elements, so the shortcut is not
taken.  A control run of the same emulation with bf16-rounded weights stays inside it.
"""
import numpy as np
import pytest

import synth

E, HIDDEN, INTER, T, TOPK = 4, 2048, 1024, 16, 2


def _unrounded_ccq(orc, arr, n, k, e):
    """(u - zp) * s of every weight of expert e in fp64 (no bf16 rounding), with stage 1 the
    single-rounded fp32 value of C' * alpha + beta (exact in fp64 before that one rounding)."""
    codes = arr["codes"][e].astype(np.float64)                      # [n, k/4]
    a = arr["code_scale"][e].astype(np.float64)[:, None]
    b = arr["code_zero"][e].astype(np.float64)[:, None]
    t = (codes * a + b).astype(np.float32).astype(np.float64)        # fmaf(C', alpha, beta)
    C = np.clip(np.rint(t), 0, 32767).astype(np.int64)
    u = np.stack([(C >> (9 - 3 * j)) & 0x3F for j in range(4)], axis=-1).reshape(n, k)
    qs = arr["qscale"][e].astype(np.int64)
    sq = np.stack([qs & 0xF, qs >> 4], axis=-1).reshape(n, -1)[:, :k // 64]
    s = (sq.astype(np.float32) * arr["super_scale"][e][:, None]).astype(np.float64)
    return (u - 32).astype(np.float64) * np.repeat(s, 64, axis=1)


def _moe(orc, x64, ids, wts, wg, wu, wd):
    """The MoE layer with the given decoded weights per expert, fp64 sums, h and y rounded to
    bf16 as the path does."""
    d = np.zeros((T, TOPK, HIDDEN))
    for e in range(E):
        sel = np.argwhere(ids == e)
        if sel.size == 0:
            continue
        xe = x64[sel[:, 0]]
        g = xe @ wg[e].T
        u = xe @ wu[e].T
        h = orc.bf16_to_f32(orc.f64_to_bf16(g / (1.0 + np.exp(-g)) * u)).astype(np.float64)
        d[sel[:, 0], sel[:, 1]] = h @ wd[e].T
    return orc.f64_to_bf16((wts.astype(np.float64)[:, :, None] * d).sum(axis=1))


def _outside(y, ref):
    yv = np.asarray(y, np.uint16).astype(np.uint32) << 16
    rv = np.asarray(ref, np.uint16).astype(np.uint32) << 16
    g = yv.view(np.float32).astype(np.float64)
    r = rv.view(np.float32).astype(np.float64)
    rms = np.sqrt(np.mean(r * r))
    err = np.abs(g - r)
    return int((err > 1e-2 * (np.abs(r) + rms)).sum()), float((err / (np.abs(r) + rms)).max())


@pytest.mark.slow
def test_unrounded_weights_leave_the_tolerance(orc):
    mats = {}
    for name, (n, k) in (("gate", (INTER, HIDDEN)), ("up", (INTER, HIDDEN)), ("down", (HIDDEN, INTER))):
        mats[name] = (synth.random_packed(synth.FMT_CCQ, E, n, k, 4201, len(mats)), n, k)
    packed = {nm: orc.Packed(orc.CCQ, n, k, E, 64, arr["codes"], qscale=arr["qscale"],
                             super_scale=arr["super_scale"], code_scale=arr["code_scale"],
                             code_zero=arr["code_zero"], zp=32)
              for nm, (arr, n, k) in mats.items()}
    exact, rounded = {}, {}
    for nm, (arr, n, k) in mats.items():
        exact[nm] = [_unrounded_ccq(orc, arr, n, k, e) for e in range(E)]
        rounded[nm] = [orc.bf16_to_f32(orc.dequantize(packed[nm], e)).astype(np.float64)
                       for e in range(E)]
        # the emulation's decode is the oracle's before its roundings (fp32, then bf16)
        for e in range(E):
            assert np.array_equal(orc.f32_to_bf16(exact[nm][e].astype(np.float32)),
                                  orc.dequantize(packed[nm], e))
    x = synth.acts_bf16((T, HIDDEN), 4202)
    ids, wts = synth.routing_uniform(T, TOPK, E, 4203)
    ref = orc.moe_ffn(x, ids, wts, packed["gate"], packed["up"], packed["down"])
    x64 = orc.bf16_to_f32(x).astype(np.float64)

    control = _moe(orc, x64, ids, wts, rounded["gate"], rounded["up"], rounded["down"])
    n_ctl, worst_ctl = _outside(control, ref)
    assert n_ctl == 0, worst_ctl

    shortcut = _moe(orc, x64, ids, wts, exact["gate"], exact["up"], exact["down"])
    n_bad, worst = _outside(shortcut, ref)
    print(f"unrounded weights: {n_bad} of {ref.size} outputs outside the tolerance, worst "
          f"{worst:.4f} of (|y| + rms); bf16 weights: {n_ctl}, worst {worst_ctl:.4f}")
    assert n_bad > 0 and worst > 1e-2
