"""Shared helpers of the test suite: moving oracle-packed weights to the device and the
output tolerance.

Tolerance (the product's outputs against the oracle): element i passes when
    |y_gpu[i] - y_ref[i]| <= 1e-2 * (|y_ref[i]| + rms(y_ref))
i.e. a relative error of at most 1e-2, measured against the output's own scale for the
outputs that are near zero (where a pure ratio is meaningless).  The kernels accumulate in
fp32 and round once to bf16 (2^-9 relative); the oracle sums in fp64 and rounds once.
"""
import numpy as np

REL_TOL = 1e-2

_FIELDS = ("codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")


def to_device(p, device="cuda"):
    """oracle.Packed -> weight_only_bit_amd.PackedWeight (same bytes, on the GPU)."""
    import weight_only_bit_amd as wq

    arrays = {f: getattr(p, f) for f in _FIELDS if getattr(p, f) is not None}
    return wq.PackedWeight.from_arrays(p.format, p.experts, p.n, p.k, arrays, group=p.group,
                                       zp=p.zp, device=device)


def bf16_to_f64(bits):
    bits = np.asarray(bits).astype(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_bf16_bits(t):
    """Host uint16 bits of a bf16 / int16 torch tensor."""
    import torch

    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def assert_close(y_gpu_bits, y_ref_bits, what=""):
    g = bf16_to_f64(y_gpu_bits)
    r = bf16_to_f64(y_ref_bits)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    bound = REL_TOL * (np.abs(r) + rms)
    err = np.abs(g - r)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {np.unravel_index(i, g.shape)} "
            f"gpu={g.flat[i]:.6g} ref={r.flat[i]:.6g} rms={rms:.4g}")
    return float((err / (np.abs(r) + rms + 1e-300)).max()) if r.size else 0.0


def to_host(w):
    """weight_only_bit_amd.PackedWeight -> oracle.Packed (host copies of the same bytes)."""
    import oracle

    def h(t):
        if t is None:
            return None
        a = t.cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a

    return oracle.Packed(w.format, w.n, w.k, w.experts, w.group, h(w.codes), h(w.scales),
                         h(w.zeros), h(w.qscale), h(w.super_scale), h(w.code_scale),
                         h(w.code_zero), w.zp)
