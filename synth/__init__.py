"""Seeded synthetic inputs shared by the tests, the oracle side and the benchmark.

This module holds no arithmetic of the method (no quantizer, decoder or product): it only
draws random numbers with the shapes and distributions of the workloads -- fp32 weights
~ N(0, 0.02), bf16 activations ~ N(0, 1), expert routings -- plus random packed bytes of the
right layout for workloads too large to quantize on the host.  Every draw is keyed by a
``SeedSequence(SEED, spawn_key=path)`` so each tensor has its own reproducible stream.

Device-side draws (``*_device``) use torch's own generator on the GPU; they are inputs only,
and the host can read any slice of them back for the oracle.
"""
from __future__ import annotations

import numpy as np

SEED = 20261203

FMT_INT4, FMT_AFFINE2, FMT_CCQ, FMT_CCQ432, FMT_CCQ_HYBRID, FMT_INT8 = 1, 2, 3, 4, 5, 6
_GROUP_BYTES = {FMT_CCQ432: 22, FMT_CCQ_HYBRID: 20}
# super scale that puts a uniform group-scale field at the magnitude of a N(0, 0.02) group:
# absmax ~ 3 std over (2^(L-1) - 1) levels, spread over the field's range
_ALG2_SUPER = {FMT_CCQ432: 0.02 * 3.0 / 7.0 / 15.0, FMT_CCQ_HYBRID: 0.02 * 3.0 / 3.0 / 8191.0}


def rng(*path: int) -> np.random.Generator:
    """Independent generator for one tensor, keyed by an integer path."""
    return np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=tuple(int(p) for p in path)))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (round to nearest even) through torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def weights_f32(shape, *path: int, std: float = 0.02) -> np.ndarray:
    """Dense fp32 weights ~ N(0, std^2) standing in for a trained checkpoint."""
    return (rng(*path).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def acts_bf16(shape, *path: int) -> np.ndarray:
    """bf16 activations ~ N(0, 1), as uint16 bits."""
    return bf16_bits(rng(*path).standard_normal(shape, dtype=np.float32))


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def routing_uniform(tokens: int, topk: int, experts: int, *path: int):
    """Each token picks topk distinct experts uniformly at random; its weights are a softmax
    over topk N(0, 1) logits.  Returns (ids int32 [t, topk], weights f32 [t, topk])."""
    g = rng(*path)
    ids = np.argsort(g.random((tokens, experts)), axis=1)[:, :topk].astype(np.int32)
    w = _softmax_rows(g.standard_normal((tokens, topk)))
    return ids, w


def routing_zipf(tokens: int, topk: int, experts: int, *path: int, s: float = 1.1):
    """Skewed routing: logit[t, e] = N(0, 1) + ln p_e with p_e proportional to (e+1)^-s; each
    token takes its topk largest logits and softmaxes them.  Expert 0 is the most popular."""
    g = rng(*path)
    bias = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    logits = g.standard_normal((tokens, experts)) + bias[None, :]
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    return ids, _softmax_rows(sel)


# ---------------------------------------------------------------------------------------------
# Random packed weights (layout only; values are draws, not a quantizer's output)
# ---------------------------------------------------------------------------------------------

def packed_layout(fmt: int, experts: int, n: int, k: int, group: int = 64) -> dict:
    """Shapes and dtypes of each array of a packed weight [experts, n, k]."""
    G = k // 64
    if fmt == FMT_INT4:
        return {"codes": ((experts, n, k // 2), np.uint8),
                "scales": ((experts, n, G) if group else (experts, n), np.uint16)}
    if fmt == FMT_INT8:
        return {"codes": ((experts, n, k), np.uint8),
                "scales": ((experts, n, G) if group else (experts, n), np.uint16)}
    if fmt == FMT_AFFINE2:
        return {"codes": ((experts, n, k // 4), np.uint8),
                "scales": ((experts, n, G), np.uint16),
                "zeros": ((experts, n, G), np.uint8)}
    if fmt == FMT_CCQ:
        return {"codes": ((experts, n, k // 4), np.uint8),
                "qscale": ((experts, n, (G + 1) // 2), np.uint8),
                "super_scale": ((experts, n), np.float32),
                "code_scale": ((experts, n), np.float32),
                "code_zero": ((experts, n), np.float32)}
    if fmt in _GROUP_BYTES:
        return {"codes": ((experts, n, G * _GROUP_BYTES[fmt]), np.uint8),
                "super_scale": ((experts, n), np.float32)}
    raise ValueError(fmt)


def random_packed(fmt: int, experts: int, n: int, k: int, *path: int, group: int = 64) -> dict:
    """Random packed weights on the host: uniform code bytes; scales of the magnitude a
    N(0, 0.02) weight would get (INT4 ~ 0.02*U(2,3)/7, INT8 ~ 0.02*U(2,3)/127, affine ~ 0.02*U(3,5)/3 with zero
    points in 0..3); CCQ group scales uniform in 1..15, super scale 0.02*3/31/15, code scale
    U(64, 128) and an integral code zero that keeps 255*scale + zero below 2^15.  The CCQ
    formats without code cluster draw every code byte (scale fields included) uniformly, with
    a super scale of the magnitude of the field's mean."""
    g = rng(*path)
    lay = packed_layout(fmt, experts, n, k, group)
    out = {}
    out["codes"] = g.integers(0, 256, size=lay["codes"][0], dtype=np.uint8)
    if fmt == FMT_INT4:
        out["scales"] = bf16_bits(0.02 * g.uniform(2.0, 3.0, size=lay["scales"][0]) / 7.0)
    elif fmt == FMT_INT8:
        out["scales"] = bf16_bits(0.02 * g.uniform(2.0, 3.0, size=lay["scales"][0]) / 127.0)
    elif fmt == FMT_AFFINE2:
        out["scales"] = bf16_bits(0.02 * g.uniform(3.0, 5.0, size=lay["scales"][0]) / 3.0)
        out["zeros"] = g.integers(0, 4, size=lay["zeros"][0], dtype=np.uint8)
    elif fmt in _GROUP_BYTES:
        shp = lay["super_scale"][0]
        out["super_scale"] = (2.0 * _ALG2_SUPER[fmt] * g.uniform(0.8, 1.2, size=shp)).astype(np.float32)
    else:
        lo = g.integers(1, 16, size=lay["qscale"][0], dtype=np.uint8)
        hi = g.integers(1, 16, size=lay["qscale"][0], dtype=np.uint8)
        out["qscale"] = (lo | (hi << 4)).astype(np.uint8)
        shp = lay["super_scale"][0]
        out["super_scale"] = np.full(shp, 0.02 * 3.0 / 31.0 / 15.0, np.float32) * \
            g.uniform(0.8, 1.2, size=shp).astype(np.float32)
        alpha = g.uniform(64.0, 128.0, size=shp).astype(np.float32)
        out["code_scale"] = alpha
        span = np.maximum(32767.0 - 255.0 * alpha.astype(np.float64) - 1.0, 0.0)
        out["code_zero"] = np.floor(g.uniform(0.0, 1.0, size=shp) * span).astype(np.float32)
    return out


def random_packed_device(fmt: int, experts: int, n: int, k: int, seed: int, device="cuda",
                         group: int = 64) -> dict:
    """Same layout and distributions as ``random_packed`` but drawn on the GPU with torch's
    generator (for multi-GB stacks).  Returns torch tensors."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    lay = packed_layout(fmt, experts, n, k, group)

    def u(shape, lo, hi):
        return torch.empty(shape, dtype=torch.float32, device=device).uniform_(lo, hi, generator=gen)

    out = {"codes": torch.randint(0, 256, lay["codes"][0], dtype=torch.uint8, device=device,
                                  generator=gen)}
    if fmt == FMT_INT4:
        out["scales"] = (0.02 * u(lay["scales"][0], 2.0, 3.0) / 7.0).to(torch.bfloat16).view(torch.int16)
    elif fmt == FMT_INT8:
        out["scales"] = (0.02 * u(lay["scales"][0], 2.0, 3.0) / 127.0).to(torch.bfloat16).view(torch.int16)
    elif fmt == FMT_AFFINE2:
        out["scales"] = (0.02 * u(lay["scales"][0], 3.0, 5.0) / 3.0).to(torch.bfloat16).view(torch.int16)
        out["zeros"] = torch.randint(0, 4, lay["zeros"][0], dtype=torch.uint8, device=device,
                                     generator=gen)
    elif fmt in _GROUP_BYTES:
        out["super_scale"] = (2.0 * _ALG2_SUPER[fmt]) * u(lay["super_scale"][0], 0.8, 1.2)
    else:
        lo = torch.randint(1, 16, lay["qscale"][0], dtype=torch.uint8, device=device, generator=gen)
        hi = torch.randint(1, 16, lay["qscale"][0], dtype=torch.uint8, device=device, generator=gen)
        out["qscale"] = lo | (hi << 4)
        shp = lay["super_scale"][0]
        out["super_scale"] = (0.02 * 3.0 / 31.0 / 15.0) * u(shp, 0.8, 1.2)
        alpha = u(shp, 64.0, 128.0)
        out["code_scale"] = alpha
        span = torch.clamp(32767.0 - 255.0 * alpha.double() - 1.0, min=0.0)
        out["code_zero"] = torch.floor(u(shp, 0.0, 1.0).double() * span).float()
    return out
