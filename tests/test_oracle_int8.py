"""Pins of the oracle's WINT8 format (FastDeploy "Quantization" precision list: INT8 weights,
BF16 activations), read with the lesson E6.4 formulas at b = 8: x_hat = s q, q a signed byte,
bf16 scale per group of 64 or per output channel.  Runs on the CPU."""
import numpy as np
import pytest
import torch


def _bf16_of(x):
    return (torch.tensor(np.asarray(x, np.float64), dtype=torch.float64).float()
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def _f32_of_bf16(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("group", [64, 0])
def test_int8_decode_every_byte_is_signed_byte_times_scale(orc, group):
    n, k = 4, 256
    codes = np.tile(np.arange(256, dtype=np.uint8), (n, 1))  # every byte value, k = 256
    g = np.random.default_rng(41)
    shape = (1, n, k // 64) if group else (1, n)
    scales = _bf16_of(g.uniform(1e-4, 1e-2, shape))
    p = orc.Packed(orc.INT8, n, k, 1, group, codes[None], scales)
    got = orc.dequantize(p)
    q = codes.view(np.int8).astype(np.float32)  # numpy's two's-complement view
    s = _f32_of_bf16(scales[0])
    s = np.repeat(s, 64, axis=1) if group else s[:, None]
    ref = torch.from_numpy((q * s).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("group", [64, 0])
def test_int8_quantizer_is_the_affine_formula_with_zero_point_zero(orc, group):
    w = np.random.default_rng(42).standard_normal((3, 192)).astype(np.float32) * 0.02
    w[1, 64:128] = 0.0
    p = orc.quantize(w, orc.INT8, group=group)
    q = p.codes[0].view(np.int8).astype(np.int32)
    scales = p.scales[0]
    for r in range(3):
        for gi in range(192 // 64 if group else 1):
            sl = slice(64 * gi, 64 * (gi + 1)) if group else slice(0, 192)
            sb = scales[r, gi] if group else scales[r]
            amax = float(np.abs(w[r, sl]).max())
            assert sb == _bf16_of(np.float32(amax) / np.float32(127.0))[()]  # s = bf16(absmax/127)
            s = float(_f32_of_bf16(sb))
            if s == 0.0:
                assert np.all(q[r, sl] == 0)
                continue
            # the quotient is formed in fp32 (the oracle's arithmetic); fl32(w / s) * s is exact in
            # fp64, so the affine formula then sees that same quotient
            quot = (w[r, sl].astype(np.float32) / np.float32(s)).astype(np.float64)
            ref = orc.affine_quant(quot * s, s, 0, -128, 127)
            assert np.array_equal(q[r, sl], ref), (r, gi)


def test_int8_storage_is_one_byte_per_weight(orc):
    p = orc.quantize(np.ones((2, 128), np.float32), orc.INT8, group=0)
    assert p.codes.nbytes == 2 * 128 == orc.packed_size(256, 8)


def test_int8_round_trip_on_grid(orc):
    g = np.random.default_rng(43)
    n, k = 5, 320
    q = g.integers(-127, 128, (n, k))
    q[:, ::64] = 127  # each group reaches the top code, so absmax / 127 is the scale
    s = _f32_of_bf16(_bf16_of(g.uniform(1e-4, 1e-2, (n, k // 64))))
    w = (q * np.repeat(s, 64, axis=1)).astype(np.float32)
    p = orc.quantize(w, orc.INT8, group=64)
    assert np.array_equal(p.codes[0].view(np.int8).astype(np.int64), q)
    assert np.array_equal(_f32_of_bf16(p.scales[0]), s)
