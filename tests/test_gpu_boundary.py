"""The boundary on the GPU: the Python binding rejects tensors whose dtype, shape, layout or
device the library could not see, before anything is launched; and the products stay exact up
to the documented scale limit (every scale below 2^100 in magnitude)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from wq_testutil import assert_close, to_device, torch_bf16_bits

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def wq():
    import torch

    import weight_only_bit_amd as wq

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    wq.lib()
    return wq


def test_binding_rejects_bad_tensors(wq):
    import torch

    _say("binding argument checks")
    p = oracle.quantize(synth.weights_f32((64, 256), 71, 1), oracle.CCQ)
    w = to_device(p)
    x = torch.from_numpy(synth.acts_bf16((4, 256), 71, 2).view(np.int16)).cuda()
    with pytest.raises(TypeError, match="dtype"):
        wq.wq_gemm(x.to(torch.int64), w)
    with pytest.raises(ValueError, match="shape"):
        wq.wq_gemm(x[:, :128].contiguous(), w)
    with pytest.raises(ValueError, match="contiguous"):
        wq.wq_gemm(torch.empty((256, 4), dtype=torch.bfloat16, device="cuda").t(), w)
    with pytest.raises(ValueError, match="shape"):
        wq.wq_gemm(x, w, y=torch.empty((4, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="GPU tensor"):
        wq.wq_gemm(x.cpu(), w)
    short = wq.PackedWeight(w.format, w.n, w.k, 1, 64, w.codes[:, :-4].contiguous(), None, None,
                            w.qscale, w.super_scale, w.code_scale, w.code_zero, 32)
    with pytest.raises(ValueError, match="codes"):
        wq.wq_gemm(x, short)
    # MoE: routing ids must be int32 (torch.topk returns int64) and weights fp32
    E, H, I, T, K = 4, 256, 128, 6, 2
    mats = [to_device(oracle.quantize(synth.weights_f32(s, 72, j), oracle.CCQ))
            for j, s in enumerate(((E, I, H), (E, I, H), (E, H, I)))]
    xm = torch.from_numpy(synth.acts_bf16((T, H), 72, 4).view(np.int16)).cuda()
    ids, wts = synth.routing_uniform(T, K, E, 72, 5)
    ids_d, wts_d = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    with pytest.raises(TypeError, match="topk_ids"):
        wq.wq_moe_ffn(xm, ids_d.long(), wts_d, *mats)
    with pytest.raises(TypeError, match="topk_weights"):
        wq.wq_moe_ffn(xm, ids_d, wts_d.to(torch.bfloat16), *mats)
    with pytest.raises(ValueError, match="shape"):
        wq.wq_moe_ffn(xm, ids_d, wts_d[:-1].contiguous(), *mats)
    with pytest.raises(ValueError, match="shape"):
        wq.wq_moe_gate_up(xm, *wq.wq_moe_route(ids_d, E), K, mats[0], mats[1],
                          h=torch.empty((T * K - 1, I), dtype=torch.bfloat16, device="cuda"))
    # the same arguments with the right types still run and match the oracle
    y = wq.wq_moe_ffn(xm, ids_d, wts_d, *mats)
    torch.cuda.synchronize()
    host = [oracle.quantize(synth.weights_f32(s, 72, j), oracle.CCQ)
            for j, s in enumerate(((E, I, H), (E, I, H), (E, H, I)))]
    assert_close(torch_bf16_bits(y), oracle.moe_ffn(synth.acts_bf16((T, H), 72, 4), ids, wts, *host),
                 "binding checks moe")


# Weight magnitudes that put the largest decode scale just below 2^100 (s ~ absmax / levels;
# N(0, 0.02) weights have absmax ~ 0.06-0.1 at these sizes).
SCALE_LIMIT_CASES = [("int4", oracle.INT4, 64, 2.0 ** 106), ("int4pc", oracle.INT4, 0, 2.0 ** 106),
                     ("int8pc", oracle.INT8, 0, 2.0 ** 110), ("affine2", oracle.AFFINE2, 64, 2.0 ** 103),
                     ("ccq", oracle.CCQ, 64, 2.0 ** 108), ("ccq432", oracle.CCQ432, 64, 2.0 ** 106),
                     ("ccqh", oracle.CCQ_HYBRID, 64, 2.0 ** 104)]


@pytest.mark.parametrize("name,fmt,group,factor", SCALE_LIMIT_CASES)
def test_products_at_the_scale_limit(wq, name, fmt, group, factor):
    import torch

    n, k = 96, 512
    w = (synth.weights_f32((n, k), 73, fmt) * np.float32(factor)).astype(np.float32)
    p = oracle.quantize(w, fmt, group=group)
    dq = oracle.dequantize(p)
    big = np.abs(oracle.bf16_to_f32(dq)).max()
    _say(f"scale limit {name}: largest decoded weight 2^{np.log2(big):.1f}")
    assert np.isfinite(big) and big > 2.0 ** 98
    d = to_device(p)
    assert np.array_equal(torch_bf16_bits(wq.wq_dequantize(d))[0], dq)
    for m in (1, 24, 64):  # single-staging, chunked decode and tiled kernels
        x = synth.acts_bf16((m, k), 73, fmt, m)
        y = wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), d)
        torch.cuda.synchronize()
        assert_close(torch_bf16_bits(y), oracle.gemm(x, p), f"scale limit {name} m={m}")


def test_gemm_with_activations_of_4gib_or_more(wq):
    """The tiled kernels address an activation row by a 32-bit offset from the array's base; an
    activation array of 4 GiB or more runs the decode-streaming kernels instead.  x here is
    32768 x 65536 bf16 = 4 GiB; sampled rows (first, last, and across the array) against the
    oracle."""
    import torch

    m, k, n = 32768, 65536, 64
    _say(f"gemm with a 4 GiB activation array ({m} x {k})")
    p = oracle.quantize(synth.weights_f32((n, k), 74, 1), oracle.CCQ)
    x = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    rows = np.array([0, 1, 12345, m // 2, m - 2, m - 1])
    xs = synth.acts_bf16((len(rows), k), 74, 2)
    x.zero_()
    x[torch.from_numpy(rows).cuda()] = torch.from_numpy(xs.view(np.int16)).cuda().view(torch.bfloat16)
    y = wq.wq_gemm(x, to_device(p))
    torch.cuda.synchronize()
    got = torch_bf16_bits(y)[rows]
    del x, y
    torch.cuda.empty_cache()
    assert_close(got, oracle.gemm(xs, p), "gemm 4 GiB activations")
