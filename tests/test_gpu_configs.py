"""Parity at the full sizes of the benchmark workloads, through the same entry points and
therefore the same kernel launches that bench.py times.

The single-linear workloads compare every output against the oracle, with the weights
quantized by the oracle's own quantizers from N(0, 0.02) draws (W4A16 512 x 512 RTN INT4 g64;
WINT2 4096 x 4096 in both 2-bit formats).  The MoE layers (64 experts, hidden 8192, expert
intermediate 3584, top-8) use seeded random packed bytes of the real layout and magnitudes --
quantizing 5.6 G weights on the host would take too long -- drawn on the GPU by synth, copied
back for the oracle, and compare sampled tokens: the oracle evaluates only the experts those
tokens are routed to.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from wq_testutil import assert_close, to_device, to_host, torch_bf16_bits

pytestmark = pytest.mark.gpu

E, HIDDEN, INTER, TOPK = 64, 8192, 3584, 8


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


@pytest.mark.parametrize("m", [1, 8])
def test_w4a16_512(wq, m):
    import torch

    _say(f"w4a16 512x512 m={m}")
    w = synth.weights_f32((512, 512), 61, 1)
    p = oracle.quantize(w, oracle.INT4, group=64)
    x = synth.acts_bf16((m, 512), 61, 2, m)
    ref = oracle.gemm(x, p)
    y = wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), to_device(p))
    assert_close(torch_bf16_bits(y), ref, f"w4a16 512x512 m={m}")


@pytest.fixture(scope="module", params=["affine2", "ccq"])
def wint2_4096(request):
    fmt = {"affine2": oracle.AFFINE2, "ccq": oracle.CCQ}[request.param]
    _say(f"quantizing 4096x4096 {request.param}")
    w = synth.weights_f32((4096, 4096), 62, 1)
    return request.param, oracle.quantize(w, fmt, group=64)


@pytest.mark.parametrize("m", [1, 8, 32])
def test_wint2_4096(wq, wint2_4096, m):
    import torch

    name, p = wint2_4096
    _say(f"wint2 4096x4096 {name} m={m}")
    x = synth.acts_bf16((m, 4096), 62, 2, m)
    ref = oracle.gemm(x, p)
    y = wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), to_device(p))
    assert_close(torch_bf16_bits(y), ref, f"wint2 4096x4096 {name} m={m}")


def _layer(wq, fmt, group, seed):
    """One MoE layer of random packed weights on the GPU (gate, up, down)."""
    mats = []
    for j, (n, k) in enumerate(((INTER, HIDDEN), (INTER, HIDDEN), (HIDDEN, INTER))):
        arr = synth.random_packed_device(fmt, E, n, k, seed + j, group=group)
        mats.append(wq.PackedWeight(fmt, n, k, E, group,
                                    *(arr.get(f) for f in ("codes", "scales", "zeros", "qscale",
                                                            "super_scale", "code_scale",
                                                            "code_zero")),
                                    oracle.default_zp(fmt)))
    return mats


def _check_tokens(wq, mats, x, ids, wts, tokens, what):
    import torch

    y = wq.wq_moe_ffn(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(wts).cuda(), *mats)
    got = torch_bf16_bits(y)[tokens]
    _say(f"{what}: oracle on tokens {tokens.tolist()}")
    host = [to_host(w) for w in mats]
    ref = oracle.moe_ffn(x, ids, wts, *host, tokens=tokens)
    assert_close(got, ref, what)


@pytest.mark.parametrize("name", ["ccq", "int4pc"])
def test_moe_decode_layer_full_size(wq, name):
    # the decode step: 32 tokens, uniform top-8 of 64 experts (CCQ g64 layers and the stack's
    # INT4 per-channel layers)
    fmt, group = (oracle.CCQ, 64) if name == "ccq" else (oracle.INT4, 0)
    _say(f"moe decode full size {name}")
    mats = _layer(wq, fmt, group, 6300 + fmt)
    x = synth.acts_bf16((32, HIDDEN), 63, 1)
    ids, wts = synth.routing_uniform(32, TOPK, E, 63, 2)
    _check_tokens(wq, mats, x, ids, wts, np.arange(32, dtype=np.int32),
                  f"moe decode full size {name}")


def _tile_class(rows):
    """The tiled kernel's row tile that holds an expert's last rows: its remainder rows % 256
    goes to one tile of 256, 128, 64 or 32 rows (0: the expert fills whole 256-row tiles)."""
    rem = rows % 256
    return 0 if rem == 0 else 256 if rem > 128 else 128 if rem > 64 else 64 if rem > 32 else 32


def test_moe_prefill_layer_full_size(wq):
    # the prefill layer: 4096 tokens, Zipf-skewed top-8 of 64 experts, CCQ g64.  Sampled tokens
    # reach every row-tile class: for two experts of each remainder class (256, 128, 64, 32
    # rows) the token of the expert's first row and of its last row (which lies in the
    # remainder tile), the heaviest expert's first, middle-tile and last rows, and the last
    # token.
    _say("moe prefill full size ccq")
    mats = _layer(wq, oracle.CCQ, 64, 6400)
    T = 4096
    x = synth.acts_bf16((T, HIDDEN), 64, 1)
    ids, wts = synth.routing_zipf(T, TOPK, E, 64, 2)
    counts = np.bincount(ids.ravel(), minlength=E)
    heavy = int(np.argmax(counts))
    assert counts[heavy] > 1024
    toks_of = [np.nonzero((ids == e).any(axis=1))[0] for e in range(E)]
    picked = {T - 1}
    hv = toks_of[heavy]
    picked |= {int(hv[0]), int(hv[len(hv) // 2]), int(hv[-1])}
    for cls in (256, 128, 64, 32):
        es = [e for e in range(E) if counts[e] and _tile_class(int(counts[e])) == cls]
        assert len(es) >= 2, (cls, es)
        for e in es[:2]:
            picked |= {int(toks_of[e][0]), int(toks_of[e][-1])}
    tokens = np.array(sorted(picked), np.int32)
    _check_tokens(wq, mats, x, ids, wts, tokens, "moe prefill full size ccq")


@pytest.mark.parametrize("name,tokens", [("ccq", 1), ("ccq", 4), ("int4", 1)])
def test_moe_pages_grouped_shape(wq, name, tokens):
    # The pages' grouped-GEMM shape: 256 experts, hidden 7168, expert intermediate 512, top-8,
    # one or four tokens (the single-staging kernels); every token against the oracle.
    fmt, group = {"ccq": (oracle.CCQ, 64), "int4": (oracle.INT4, 64)}[name]
    n_exp, hidden, inter = 256, 7168, 512
    _say(f"pages grouped shape {name} tokens={tokens}: drawing weights")
    mats = []
    for j, (n, k) in enumerate(((inter, hidden), (inter, hidden), (hidden, inter))):
        arr = synth.random_packed_device(fmt, n_exp, n, k, 840 + j, group=group)
        mats.append(wq.PackedWeight(fmt, n, k, n_exp, group,
                                    *(arr.get(f) for f in ("codes", "scales", "zeros", "qscale",
                                                            "super_scale", "code_scale",
                                                            "code_zero")),
                                    oracle.default_zp(fmt)))
    x = synth.acts_bf16((tokens, hidden), 843, tokens)
    ids, wts = synth.routing_uniform(tokens, 8, n_exp, 844, tokens)
    _check_tokens(wq, mats, x, ids, wts, np.arange(tokens), f"pages grouped {name} t={tokens}")


# The pages' GEMV operator shapes (CCQ paper, section 5, GEMV table: input 4096 or 8192,
# output 1024, 4096 or 8192, one and four rows), in the two 2-bit formats the table compares;
# the seeded random packed bytes of synth (the layout and magnitudes of quantized weights),
# every output against the oracle.
PAGES_GEMV = [(4096, 4096), (4096, 1024), (8192, 8192), (8192, 1024)]


@pytest.mark.parametrize("k,n", PAGES_GEMV)
@pytest.mark.parametrize("fmt_name", ["affine2", "ccq"])
def test_pages_gemv_shapes(wq, k, n, fmt_name):
    import torch

    fmt = {"affine2": oracle.AFFINE2, "ccq": oracle.CCQ}[fmt_name]
    arr = synth.random_packed(fmt, 1, n, k, 850, k, n)
    p = oracle.Packed(fmt, n, k, 1, 64, arr["codes"], arr.get("scales"), arr.get("zeros"),
                      arr.get("qscale"), arr.get("super_scale"), arr.get("code_scale"),
                      arr.get("code_zero"), oracle.default_zp(fmt))
    w = to_device(p)
    for m in (1, 4):
        _say(f"pages gemv {fmt_name} k={k} n={n} m={m}")
        x = synth.acts_bf16((m, k), 851, k, n, m)
        y = wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), w)
        assert_close(torch_bf16_bits(y), oracle.gemm(x, p), f"pages gemv {fmt_name} {k}x{n} m={m}")


# The pages' grouped-GEMM shape at the table's larger token counts (16 and 64 tokens, 8 of 256
# experts each), CCQ and W8A16 (INT8 per channel): every token against the oracle.
@pytest.mark.parametrize("name,tokens", [("ccq", 16), ("int8pc", 16), ("ccq", 64)])
def test_moe_pages_grouped_shape_more_tokens(wq, name, tokens):
    fmt, group = {"ccq": (oracle.CCQ, 64), "int8pc": (oracle.INT8, 0)}[name]
    n_exp, hidden, inter = 256, 7168, 512
    _say(f"pages grouped shape {name} tokens={tokens}: drawing weights")
    mats = []
    for j, (n, k) in enumerate(((inter, hidden), (inter, hidden), (hidden, inter))):
        arr = synth.random_packed_device(fmt, n_exp, n, k, 860 + j, group=group)
        mats.append(wq.PackedWeight(fmt, n, k, n_exp, group,
                                    *(arr.get(f) for f in ("codes", "scales", "zeros", "qscale",
                                                            "super_scale", "code_scale",
                                                            "code_zero")),
                                    oracle.default_zp(fmt)))
    x = synth.acts_bf16((tokens, hidden), 863, tokens)
    ids, wts = synth.routing_uniform(tokens, 8, n_exp, 864, tokens)
    _check_tokens(wq, mats, x, ids, wts, np.arange(tokens), f"pages grouped {name} t={tokens}")
