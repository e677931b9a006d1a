"""Parity of the HIP path (through the C ABI) against the CPU oracle, on seeded inputs.

Sizes here are ones the oracle finishes in seconds but that span several tiles, K chunks and
ragged tails.  Decode is compared bit for bit; products within the tolerance of
tests/wq_testutil.py.  Inputs come from synth (weights, activations, routing) and the
oracle's quantizers (packed bytes) -- never from the HIP path.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from wq_testutil import assert_close, to_device, torch_bf16_bits

pytestmark = pytest.mark.gpu

FMTS = {"int4": oracle.INT4, "affine2": oracle.AFFINE2, "ccq": oracle.CCQ,
        "ccq432": oracle.CCQ432, "ccqh": oracle.CCQ_HYBRID, "int8": oracle.INT8}
ALL = ["int4", "int4pc", "affine2", "ccq", "ccq432", "ccqh", "int8", "int8pc"]


def _fmt_group(name):
    """Format id and group of a test name (the "pc" names are per-channel INT4 / INT8)."""
    if name.endswith("pc"):
        return FMTS[name[:-2]], 0
    return FMTS[name], 64


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


def _quant(fmt, shape, seed, group=64):
    w = synth.weights_f32(shape, *seed)
    return oracle.quantize(w, fmt, group=group)


def _product_bits(decoded):
    """What a product with identity activations returns for decoded weight bits: the sum
    starts at +0, so a -0 weight (a zero group scale times a state below the zero point)
    comes back as +0."""
    out = np.array(decoded, copy=True)
    out[out == 0x8000] = 0
    return out


def _random_packed(fmt, E, n, k, seed, group=64):
    arr = synth.random_packed(fmt, E, n, k, *seed, group=group)
    return oracle.Packed(fmt, n, k, E, group, arr.get("codes"), arr.get("scales"), arr.get("zeros"),
                         arr.get("qscale"), arr.get("super_scale"), arr.get("code_scale"),
                         arr.get("code_zero"), oracle.default_zp(fmt))


# ---------------------------------------------------------------------------------------------
# Dequantize: bit-exact
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("src", ["quantized", "random"])
def test_dequantize_bit_exact(wq, name, src):
    fmt, group = _fmt_group(name)
    E, n, k = 2, 40, 320  # 5 groups: an odd count exercises the half-used qscale byte
    _say(f"dequant {name} {src} E={E} n={n} k={k}")
    if src == "quantized":
        p = _quant(fmt, (E, n, k), (1, fmt, group), group=group)
    else:
        p = _random_packed(fmt, E, n, k, (2, fmt, group), group=group)
    got = torch_bf16_bits(wq.wq_dequantize(to_device(p)))
    for e in range(E):
        ref = oracle.dequantize(p, e)
        assert np.array_equal(got[e], ref), f"expert {e}: {(got[e] != ref).sum()} mismatches"


@pytest.mark.parametrize("name", ["ccq432", "ccqh"])
def test_dequantize_alg2_every_word_value(wq, name):
    # every u8 / u16 word value in every non-last position class, random last words (weight 63
    # and the group scale field), odd group count (groups start 2 bytes into a dword)
    fmt = FMTS[name]
    P, nvals = (22, 256) if name == "ccq432" else (10, 65536)
    g = np.random.default_rng(31)
    n, G = 16, 5 if name == "ccq432" else 457
    body = np.resize(np.arange(nvals), n * G * (P - 1)).reshape(n, G, P - 1)
    words = np.concatenate([body, g.integers(0, nvals, (n, G, 1))], axis=2)
    sup = g.uniform(1e-5, 1e-3, (1, n)).astype(np.float32)
    p = oracle.alg2_pack(fmt, words[None], sup)
    got = torch_bf16_bits(wq.wq_dequantize(to_device(p)))[0]
    assert np.array_equal(got, oracle.dequantize(p))


def test_dequantize_ccq_every_code(wq):
    # rows r with code scale 1 and code zero 256 r: the 128 rows cover all 2^15 codes, every
    # group scale 0..15, and a non-trivial super scale per row
    rows, k = 128, 1024
    g = np.random.default_rng(21)
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))[None]
    sq = g.integers(0, 16, (rows, k // 64), dtype=np.uint8)
    qscale = (sq[:, 0::2] | (sq[:, 1::2] << 4)).astype(np.uint8)[None]
    p = oracle.Packed(oracle.CCQ, rows, k, 1, 64, codes, qscale=qscale,
                      super_scale=g.uniform(1e-4, 1e-3, (1, rows)).astype(np.float32),
                      code_scale=np.ones((1, rows), np.float32),
                      code_zero=(256.0 * np.arange(rows, dtype=np.float32))[None], zp=32)
    got = torch_bf16_bits(wq.wq_dequantize(to_device(p)))[0]
    assert np.array_equal(got, oracle.dequantize(p))


def test_dequantize_ccq_rounding_and_clamp_edges(wq):
    # code scales / zeros that put fma results on .5 ties, below 0 and above 2^15 - 1
    rows, k = 16, 256
    g = np.random.default_rng(22)
    cs = np.array([0.5, 1.5, 128.5, 127.25, 200.0, 300.0, 1.0, 64.0625,
                   0.75, 2.5, 128.0, 129.0, 1e-3, 255.0, 128.49, 97.7], np.float32)
    cz = np.array([0.5, -0.5, -100.0, 0.25, 0.0, -5.0, 32760.0, 10.5,
                   -0.49, 0.5, 32767.0, -129.0, 0.5, 0.0, 1.5, 3.0], np.float32)
    codes = g.integers(0, 256, (1, rows, k // 4), dtype=np.uint8)
    codes[0, :, :256 // 4] = np.arange(64, dtype=np.uint8)[None] * 4 + 3
    sq = g.integers(1, 16, (rows, k // 128), dtype=np.uint8)
    p = oracle.Packed(oracle.CCQ, rows, k, 1, 64, codes, qscale=(sq | (sq << 4))[None],
                      super_scale=np.full((1, rows), 3e-4, np.float32), code_scale=cs[None],
                      code_zero=cz[None], zp=32)
    got = torch_bf16_bits(wq.wq_dequantize(to_device(p)))[0]
    assert np.array_equal(got, oracle.dequantize(p))


# ---------------------------------------------------------------------------------------------
# Dense product
# ---------------------------------------------------------------------------------------------

DENSE_SHAPES = [(80, 576), (128, 1024), (512, 512)]


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("nk", DENSE_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("m", [1, 3, 16, 17, 32, 33, 70, 150, 276])
def test_gemm_parity(wq, name, nk, m):
    import torch

    fmt, group = _fmt_group(name)
    n, k = nk
    _say(f"gemm {name} n={n} k={k} m={m}")
    p = _quant(fmt, (n, k), (3, fmt, group, n, k), group=group)
    x = synth.acts_bf16((m, k), 4, m, k)
    ref = oracle.gemm(x, p)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    y = wq.wq_gemm(xd, to_device(p))
    assert_close(torch_bf16_bits(y), ref, f"gemm {name} {n}x{k} m={m}")


# Few rows whose activations fit in LDS whole (rows x (2 K + 16) + 128 bytes <= 132 KiB, K a
# multiple of 256) take the single-staging kernel: 4 waves split K, or 16 when the output tiles
# are few and K % 1024 == 0.  K = 8448 (4 waves) gives each wave 2112 columns and K = 17408 (16
# waves) 1088: more steps than a lane holds at once for every format, and a last step that runs
# past the wave's part.  m = 8 at K = 8448 and m = 4 at K = 17408 just miss the LDS limit and
# take the chunked kernel; m = 7 and m = 16 stage in two rounds; n = 40 leaves a partial tile.
GEMV_CASES = [(40, 8448, 1), (40, 8448, 3), (40, 8448, 7), (40, 8448, 8), (200, 2048, 16),
              (24, 768, 5), (40, 17408, 1), (40, 17408, 3), (40, 17408, 4), (64, 4096, 16)]


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "x".join(map(str, c)))
def test_gemv_path_parity(wq, name, case):
    import torch

    fmt, group = _fmt_group(name)
    n, k, m = case
    _say(f"gemv {name} n={n} k={k} m={m}")
    p = _quant(fmt, (n, k), (41, fmt, group, n, k), group=group)
    x = synth.acts_bf16((m, k), 42, m, k)
    ref = oracle.gemm(x, p)
    y = wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), to_device(p))
    assert_close(torch_bf16_bits(y), ref, f"gemv {name} {n}x{k} m={m}")


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("k", [768, 1024])
def test_gemv_decodes_every_weight_bit_exact(wq, name, k):
    # The identity-activation check of the decode, 16 rows at a time (single-staging kernel):
    # k = 768 gives each of 4 waves 192 columns (CCQ lanes 2 and 3 and INT4's second step run
    # past the part and must read zeros); k = 1024 gives each of 16 waves 64 columns.
    import torch

    fmt, group = _fmt_group(name)
    n = 40
    p = _quant(fmt, (n, k), (43, fmt, group), group=group)
    ref = oracle.dequantize(p)
    d = to_device(p)
    for c0 in range(0, k, 16):
        x = np.zeros((16, k), np.uint16)
        x[np.arange(16), c0 + np.arange(16)] = 0x3F80
        y = torch_bf16_bits(wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), d))
        assert np.array_equal(y.T, _product_bits(ref[:, c0:c0 + 16])), f"columns {c0}..{c0 + 15}"


def test_gemm_row_chunks(wq):
    # Group-64 INT8 runs the decode-streaming kernel for every row count; past 65535 blocks of
    # 32 rows the product is split into several launches.  Rows on both sides of the split.
    import torch

    n, k = 32, 64
    chunk = 65535 * 32
    m = chunk + 77
    _say(f"gemm row chunks int8 m={m}")
    p = _quant(oracle.INT8, (n, k), (7, 1), group=64)
    x = synth.acts_bf16((m, k), 7, 2)
    y = wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), to_device(p))
    rows = np.array([0, 1, chunk - 1, chunk, chunk + 1, m - 1])
    ref = oracle.gemm(np.ascontiguousarray(x[rows]), p)
    assert_close(torch_bf16_bits(y)[rows], ref, "gemm row chunks")


def test_gemm_deterministic(wq):
    import torch

    p = _quant(oracle.CCQ, (256, 2048), (5,))
    x = torch.from_numpy(synth.acts_bf16((8, 2048), 6).view(np.int16)).cuda()
    d = to_device(p)
    a = torch_bf16_bits(wq.wq_gemm(x, d))
    b = torch_bf16_bits(wq.wq_gemm(x, d))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ALL)
def test_tiled_gemm_repeatable_short_k(wq, name):
    # Many activation rows (tiled kernel) with short K: every step of the pipeline is a
    # prologue or tail step.  Repeated launches must give identical bits within tolerance of
    # the oracle (a read of the packed codes that raced its own results once gave wrong
    # 32-column blocks here, intermittently).
    import torch

    fmt, group = _fmt_group(name)
    # 1, 2, 3 steps (tails only), 4 (one unrolled loop pass), 5 and 7 (a pass plus odd tails)
    for k in (64, 128, 192, 256, 320, 448):
        n, m = 320, 64
        p = _quant(fmt, (n, k), (21, fmt, group, k), group=group)
        x = synth.acts_bf16((m, k), 22, k)
        ref = oracle.gemm(x, p)
        d = to_device(p)
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        first = None
        for rep in range(6):
            y = torch_bf16_bits(wq.wq_gemm(xd, d))
            assert_close(y, ref, f"tiled {name} k={k} rep {rep}")
            if first is None:
                first = y
            assert np.array_equal(y, first), f"tiled {name} k={k}: run {rep} differs from run 0"


@pytest.mark.parametrize("name", ALL)
def test_gemm_decodes_every_weight_bit_exact(wq, name):
    # Identity activations: row m of x = e_(c0+m) makes y[m][n] = W_hat[n][c0+m], one exact
    # product rounded back to the same bf16 -- so the product path's decode of every weight
    # must equal the oracle's decoded bits.
    import torch

    fmt, group = _fmt_group(name)
    n, k = 48, 320
    p = _quant(fmt, (n, k), (7, fmt, group), group=group)
    ref = oracle.dequantize(p)
    d = to_device(p)
    for c0 in range(0, k, 32):
        x = np.zeros((32, k), np.uint16)
        x[np.arange(32), c0 + np.arange(32)] = 0x3F80
        y = torch_bf16_bits(wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), d))
        assert np.array_equal(y.T, _product_bits(ref[:, c0:c0 + 32])), f"columns {c0}..{c0 + 31}"


@pytest.mark.parametrize("name", ["ccq432", "ccqh"])
def test_gemm_alg2_random_words_bit_exact(wq, name):
    # uniformly random code words (any scale field, any states) through the product path's
    # decode; k = 576 gives 9 groups per row, so (4,3,2) groups start at both byte offsets
    import torch

    fmt = FMTS[name]
    n, k = 48, 576
    p = _random_packed(fmt, 1, n, k, (32, fmt))
    ref = oracle.dequantize(p)
    d = to_device(p)
    for c0 in range(0, k, 32):
        x = np.zeros((32, k), np.uint16)
        x[np.arange(32), c0 + np.arange(32)] = 0x3F80
        y = torch_bf16_bits(wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), d))
        assert np.array_equal(y.T, _product_bits(ref[:, c0:c0 + 32])), f"columns {c0}..{c0 + 31}"


# ---------------------------------------------------------------------------------------------
# MoE routing and expert FFN
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("t,topk,experts,kind", [(1, 8, 64, "uniform"), (7, 2, 8, "uniform"),
                                                 (300, 8, 64, "uniform"), (4096, 8, 64, "zipf"),
                                                 (33, 4, 300, "uniform"), (50, 1, 1, "uniform"),
                                                 (20, 8, 512, "uniform"), (1000, 6, 16, "zipf"),
                                                 (0, 8, 64, "uniform"), (128, 8, 64, "zipf"),
                                                 (129, 8, 64, "zipf"),
                                                 # above 4096 pairs: sorted in chunks of >= 2048
                                                 (513, 8, 64, "uniform"), (700, 8, 300, "zipf"),
                                                 (3000, 2, 1, "uniform"), (12501, 8, 512, "uniform"),
                                                 (131072, 8, 64, "zipf")])
def test_route_exact(wq, t, topk, experts, kind):
    # both the one-workgroup sort and, for long arrays, the chunked one (its workspace from
    # wq_moe_route_workspace_bytes) against the oracle's stable sort
    import torch

    _say(f"route t={t} topk={topk} E={experts} {kind}")
    gen = synth.routing_zipf if kind == "zipf" else synth.routing_uniform
    ids, _ = gen(t, topk, experts, 8, t)
    off_ref, pairs_ref = oracle.moe_route(ids, experts)
    ids_d = torch.from_numpy(ids).cuda()
    for chunked in (True, False):
        off, pairs = wq.wq_moe_route(ids_d, experts, chunked=chunked)
        assert np.array_equal(off.cpu().numpy(), off_ref), chunked
        assert np.array_equal(pairs.cpu().numpy(), pairs_ref), chunked


@pytest.mark.parametrize("t,experts", [(40, 64), (300, 16), (1000, 64)])
def test_route_drops_ids_out_of_range(wq, t, experts):
    # Ids outside [0, E) are dropped: the offsets count the valid pairs only and the first
    # offsets[E] slots hold the valid pairs grouped by expert in increasing pair order (checked
    # against a direct count, since the oracle refuses such tables).  40 x 8 pairs take the
    # few-pairs kernel, 300 x 8 the counter-row kernel, 1000 x 8 the chunked sort.
    import torch

    ids, _ = synth.routing_uniform(t, 8, experts, 9, t)
    flat = ids.reshape(-1).copy()
    bad = np.random.default_rng(10).random(flat.size) < 0.1
    flat[bad] = np.where(np.arange(flat.size)[bad] % 2 == 0, -1, experts)
    ids = flat.reshape(ids.shape)
    off, pairs = wq.wq_moe_route(torch.from_numpy(ids).cuda(), experts)
    off, pairs = off.cpu().numpy(), pairs.cpu().numpy()
    counts = np.array([(flat == e).sum() for e in range(experts)])
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
    want = np.concatenate([np.flatnonzero(flat == e) for e in range(experts)])
    assert np.array_equal(pairs[:off[-1]], want)


MOE_CASES = [
    # name, E, hidden, inter, tokens, topk  (avg rows per expert >= 32 runs the tiled kernels)
    ("ccq", 8, 256, 192, 5, 2),
    ("ccq", 8, 512, 320, 40, 4),
    ("int4pc", 6, 256, 128, 12, 3),
    ("affine2", 4, 256, 192, 9, 2),
    ("int4", 4, 192, 128, 70, 2),
    ("ccq", 4, 256, 192, 64, 2),        # tiled, 32 rows per expert on average
    ("int4pc", 8, 512, 320, 200, 4),    # tiled, ragged row tiles
    ("affine2", 4, 320, 128, 96, 2),    # tiled
    ("ccq432", 8, 320, 192, 12, 2),
    ("ccqh", 8, 576, 320, 40, 4),
    ("ccq432", 4, 576, 192, 64, 2),     # 32 rows per expert on average
    ("ccqh", 8, 512, 320, 200, 4),
    ("int8", 8, 256, 192, 12, 2),
    ("int8pc", 4, 320, 192, 70, 2),      # tiled
    ("int8", 4, 256, 128, 96, 2),        # group-64 INT8: decode-streaming kernels at every size
]


@pytest.mark.parametrize("case", MOE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_moe_ffn_parity(wq, case):
    import torch

    name, E, H, I, T, topk = case
    fmt, group = _fmt_group(name)
    _say(f"moe {case}")
    gate = _quant(fmt, (E, I, H), (9, 1, E, H, I), group=group)
    up = _quant(fmt, (E, I, H), (9, 2, E, H, I), group=group)
    down = _quant(fmt, (E, H, I), (9, 3, E, H, I), group=group)
    x = synth.acts_bf16((T, H), 10, T, H)
    ids, wts = synth.routing_uniform(T, topk, E, 11, T)
    ref = oracle.moe_ffn(x, ids, wts, gate, up, down)
    y = wq.wq_moe_ffn(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(wts).cuda(), to_device(gate), to_device(up), to_device(down))
    assert_close(torch_bf16_bits(y), ref, f"moe {case}")


# MoE products of at most 16 tokens whose (expert, 16-row tile) pairs number at most 256 take the
# single-staging kernel: 16 waves per workgroup when K splits, else 4 ((4,3,2) and hybrid: always
# 4); an expert with more rows than fit in LDS at once takes several passes.  The other products
# of these cases take the chunked kernel.
MOE_GEMV_CASES = [
    # name, E, hidden, inter, tokens, topk, routing
    ("ccq", 8, 1024, 512, 1, 2, "uniform"),      # gate+up 16 waves, down 4
    ("int4", 8, 768, 256, 3, 2, "uniform"),      # gate+up 4 waves, ragged parts
    ("int8pc", 4, 8192, 256, 16, 2, "expert0"),  # gate+up: expert 0 has 16 rows, two passes of 8
    ("ccq432", 8, 512, 256, 4, 2, "uniform"),    # both products, 4 waves
    ("affine2", 8, 768, 512, 2, 2, "uniform"),   # both products, 4 waves
    ("ccq", 8, 2048, 1024, 1, 1, "uniform"),     # down 16 waves
    ("int4pc", 8, 1024, 512, 5, 3, "uniform"),   # gate+up 16 waves at 256 pairs
    ("ccqh", 6, 1024, 256, 2, 2, "uniform"),     # both products, 4 waves
]


@pytest.mark.parametrize("case", MOE_GEMV_CASES, ids=lambda c: "-".join(map(str, c)))
def test_moe_gemv_path_parity(wq, case):
    import torch

    name, E, H, I, T, topk, kind = case
    fmt, group = _fmt_group(name)
    _say(f"moe gemv {case}")
    gate = _quant(fmt, (E, I, H), (13, 1, E, H, I), group=group)
    up = _quant(fmt, (E, I, H), (13, 2, E, H, I), group=group)
    down = _quant(fmt, (E, H, I), (13, 3, E, H, I), group=group)
    x = synth.acts_bf16((T, H), 14, T, H)
    ids, wts = synth.routing_uniform(T, topk, E, 15, T)
    if kind == "expert0":  # every token's first expert is 0, the others distinct from it
        for t in range(T):
            ids[t] = [0] + [1 + (t + j) % (E - 1) for j in range(topk - 1)]
    ref = oracle.moe_ffn(x, ids, wts, gate, up, down)
    y = wq.wq_moe_ffn(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(wts).cuda(), to_device(gate), to_device(up), to_device(down))
    assert_close(torch_bf16_bits(y), ref, f"moe gemv {case}")


def test_empty_inputs(wq):
    # no rows, no tokens: nothing to compute, no error, empty outputs
    import torch

    p = _quant(oracle.CCQ, (64, 128), (8, 1))
    y = wq.wq_gemm(torch.zeros((0, 128), dtype=torch.int16).cuda(), to_device(p))
    assert tuple(y.shape) == (0, 64)
    gate = _quant(oracle.CCQ, (4, 64, 128), (8, 2))
    up = _quant(oracle.CCQ, (4, 64, 128), (8, 3))
    down = _quant(oracle.CCQ, (4, 128, 64), (8, 4))
    ym = wq.wq_moe_ffn(torch.zeros((0, 128), dtype=torch.int16).cuda(),
                       torch.zeros((0, 2), dtype=torch.int32).cuda(),
                       torch.zeros((0, 2), dtype=torch.float32).cuda(),
                       to_device(gate), to_device(up), to_device(down))
    torch.cuda.synchronize()
    assert tuple(ym.shape) == (0, 128)


@pytest.mark.parametrize("name", ["int4", "ccq", "int8pc"])
@pytest.mark.parametrize("m", [8, 300])
def test_zero_activations_give_plus_zero(wq, name, m):
    # a zero activation row gives exactly +0 in every output (sums start at +0 and add +0 / -0
    # products), in both the decode-streaming and the tiled kernels
    import torch

    fmt, group = _fmt_group(name)
    p = _quant(fmt, (96, 256), (8, 5, fmt), group=group)
    y = wq.wq_gemm(torch.zeros((m, 256), dtype=torch.int16).cuda(), to_device(p))
    assert np.all(torch_bf16_bits(y) == 0)


def test_moe_all_tokens_one_expert(wq):
    # every token routed to experts 0 and 1: a 40-row expert exercises two row super-tiles
    import torch

    E, H, I, T = 4, 256, 128, 40
    gate = _quant(oracle.CCQ, (E, I, H), (12, 1))
    up = _quant(oracle.CCQ, (E, I, H), (12, 2))
    down = _quant(oracle.CCQ, (E, H, I), (12, 3))
    x = synth.acts_bf16((T, H), 13)
    ids = np.tile(np.array([[1, 0]], np.int32), (T, 1))
    wts = np.tile(np.array([[0.75, 0.25]], np.float32), (T, 1))
    ref = oracle.moe_ffn(x, ids, wts, gate, up, down)
    y = wq.wq_moe_ffn(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(wts).cuda(), to_device(gate), to_device(up), to_device(down))
    assert_close(torch_bf16_bits(y), ref, "moe one expert")


def test_moe_stages_compose_to_ffn(wq):
    # route + gate/up + down + combine called one by one give the bits of wq_moe_ffn
    import torch

    E, H, I, T, topk = 8, 512, 192, 20, 4
    gate = to_device(_quant(oracle.CCQ, (E, I, H), (14, 1)))
    up = to_device(_quant(oracle.CCQ, (E, I, H), (14, 2)))
    down = to_device(_quant(oracle.CCQ, (E, H, I), (14, 3)))
    x = torch.from_numpy(synth.acts_bf16((T, H), 15).view(np.int16)).cuda()
    ids, wts = synth.routing_uniform(T, topk, E, 16)
    ids_d, wts_d = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    y_ffn = torch_bf16_bits(wq.wq_moe_ffn(x, ids_d, wts_d, gate, up, down))
    off, pairs = wq.wq_moe_route(ids_d, E)
    h = wq.wq_moe_gate_up(x, off, pairs, topk, gate, up)
    d = wq.wq_moe_down(h, T, topk, off, pairs, down)
    y = torch_bf16_bits(wq.wq_moe_combine(d, wts_d))
    assert np.array_equal(y, y_ffn)


def test_tiled_gemm_decodes_every_weight_bit_exact(wq):
    # 128-row identity blocks go through the tiled kernel (more than 32 rows): y[m][n] =
    # W_hat[n][c0 + m] exactly, for every weight, in every format.
    import torch

    for name in ALL:
        fmt, group = _fmt_group(name)
        n, k = 136, 320
        p = _quant(fmt, (n, k), (17, fmt, group), group=group)
        ref = oracle.dequantize(p)
        d = to_device(p)
        for c0 in range(0, k, 128):
            w = min(128, k - c0)
            x = np.zeros((w, k), np.uint16)
            x[np.arange(w), c0 + np.arange(w)] = 0x3F80
            y = torch_bf16_bits(wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), d))
            assert np.array_equal(y.T, _product_bits(ref[:, c0:c0 + w])), f"{name} columns {c0}.."


@pytest.mark.parametrize("name", ["ccq", "int4pc", "ccq432", "ccqh", "int8pc"])
def test_moe_prefill_skewed_routing(wq, name):
    # Zipf-biased routing as in the prefill workload, at reduced sizes: most rows go to the
    # first experts (several 128-row tiles), the tail experts get a few rows or none.
    import torch

    fmt, group = _fmt_group(name)
    E, H, I, T, topk = 16, 512, 256, 384, 4
    gate = _quant(fmt, (E, I, H), (18, 1), group=group)
    up = _quant(fmt, (E, I, H), (18, 2), group=group)
    down = _quant(fmt, (E, H, I), (18, 3), group=group)
    x = synth.acts_bf16((T, H), 19)
    ids, wts = synth.routing_zipf(T, topk, E, 20)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 128 and counts.min() < 32
    tokens = np.array([0, 1, 2, 100, 200, 383], np.int32)
    ref = oracle.moe_ffn(x, ids, wts, gate, up, down, tokens=tokens)
    y = wq.wq_moe_ffn(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(wts).cuda(), to_device(gate), to_device(up), to_device(down))
    assert_close(torch_bf16_bits(y)[tokens], ref, f"moe prefill {name}")


@pytest.mark.parametrize("name", ["ccq", "int4", "int4pc", "affine2", "ccq432", "ccqh", "int8pc"])
def test_moe_tiled_remainder_classes(wq, name):
    # Experts whose routed rows hit every side of the tiled kernel's tile classes (256, 128, 64
    # and 32 rows): remainders modulo 256 of 0, 1, 16, 17, 31, 32, 33, 64, 65, 128, 129 and 255,
    # with and without full 256-row tiles before them; every token checked.
    import torch

    fmt, group = _fmt_group(name)
    counts = [0, 1, 16, 17, 31, 32, 33, 64, 65, 128, 129, 255, 256, 257, 288, 289, 544, 561]
    E, H, I, topk = len(counts), 256, 192, 2
    flat = np.repeat(np.arange(E, dtype=np.int32), counts)
    T = len(flat) // 2
    assert max(counts) <= T  # pairs (flat[t], flat[t + T]) of the sorted list are distinct
    ids = np.stack([flat[:T], flat[T:]], axis=1)
    _, wts = synth.routing_uniform(T, topk, E, 21)
    _say(f"moe remainder classes {name} T={T}")
    gate = _quant(fmt, (E, I, H), (22, 1), group=group)
    up = _quant(fmt, (E, I, H), (22, 2), group=group)
    down = _quant(fmt, (E, H, I), (22, 3), group=group)
    x = synth.acts_bf16((T, H), 23)
    ref = oracle.moe_ffn(x, ids, wts, gate, up, down)
    y = wq.wq_moe_ffn(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(wts).cuda(), to_device(gate), to_device(up), to_device(down))
    assert_close(torch_bf16_bits(y), ref, f"moe remainder classes {name}")


def _bf16(v):
    """bf16 bits of a value that bf16 holds exactly."""
    b = int(np.array(v, np.float32).view(np.uint32))
    assert b & 0xFFFF == 0, v
    return b >> 16


_BF16_MAX = float(np.array(0x7F7F0000, np.uint32).view(np.float32))
# (a, b, bf16 bits of the correctly rounded a + b): pairs of bf16 values whose fp32 sum is exact
# and lies on or next to a bf16 rounding boundary.
ROUNDING_PAIRS = [
    (1.0, 2.0 ** -8, 0x3F80),                  # tie: down to the even 1.0
    (1.0 + 2.0 ** -7, 2.0 ** -8, 0x3F82),      # tie: up to the even 1 + 2^-6
    (1.0, 2.0 ** -8 + 2.0 ** -15, 0x3F81),     # just above the tie: up
    (1.0, 3 * 2.0 ** -9, 0x3F81),              # above the tie: up
    (-1.0, -(2.0 ** -8), 0xBF80),              # negative tie: down in magnitude
    (-(1.0 + 2.0 ** -7), -(2.0 ** -8), 0xBF82),
    (2.0 - 2.0 ** -7, 2.0 ** -8, 0x4000),      # tie at the top of a binade: carries to 2
    (256.0, 1.0, 0x4380), (258.0, 1.0, 0x4382),  # ties where the bf16 step is 2
    (3.0, -3.0, 0x0000),                       # exact cancellation: +0
    (_BF16_MAX, 2.0 ** 119, 0x7F80),           # tie above the largest bf16: +inf
    (-_BF16_MAX, -(2.0 ** 119), 0xFF80),       # and -inf
    (1.5, 0.0, 0x3FC0),                        # exact
]


@pytest.mark.parametrize("n", [64, 60])
@pytest.mark.parametrize("m", [1, 9, 24, 40, 300])
def test_products_round_half_to_even_bit_exact(wq, m, n):
    # The output rounding of every product kernel (single-staging up to 16 rows, chunked up to
    # 32, tiled beyond; n = 60 takes the tiled kernel's register epilogue, 64 its staged one),
    # bit for bit: every weight is exactly 1 and row i of x holds a pair (a, b) in columns 0
    # and 1, so y[i][c] = bf16(a + b) for every column c.
    import torch

    k = 256
    p = oracle.Packed(oracle.INT8, n, k, 1, 0, np.ones((1, n, k), np.uint8),
                      np.full((1, n), 0x3F80, np.uint16))
    assert np.all(oracle.dequantize(p) == 0x3F80)
    x = np.zeros((m, k), np.uint16)
    want = np.zeros(m, np.uint16)
    for i in range(m):
        a, b, r = ROUNDING_PAIRS[i % len(ROUNDING_PAIRS)]
        x[i, 0], x[i, 1], want[i] = _bf16(a), _bf16(b), r
    ref = oracle.gemm(x, p)
    assert np.array_equal(ref, np.repeat(want[:, None], n, axis=1))
    y = torch_bf16_bits(wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), to_device(p)))
    assert np.array_equal(y, ref), np.argwhere(y != ref)[:5]


def test_combine_rounds_like_the_oracle(wq):
    # wq_moe_combine with one slot of weight 1 returns bf16(1 * d + 0): checked bit for bit
    # against the oracle's fp32 -> bf16 conversion on random fp32 patterns (subnormals left
    # out), every rounding tie class of the low half, infinities, zeros and NaNs with payloads
    # (all to 0x7FC0).
    import torch

    g = np.random.default_rng(41)
    bits = g.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    hi = g.integers(0, 1 << 16, 4096, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    special = np.array([0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x7FC00000,
                        0xFFC00001, 0x7F800001, 0x7FBFFFFF, 0x7F7FFFFF, 0x7F7F8000], np.uint32)
    bits = np.concatenate([bits, (hi[:, None] | lows[None, :]).ravel(), special])
    expo = (bits >> 23) & 0xFF
    bits = bits[(expo != 0) | ((bits & 0x7FFFFF) == 0)]  # no subnormals
    hidden = 4096
    bits = np.resize(bits, (bits.size + hidden - 1) // hidden * hidden)
    d = bits.view(np.float32).reshape(-1, hidden)
    t = d.shape[0]
    w = np.ones((t, 1), np.float32)
    with np.errstate(invalid="ignore"):
        want = oracle.f32_to_bf16(d * np.float32(1.0) + np.float32(0.0))
    y = torch_bf16_bits(wq.wq_moe_combine(torch.from_numpy(d.copy()).cuda(),
                                          torch.from_numpy(w).cuda()))
    assert np.array_equal(y, want), np.argwhere(y != want)[:5]


def test_gemm_ccq_clamped_rows_bit_exact(wq):
    # Rows whose code scale / zero push the expanded code below 0 or above 2^15 - 1 (and rows
    # that stay inside, in the same 16-row tile): the product path's decode must still equal
    # the oracle's bits (identity activations read the weights back).
    import torch

    rows, k = 32, 256
    g = np.random.default_rng(23)
    cs = np.tile(np.array([0.5, 1.5, 128.5, 127.25, 200.0, 300.0, 1.0, 64.0625,
                           0.75, 2.5, 128.0, 129.0, 1e-3, 255.0, 128.49, 97.7], np.float32), 2)
    cz = np.tile(np.array([0.5, -0.5, -100.0, 0.25, 0.0, -5.0, 32760.0, 10.5,
                           -0.49, 0.5, 32767.0, -129.0, 0.5, 0.0, 1.5, 3.0], np.float32), 2)
    codes = g.integers(0, 256, (1, rows, k // 4), dtype=np.uint8)
    sq = g.integers(1, 16, (rows, k // 128), dtype=np.uint8)
    p = oracle.Packed(oracle.CCQ, rows, k, 1, 64, codes, qscale=(sq | (sq << 4))[None],
                      super_scale=np.full((1, rows), 3e-4, np.float32), code_scale=cs[None],
                      code_zero=cz[None], zp=32)
    ref = oracle.dequantize(p)
    d = to_device(p)
    for m in (32, 128):  # decode-streaming and tiled kernels
        for c0 in range(0, k, m):
            w = min(m, k - c0)
            x = np.zeros((w, k), np.uint16)
            x[np.arange(w), c0 + np.arange(w)] = 0x3F80
            y = torch_bf16_bits(wq.wq_gemm(torch.from_numpy(x.view(np.int16)).cuda(), d))
            assert np.array_equal(y.T, _product_bits(ref[:, c0:c0 + w])), (m, c0)


# ---------------------------------------------------------------------------------------------
# CCQ encoder on the GPU: bit-identical to the oracle's quantizer
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape,zp,refine", [((1, 40, 320), 32, True), ((1, 40, 320), 32, False),
                                             ((1, 40, 320), 32, oracle.CCQ_REPICK),
                                             ((1, 40, 320), 32, oracle.CCQ_SCALE_UPDATE),
                                             ((2, 24, 1024), 32, True), ((1, 6, 8192), 32, True),
                                             ((1, 16, 448), 0, True), ((1, 16, 448), 16, False),
                                             ((1, 3, 131072), 32, True)])
def test_quantize_ccq_matches_oracle(wq, shape, zp, refine):
    import torch

    E, n, k = shape
    _say(f"ccq encode {shape} zp={zp} refine={refine}")
    w = synth.weights_f32(shape, 33, E, n, k)
    w[0, 0] = 0.0                                  # a zero row: super scale 1
    w[0, 1] = 0.01                                 # a constant row: one code, code scale 1
    w[0, 2, 5] = 0.9                               # an outlier
    ref = oracle.quantize(w, oracle.CCQ, refine=refine, zp=zp)
    got = wq.wq_quantize_ccq(torch.from_numpy(w).cuda(), zp=zp, refine=refine)
    for name in ("codes", "qscale", "super_scale", "code_scale", "code_zero"):
        g = getattr(got, name).cpu().numpy()
        r = getattr(ref, name).reshape(g.shape)
        assert g.dtype.itemsize == r.dtype.itemsize, name
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8)), \
            f"{name}: {(g.view(np.uint8) != r.view(np.uint8)).sum()} bytes differ"
