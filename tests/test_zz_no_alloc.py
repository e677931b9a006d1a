"""wq_moe_ffn_noalloc (the MoE FFN with the library's own scratch array as workspace) against
wq_moe_ffn with a caller workspace: identical bits on two calls in a row, the second with a
smaller input, at the decode layer's full shape and on a small oracle-checked layer; and a call
whose workspace exceeds the array is refused before anything runs."""
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


def _run_both(wq, x, ids, wts, mats):
    import torch

    t, hidden = x.shape
    ref = wq.wq_moe_ffn(x, ids, wts, *mats)
    y = torch.full((t, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    wq.wq_moe_ffn_noalloc(x, ids, wts, *mats, y=y)
    torch.cuda.synchronize()
    return torch_bf16_bits(y), torch_bf16_bits(ref)


def test_noalloc_matches_workspace_call_full_decode_shape(wq):
    import torch

    E, H, I, K = 64, 8192, 3584, 8
    fields = ("codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")
    mats = []
    for j, (n, k) in enumerate(((I, H), (I, H), (H, I))):
        arr = synth.random_packed_device(wq.FMT_CCQ2, E, n, k, 9100 + j)
        mats.append(wq.PackedWeight(wq.FMT_CCQ2, n, k, E, 64, *(arr.get(f) for f in fields), 32))
    for call, T in enumerate((32, 4)):  # the chunked decode kernels, then the single-staging ones
        _say(f"noalloc full decode shape: call {call}, {T} tokens")
        x = torch.from_numpy(synth.acts_bf16((T, H), 9101, T).view(np.int16)).cuda()
        ids, wts = synth.routing_uniform(T, K, E, 9102, T)
        got, ref = _run_both(wq, x, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), mats)
        assert np.array_equal(got, ref), (call, T)
    # a workspace above the scratch array is refused on the host
    T = 128
    need = wq.wq_moe_workspace_bytes(T, K, E, H, I)
    assert need > wq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    ids, wts = synth.routing_uniform(T, K, E, 9103)
    y = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="WQ_ERR_WORKSPACE"):
        wq.wq_moe_ffn_noalloc(x, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), *mats, y=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.view(torch.int16)).item() == 0  # nothing ran


def test_noalloc_small_layer_against_oracle(wq):
    import torch

    E, H, I, K = 8, 1024, 512, 2
    host = [oracle.quantize(synth.weights_f32(s, 9110, j), oracle.CCQ)
            for j, s in enumerate(((E, I, H), (E, I, H), (E, H, I)))]
    mats = [to_device(p) for p in host]
    for call, T in enumerate((200, 7)):  # the tiled kernels (50 rows per expert), then decode
        _say(f"noalloc small layer: call {call}, {T} tokens")
        xh = synth.acts_bf16((T, H), 9111, T)
        ids, wts = synth.routing_uniform(T, K, E, 9112, T)
        got, ref = _run_both(wq, torch.from_numpy(xh.view(np.int16)).cuda(),
                             torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(), mats)
        assert np.array_equal(got, ref), (call, T)
        assert_close(got, oracle.moe_ffn(xh, ids, wts, *host), f"noalloc small layer call {call}")


def test_noalloc_captured_in_a_graph(wq):
    """The callers this entry point is for include code under HIP graph capture: a captured
    call replays the eager result bit for bit, also after eager calls with other inputs have
    overwritten the scratch array in between (nothing in it needs clearing)."""
    import torch

    E, H, I, K = 8, 1024, 512, 2
    host = [oracle.quantize(synth.weights_f32(s, 9120, j), oracle.CCQ)
            for j, s in enumerate(((E, I, H), (E, I, H), (E, H, I)))]
    mats = [to_device(p) for p in host]

    def inputs(T, seed):
        xh = synth.acts_bf16((T, H), 9121, seed)
        ids, wts = synth.routing_uniform(T, K, E, 9122, seed)
        return (xh, ids, wts, torch.from_numpy(xh.view(np.int16)).cuda(),
                torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda())

    xh, ids, wts, x, ids_d, wts_d = inputs(12, 1)
    y = torch.empty((12, H), dtype=torch.bfloat16, device="cuda")
    wq.wq_moe_ffn_noalloc(x, ids_d, wts_d, *mats, y=y)  # warm-up: one-time set-up outside capture
    torch.cuda.synchronize()
    eager = torch_bf16_bits(y).copy()
    assert_close(eager, oracle.moe_ffn(xh, ids, wts, *host), "noalloc eager before capture")
    _say("noalloc: graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wq.wq_moe_ffn_noalloc(x, ids_d, wts_d, *mats, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.wq_moe_ffn_noalloc(x, ids_d, wts_d, *mats, y=y)
    other = inputs(20, 2)
    y2 = torch.empty((20, H), dtype=torch.bfloat16, device="cuda")
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(torch_bf16_bits(y), eager), rep
        wq.wq_moe_ffn_noalloc(other[3], other[4], other[5], *mats, y=y2)  # overwrites the scratch
        torch.cuda.synchronize()
    assert_close(torch_bf16_bits(y2), oracle.moe_ffn(other[0], other[1], other[2], *host),
                 "noalloc eager between replays")
