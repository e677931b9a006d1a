"""The products captured in a HIP graph (torch.cuda.CUDAGraph) and replayed, as a serving loop
or the operator benchmarks run them.  Every replay, with eager work of the same library and
synchronizations between replays, must give the eager result bit for bit.  The library issues
only kernel launches on the caller's stream (no memsets, no allocations), so its calls can be
captured once their first eager call has run.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from wq_testutil import to_device, torch_bf16_bits

pytestmark = pytest.mark.gpu

REPLAYS = 4


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


def _capture(fn):
    """Warm up on a side stream, then capture fn() once."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("name,m", [("ccq", 1), ("ccq", 300), ("int4", 8), ("int8pc", 64)])
def test_graph_replay_gemm(wq, name, m):
    import torch

    fmt, group = {"ccq": (oracle.CCQ, 64), "int4": (oracle.INT4, 64), "int8pc": (oracle.INT8, 0)}[name]
    _say(f"graph gemm {name} m={m}")
    p = oracle.quantize(synth.weights_f32((320, 512), 80, fmt, group), fmt, group=group)
    w = to_device(p)
    x = torch.from_numpy(synth.acts_bf16((m, 512), 81, m).view(np.int16)).cuda()
    x2 = torch.from_numpy(synth.acts_bf16((m, 512), 82, m).view(np.int16)).cuda()
    ref = torch_bf16_bits(wq.wq_gemm(x, w))
    ref2 = torch_bf16_bits(wq.wq_gemm(x2, w))
    y = torch.empty((m, 320), dtype=torch.bfloat16, device="cuda")
    g = _capture(lambda: wq.wq_gemm(x, w, y=y))
    for r in range(REPLAYS):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(torch_bf16_bits(y), ref), f"replay {r}"
        # eager work of the same library between replays
        assert np.array_equal(torch_bf16_bits(wq.wq_gemm(x2, w)), ref2)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [6, 200, 2500])  # 2500 x 2 pairs: the chunked routing sort
def test_graph_replay_moe_ffn(wq, T):
    import torch

    E, H, I, topk = 8, 256, 192, 2
    _say(f"graph moe T={T}")
    gate, up, down = (to_device(oracle.quantize(synth.weights_f32(shape, 83, j), oracle.CCQ))
                      for j, shape in enumerate(((E, I, H), (E, I, H), (E, H, I))))
    x = torch.from_numpy(synth.acts_bf16((T, H), 84, T).view(np.int16)).cuda()
    ids, wts = synth.routing_uniform(T, topk, E, 85, T)
    ids_d, wts_d = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    ref = torch_bf16_bits(wq.wq_moe_ffn(x, ids_d, wts_d, gate, up, down))
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(wq.wq_moe_workspace_bytes(T, topk, E, H, I), 256), dtype=torch.uint8,
                     device="cuda")
    g = _capture(lambda: wq.wq_moe_ffn(x, ids_d, wts_d, gate, up, down, y=y, ws=ws))
    for r in range(REPLAYS):
        y.zero_()
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(torch_bf16_bits(y), ref), f"replay {r}"
        assert np.array_equal(torch_bf16_bits(wq.wq_moe_ffn(x, ids_d, wts_d, gate, up, down)), ref)
        torch.cuda.synchronize()
