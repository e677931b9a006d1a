"""The mixed-precision MoE stack at full layer shape through the stack runner the benchmark
times: 64 experts, hidden 8192, expert intermediate 3584, top-8 routing of 32 tokens, one
WINT4 per-channel layer followed by two CCQ (6,4,3) group-64 layers (the FastDeploy "WINT2
Quantization" w4w2 layer map, shortened), all layers sharing one set of routing arrays and
h / d workspaces.  Every token of every layer is checked against the oracle, and a captured
HIP graph of the step must replay the eager outputs bit for bit."""
import sys

import numpy as np
import pytest

import oracle
import synth
from wq_testutil import assert_close, to_host, torch_bf16_bits

pytestmark = pytest.mark.gpu

E, H, I, T, K = 64, 8192, 3584, 32, 8


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _layer(wq, fmt, group, seed):
    zp = 32
    out = []
    for j, (n, k) in enumerate(((I, H), (I, H), (H, I))):
        arr = synth.random_packed_device(fmt, E, n, k, seed * 16 + j, group=group)
        out.append(wq.PackedWeight(fmt, n, k, E, group, *(arr.get(f) for f in (
            "codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")), zp))
    return tuple(out)


def test_mixed_stack_every_token_every_layer():
    import torch

    import weight_only_bit_amd as wq
    from weight_only_bit_amd.stack import MoeStack

    assert torch.cuda.is_available()
    wq.lib()
    plan = [(wq.FMT_INT4, 0), (wq.FMT_CCQ2, 64), (wq.FMT_CCQ2, 64)]
    _say("stack: generating 3 layers (INT4 per channel, CCQ, CCQ) at 64 x 8192 x 3584")
    layers = [_layer(wq, fmt, group, 5100 + l) for l, (fmt, group) in enumerate(plan)]
    x_h = synth.acts_bf16((T, H), 5200)
    x = torch.from_numpy(x_h.view(np.int16)).cuda()
    routes_h = [synth.routing_uniform(T, K, E, 5201, l) for l in range(len(layers))]
    routes = [(torch.from_numpy(i).cuda(), torch.from_numpy(w).cuda()) for i, w in routes_h]
    ys = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in layers]
    st = MoeStack(layers, T, K)
    _say("stack: eager step")
    st.step(x, routes, ys)
    torch.cuda.synchronize()
    eager = [torch_bf16_bits(y).copy() for y in ys]
    for l, (fmt, _) in enumerate(plan):
        _say(f"stack: oracle layer {l} (format {fmt}), all {T} tokens")
        g, u, dn = (to_host(w) for w in layers[l])
        ref = oracle.moe_ffn(x_h, routes_h[l][0], routes_h[l][1], g, u, dn)
        assert_close(eager[l], ref, f"stack layer {l}")
    # the captured step replays the eager result bit for bit, with eager work in between
    _say("stack: graph capture and replays")
    st.capture(x, routes, ys)
    for rep in range(3):
        for y in ys:
            y.zero_()
        st.replay()
        torch.cuda.synchronize()
        for l in range(len(layers)):
            assert np.array_equal(torch_bf16_bits(ys[l]), eager[l]), (rep, l)
        st.step(x, routes, ys)  # eager work between replays
        torch.cuda.synchronize()
