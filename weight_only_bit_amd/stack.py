"""A stack of MoE expert-FFN layers run as one decode step, with workspaces shared by the
layers.

The pages' deployment keeps every layer's experts resident on one GPU and runs the layers in
sequence: the FastDeploy "WINT2 Quantization" page's w4w2 map quantizes the experts of layers
0-6 to WINT4 (per channel) and those of layers 7-53 to the 2-bit CCQ format.  One step calls,
per layer, the four stages of ``wq_moe_ffn`` (routing, grouped gate+up with SiLU * up, grouped
down, routing-weighted combine) on the caller's stream, reusing one set of routing arrays and
one h / d workspace for every layer.  The step can be captured in a HIP graph (``capture``)
and replayed; nothing in it allocates.

Argument marshalling only: every stage runs in libwq.so's kernels.
"""
from __future__ import annotations

from . import _check, _need, _ptr, _stream, lib, wq_moe_combine, wq_moe_down, wq_moe_gate_up


class MoeStack:
    """layers: list of (gate, up, down) PackedWeight, all with the same experts, hidden and
    inter; tokens, topk: the step's batch."""

    def __init__(self, layers, tokens: int, topk: int, device="cuda"):
        import torch

        if not layers:
            raise ValueError("MoeStack: no layers")
        g0 = layers[0][0]
        self.E, self.I, self.H = g0.experts, g0.n, g0.k
        for gate, up, down in layers:
            if (gate.experts, gate.n, gate.k) != (self.E, self.I, self.H) or \
                    (up.experts, up.n, up.k) != (self.E, self.I, self.H) or \
                    (down.experts, down.n, down.k) != (self.E, self.H, self.I):
                raise ValueError("MoeStack: every layer must have the same expert shapes")
        self.layers = layers
        self.T, self.K = tokens, topk
        P = tokens * topk
        self.offsets = torch.empty(self.E + 1, dtype=torch.int32, device=device)
        self.pairs = torch.empty(P, dtype=torch.int32, device=device)
        self.h = torch.empty((P, self.I), dtype=torch.bfloat16, device=device)
        self.d = torch.empty((P, self.H), dtype=torch.float32, device=device)
        self._graph = None

    def layer(self, l: int, x, ids, wts, y, gate_up_events=None):
        """One layer: y = MoE-FFN_l(x) routed by ids / wts (int32 / f32 [tokens, topk]).
        gate_up_events: optional (start, end) events recorded around the gate+up launch."""
        import torch

        gate, up, down = self.layers[l]
        _need(ids, "MoeStack ids", "i32", shape=(self.T, self.K))
        _check(lib().wq_moe_route(_ptr(ids), self.T, self.K, self.E, _ptr(self.offsets),
                                  _ptr(self.pairs), None, 0, _stream()), "MoeStack route")
        if gate_up_events is not None:
            gate_up_events[0].record(torch.cuda.current_stream())
        wq_moe_gate_up(x, self.offsets, self.pairs, self.K, gate, up, h=self.h)
        if gate_up_events is not None:
            gate_up_events[1].record(torch.cuda.current_stream())
        wq_moe_down(self.h, self.T, self.K, self.offsets, self.pairs, down, d=self.d)
        wq_moe_combine(self.d, wts, y=y)

    def step(self, x, routes, ys, events=None):
        """Every layer in order: layer l reads x, routes[l] = (ids, wts) and writes ys[l].
        events: optional {layer: (start, end)} around the gate+up launches."""
        for l in range(len(self.layers)):
            self.layer(l, x, routes[l][0], routes[l][1], ys[l],
                       None if events is None else events.get(l))

    def capture(self, x, routes, ys):
        """Capture one step in a HIP graph (after at least one eager step has run, so every
        kernel's one-time set-up is done); replay() then re-runs it on the current stream."""
        import torch

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step(x, routes, ys)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(x, routes, ys)
        self._graph = g
        return g

    def replay(self):
        if self._graph is None:
            raise RuntimeError("MoeStack.replay: capture() first")
        self._graph.replay()


__all__ = ["MoeStack"]
