#!/usr/bin/env python3
"""Benchmark of the weight-only low-bit decode path on one MI355X.

Default workload (one step): a mixed-precision MoE stack decode step at batch 32 -- 54 MoE
layers, each 64 experts with hidden 8192 and expert intermediate 3584, top-8 routing; layers
0-6 hold INT4 per-channel weights and layers 7-53 CCQ (6,4,3) group-64 weights (the w4w2 layer
map of the FastDeploy WINT2 deployment).  All 88.6 GB of packed weights are resident in HBM;
every layer reads the same bf16 activations and writes its own output.  One step runs, per
layer: routing, expert gate+up (fused SiLU*up), expert down and the weighted combine.

Reported: weight-stream GB/s (packed bytes of the experts a step routes to / step time),
tokens/s, the roofline of the dominant kernel (CCQ gate+up) from HIP events around each of
its launches in the timed region, and the CPU oracle timed on a bounded sample.

Inputs are synthetic: packed codes and scales are seeded random draws with the layout and
magnitudes of quantized N(0, 0.02) weights (the kernels' cost does not depend on code values);
activations N(0, 1); uniform top-8 routing with softmax weights.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_skinny_ccq_gateup_moe_decode.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_tiled_ccq_gateup_moe_prefill.json")


def kernel_record(path=TRAFFIC_FILE):
    """The committed record of a roofline kernel (rocprofv3 counter runs, for the decode kernel
    also the instruction count of its compiled loop), or None when the kernel sources changed
    since it was taken."""
    import hashlib

    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["kernel_sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return rec if h.hexdigest() == rec["kernel_sources_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of a roofline kernel from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy), or None when the kernel sources changed
    since those counters were taken."""
    rec = kernel_record(path)
    return int(rec["traffic_bytes_per_launch"]) if rec and "traffic_bytes_per_launch" in rec else None


# Vector-ALU issue peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes at the 2.4 GHz peak clock
# (a 64-lane instruction occupies a SIMD for 4 cycles).
VALU_LANE_OPS_PEAK = 256 * 4 * 16 * 2.4e9


def alu_roofline(weights_per_launch, launch_s):
    """The gate+up kernel against the vector-ALU issue roofline: decoded weights per second
    against the VALU peak divided by the loop's instructions per weight (counted in the
    compiled gfx950 loop and kept with the kernel record), or None without a current record."""
    rec = kernel_record()
    if not rec or "valu_per_weight" not in rec:
        return None
    ipw = float(rec["valu_per_weight"])
    peak = VALU_LANE_OPS_PEAK / ipw / 1e9
    achieved = weights_per_launch / launch_s / 1e9
    return {"bound": "alu", "achieved": round(achieved, 1), "peak": round(peak, 1),
            "unit": "G weights/s", "frac": round(achieved / peak, 4), "valu_per_weight": ipw}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baselines."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def omp_threads(n):
    """Set the OpenMP thread count of this thread's later parallel regions (the oracle's)."""
    import ctypes

    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


# --wformat name -> (wq format id, zero point, label)
WFORMATS = {"ccq": (3, 32, "CCQ (6,4,3) code cluster g64"),
            "ccq432": (4, 8, "CCQ (4,3,2) g64"),
            "ccqh": (5, 4, "CCQ hybrid (3,3,2)+(3,4,2) g64")}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=54, help="MoE layers in the stack")
    ap.add_argument("--int4-layers", type=int, default=7, help="leading INT4 per-channel layers")
    ap.add_argument("--tokens", type=int, default=32)
    ap.add_argument("--cpu-tokens", type=int, default=32, help="tokens per sampled layer for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg of the default run")
    ap.add_argument("--prefill-cpu-tokens", type=int, default=6,
                    help="tokens of the prefill layer the oracle runs for the prefill CPU baseline")
    ap.add_argument("--wformat", default="ccq", choices=list(WFORMATS),
                    help="2-bit-class format of the MoE layers (moe_stack_decode, moe_prefill): "
                         "ccq = (6,4,3) code cluster, 2.06 bpw (default); ccq432 = (4,3,2), "
                         "2.75 bpw; ccqh = hybrid (3,3,2)+(3,4,2), 2.5 bpw")
    ap.add_argument("--workload", default="moe_stack_decode",
                    choices=["moe_stack_decode", "moe_prefill", "dense_decode", "copy_calibration",
                             "pages_shapes", "ccq_encode", "hbm_achievable"],
                    help="moe_stack_decode (default): the 54-layer stack step; moe_prefill: one "
                         "CCQ MoE layer at 4096 tokens with Zipf-skewed routing; dense_decode: "
                         "one 4096x4096 CCQ / 2-bit affine linear at 1, 8, 32 rows; pages_shapes: "
                         "the GEMV and grouped-GEMM shapes of the CCQ paper's operator tables; "
                         "ccq_encode: the GPU CCQ encoder on one expert gate tensor; "
                         "hbm_achievable: torch's read-only reduction and copy bandwidth (context)")
    return ap.parse_args()


def make_layer(wq, synth, fmt, E, H, I, seed, group):
    """gate, up, down PackedWeight for one layer, drawn on the GPU."""
    zp = {f: z for f, z, _ in WFORMATS.values()}.get(fmt, 32)
    ws = []
    for j, (n, k) in enumerate(((I, H), (I, H), (H, I))):
        arr = synth.random_packed_device(fmt, E, n, k, seed * 16 + j, group=group)
        ws.append(wq.PackedWeight(fmt, n, k, E, group, *(arr.get(f) for f in (
            "codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")), zp))
    return ws


def to_host_packed(oracle, w):
    """Device PackedWeight -> oracle.Packed (host copies of the same bytes)."""
    import numpy as np

    def h(t):
        if t is None:
            return None
        a = t.cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a

    return oracle.Packed(w.format, w.n, w.k, w.experts, w.group, h(w.codes), h(w.scales),
                         h(w.zeros), h(w.qscale), h(w.super_scale), h(w.code_scale),
                         h(w.code_zero), w.zp)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the decode path keeps every expert of a layer on "
              f"one device (no sharding, no collectives); got --gpus {args.gpus}, WORLD_SIZE {world}.",
              flush=True)
        sys.exit(2)
    if args.workload == "moe_prefill":
        return moe_prefill(args)
    if args.workload == "dense_decode":
        return dense_decode(args)
    if args.workload == "copy_calibration":
        return copy_calibration(args)
    if args.workload == "pages_shapes":
        return pages_shapes(args)
    if args.workload == "ccq_encode":
        return ccq_encode(args)
    if args.workload == "hbm_achievable":
        return hbm_achievable(args)

    import numpy as np
    import torch

    import synth
    import weight_only_bit_amd as wq
    from weight_only_bit_amd.stack import MoeStack

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wq.lib()
    dev = torch.device("cuda:0")
    E, H, I, K = 64, 8192, 3584, 8
    T = args.tokens
    L = args.layers
    n4 = min(args.int4_layers, L)

    # ---------------- resident stack ----------------
    t0 = time.time()
    layers = []
    for l in range(L):
        fmt, group = (wq.FMT_INT4, 0) if l < n4 else (WFORMATS[args.wformat][0], 64)
        layers.append(make_layer(wq, synth, fmt, E, H, I, 1000 + l, group))
        if l % 8 == 7 or l == L - 1:
            torch.cuda.synchronize()
            log(f"generated layers 0..{l} ({time.time() - t0:.1f} s)")
    resident = sum(w.nbytes() for lay in layers for w in lay)
    x = torch.from_numpy(synth.acts_bf16((T, H), 500).view(np.int16)).to(dev)
    routes_h = [synth.routing_uniform(T, K, E, 600, l) for l in range(L)]
    routes = [(torch.from_numpy(i).to(dev), torch.from_numpy(w).to(dev)) for i, w in routes_h]
    ys = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    stack = MoeStack(layers, T, K, device=dev)

    # Algorithmic bytes: packed weights of the experts each layer routes to.
    per_expert = [[w.nbytes() // E for w in lay] for lay in layers]
    touched = [len(np.unique(r[0])) for r in routes_h]
    step_weight_bytes = sum(touched[l] * sum(per_expert[l]) for l in range(L))
    step_act_bytes = L * 2 * T * H * 2  # x read + y written per layer
    ccq_layers = [l for l in range(L) if l >= n4]

    # ---------------- warmup, graph capture, timed steps (graph replays) ----------------
    for _ in range(max(args.warmup, 1)):
        stack.step(x, routes, ys)
    torch.cuda.synchronize()
    stack.capture(x, routes, ys)
    stack.replay()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for s in range(args.steps):
        stack.replay()
        marks[s + 1].record()
    torch.cuda.synchronize()
    step_ms = [marks[s].elapsed_time(marks[s + 1]) for s in range(args.steps)]
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    half = step_ms[args.steps // 2:] if args.steps > 1 else step_ms
    ms_step_latter = float(np.mean(half))

    # ---------------- eager passes: plain (context) and with events around CCQ gate+up ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        stack.step(x, routes, ys)
    e1.record()
    torch.cuda.synchronize()
    ms_step_eager = e0.elapsed_time(e1) / args.steps
    evs_all = [{l: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for l in ccq_layers} for _ in range(args.steps)]
    for s in range(args.steps):
        stack.step(x, routes, ys, events=evs_all[s])
    torch.cuda.synchronize()
    gu_ms = [evs[l][0].elapsed_time(evs[l][1]) for evs in evs_all for l in ccq_layers]
    gu_avg_ms = float(np.mean(gu_ms)) if gu_ms else float("nan")
    # bytes of one CCQ gate+up launch: gate and up of the touched experts + x read + h written
    gu_bytes = float(np.mean([touched[l] * (per_expert[l][0] + per_expert[l][1]) for l in ccq_layers])) \
        + T * H * 2 + T * K * I * 2
    gu_gbs = gu_bytes / (gu_avg_ms * 1e-3) / 1e9
    # weights one CCQ gate+up launch decodes: gate and up rows of the touched experts
    gu_weights = float(np.mean([touched[l] for l in ccq_layers])) * 2 * I * H if ccq_layers else 0.0

    value = step_weight_bytes / (ms_step * 1e-3) / 1e9
    tok_s = T / (ms_step * 1e-3)
    log(f"step {ms_step:.3f} ms (graph replay; latter half {ms_step_latter:.3f}, eager {ms_step_eager:.3f}), "
        f"weight stream {value:.1f} GB/s, {tok_s:.1f} tok/s; CCQ gate+up {gu_avg_ms * 1e3:.1f} us avg "
        f"-> {gu_gbs:.1f} GB/s")

    # ---------------- CPU baseline (oracle on a bounded sample) + spot parity ----------------
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from wq_testutil import assert_close, torch_bf16_bits

        stack.replay()  # the outputs the parity check reads: one more replay of the step
        torch.cuda.synchronize()
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        # up to three of the 2-bit-class layers and two INT4 per-channel layers: ~10 s of oracle
        # work on 16 host cores (each layer's touched experts are decoded and multiplied)
        sample_layers = [l for l in (n4, n4 + 1, n4 + 2) if l < L] + [l for l in (0, 1) if l < n4]
        tot_bytes, tot_s, errs = 0, 0.0, []
        xh = x.cpu().numpy().view(np.uint16)
        for l in sample_layers:
            g, u, dn = (to_host_packed(oracle, w) for w in layers[l])
            ids, wts = routes_h[l]
            toks = np.arange(min(args.cpu_tokens, T), dtype=np.int32)
            t1 = time.perf_counter()
            yref = oracle.moe_ffn(xh, ids, wts, g, u, dn, tokens=toks)
            tot_s += time.perf_counter() - t1
            tot_bytes += len(np.unique(ids[toks])) * sum(per_expert[l])
            errs.append(assert_close(torch_bf16_bits(ys[l])[toks], yref, f"bench spot parity layer {l}"))
            log(f"oracle layer {l}: {len(toks)} token(s) in {tot_s:.1f} s cumulative")
        cpu = {"value": round(tot_bytes / tot_s / 1e9, 4), "unit": "GB/s", "cores": threads,
               "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": f"{args.cpu_tokens} token(s) of layer(s) {sample_layers} "
                         f"(CCQ and INT4 per-channel), all 8 routed experts decoded and multiplied; "
                         f"{tot_bytes / 1e9:.3f} GB of packed weights in {tot_s:.1f} s"}
        parity = max(errs)

    prefill = None if args.no_prefill else prefill_leg(args, wq, synth, dev)
    out = {
        "metric": METRIC + ("" if args.wformat == "ccq" else f" [{WFORMATS[args.wformat][2]}]"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random packed codes/scales, N(0,1) activations, uniform top-8 routing)",
        "config": {"workload": "moe_stack_decode", "layers": L, "int4_per_channel_layers": n4,
                   "ccq_g64_layers": L - n4, "ccq_format": WFORMATS[args.wformat][2], "experts": E, "topk": K, "hidden": H, "inter": I,
                   "tokens": T, "resident_weight_bytes": resident,
                   "step_weight_bytes": step_weight_bytes, "step_activation_bytes": step_act_bytes},
        "value_note": "the decode half of the metric (weight bytes the step streams / step time); the "
                      "prefill half is prefill.value (TFLOP/s)",
        "timing": {"protocol": f"one step ({L} layers) captured in a HIP graph; exactly `steps` replays "
                               "timed with events around all of them (ms_per_step); per-replay events "
                               "give the latter half's mean; an eager pass without events for context",
                   "ms_per_step_latter_half": round(ms_step_latter, 4),
                   "ms_per_step_eager": round(ms_step_eager, 4)},
        "tokens_per_s": round(tok_s, 2),
        "roofline": {"kernel": f"skinny_kernel {WFORMATS[args.wformat][2]} gate+up (MODE_GATEUP)",
                     "bound": "hbm",
                     "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic() if args.wformat == "ccq" else None,
                     "avg_launch_us": round(gu_avg_ms * 1e3, 2),
                     "launch_timing": "HIP events around every CCQ gate+up launch of an eager pass of "
                                      "`steps` steps after the timed replays, on the launch stream",
                     "algorithmic_bytes_per_launch": int(gu_bytes),
                     "alu": alu_roofline(gu_weights, gu_avg_ms * 1e-3) if args.wformat == "ccq" else None},
        "cpu_baseline": cpu,
        "spot_parity_max_rel_err": parity,
        "prefill": prefill,
    }
    print(json.dumps(out), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


METRIC = "weight-stream HBM GB/s (decode M\u226432) + bf16 TFLOP/s (prefill) for w2/w4 GEMM"


def prefill_measure(args, wq, synth, dev, cpu_tokens=0):
    """One MoE layer at prefill size: 4096 tokens, top-8 of 64 experts, Zipf(1.1)-biased routing,
    weights in the --wformat 2-bit-class format.  Layer TFLOP/s (unpadded: 2 * pairs * 3 *
    hidden * inter per call, routing and combine included) from events around `steps` calls;
    the stages one by one from events around each launch, the gate+up stage being the MFMA
    roofline kernel.  cpu_tokens > 0: the oracle on that many tokens of the same layer (its
    rate, and the spot parity of those tokens)."""
    import numpy as np
    import torch

    E, H, I, K, T = 64, 8192, 3584, 8, 4096
    g, u, dn = make_layer(wq, synth, WFORMATS[args.wformat][0], E, H, I, 2000, 64)
    xh = synth.acts_bf16((T, H), 501)
    x = torch.from_numpy(xh.view(np.int16)).to(dev)
    ids, wts = synth.routing_zipf(T, K, E, 601)
    ids_d, wts_d = torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(wq.wq_moe_workspace_bytes(T, K, E, H, I), dtype=torch.uint8, device=dev)
    P = T * K
    flops = 2.0 * P * 3 * H * I
    for _ in range(max(args.warmup, 1)):
        wq.wq_moe_ffn(x, ids_d, wts_d, g, u, dn, y=y, ws=ws)
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(args.steps):
        wq.wq_moe_ffn(x, ids_d, wts_d, g, u, dn, y=y, ws=ws)
    en.record()
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / args.steps
    tf = flops / (ms * 1e-3) / 1e12

    # the stages one by one (same kernels as wq_moe_ffn), each launch bracketed by events
    off, pairs = wq.wq_moe_route(ids_d, E)
    h = torch.empty((P, I), dtype=torch.bfloat16, device=dev)
    d = torch.empty((P, H), dtype=torch.float32, device=dev)
    stages = {"route": lambda: wq.wq_moe_route(ids_d, E),
              "gate_up": lambda: wq.wq_moe_gate_up(x, off, pairs, K, g, u, h=h),
              "down": lambda: wq.wq_moe_down(h, T, K, off, pairs, dn, d=d),
              "combine": lambda: wq.wq_moe_combine(d, wts_d, y=y)}
    stage_us = {}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(max(args.steps, 1)):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            fn()
            a1.record()
            evs.append((a0, a1))
        torch.cuda.synchronize()
        stage_us[name] = float(np.mean([a0.elapsed_time(a1) for a0, a1 in evs])) * 1e3
    gu_flops = 2.0 * P * 2 * H * I
    gu_tf = gu_flops / (stage_us["gate_up"] * 1e-6) / 1e12
    dn_tf = 2.0 * P * H * I / (stage_us["down"] * 1e-6) / 1e12
    counts = np.bincount(ids.ravel(), minlength=E)
    log(f"prefill layer {ms * 1e3:.0f} us ({tf:.1f} TFLOP/s); stages: " +
        ", ".join(f"{k} {v:.0f} us" for k, v in stage_us.items()) +
        f"; gate+up {gu_tf:.1f} TFLOP/s, down {dn_tf:.1f} TFLOP/s")
    res = {"value": round(tf, 2), "unit": "TFLOP/s", "ms_per_layer": round(ms, 4),
           "tokens_per_s": round(T / (ms * 1e-3), 1),
           "config": {"workload": "moe_prefill", "tokens": T, "topk": K, "experts": E,
                      "hidden": H, "inter": I, "routing": "zipf s=1.1",
                      "format": WFORMATS[args.wformat][2],
                      "max_rows_per_expert": int(counts.max()), "min_rows_per_expert": int(counts.min()),
                      "flops_per_layer": flops},
           "stage_us": {k: round(v, 1) for k, v in stage_us.items()},
           "down_tflops": round(dn_tf, 2),
           "roofline": {"kernel": f"tiled_kernel {WFORMATS[args.wformat][2]} gate+up (MODE_GATEUP)",
                        "bound": "mfma",
                        "achieved": round(gu_tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic(PREFILL_TRAFFIC_FILE) if args.wformat == "ccq" else None,
                        "traffic_note": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB "
                                        "copy) against 1.276e9 algorithmic bytes (packed gate+up weights "
                                        "of the 64 experts, x, h)",
                        "avg_launch_us": round(stage_us["gate_up"], 1),
                        "algorithmic_flops_per_launch": gu_flops}}
    if cpu_tokens > 0:
        import oracle

        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from wq_testutil import assert_close, torch_bf16_bits

        wq.wq_moe_ffn(x, ids_d, wts_d, g, u, dn, y=y, ws=ws)
        torch.cuda.synchronize()
        toks = np.linspace(0, T - 1, cpu_tokens).astype(np.int32)
        host = [to_host_packed(oracle, w) for w in (g, u, dn)]
        t1 = time.perf_counter()
        yref = oracle.moe_ffn(xh, ids, wts, *host, tokens=toks)
        dt = time.perf_counter() - t1
        err = assert_close(torch_bf16_bits(y)[toks], yref, "bench prefill spot parity")
        res["cpu_baseline"] = {
            "value": round(2.0 * len(toks) * K * 3 * H * I / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{len(toks)} token(s) of the prefill layer (each with its 8 routed experts "
                      f"decoded and multiplied), {dt:.1f} s"}
        res["spot_parity_max_rel_err"] = err
        log(f"oracle prefill: {len(toks)} tokens in {dt:.1f} s")
    return res


def prefill_leg(args, wq, synth, dev):
    return prefill_measure(args, wq, synth, dev, 0 if args.no_cpu_baseline else args.prefill_cpu_tokens)


def moe_prefill(args):
    """The prefill layer alone (see prefill_measure); `value` is its TFLOP/s."""
    import torch

    import synth
    import weight_only_bit_amd as wq

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    res = prefill_measure(args, wq, synth, dev, 0 if args.no_cpu_baseline else args.prefill_cpu_tokens)
    out = {"metric": f"bf16 TFLOP/s (prefill MoE layer, {WFORMATS[args.wformat][2]})",
           "value": res["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res["ms_per_layer"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": res["config"], "tokens_per_s": res["tokens_per_s"], "stage_us": res["stage_us"],
           "down_tflops": res["down_tflops"], "roofline": res["roofline"],
           "cpu_baseline": res.get("cpu_baseline")}
    print(json.dumps(out), flush=True)


def graph_us(fn, calls, replays=3):
    """Mean GPU time per call of fn(i), i = 0 .. calls-1, with no host launch cost: the calls are
    captured once in a HIP graph (after eager warm-up calls) and the graph is replayed.  Also
    returns the same calls' mean when launched eagerly one by one from Python."""
    import torch

    for i in range(min(calls, 4)):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(calls):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / calls * 1e3
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (replays * calls) * 1e3
    del g
    return us, eager


def dense_decode(args):
    """One 4096 x 4096 linear at 1, 8 and 32 rows, CCQ, 2-bit affine and WINT8 (per channel, the
    deployment's dense layers); each call reads one of
    enough distinct weight copies (>= 1 GiB in total) that the 256 MB last-level cache holds no
    weights between calls.  Also the 512 x 512 W4A16 linear (INT4 g64) at 1 and 8 rows over
    >= 512 MB of copies, and for every case a "hot" time: one copy called again and again, its
    weights in cache."""
    import numpy as np
    import torch

    import synth
    import weight_only_bit_amd as wq

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    N = Kd = 4096
    res = {}
    for fmt, name, group in ((wq.FMT_CCQ2, "ccq", 64), (wq.FMT_INT2_AFFINE, "affine2", 64),
                             (wq.FMT_INT8, "int8pc", 0)):
        one = None
        copies = []
        for c in range(256):
            arr = synth.random_packed_device(fmt, 1, N, Kd, 3000 + c, group=group)
            w = wq.PackedWeight(fmt, N, Kd, 1, group, *(arr.get(f) for f in (
                "codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")), 32)
            copies.append(w)
            one = w.nbytes()
            if one * len(copies) >= (1 << 30):
                break
        for m in (1, 8, 32):
            x = torch.from_numpy(synth.acts_bf16((m, Kd), 502, m).view(np.int16)).to(dev)
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            us, eager = graph_us(lambda i: wq.wq_gemm(x, copies[i % len(copies)], y=y), len(copies),
                                 max(args.steps, 1))
            hot, _ = graph_us(lambda i: wq.wq_gemm(x, copies[0], y=y), 256, max(args.steps, 1))
            res[f"{name}_m{m}"] = {"us": round(us, 2), "GB/s": round(one / (us * 1e-6) / 1e9, 1),
                                   "eager_us": round(eager, 2), "hot_us": round(hot, 2)}
        del copies
    # W4A16 512 x 512: the copies are views into one [R, 512, 512] packed array
    n1 = k1 = 512
    one1 = n1 * k1 // 2 + n1 * (k1 // 64) * 2
    R = -(-(512 << 20) // one1)
    arr = synth.random_packed_device(wq.FMT_INT4, R, n1, k1, 3500, group=64)
    c1 = [wq.PackedWeight(wq.FMT_INT4, n1, k1, 1, 64, arr["codes"][i:i + 1], arr["scales"][i:i + 1],
                          None, None, None, None, None, 8) for i in range(R)]
    for m in (1, 8):
        x = torch.from_numpy(synth.acts_bf16((m, k1), 503, m).view(np.int16)).to(dev)
        y = torch.empty((m, n1), dtype=torch.bfloat16, device=dev)
        us, eager = graph_us(lambda i: wq.wq_gemm(x, c1[i], y=y), R, max(args.steps, 1))
        hot, _ = graph_us(lambda i: wq.wq_gemm(x, c1[0], y=y), 256, max(args.steps, 1))
        res[f"w4a16_512_m{m}"] = {"us": round(us, 2), "GB/s": round(one1 / (us * 1e-6) / 1e9, 1),
                                  "eager_us": round(eager, 2), "hot_us": round(hot, 2)}
    # The oracle on the host (context only): one row of each linear, all threads and one.
    import oracle

    cpu = {}
    ncores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    for name, fmt, n, k in (("ccq_m1", oracle.CCQ, 4096, 4096), ("w4a16_512_m1", oracle.INT4, 512, 512)):
        a = synth.random_packed(fmt, 1, n, k, 3600)
        pk = oracle.Packed(fmt, n, k, 1, 64, a["codes"], a.get("scales"), a.get("zeros"), a.get("qscale"),
                           a.get("super_scale"), a.get("code_scale"), a.get("code_zero"),
                           oracle.default_zp(fmt))
        xh = synth.acts_bf16((1, k), 504)
        nbytes = sum(v.nbytes for v in a.values())
        row = {}
        for threads in (ncores, 1):
            omp_threads(threads)
            oracle.gemm(xh, pk)
            calls, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < 1.0:
                oracle.gemm(xh, pk)
                calls += 1
            s = (time.perf_counter() - t0) / calls
            row[f"{threads}_threads"] = {"us": round(s * 1e6, 1), "GB/s": round(nbytes / s / 1e9, 3)}
        omp_threads(ncores)
        cpu[name] = row
    out = {"metric": "weight-stream GB/s, dense 4096x4096 linear", "value": res["ccq_m1"]["GB/s"],
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "dense_decode", "n": N, "k": Kd}, "results": res,
           "cpu_baseline": {"kind": "oracle", "cpu_model": cpu_model(), "results": cpu,
                            "sample": "one row through each linear (the whole weight decoded), "
                                      "repeated for 1 s, at all host threads and at one"},
           "note": "us: per call from HIP-graph replay of the calls (no host launch cost), each "
                   "call on a weight copy not in cache; eager_us: the same calls launched one by "
                   "one from Python; hot_us: graph replay of one copy called again and again "
                   "(weights in cache); w4a16_512: the 512 x 512 INT4 g64 linear"}
    print(json.dumps(out), flush=True)


# The operator tables of the CCQ paper's inference-performance section (execution time in ms on
# one NVIDIA H20; quoted as context only, another machine's numbers): GEMV input x output at
# M = 1 and 4 (columns WINT2-standard, CCQ) and grouped GEMM groups x output x input at M = 1,
# 4, 16, 64 (columns W8A16, W4A16, W2A16-CCQ).
PAGES_GEMV_MS = {(4096, 4096, 1): (0.027, 0.034), (4096, 1024, 1): (0.015, 0.017),
                 (8192, 8192, 1): (0.073, 0.090), (8192, 1024, 1): (0.019, 0.022),
                 (4096, 4096, 4): (0.028, 0.035), (4096, 1024, 4): (0.015, 0.017),
                 (8192, 8192, 4): (0.076, 0.104), (8192, 1024, 4): (0.019, 0.024)}
PAGES_GROUPED_MS = {(7168, 512, 1): (0.044, 0.030, 0.021), (1024, 7168, 1): (0.100, 0.068, 0.058),
                    (7168, 512, 4): (0.053, 0.035, 0.027), (1024, 7168, 4): (0.315, 0.199, 0.166),
                    (7168, 512, 16): (0.104, 0.071, 0.059), (1024, 7168, 16): (1.052, 0.624, 0.527),
                    (7168, 512, 64): (0.297, 0.193, 0.161), (1024, 7168, 64): (2.655, 1.628, 1.386)}


def pages_shapes(args):
    """The pages' operator shapes on this GPU.  GEMV: dense wq_gemm, input K x output N, M rows,
    2-bit affine (the WINT2-standard column) and CCQ.  Grouped GEMM: 256 experts, M tokens each
    routed to 8 distinct experts uniformly; output x input 1024 x 7168 is the fused gate+up
    product (2 x 512 outputs per pair, wq_moe_gate_up) and 7168 x 512 the down product
    (wq_moe_down), INT8 per channel (W8A16), INT4 g64 (W4A16) and CCQ (W2A16).  Every call reads weights that are not in
    the 256 MB last-level cache: GEMVs rotate over >= 1 GiB of weight copies, grouped products
    over 64 routing tables (each touches 8 M of the 256 experts)."""
    import numpy as np
    import torch

    import synth
    import weight_only_bit_amd as wq

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    fields = ("codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")

    def timed(fn, calls):
        return graph_us(fn, calls, max(args.steps, 1))[0]  # us per call, graph replay

    gemv = {}
    for (k, n, m), (ms_w2, ms_ccq) in PAGES_GEMV_MS.items():
        row = {}
        for fmt, name in ((wq.FMT_INT2_AFFINE, "wint2"), (wq.FMT_CCQ2, "ccq")):
            copies = []
            while True:
                arr = synth.random_packed_device(fmt, 1, n, k, 7000 + len(copies))
                copies.append(wq.PackedWeight(fmt, n, k, 1, 64, *(arr.get(f) for f in fields), 32))
                if copies[0].nbytes() * len(copies) >= (1 << 30):
                    break
            x = torch.from_numpy(synth.acts_bf16((m, k), 701, m, k).view(np.int16)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            us = timed(lambda i: wq.wq_gemm(x, copies[i % len(copies)], y=y), len(copies))
            row[name] = {"us": round(us, 2), "GB/s": round(copies[0].nbytes() / (us * 1e-6) / 1e9, 1)}
            del copies
        row["pages_h20_ms"] = {"wint2_standard": ms_w2, "ccq": ms_ccq}
        gemv[f"{k}x{n}_m{m}"] = row

    grouped = {}
    E, topk = 256, 8
    for fmt, name, group in ((wq.FMT_INT8, "w8a16", 0), (wq.FMT_INT4, "w4a16", 64),
                             (wq.FMT_CCQ2, "w2a16_ccq", 64)):
        g = synth.random_packed_device(fmt, E, 512, 7168, 7101, group=group)
        u = synth.random_packed_device(fmt, E, 512, 7168, 7102, group=group)
        dn = synth.random_packed_device(fmt, E, 7168, 512, 7103, group=group)
        gw = wq.PackedWeight(fmt, 512, 7168, E, group, *(g.get(f) for f in fields), 32)
        uw = wq.PackedWeight(fmt, 512, 7168, E, group, *(u.get(f) for f in fields), 32)
        dw = wq.PackedWeight(fmt, 7168, 512, E, group, *(dn.get(f) for f in fields), 32)
        per_expert_gu = (gw.nbytes() + uw.nbytes()) // E
        per_expert_dn = dw.nbytes() // E
        for m in (1, 4, 16, 64):
            x = torch.from_numpy(synth.acts_bf16((m, 7168), 702, m).view(np.int16)).to(dev)
            routes = []
            for r in range(64):
                ids, _ = synth.routing_uniform(m, topk, E, 703, m, r)
                off, pairs = wq.wq_moe_route(torch.from_numpy(ids).to(dev), E)
                routes.append((off, pairs, len(np.unique(ids))))
            h = torch.empty((m * topk, 512), dtype=torch.bfloat16, device=dev)
            d = torch.empty((m * topk, 7168), dtype=torch.float32, device=dev)
            reps = len(routes)
            us_gu = timed(lambda i: wq.wq_moe_gate_up(x, routes[i % 64][0], routes[i % 64][1], topk, gw, uw, h=h), reps)
            us_dn = timed(lambda i: wq.wq_moe_down(h, m, topk, routes[i % 64][0], routes[i % 64][1], dw, d=d), reps)
            touched = float(np.mean([r[2] for r in routes]))
            for (o, i_, us, per) in ((1024, 7168, us_gu, per_expert_gu), (7168, 512, us_dn, per_expert_dn)):
                key = f"256x{o}x{i_}_m{m}"
                grouped.setdefault(key, {})[name] = {"us": round(us, 2),
                                                     "GB/s": round(touched * per / (us * 1e-6) / 1e9, 1)}
                grouped[key]["pages_h20_ms"] = dict(zip(("w8a16", "w4a16", "w2a16_ccq"),
                                                        PAGES_GROUPED_MS[(o, i_, m)]))
                grouped[key]["experts_touched"] = round(touched, 1)
        del gw, uw, dw
        torch.cuda.empty_cache()
    for key, row in list(gemv.items()) + list(grouped.items()):
        log(key, json.dumps(row))
    out = {"metric": "latency of the pages' operator shapes (us)", "value": gemv["4096x4096_m1"]["ccq"]["us"],
           "unit": "us", "n_gpus": 1, "steps": args.steps, "higher_is_better": False, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": "pages_shapes"}, "gemv": gemv, "grouped_gemm": grouped,
           "note": "us per call from HIP-graph replay (no host launch cost); pages_h20_ms are the "
                   "pages' own H20 timings, context only"}
    print(json.dumps(out), flush=True)


FP64_PEAK_TFLOPS = 78.6  # MI355X vector fp64


def ccq_encode(args):
    """The CCQ (6,4,3) code-cluster encoder (wq_quantize_ccq, refine on) on the gate tensor of
    one MoE layer: 64 experts x 3584 x 8192 fp32 weights ~ N(0, 0.02) drawn on the GPU.  Rate in
    weights/s; roofline against the fp64 vector peak with about 5,050 fp64 operations per
    4-weight vector (the 960 of the trellis search and 4,096 of the 256-candidate re-pick)."""
    import numpy as np
    import torch

    import weight_only_bit_amd as wq

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    E, n, k = 64, 3584, 8192
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    w = torch.randn((E, n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02
    for _ in range(max(args.warmup, 1)):
        wq.wq_quantize_ccq(w)
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(args.steps):
        wq.wq_quantize_ccq(w)
    en.record()
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / args.steps
    weights = E * n * k
    flops = weights / 4 * (960 + 4096)
    tf = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        rows = 256
        sample = w[0, :rows].cpu().numpy()
        t1 = time.perf_counter()
        oracle.quantize(sample, oracle.CCQ, refine=True)
        dt = time.perf_counter() - t1
        cpu = {"value": round(rows * k / dt / 1e6, 3), "unit": "M weights/s",
               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "cpu_model": cpu_model(),
            "kind": "oracle",
               "sample": f"{rows} rows x {k} of expert 0, refine on, {dt:.1f} s"}
    log(f"encode {ms:.1f} ms for {weights / 1e9:.2f} G weights ({weights / (ms * 1e-3) / 1e9:.1f} G weights/s), "
        f"{tf:.1f} fp64 TFLOP/s")
    out = {"metric": "CCQ encode rate (weights/s)", "value": round(weights / (ms * 1e-3), 1),
           "unit": "weights/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 3), "higher_is_better": True, "dtype": "f64", "data": "synthetic",
           "config": {"workload": "ccq_encode", "experts": E, "rows": n, "k": k, "refine": True},
           "roofline": {"kernel": "ccq_encode_kernel<true>", "bound": "alu", "achieved": round(tf, 2),
                        "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / FP64_PEAK_TFLOPS, 4),
                        "traffic": None, "algorithmic_flops_per_launch": flops},
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def copy_calibration(args):
    """A plain device-to-device copy of exactly 1 GiB (one dispatch per step): the reference
    for scaling the FETCH_SIZE / WRITE_SIZE hardware counters to bytes."""
    import torch

    torch.cuda.set_device(0)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(max(args.steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy_calibration", "bytes_read": n, "bytes_written": n,
                      "copies": max(args.steps, 1)}), flush=True)


def hbm_achievable(args):
    """Context for the HBM fractions: what plain library kernels (torch) reach on this GPU --
    a read-only reduction over 4 GiB of bf16 and a 2 GiB device-to-device copy, timed with
    events over repeated calls.  Not part of the path."""
    import torch

    torch.cuda.set_device(0)
    out = {"workload": "hbm_achievable", "unit": "GB/s"}
    x = torch.ones(2 << 30, dtype=torch.bfloat16, device="cuda:0")  # 4 GiB
    src = torch.ones(2 << 30, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for name, fn, nbytes in (("read_reduce", lambda: x.sum(dtype=torch.float32), x.numel() * 2),
                             ("copy", lambda: dst.copy_(src), 2 * src.numel())):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps, 5)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["hbm_peak"] = HBM_PEAK_GBS
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
