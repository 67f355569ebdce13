"""Benchmark of the sync-free MoE expert MLP step on one MI355X.

Workload: the DeepSeek-V3-like one-GPU expert share -- 32 experts, 16384
routed rows with Zipf(1.1) counts (device-resident), hidden 7168, expert
intermediate 2048, bf16 weights and activations, fp32 accumulation.  One step
is the whole hot path:

    FC1 + SwiGLU  (GroupGemm + Activation, packed W1, saves the pre-activation)
    FC2           (GroupGemm, W2 [E][I][H])
    dgrad + dSwiGLU (GroupGemm + dActivation: dY2 . W2^T, reads the pre-activation)
    dX            (GroupGemm: d(gate|up) . W1^T through the packed W1)

Inputs are synthetic and seeded (workloads.py) and already resident in HBM
when the timed region starts.  `value` is the step's algorithmic TFLOP/s
(sum over experts of 2 m_e K N for the four GEMMs) divided by the measured
step time.  The dominant kernel (FC1) is also timed on its own with HIP events
on the launch stream, for the roofline entry.  The CPU oracle is timed on a
the whole step (every routed row, float64) for `cpu_baseline`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baselines", action="store_true", help="skip the unfused B1 timing")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads (tiny, GPT-OSS-like, MXFP8) and B2")
    ap.add_argument("--traffic", type=str,
                    default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                         "fc1_glu_dsv3_traffic.json"),
                    help="JSON with HBM bytes per FC1 launch measured by rocprofv3 counters "
                         "(used only while the kernel source still matches its recorded hash)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (a known-size "
                         "reference for the HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import workloads as W
    import grouped_gemm_glu_amd as G

    torch.cuda.set_device(0)
    G.moe_init(0)
    dev = "cuda"

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    t0 = time.time()
    d = W.dsv3(with_w2=True)
    dy2_h = W.dsv3_dy2()
    counts_h = d["counts"]
    E, M, H, I = d["E"], d["M"], d["H"], d["I"]
    log(f"inputs generated in {time.time() - t0:.1f}s; counts max {counts_h.max()} min {counts_h.min()}")

    x = up(d["x"])
    w1 = up(d["w1"])
    w2 = up(d["w2"])
    dy2 = up(dy2_h)
    counts = torch.from_numpy(counts_h.astype(np.int32)).to(dev)
    # offline weight preparation (not timed): the gate/up-repacked W1 for FC1 and
    # tile-blocked copies of W1 (dX) and W2 (FC2, dgrad)
    def packed(n_bytes):
        return torch.empty(n_bytes // 2, dtype=torch.int16, device=dev)
    w1p = packed(G.moe_packed_w1_bytes(E, H, I))
    G.moe_repack_gate_up(w1, E, H, I, w1p)
    w1x = packed(G.moe_packed_weight_bytes(E, H, 2 * I))
    G.moe_pack_weight(w1, E, H, 2 * I, G.B_NK, w1x)
    w2f = packed(G.moe_packed_weight_bytes(E, H, I))
    G.moe_pack_weight(w2, E, H, I, G.B_KN, w2f)
    w2d = packed(G.moe_packed_weight_bytes(E, I, H))
    G.moe_pack_weight(w2, E, I, H, G.B_NK, w2d)
    y = torch.empty((M, I), dtype=torch.int16, device=dev)
    pre = torch.empty((M, 2 * I), dtype=torch.int16, device=dev)
    out2 = torch.empty((M, H), dtype=torch.int16, device=dev)
    dgu = torch.empty((M, 2 * I), dtype=torch.int16, device=dev)
    dx = torch.empty((M, H), dtype=torch.int16, device=dev)
    grp = G.groups(counts, M)
    ep = G.epilogue("swiglu")
    op_y = G.operand(y)
    op_w2 = G.operand(w2f, layout=G.B_PACKED)
    op_w2d = G.operand(w2d, layout=G.B_PACKED)
    op_dgu = G.operand(dgu)
    op_w1x = G.operand(w1x, layout=G.B_PACKED)
    torch.cuda.synchronize()

    def fc1():
        G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, y, pre)

    def fc2():
        G.moe_group_gemm_quant(op_y, op_w2, H, I, grp, out2)

    def dglu():
        G.moe_group_gemm_dglu_bwd(dy2, op_w2d, H, I, grp, pre, ep, dgu)

    def dxk():
        G.moe_group_gemm_quant(op_dgu, op_w1x, H, 2 * I, grp, dx)

    def step():
        fc1()
        fc2()
        dglu()
        dxk()

    flop_row = 2 * H * 2 * I + 2 * I * H + 2 * H * I + 2 * 2 * I * H
    step_flops = float(M) * flop_row
    fc1_flops = 2.0 * M * H * 2 * I

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K eager steps; HIP events bracket every FC1 launch on
    # the launch stream (torch's current stream, which the binding uses)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        fc1()
        evs[i][1].record(stream)
        fc2()
        dglu()
        dxk()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    fc1_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # ---- per-kernel times (events around each kernel alone), for the record
    def time_kernel(fn, n=10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    kern_ms = {"fc1_glu": time_kernel(fc1), "fc2": time_kernel(fc2),
               "dgrad_dglu": time_kernel(dglu), "dx": time_kernel(dxk)}
    # weight gradients (K-grouped, fp32 out)
    dW1 = torch.empty((E, H, 2 * I), dtype=torch.float32, device=dev)
    dW2 = torch.empty((E, I, H), dtype=torch.float32, device=dev)

    def dw1():
        G.moe_group_gemm_wgrad(x, dgu, H, 2 * I, grp, dW1)

    def dw2():
        G.moe_group_gemm_wgrad(y, dy2, I, H, grp, dW2)

    kern_ms["dw1"] = time_kernel(dw1)
    kern_ms["dw2"] = time_kernel(dw2)

    def train_step():
        step()
        dw1()
        dw2()

    ts_ms = _ev_ms(torch, train_step, args.steps)
    train = {"ms": round(ts_ms, 4),
             "tflops": round((step_flops + 2.0 * M * H * 2 * I + 2.0 * M * I * H) / ts_ms / 1e9, 1),
             "what": "the step plus the weight gradients dW1 = Xg^T dgu [E][H][2I] and "
                     "dW2 = y^T dY2 [E][I][H] (K-grouped, fp32 out)"}
    del dW1, dW2

    # ---- the same step as one hipGraph replay (no host sync inside)
    graph_ms = None
    graph_pair = None
    try:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / args.steps
        # the same comparison interleaved (same clock and thermal state)
        pg = paired_ms(torch, {"eager": step, "graph": g.replay})
        graph_pair = {"eager_ms": round(pg["eager"], 4), "graph_ms": round(pg["graph"], 4),
                      "timing": "interleaved, best of 3 rounds of 10"}
    except Exception as exc:  # reported, never hides the eager number
        log(f"graph capture failed: {exc!r}")

    # ---- B1: the unfused chain on the same main loop (GEMM -> HBM -> GLU)
    b1 = None
    if not args.no_baselines:
        # same main loop on a tile-blocked W1 in PLAIN column order (N = 2I, K = H),
        # writing the bf16 pre-activation, then the unfused GLU kernel
        w1t_plain = packed(G.moe_packed_weight_bytes(E, 2 * I, H))
        G.moe_pack_weight(w1, E, 2 * I, H, G.B_KN, w1t_plain)
        z = torch.empty((M, 2 * I), dtype=torch.int16, device=dev)
        op_x = G.operand(x)
        op_w1t = G.operand(w1t_plain, layout=G.B_PACKED)

        def b1_chain():
            G.moe_group_gemm_quant(op_x, op_w1t, 2 * I, H, grp, z)
            G.moe_glu_unfused(z, grp, I, ep, y)

        def b1_gemm_only():
            G.moe_group_gemm_quant(op_x, op_w1t, 2 * I, H, grp, z)

        def fc1_no_preact():   # inference, or a backward that recomputes z
            G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, y, None)

        pm = paired_ms(torch, {"fused": fc1, "b1": b1_chain, "fused_y_only": fc1_no_preact,
                               "b1_gemm": b1_gemm_only})
        b1 = {"fc1_fused_ms": round(pm["fused"], 4), "fc1_unfused_ms": round(pm["b1"], 4),
              "fused_speedup": round(pm["b1"] / pm["fused"], 3),
              "fc1_fused_y_only_ms": round(pm["fused_y_only"], 4),
              "fused_y_only_speedup": round(pm["b1"] / pm["fused_y_only"], 3),
              "b1_gemm_ms": round(pm["b1_gemm"], 4),
              "timing": "interleaved, best of 3 rounds of 10"}
        del w1t_plain, z
        # the backward counterpart: dgrad GroupGemm writing dL/dy in bf16, then
        # the unfused dGLU pass (and, with MXFP8 outputs, the standalone
        # quantize/transpose of dgu), against the fused dgrad + dGLU
        gmat = torch.empty((M, I), dtype=torch.int16, device=dev)
        op_dy2 = G.operand(dy2)
        dq = torch.empty((M, 2 * I), dtype=torch.uint8, device=dev)
        ds = torch.empty((M, 2 * I // 32), dtype=torch.uint8, device=dev)
        dcq = torch.empty((2 * I, M), dtype=torch.uint8, device=dev)
        dcs = torch.empty((2 * I, (M + 31) // 32 + E), dtype=torch.uint8, device=dev)
        mx_dgu = G.mx_out(row_q=dq, row_s=ds, col_q=dcq, col_s=dcs)
        # the same copies with the transposed one in the K-tiled layout that the
        # MXFP8 weight gradient reads
        S = G.mx_col_slots(M, E, blocked=True)
        dkq = torch.empty((2 * I, 32 * S), dtype=torch.uint8, device=dev)
        dks = torch.empty((2 * I, S), dtype=torch.uint8, device=dev)
        mx_dgu_k = G.mx_out(row_q=dq, row_s=ds, col_q=dkq, col_s=dks, col_blocked=True)

        def b1_bwd():
            G.moe_group_gemm_quant(op_dy2, op_w2d, I, H, grp, gmat)
            G.moe_dglu_unfused(gmat, pre, grp, I, ep, dgu)

        def b1_bwd_mx():
            b1_bwd()
            G.moe_mxfp8_quantize(dgu, M, 2 * I, grp, mx_dgu)

        def fused_bwd_mx():
            G.moe_group_gemm_dglu_bwd(dy2, op_w2d, H, I, grp, pre, ep, dgu, mx_dgu)

        def b1_bwd_mx_k():
            b1_bwd()
            G.moe_mxfp8_quantize(dgu, M, 2 * I, grp, mx_dgu_k)

        def fused_bwd_mx_k():
            G.moe_group_gemm_dglu_bwd(dy2, op_w2d, H, I, grp, pre, ep, dgu, mx_dgu_k)

        pb = paired_ms(torch, {"fused": dglu, "b1": b1_bwd, "fused_mx": fused_bwd_mx,
                               "b1_mx": b1_bwd_mx, "fused_mx_k": fused_bwd_mx_k,
                               "b1_mx_k": b1_bwd_mx_k})
        b1["dgrad_dglu_fused_ms"] = round(pb["fused"], 4)
        b1["dgrad_dglu_unfused_ms"] = round(pb["b1"], 4)
        b1["dgrad_dglu_fused_speedup"] = round(pb["b1"] / pb["fused"], 3)
        b1["dgrad_dglu_mx_fused_ms"] = round(pb["fused_mx"], 4)
        b1["dgrad_dglu_mx_unfused_ms"] = round(pb["b1_mx"], 4)
        b1["dgrad_dglu_mx_fused_speedup"] = round(pb["b1_mx"] / pb["fused_mx"], 3)
        b1["dgrad_dglu_mx_ktiled_fused_ms"] = round(pb["fused_mx_k"], 4)
        b1["dgrad_dglu_mx_ktiled_unfused_ms"] = round(pb["b1_mx_k"], 4)
        b1["dgrad_dglu_mx_ktiled_fused_speedup"] = round(pb["b1_mx_k"] / pb["fused_mx_k"], 3)
        del gmat, dq, ds, dcq, dcs, dkq, dks

    fc1_tflops = fc1_flops / (fc1_ms * 1e-3) / 1e12
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    extra = None
    if not args.no_extra:
        extra = {"training_step_with_wgrads": train}
        log("secondary: B2 traditional path")
        extra["b2_traditional_fc1"] = bench_b2(G, torch, time_kernel, x, counts, counts_h, w1, E,
                                               M, H, I, ep, y, kern_ms["fc1_glu"])
        log("secondary: vendor GEMM libraries on the same FC1")
        extra["vendor_fc1"] = bench_vendor(torch, x, w1, counts_h, E, M, H, I, kern_ms["fc1_glu"])
        log("secondary: CU margin with a concurrent copy")
        extra["cu_margin_overlap"] = bench_overlap(G, torch, x, grp, w1p, H, I, ep, y, pre)
        log("secondary: amax outputs and parameter gradients")
        extra["epilogue_extras"] = bench_amax(G, torch, x, grp, w1p, E, H, I, y, pre, dy2, op_w2d,
                                               dgu)
        log("secondary: MXFP8 forward")
        extra["mxfp8_dsv3_share"] = bench_mxfp8(G, torch, time_kernel, w1, w1p, w2, counts,
                                                counts_h, E, M, H, I, kern_ms)
        del w1x, w2d
        log("secondary: GPT-OSS-like routed FC1")
        extra["gptoss_fc1"] = bench_gptoss(G, torch, time_kernel)
        log("secondary: tiny routed FC1")
        extra["tiny_route_fc1"] = bench_tiny(G, torch)

    traffic = read_traffic(args.traffic)

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 2
        src_c = torch.empty(n, dtype=torch.int16, device=dev).fill_(1)
        dst_c = torch.empty_like(src_c)
        torch.cuda.synchronize()
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.calibrate_copy_mib} MiB device copies")
        del src_c, dst_c

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(d, dy2_h)

    rec = {
        "metric": "fused MoE GroupGEMM+GLU TFLOP/s fwd & bwd and % MFMA peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Zipf(1.1) expert counts, N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "DeepSeek-V3-like one-GPU expert share: FC1+SwiGLU, FC2, "
                               "dgrad+dSwiGLU, dX",
                   "experts": E, "routed_rows": M, "hidden": H, "intermediate": I,
                   "parallelism": "single GPU"},
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": "moe_group_gemm_glu_fwd (FC1 + SwiGLU)",
                     "achieved": round(fc1_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fc1_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "avg_launch_ms": round(fc1_ms, 4),
                     "algorithmic_flops_per_launch": fc1_flops},
        "kernel_ms": {k: round(v, 4) for k, v in kern_ms.items()},
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "graph_vs_eager": graph_pair,
        "unfused_b1": b1,
        "secondary": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def paired_ms(torch, fns, rounds=3, n=10):
    """Times several chains interleaved (round robin, `rounds` times, `n`
    launches each) and keeps each one's best round, so a fused kernel and its
    unfused baseline see the same clock and thermal state."""
    best = {k: float("inf") for k in fns}
    for _ in range(rounds):
        for k, fn in fns.items():
            best[k] = min(best[k], _ev_ms(torch, fn, n))
    return best


def _ev_ms(torch, fn, n=5):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def bench_b2(G, torch, time_kernel, x, counts, counts_h, w1, E, M, H, I, ep, y, fused_ms):
    """B2, the traditional path the sync-free kernels replace: read the group
    sizes back to the host (a synchronisation), then one single-group GEMM per
    expert over 4 streams (plain-order W1, bf16 pre-activation to HBM), then
    the GLU pass.  Timed wall-clock around the whole chain."""
    dev = x.device
    w1t = torch.empty(G.moe_packed_weight_bytes(E, 2 * I, H) // 2, dtype=torch.int16, device=dev)
    G.moe_pack_weight(w1, E, 2 * I, H, G.B_KN, w1t)
    per_e = G.moe_packed_weight_bytes(1, 2 * I, H) // 2
    z = torch.empty((M, 2 * I), dtype=torch.int16, device=dev)
    streams = [torch.cuda.Stream() for _ in range(4)]
    grp = G.groups(counts, M)
    main = torch.cuda.current_stream()

    def chain():
        c = counts.cpu().numpy()                     # host readback: the sync
        off = np.concatenate([[0], np.cumsum(c)])
        for s in streams:
            s.wait_stream(main)
        for e in range(E):
            m = int(c[e])
            if m == 0:
                continue
            s = streams[e % 4]
            G.moe_group_gemm_quant(G.operand(x[off[e]:off[e + 1]]),
                                   G.operand(w1t[e * per_e:(e + 1) * per_e], layout=G.B_PACKED),
                                   2 * I, H, G.groups(counts[e:e + 1], m), z[off[e]:off[e + 1]],
                                   stream=s)
        for s in streams:
            main.wait_stream(s)
        G.moe_glu_unfused(z, grp, I, ep, y)

    chain()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(5):
        chain()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) * 1e3 / 5
    del w1t, z
    return {"ms": round(ms, 4), "fused_speedup": round(ms / fused_ms, 3),
            "what": "host readback of counts + 32 per-expert GEMM launches on 4 streams + GLU pass"}


def bench_vendor(torch, x, w1, counts_h, E, M, H, I, fused_ms):
    """Context for the FC1 kernel: the ROCm GEMM libraries behind torch on the
    same FC1 GEMM (bf16 in, fp32 accumulation, bf16 pre-activation out, no
    activation), with both operands K-contiguous: one hipBLASLt GEMM per
    expert (the counts taken as known on the host: no readback charged),
    torch._grouped_mm over the group offsets, and one dense GEMM of the same FLOPs (all rows against a
    single expert's weights, whose panels the last-level cache holds) as the
    ceiling that the library reaches on this chip for this shape."""
    dev = x.device
    xb = x.view(torch.bfloat16)
    wkn = w1.view(torch.bfloat16).view(E, H, 2 * I)            # [E][K][N]
    wnk = wkn.transpose(1, 2).contiguous()                      # [E][N][K]
    out = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    off = np.concatenate([[0], np.cumsum(counts_h)]).astype(np.int64)
    flops = 2.0 * M * H * 2 * I

    def per_expert():
        for e in range(E):
            if counts_h[e]:
                torch.mm(xb[off[e]:off[e + 1]], wnk[e].t(), out=out[off[e]:off[e + 1]])

    def dense():
        torch.mm(xb, wnk[0].t(), out=out)

    res = {}
    for name, fn in (("per_expert_hipblaslt", per_expert), ("dense_same_flops", dense)):
        ms = min(_ev_ms(torch, fn, 10) for _ in range(3))
        res[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                     "fused_fc1_speedup": round(ms / fused_ms, 3)}
    try:
        offs = torch.from_numpy(off[1:].astype(np.int32)).to(dev)
        torch._grouped_mm(xb, wkn, offs=offs)
        ms = min(_ev_ms(torch, lambda: torch._grouped_mm(xb, wkn, offs=offs), 10) for _ in range(3))
        res["torch_grouped_mm"] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                                   "fused_fc1_speedup": round(ms / fused_ms, 3)}
    except Exception as exc:   # not every torch build has it on ROCm
        res["torch_grouped_mm"] = {"error": repr(exc)[:200]}
    res["what"] = ("FC1 GEMM only (no SwiGLU), bf16, library kernels chosen by torch; "
                   "fused_fc1_speedup = library ms / this library's FC1 + SwiGLU ms")
    del wnk, out
    return res


def bench_overlap(G, torch, x, grp, w1p, H, I, ep, y, pre, margin=32, copy_mib=2048):
    """FC1 leaving `margin` CUs free while a bandwidth-bound copy runs on a
    second stream (both at default priority), against each alone and against
    the same pair with no margin: the knob the pages use to let communication
    kernels run beside the GEMMs."""
    dev = x.device
    n = copy_mib * (1 << 20) // 2
    src = torch.empty(n, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def fc1(m):
        G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, y, pre, cu_margin=m)

    def copy():
        dst.copy_(src)

    def both(m):
        side.wait_stream(main)
        fc1(m)
        with torch.cuda.stream(side):
            copy()
        main.wait_stream(side)

    def wall(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / reps

    res = {"fc1_ms": round(wall(lambda: fc1(0)), 4),
           f"fc1_margin{margin}_ms": round(wall(lambda: fc1(margin)), 4),
           "copy_ms": round(wall(copy), 4),
           "fc1_and_copy_ms": round(wall(lambda: both(0)), 4),
           f"fc1_margin{margin}_and_copy_ms": round(wall(lambda: both(margin)), 4),
           "copy_gib": copy_mib / 1024}
    res["copy_gbs_alone"] = round(2 * copy_mib * (1 << 20) / res["copy_ms"] / 1e6, 1)
    del src, dst
    return res


def bench_amax(G, torch, x, grp, w1p, E, H, I, y, pre, dy2, op_w2d, dgu):
    """FC1 with the per-tensor amax of y, and dgrad + dSwiGLU with the amax of
    the 16-row Hadamard rotation of dgu^T, each beside the same kernel without
    it (interleaved timing)."""
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    db = torch.zeros((E, 2 * I), dtype=torch.float32, device="cuda")
    drs = torch.zeros(y.shape[0], dtype=torch.float32, device="cuda")
    ep0 = G.epilogue("swiglu")
    ep1 = G.epilogue("swiglu", amax_out=amax, rht_signs=0x5A3C)
    ep2 = G.epilogue("swiglu", dbias_out=db, drow_scale_out=drs)
    ep3 = G.epilogue("swiglu", dbias_out=db)
    ep4 = G.epilogue("swiglu", drow_scale_out=drs)

    def fc1(ep):
        return lambda: G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, y, pre)

    def dglu(ep):
        return lambda: G.moe_group_gemm_dglu_bwd(dy2, op_w2d, H, I, grp, pre, ep, dgu)

    pm = paired_ms(torch, {"fc1": fc1(ep0), "fc1_amax": fc1(ep1),
                           "dglu": dglu(ep0), "dglu_rht_amax": dglu(ep1),
                           "dglu_param_grads": dglu(ep2), "dglu_dbias": dglu(ep3),
                           "dglu_drow_scale": dglu(ep4)})
    return {k: round(v, 4) for k, v in pm.items()} | {
        "what": "FC1 + SwiGLU with max|y|; dgrad + dSwiGLU with the amax of H16 S / 4 over "
                "16-row runs of dgu^T, and with d(bias) and d(row_scale) added; against the "
                "same kernels without them",
        "timing": "interleaved, best of 3 rounds of 10"}


def bench_mxfp8(G, torch, time_kernel, w1, w1p, w2, counts, counts_h, E, M, H, I, kern_ms):
    """The MXFP8 forward on the same expert share with student-t activations:
    FC1 + SwiGLU writing the pre-activation and the row-wise and transposed
    MXFP8 copies of y in its epilogue, then FC2 as MXFP8 x MXFP8 on the
    block-scaled MFMA with W2 quantised offline along I.  B1 here: plain GEMM
    -> GLU pass -> standalone MXFP8 quantize/transpose."""
    import workloads as W
    dev = w1.device
    x = torch.from_numpy(W.student_t_rows_bf16(W.DSV3_MX["seed"], M, H).view(np.int16)).to(dev)
    grp = G.groups(counts, M)
    ep = G.epilogue("swiglu")
    pre = torch.empty((M, 2 * I), dtype=torch.int16, device=dev)
    y = torch.empty((M, I), dtype=torch.int16, device=dev)
    row_q = torch.empty((M, I), dtype=torch.uint8, device=dev)
    row_s = torch.empty((M, I // 32), dtype=torch.uint8, device=dev)
    col_q = torch.empty((I, M), dtype=torch.uint8, device=dev)
    col_s = torch.empty((I, (M + 31) // 32 + E), dtype=torch.uint8, device=dev)
    mx = G.mx_out(row_q=row_q, row_s=row_s, col_q=col_q, col_s=col_s)
    w2q = torch.empty(G.moe_packed_mx_weight_bytes(E, H, I), dtype=torch.uint8, device=dev)
    w2s = torch.empty(G.moe_packed_mx_scale_bytes(E, H, I), dtype=torch.uint8, device=dev)
    G.moe_pack_weight_mx(w2, E, H, I, G.B_KN, w2q, w2s)
    out2 = torch.empty((M, H), dtype=torch.int16, device=dev)
    op_a = G.operand(row_q, dtype=G.DT_MXFP8, scales=row_s)
    op_b = G.operand(w2q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=w2s)

    def fc1_mx():
        G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, None, pre, mx)

    def fc2_mx():
        G.moe_group_gemm_quant(op_a, op_b, H, I, grp, out2)

    fc2_ms = time_kernel(fc2_mx)
    # B1 for the MXFP8 forward
    w1t = torch.empty(G.moe_packed_weight_bytes(E, 2 * I, H) // 2, dtype=torch.int16, device=dev)
    G.moe_pack_weight(w1, E, 2 * I, H, G.B_KN, w1t)
    z = torch.empty((M, 2 * I), dtype=torch.int16, device=dev)
    op_x, op_w1t = G.operand(x), G.operand(w1t, layout=G.B_PACKED)

    def b1():
        G.moe_group_gemm_quant(op_x, op_w1t, 2 * I, H, grp, z)
        G.moe_glu_unfused(z, grp, I, ep, y)
        G.moe_mxfp8_quantize(y, M, I, grp, mx)

    # the transposed copy in the K-tiled layout the MXFP8 weight gradient reads
    Sk = G.mx_col_slots(M, E, blocked=True)
    col_qk = torch.empty((I, 32 * Sk), dtype=torch.uint8, device=dev)
    col_sk = torch.empty((I, Sk), dtype=torch.uint8, device=dev)
    mx_k = G.mx_out(row_q=row_q, row_s=row_s, col_q=col_qk, col_s=col_sk, col_blocked=True)

    def fc1_mx_k():
        G.moe_group_gemm_glu_fwd(x, grp, w1p, H, I, ep, None, pre, mx_k)

    pm = paired_ms(torch, {"fused": fc1_mx, "b1": b1, "fused_k": fc1_mx_k})
    fc1_ms, b1_ms = pm["fused"], pm["b1"]
    del col_qk, col_sk
    # the MXFP8 recipe's FC1 itself on the block-scaled MFMA: rows of x
    # quantised on the GPU, gate/up-repacked MXFP8 W1
    xq = torch.empty((M, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    G.moe_mxfp8_quantize(x, M, H, None, G.mx_out(row_q=xq, row_s=xs))
    w1q = torch.empty(G.moe_packed_mx_weight_bytes(E, 2 * I, H), dtype=torch.uint8, device=dev)
    w1s = torch.empty(G.moe_packed_mx_scale_bytes(E, 2 * I, H), dtype=torch.uint8, device=dev)
    G.moe_repack_gate_up_mx(w1, E, H, I, w1q, w1s)
    op_xq = G.operand(xq, dtype=G.DT_MXFP8, scales=xs)
    op_w1q = G.operand(w1q, dtype=G.DT_MXFP8, layout=G.B_PACKED, scales=w1s)

    def fc1_mxin():
        G.moe_group_gemm_glu_fwd_mx(op_xq, grp, op_w1q, H, I, ep, None, pre, mx)

    fc1_mxin_ms = time_kernel(fc1_mxin)
    del xq, xs, w1q, w1s
    # MXFP8 weight gradient dW1 = Xg^T dgu from K-tiled transposed copies
    # (e4m3 for Xg, e5m2 for the gradient; the FC1 pre-activation of this run
    # stands in for dgu, which has its shape), fp32 out; the two column
    # quantisations that write the copies are timed with it
    S = G.mx_col_slots(M, E, blocked=True)
    xcq = torch.empty((H, 32 * S), dtype=torch.uint8, device=dev)
    xcs = torch.empty((H, S), dtype=torch.uint8, device=dev)
    gcq = torch.empty((2 * I, 32 * S), dtype=torch.uint8, device=dev)
    gcs = torch.empty((2 * I, S), dtype=torch.uint8, device=dev)
    dw1 = torch.empty((E, H, 2 * I), dtype=torch.float32, device=dev)
    op_xc = G.operand(xcq, dtype=G.DT_MXFP8, scales=xcs)
    op_gc = G.operand(gcq, dtype=G.DT_MXFP8_E5M2, scales=gcs)

    def quant_cols():
        G.moe_mxfp8_quantize(x, M, H, grp, G.mx_out(col_q=xcq, col_s=xcs, col_blocked=True))
        G.moe_mxfp8_quantize(pre, M, 2 * I, grp, G.mx_out(col_q=gcq, col_s=gcs, e5m2=True,
                                                          col_blocked=True))

    def wgrad_mx():
        G.moe_group_gemm_wgrad_mx(op_xc, op_gc, H, 2 * I, grp, dw1)

    quant_cols()
    qcols_ms = time_kernel(quant_cols)
    wgrad_mx_ms = time_kernel(wgrad_mx)
    del xcq, xcs, gcq, gcs, dw1
    fc2_flops = 2.0 * M * I * H
    fc1_flops = 2.0 * M * H * 2 * I
    del x, w1t, z, w2q, w2s
    return {"fc1_swiglu_mx_ms": round(fc1_ms, 4),
            "fc1_swiglu_mx_ktiled_cols_ms": round(pm["fused_k"], 4),
            "fc1_tflops": round(fc1_flops / fc1_ms / 1e9, 1),
            "fc1_b1_unfused_ms": round(b1_ms, 4), "fc1_fused_speedup": round(b1_ms / fc1_ms, 3),
            "fc2_mxfp8_ms": round(fc2_ms, 4), "fc2_tflops": round(fc2_flops / fc2_ms / 1e9, 1),
            "fc2_frac_fp8_peak": round(fc2_flops / fc2_ms / 1e9 / 5000.0, 4),
            "fc2_bf16_ms": round(kern_ms["fc2"], 4),
            "fc1_mxfp8_inputs_ms": round(fc1_mxin_ms, 4),
            "fc1_mxfp8_inputs_tflops": round(fc1_flops / fc1_mxin_ms / 1e9, 1),
            "fc1_mxfp8_inputs_frac_fp8_peak": round(fc1_flops / fc1_mxin_ms / 1e9 / 5000.0, 4),
            "dw1_mxfp8_ms": round(wgrad_mx_ms, 4),
            "dw1_mxfp8_tflops": round(fc1_flops / wgrad_mx_ms / 1e9, 1),
            "dw1_mxfp8_frac_fp8_peak": round(fc1_flops / wgrad_mx_ms / 1e9 / 5000.0, 4),
            "dw1_mxfp8_hbm_bound_ms": round(E * H * 2 * I * 4 / PEAK_HBM_GBS / 1e6, 4),
            "k_tiled_copies_x_and_dgu_ms": round(qcols_ms, 4),
            "activations": "student-t(3) x 0.5, bf16"}


def bench_gptoss(G, torch, time_kernel):
    """GPT-OSS-like routed FC1: 8192 tokens, 32 experts, top-4, hidden and
    intermediate 2880, SwiGLU with alpha 1.702, clamp 7, bias; routing and
    grouping on the device, then the fused FC1 (vs GEMM -> GLU pass)."""
    import workloads as W
    d = W.gptoss(with_weights=True)
    T, E, k, H, I = d["T"], d["E"], d["k"], d["H"], d["I"]
    dev = "cuda"
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev)
    logits = torch.from_numpy(d["logits"]).to(dev)
    x, w1, b1 = up(d["x"]), up(d["w1"]), up(d["b1"])
    TK = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    dst = torch.empty((T, k), dtype=torch.int32, device=dev)
    src = torch.empty(TK, dtype=torch.int32, device=dev)
    xg = torch.empty((TK, H), dtype=torch.int16, device=dev)
    w1p = torch.empty(G.moe_packed_w1_bytes(E, H, I) // 2, dtype=torch.int16, device=dev)
    G.moe_repack_gate_up(w1, E, H, I, w1p)
    y = torch.empty((TK, I), dtype=torch.int16, device=dev)
    pre = torch.empty((TK, 2 * I), dtype=torch.int16, device=dev)
    lim = d["limit"]
    ep = G.epilogue("swiglu", alpha=d["alpha"], gate_lo=-lim, gate_hi=lim, up_lo=-lim, up_hi=lim,
                    bias=b1)
    grp = G.groups(cnt, TK)

    def route():
        G.moe_route_group(logits, None, T, E, k, ids, cnt, off, dst, src, x, H, xg)

    def fc1():
        G.moe_group_gemm_glu_fwd(xg, grp, w1p, H, I, ep, y, pre)

    route_ms = time_kernel(route)
    w1t = torch.empty(G.moe_packed_weight_bytes(E, 2 * I, H) // 2, dtype=torch.int16, device=dev)
    G.moe_pack_weight(w1, E, 2 * I, H, G.B_KN, w1t)
    z = torch.empty((TK, 2 * I), dtype=torch.int16, device=dev)
    op_x, op_w1t = G.operand(xg), G.operand(w1t, layout=G.B_PACKED)

    def b1c():
        G.moe_group_gemm_quant(op_x, op_w1t, 2 * I, H, grp, z)
        G.moe_glu_unfused(z, grp, I, ep, y)

    pm = paired_ms(torch, {"fused": fc1, "b1": b1c})
    fc1_ms, b1_ms = pm["fused"], pm["b1"]
    flops = 2.0 * TK * H * 2 * I
    del x, w1, w1p, w1t, z, xg, y, pre
    return {"route_group_ms": round(route_ms, 4), "fc1_ms": round(fc1_ms, 4),
            "fc1_tflops": round(flops / fc1_ms / 1e9, 1),
            "fc1_b1_unfused_ms": round(b1_ms, 4), "fc1_fused_speedup": round(b1_ms / fc1_ms, 3),
            "tokens": T, "experts": E, "top_k": k, "hidden": H, "intermediate": I}


def bench_tiny(G, torch):
    """The tiny routed case (512 tokens, 4 experts, top-2, hidden 256,
    intermediate 512): launch-bound, so reported as microseconds per forward
    (route + fused FC1) against B1 (route + GEMM + GLU pass), eager and as one
    graph replay, and the FC1 step alone (one fused launch against GEMM + GLU
    pass) as a graph replay."""
    import workloads as W
    d = W.tiny()
    T, E, k, H, I = d["T"], d["E"], d["k"], d["H"], d["I"]
    dev = "cuda"
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev)
    logits = torch.from_numpy(d["logits"]).to(dev)
    x, w1 = up(d["x"]), up(d["w1"])
    TK = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    dst = torch.empty((T, k), dtype=torch.int32, device=dev)
    src = torch.empty(TK, dtype=torch.int32, device=dev)
    xg = torch.empty((TK, H), dtype=torch.int16, device=dev)
    w1p = torch.empty(G.moe_packed_w1_bytes(E, H, I) // 2, dtype=torch.int16, device=dev)
    G.moe_repack_gate_up(w1, E, H, I, w1p)
    w1t = torch.empty(G.moe_packed_weight_bytes(E, 2 * I, H) // 2, dtype=torch.int16, device=dev)
    G.moe_pack_weight(w1, E, 2 * I, H, G.B_KN, w1t)
    y = torch.empty((TK, I), dtype=torch.int16, device=dev)
    z = torch.empty((TK, 2 * I), dtype=torch.int16, device=dev)
    grp = G.groups(cnt, TK)
    ep = G.epilogue("swiglu")
    op_x, op_w1t = G.operand(xg), G.operand(w1t, layout=G.B_PACKED)

    def fused():
        G.moe_route_group(logits, None, T, E, k, ids, cnt, off, dst, src, x, H, xg)
        G.moe_group_gemm_glu_fwd(xg, grp, w1p, H, I, ep, y)

    def b1():
        G.moe_route_group(logits, None, T, E, k, ids, cnt, off, dst, src, x, H, xg)
        G.moe_group_gemm_quant(op_x, op_w1t, 2 * I, H, grp, z)
        G.moe_glu_unfused(z, grp, I, ep, y)

    # the FC1 step alone on the routed rows: one fused launch vs GEMM -> GLU pass
    fused()
    torch.cuda.synchronize()

    def fc1_only():
        G.moe_group_gemm_glu_fwd(xg, grp, w1p, H, I, ep, y)

    def b1_only():
        G.moe_group_gemm_quant(op_x, op_w1t, 2 * I, H, grp, z)
        G.moe_glu_unfused(z, grp, I, ep, y)

    res = {"fused_us": round(_ev_ms(torch, fused, 50) * 1e3, 2),
           "b1_us": round(_ev_ms(torch, b1, 50) * 1e3, 2)}
    for name, fn in (("fused", fused), ("b1", b1), ("fc1_only_fused", fc1_only),
                     ("fc1_only_b1", b1_only)):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        res[f"{name}_graph_us"] = round(_ev_ms(torch, g.replay, 50) * 1e3, 2)
    res["fused_speedup_graph"] = round(res["b1_graph_us"] / res["fused_graph_us"], 3)
    res["fc1_only_speedup_graph"] = round(res["fc1_only_b1_graph_us"] / res["fc1_only_fused_graph_us"], 3)
    return res


def read_traffic(path):
    """HBM bytes per FC1 launch from the committed counter record, or None when
    the record is missing or the GEMM kernel source changed since it was taken."""
    import hashlib
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    root = os.path.dirname(os.path.abspath(__file__))
    src = os.path.join(root, rec.get("kernel_source", ""))
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()[:16]
    if h != rec.get("source_sha256_16"):
        return None
    return rec.get("fc1_hbm_bytes_per_launch")


def _host_info():
    """CPU model and the BLAS library numpy calls (for the cpu_baseline record)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:   # numpy without the dict form: leave it unknown
        pass
    return model, blas


def cpu_baseline(d, dy2_h, rows_per_expert=None):
    """The oracle, as it stands, on the same step: by default every routed row
    of every expert (the whole workload) through FC1+SwiGLU, FC2,
    dgrad+dSwiGLU and dX, timed on this host's cores.  `value` is the float64
    run (the oracle's arithmetic); the same functions in float32 (BLAS sgemm,
    closer to the GPU's fp32 accumulation) are timed after it as `fp32`.
    About 15-30 s of CPU work in all; rows_per_expert caps each expert's rows."""
    from oracle import moe as O
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))       # BLAS threads actually used
    counts = d["counts"]
    off = np.concatenate([[0], np.cumsum(counts)])
    H, I = d["H"], d["I"]
    cap = int(counts.max()) if rows_per_expert is None else rows_per_expert
    c = np.minimum(counts, cap).astype(np.int64)
    sel = np.concatenate([np.arange(off[e], off[e] + c[e]) for e in range(len(counts))])
    xs, dys = d["x"][sel], dy2_h[sel]
    ep = O.Epilogue()

    def run(dtype):
        t = time.perf_counter()
        pre, y = O.fc1_glu(xs, c, d["w1"], ep, dtype=dtype)
        O.group_gemm(y, c, d["w2"], dtype=dtype)
        dgu = O.dgrad_dglu(dys, c, d["w2"], pre, ep, dtype=dtype)
        O.dx(dgu, c, d["w1"], dtype=dtype)
        return time.perf_counter() - t

    flops = float(c.sum()) * (2 * H * 2 * I + 2 * I * H + 2 * H * I + 2 * 2 * I * H)
    dt = run(np.float64)
    dt32 = run(np.float32)
    model, blas = _host_info()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 2), "dtype": "float64",
            "fp32": {"value": round(flops / dt32 / 1e12, 6), "seconds": round(dt32, 2)},
            "cpu_model": model, "blas": blas,
            "sample": (f"all {int(c.sum())} routed rows of the 32 experts" if rows_per_expert is None
                       else f"first min(m_e, {cap}) rows of each of the 32 experts "
                            f"({int(c.sum())} of {int(counts.sum())} rows)")
                      + " through the full step (FC1+SwiGLU, FC2, dgrad+dSwiGLU, dX)"}

if __name__ == "__main__":
    main()
