"""Throughput of the W4 (NVFP4) + dynamic LoRA linear on one MI355X.

One step = the four projections of one synthetic MiniMax-H3 DiT block at the packed sequence length
S = 37726 (fused QKV 18432x6144 r=384, attention-out 6144x6144 r=128, fused gate/up 32768x6144 r=128,
down 6144x16384 r=128; rank = alpha; strength 1; adapter active), each through h3q_linear: LoRA-down
(+ x * pqs) and the W4 GEMM with the folded LoRA-up and the epilogue. Inputs are synthetic (seeded),
resident in HBM before timing starts.

  metric  effective TFLOP/s = sum over projections of 2 S N K + 2 S r (K + N), per second of wall time;
          the median of 5 loops of K steps each, with the library's per-kernel timing off
  roofline  the main GEMM kernel (MFMA-bound): 2 S N (K + r) FLOP per launch over its HIP-event time,
          from one more loop of K steps with the per-kernel events on
  cpu_baseline  the fp64 oracle on a fixed row subset of the same workload (the first 256 rows, the
          last 256 and every 64th), on the host cores, with the full-S time extrapolated
Side sections time the other workload configurations with the same protocol: the block at S = 8192,
at S = 37728 (the canvas's second packed length), and adapter switching at S = 16384 (two resident
adapters x strengths 0, 0.5, 1, and adapter none).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--loops L] [--S 37726] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU (published 2.5 PF)
PEAK_HBM_GBS = 8000.0

# HBM bytes per GEMM launch of this workload from rocprofv3 FETCH_SIZE (x 2.00) and WRITE_SIZE (x 1.00)
# counter runs, mean over the four projections (profiles/gemm_w4_block_S37726.md), valid only for the
# GEMM sources they were taken with (SHA-256 prefix of the files below, in this order).
GEMM_TRAFFIC_BYTES = 9.026e9
GEMM_TRAFFIC_SOURCES = ("gemm_w4.hip", "gemm_w4_steps.inc", "h3q_device.hpp", "h3q_kernels.hpp", "h3q_layout.hpp")
GEMM_TRAFFIC_SHA = "6ada36f57eadc907"


def gemm_traffic():
    """The counter-derived traffic if the GEMM sources are the ones it was measured on, else None."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "bit_linear_dynamic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return GEMM_TRAFFIC_BYTES if h.hexdigest()[:16] == GEMM_TRAFFIC_SHA else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--loops", type=int, default=5, help="timed loops of --steps steps; the median is reported")
    ap.add_argument("--S", type=int, default=37726)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--proj", choices=["qkv", "attn_out", "gate_up", "down"], default=None,
                    help="profiling aid: time one projection only (the JSON line then covers only it)")
    ap.add_argument("--timed-only", action="store_true",
                    help="profiling aid: skip the per-projection, Q/K-epilogue and merged-vs-dynamic passes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="profiling aid: run only a plain device copy of MIB MiB (HBM counter calibration)")
    return ap.parse_args()


def build_block(S, device, only=None):
    """Pack the four projections (weights quantized on the device by h3q_debug_quantize_act from
    N(0, 0.02) draws) and register two adapters each (ids 1 and 2: distinct seeds, the projection's
    rank with alpha = rank); x and y hold S rows (the side sections use row prefixes of them)."""
    import torch

    import bit_linear_dynamic_amd as h3q
    from bit_linear_dynamic_amd import synth
    from bit_linear_dynamic_amd import workloads as wl

    projs = []
    xs = {}
    for i, p in enumerate(wl.BLOCK):
        if only is not None and p.name != only:
            continue
        w = synth.weight_fp32(p.N, p.K, synth.seed_of(3, i, synth.W), device).to(torch.bfloat16)
        codes, scales, ts = h3q.h3q_debug_quantize_act(w)
        torch.cuda.synchronize()
        del w
        handle = h3q.h3q_pack_weight(codes.cpu(), scales.cpu(), ts.item(), p.N, p.K,
                                     h3q.H3Q_PACK_GATE_UP if p.gate_up else 0)
        host = (codes.cpu(), scales.cpu(), ts.item())
        del codes, scales
        A, B = synth.lora_factors(p.N, p.K, p.rank, synth.seed_of(3, i, synth.A1), synth.seed_of(3, i, synth.B1), device)
        h3q.h3q_register_adapter(handle, 1, A.cpu(), B.cpu(), p.rank, p.alpha)
        A2, B2 = synth.lora_factors(p.N, p.K, p.rank, synth.seed_of(3, i, synth.A2), synth.seed_of(3, i, synth.B2))
        h3q.h3q_register_adapter(handle, 2, A2, B2, p.rank, p.alpha)
        del A2, B2
        if p.K not in xs:
            xs[p.K] = (synth.activation(S, p.K, synth.seed_of(3, i, synth.X), device),
                       synth.pre_quant_scale(p.K, synth.seed_of(3, i, synth.PQS), device))
        x, pqs = xs[p.K]
        y = torch.empty((S, p.N), dtype=torch.bfloat16, device=device)
        projs.append(dict(p=p, handle=handle, x=x, pqs=pqs, y=y, host=host, A=A, B=B))
    torch.cuda.synchronize()
    return projs


def step(projs, stream, S, adapter_id=1, strength=1.0):
    """One block pass: the four projections on the first S rows of x (all rows by default)."""
    import bit_linear_dynamic_amd as h3q
    for d in projs:
        x, y = d["rows"][S]
        h3q.h3q_linear(x, d["pqs"], d["handle"], adapter_id, strength, y=y, stream=stream)


def time_loops(run, steps, loops, stream):
    """Per-step milliseconds of `loops` timed loops of `steps` calls of run(), each loop bracketed by
    device synchronization and events on `stream`; returns (median, every loop's value)."""
    import torch
    per = []
    for _ in range(loops):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / steps)
    return sorted(per)[len(per) // 2], [round(v, 4) for v in per]


def block_side(projs, stream, S, steps, loops):
    """The block at another sequence length (a row prefix of the same inputs), same protocol."""
    from bit_linear_dynamic_amd import workloads as wl
    step(projs, stream, S)
    ms, per = time_loops(lambda: step(projs, stream, S), steps, loops, stream)
    flops = sum(wl.effective_flops(S, d["p"]) for d in projs)
    tf = flops / (ms * 1e-3) / 1e12
    return {"S": S, "ms_per_step": round(ms, 4), "loops_ms_per_step": per, "effective_tflops": round(tf, 1),
            "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "tflop_per_step": round(flops / 1e12, 4)}


def switching(projs, stream, S, steps, loops):
    """Adapter switching at S: per block pass (four projections), every (adapter, strength) pair of
    {none, 1, 2} x {0, 0.5, 1}, and a pass that alternates adapters 1 and 2 from call to call; a
    switch is a host-side lookup, so the alternating pass costs what the single-adapter ones do and
    adapter none or strength 0 costs the base-only call."""
    from bit_linear_dynamic_amd import workloads as wl
    import bit_linear_dynamic_amd as h3q

    per_call = {}
    for aid in (h3q.H3Q_ADAPTER_NONE, 1, 2):
        for st in (0.0, 0.5, 1.0):
            step(projs, stream, S, aid, st)
            ms, _ = time_loops(lambda: step(projs, stream, S, aid, st), steps, loops, stream)
            per_call[f"{'none' if aid < 0 else aid}@{st}"] = round(ms, 4)
    flip = [0]

    def alternating():
        for d in projs:
            x, y = d["rows"][S]
            flip[0] ^= 1
            h3q.h3q_linear(x, d["pqs"], d["handle"], 1 + flip[0], 1.0, y=y, stream=stream)

    alt, _ = time_loops(alternating, steps, loops, stream)
    active = [per_call[k] for k in ("1@0.5", "1@1.0", "2@0.5", "2@1.0")]
    base = [per_call[k] for k in ("none@0.0", "none@0.5", "none@1.0", "1@0.0", "2@0.0")]
    same = (per_call["1@1.0"] + per_call["2@1.0"]) / 2
    flops_a = sum(wl.effective_flops(S, d["p"]) for d in projs)
    return {"S": S, "block_ms_per_pass": per_call, "alternating_1_2_ms": round(alt, 4),
            "switch_overhead_pct": round(100 * (alt - same) / same, 2),
            "adapter_spread_pct": round(100 * (max(active) - min(active)) / min(active), 2),
            "base_spread_pct": round(100 * (max(base) - min(base)) / min(base), 2),
            "adapter_cost_pct": round(100 * (same - min(base)) / min(base), 2),
            "effective_tflops_adapter": round(flops_a / (same * 1e-3) / 1e12, 1)}


def subset_rows(S):
    """The oracle's fixed row subset: the first 256 rows, the last 256 (holding the ragged last row
    tile) and every 64th row."""
    import numpy as np
    return np.unique(np.concatenate([np.arange(min(256, S)), np.arange(max(0, S - 256), S), np.arange(0, S, 64)]))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(projs, S):
    """The oracle as it stands, on the row subset of each projection, timed with a wall clock
    around the oracle calls only; the full-S time is extrapolated from it (rows are independent)."""
    import numpy as np

    import oracle
    from bit_linear_dynamic_amd import synth
    from bit_linear_dynamic_amd import workloads as wl

    rows = subset_rows(S)
    lib = oracle.load()
    inputs = []
    for d in projs:
        p = d["p"]
        idx = __import__("torch").from_numpy(rows).to(d["x"].device)
        xb = synth.bf16_bits(d["x"].index_select(0, idx))
        codes, scales, ts = d["host"]
        inputs.append((xb, d["pqs"].cpu().numpy(), codes.numpy(), scales.numpy(), ts,
                       synth.bf16_bits(d["A"]), synth.bf16_bits(d["B"]), p))
    t0 = time.perf_counter()
    for xb, pqs, codes, scales, ts, A, B, p in inputs:
        oracle.linear(xb, pqs, codes, scales, ts, A, B, p.rank, p.alpha, 1.0, lib=lib)
    dt = time.perf_counter() - t0
    flops = sum(wl.effective_flops(len(rows), p) for *_, p in inputs)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(lib), "kind": "oracle",
            "sample": f"row subset R of S={S} (the first 256 rows, the last 256, every 64th: {len(rows)} rows) "
                      f"through each of the 4 projections, adapter 1 at strength 1; {dt:.1f} s wall for "
                      f"{flops / 1e9:.1f} GFLOP effective (each projection's whole-weight fp64 decode included)",
            "seconds": round(dt, 3), "rows": int(len(rows)), "block_rows_per_s": round(len(rows) / dt, 2),
            "extrapolated_full_s": round(dt * S / len(rows), 1),
            "extrapolated_note": "extrapolated, not measured: the subset's time scaled by S / rows",
            "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def merged_vs_dynamic(projs, stream, S, calls=5):
    """Per projection: the dynamic call (LoRA-down + GEMM over K + r_pad) against a base-only call on
    the weight with the update merged in before quantizing (h3q_merge_adapter, then packed), both with
    pqs; plus what one merge costs (device merge + quantize, synchronous) and the host-side pack. The
    accuracy side of the comparison (the merged route re-rounds the adapted weight to NVFP4) is
    measured against the oracle by the tests, not here."""
    import torch

    import bit_linear_dynamic_amd as h3q

    def per_call_ms(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(calls):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls

    out, tot = {}, {"dynamic_ms": 0.0, "merged_ms": 0.0}
    for d in projs:
        p = d["p"]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        codes, scales, ts = h3q.h3q_merge_adapter(d["handle"], 1, 1.0, d["pqs"])
        merge_ms = (time.perf_counter() - t0) * 1e3
        t0 = time.perf_counter()
        mh = h3q.h3q_pack_weight(codes.cpu(), scales.cpu(), ts.item(), p.N, p.K,
                                 h3q.H3Q_PACK_GATE_UP if p.gate_up else 0)
        pack_ms = (time.perf_counter() - t0) * 1e3
        del codes, scales
        x, y = d["rows"][S]
        try:
            dyn = per_call_ms(lambda: h3q.h3q_linear(x, d["pqs"], d["handle"], 1, 1.0, y=y, stream=stream))
            mrg = per_call_ms(lambda: h3q.h3q_linear(x, d["pqs"], mh, h3q.H3Q_ADAPTER_NONE, 0.0, y=y, stream=stream))
        finally:
            h3q.h3q_free_weight(mh)
        out[p.name] = {"dynamic_ms": round(dyn, 4), "merged_ms": round(mrg, 4),
                       "dynamic_overhead_pct": round(100.0 * (dyn - mrg) / mrg, 2),
                       "merge_ms": round(merge_ms, 2), "pack_host_ms": round(pack_ms, 1)}
        tot["dynamic_ms"] += dyn
        tot["merged_ms"] += mrg
    out["block"] = {"dynamic_ms": round(tot["dynamic_ms"], 4), "merged_ms": round(tot["merged_ms"], 4),
                    "dynamic_overhead_pct": round(100.0 * (tot["dynamic_ms"] - tot["merged_ms"]) / tot["merged_ms"], 2)}
    return out


def producer_fusion(projs, stream, S, calls=5):
    """The MLP pair gate/up -> down per call, unfused (SwiGLU writes h; the down call makes its own
    base operand bf16(h * pqs) in LoRA-down or the prescale pass) against fused (the SwiGLU epilogue
    also writes that operand; the down call takes it as given), with adapter 1 at strength 1 and with
    no adapter."""
    import torch

    import bit_linear_dynamic_amd as h3q

    by = {d["p"].name: d for d in projs}
    if "gate_up" not in by or "down" not in by:
        return None
    gu, dn = by["gate_up"], by["down"]
    F = gu["p"].N // 2
    gx, dy = gu["rows"][S][0], dn["rows"][S][1]
    h = torch.empty((S, F), dtype=torch.bfloat16, device=gx.device)
    xs = torch.empty_like(h)

    def unfused(aid, st):
        h3q.h3q_linear_swiglu(gx, gu["pqs"], gu["handle"], aid, st, h=h, stream=stream)
        h3q.h3q_linear(h, dn["pqs"], dn["handle"], aid, st, y=dy, stream=stream)

    def fused(aid, st):
        h3q.h3q_linear_swiglu_emit(gx, gu["pqs"], gu["handle"], aid, st, dn["pqs"], h=h, xs_next=xs,
                                   stream=stream)
        h3q.h3q_linear_prescaled(h, xs, dn["handle"], aid, st, y=dy, stream=stream)

    def per_call_ms(fn, aid, st):
        fn(aid, st)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(calls):
            fn(aid, st)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls

    out = {}
    for name, aid, st in (("adapter", 1, 1.0), ("no_adapter", h3q.H3Q_ADAPTER_NONE, 0.0)):
        # alternate the two orders so that neither always runs on a warmer or cooler chip
        u1, f1 = per_call_ms(unfused, aid, st), per_call_ms(fused, aid, st)
        f2, u2 = per_call_ms(fused, aid, st), per_call_ms(unfused, aid, st)
        u, f = (u1 + u2) / 2, (f1 + f2) / 2
        out[name] = {"unfused_ms": round(u, 4), "fused_ms": round(f, 4), "fused_vs_unfused_pct": round(100 * (f - u) / u, 2)}
    return out


def w4a4_gate_up(projs, stream, S, calls=5):
    """The W4A4 variant on the fused gate/up projection at the bench's S: activations quantized to
    NVFP4 per call for the base GEMM, LoRA on the original x, SiLU(gate) * up in the epilogue. Per
    call: wall time, and each kernel's share from the library's HIP events (the quantizer's two passes
    read x twice and write the decoded operand)."""
    import torch

    import bit_linear_dynamic_amd as h3q
    from bit_linear_dynamic_amd import workloads as wl

    d = next((d for d in projs if d["p"].name == "gate_up"), None)
    if d is None:
        return None
    p = d["p"]
    x = d["rows"][S][0]
    h = torch.empty((S, p.N // 2), dtype=torch.bfloat16, device=x.device)
    flags = h3q.H3Q_ACT_NVFP4 | h3q.H3Q_EPI_SWIGLU

    def call():
        h3q.h3q_linear_ex(x, d["pqs"], d["handle"], 1, 1.0, flags, out=h, stream=stream)

    call()
    torch.cuda.synchronize()
    h3q.h3q_timing_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(calls):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    call_ms = a.elapsed_time(b) / calls
    g, gn = h3q.h3q_timing_get(h3q.H3Q_KERNEL_GEMM)
    q, qn = h3q.h3q_timing_get(h3q.H3Q_KERNEL_ACT_QUANT)
    l, ln = h3q.h3q_timing_get(h3q.H3Q_KERNEL_LORA_DOWN)
    h3q.h3q_timing_enable(False)
    g, q, l = g / gn, q / qn, l / ln
    K_pad = (p.K + 63) // 64 * 64
    q_bytes = 2 * S * p.K * 2 + S * K_pad * 2 + p.K * 4
    return {"S": S, "projection": [p.N, p.K, p.rank], "call_ms": round(call_ms, 4),
            "effective_tflops": round(wl.effective_flops(S, p) / (call_ms * 1e-3) / 1e12, 1),
            "gemm_ms": round(g, 4), "gemm_tflops": round(2 * S * p.N * (p.K + p.rank) / (g * 1e-3) / 1e12, 1),
            "act_quant_ms": round(q, 4), "act_quant_bytes": q_bytes,
            "act_quant_GBps": round(q_bytes / (q * 1e-3) / 1e9, 1), "lora_down_ms": round(l, 4)}


def small_s_graph(device, calls=20, replays=10):
    """The small case (one fused-QKV-like projection 3072 x 1024, rank = alpha = 384, S = 256) is
    launch-bound: per-call time issued eagerly against the same calls captured once into a HIP graph
    and replayed (after one eager call has sized the stream's workspace)."""
    import torch

    import bit_linear_dynamic_amd as h3q
    from bit_linear_dynamic_amd import synth
    from bit_linear_dynamic_amd import workloads as wl

    p, S = wl.SMALL_QKV, wl.S_SMALL
    w = synth.weight_fp32(p.N, p.K, synth.seed_of(1, 0, synth.W), device).to(torch.bfloat16)
    codes, scales, ts = h3q.h3q_debug_quantize_act(w)
    torch.cuda.synchronize()
    handle = h3q.h3q_pack_weight(codes.cpu(), scales.cpu(), ts.item(), p.N, p.K)
    try:
        A, B = synth.lora_factors(p.N, p.K, p.rank, synth.seed_of(1, 0, synth.A1), synth.seed_of(1, 0, synth.B1))
        h3q.h3q_register_adapter(handle, 1, A, B, p.rank, p.alpha)
        x = synth.activation(S, p.K, synth.seed_of(1, 0, synth.X), device)
        pqs = synth.pre_quant_scale(p.K, synth.seed_of(1, 0, synth.PQS), device)
        y = torch.empty((S, p.N), dtype=torch.bfloat16, device=device)
        s = torch.cuda.Stream()

        def run():
            for _ in range(calls):
                h3q.h3q_linear(x, pqs, handle, 1, 1.0, y=y, stream=s)

        with torch.cuda.stream(s):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            a.record(s)
            for _ in range(replays):
                run()
            b.record(s)
        torch.cuda.synchronize()
        eager_us = a.elapsed_time(b) * 1e3 / (calls * replays)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
            a.record(s)
            for _ in range(replays):
                g.replay()
            b.record(s)
        torch.cuda.synchronize()
        graph_us = a.elapsed_time(b) * 1e3 / (calls * replays)
        flops = wl.effective_flops(S, p)
        return {"projection": [p.N, p.K, p.rank], "S": S, "eager_us_per_call": round(eager_us, 2),
                "graph_us_per_call": round(graph_us, 2), "graph_tflops": round(flops / (graph_us * 1e-6) / 1e12, 1),
                "eager_tflops": round(flops / (eager_us * 1e-6) / 1e12, 1)}
    finally:
        torch.cuda.synchronize()
        h3q.h3q_free_weight(handle)


def mfma_ceiling(stream, device, gemm_achieved):
    """The matrix-core rate the board sustains under its power limit (h3q_mfma_loop: rotating operand
    pairs, two waves per SIMD, no memory traffic), on activation-like bf16 N(0, 1) operands against
    decoded-weight-like ones (E2M1 value times an E4M3 block scale, exact in bf16); the median of three
    ~20 ms runs. The GEMM's rate is then also read against this practical ceiling."""
    import torch

    import bit_linear_dynamic_amd as h3q
    from bit_linear_dynamic_amd import synth

    ops_a = synth.normal((8, 256, 8), 1.0, synth.seed_of(11, 0, 0), device, torch.bfloat16)
    e2m1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device=device)
    g = torch.Generator(device=device)
    g.manual_seed(synth.seed_of(11, 0, 1))
    mag = e2m1[torch.randint(0, 8, (8, 256, 8), generator=g, device=device)]
    sign = torch.randint(0, 2, (8, 256, 8), generator=g, device=device) * 2.0 - 1.0
    scale = torch.exp2(torch.randint(-8, -5, (8, 256, 1), generator=g, device=device).float()) * \
        (1.0 + torch.randint(0, 8, (8, 256, 1), generator=g, device=device).float() / 8.0)
    ops_b = (sign * mag * scale).to(torch.bfloat16)
    wgs = 2 * torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    flop_per_iter = wgs * 4 * 64 * 32768
    sink = h3q.h3q_mfma_loop(ops_a, ops_b, 100, wgs, stream=stream)
    iters = max(1, int(0.02 * 1.7e15 / flop_per_iter))
    runs = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        h3q.h3q_mfma_loop(ops_a, ops_b, iters, wgs, sink=sink, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        runs.append(flop_per_iter * iters / (a.elapsed_time(b) * 1e-3) / 1e12)
    tf = sorted(runs)[1]
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "gemm_frac_of_loop": round(gemm_achieved / tf, 4), "workgroups": wgs, "iters": iters}


def adaln_curve(stream, device, reps=50):
    """The AdaLN modulation curve of all 50 blocks ([96768, 24] each, 1025 samples, rank 8 + 16) at
    T = 2 times per call: apply time and its HBM rate (bytes = blocks * rows * (2 R + 4 + 4 T)), and
    the one-off table build."""
    import torch

    import bit_linear_dynamic_amd as h3q
    from bit_linear_dynamic_amd import synth
    from bit_linear_dynamic_amd import workloads as wl

    c = wl.ADALN
    u, emb, A, M, bias = synth.adaln_curve_inputs(c.blocks, c.samples, c.emb_dim, c.base_rank, c.lora_rank, c.rows,
                                                  synth.seed_of(9, 0, 0), device)
    u, emb = u.to(device), emb.to(device)
    t = torch.tensor([0.8125, 0.30078125], dtype=torch.float32, device=device)
    table = h3q.h3q_adaln_table(u, emb, A, 1.0, stream=stream)
    out = h3q.h3q_adaln_apply(M, bias, table, t, stream=stream)

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    build_ms = timed(lambda: h3q.h3q_adaln_table(u, emb, A, 1.0, stream=stream))
    apply_ms = timed(lambda: h3q.h3q_adaln_apply(M, bias, table, t, out=out, stream=stream))
    R, T = c.base_rank + c.lora_rank, t.shape[0]
    bytes_apply = c.blocks * c.rows * (2 * R + 4 + 4 * T)
    gbs = bytes_apply / (apply_ms * 1e-3) / 1e9
    return {"blocks": c.blocks, "rows": c.rows, "R": R, "samples": c.samples, "T": T,
            "apply_us": round(apply_ms * 1e3, 2), "apply_bytes": bytes_apply, "apply_GBps": round(gbs, 1),
            "apply_hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "table_build_us": round(build_ms * 1e3, 2),
            "table_flop": 2 * c.blocks * c.samples * c.lora_rank * c.emb_dim}


def library_bf16_gemm(projs, S, device, calls=5):
    """Context, not a product path: torch's bf16 matrix product (the ROCm BLAS library it dispatches
    to) on each projection's contraction, x [S, K + r] times a dense bf16 weight [K + r, N] (N(0, 1)
    activations, N(0, 0.02) weights): what a tuned library reaches on the same dense shapes with no
    4-bit decode and no adapter pass. Per-call time is the mean of `calls` calls after two warm-ups."""
    import torch

    from bit_linear_dynamic_amd import synth

    out, flop_sum, ms_sum = {}, 0.0, 0.0
    for i, d in enumerate(projs):
        p = d["p"]
        kt = p.K + p.rank
        x = synth.normal((S, kt), 1.0, synth.seed_of(12, i, 0), device, torch.bfloat16)
        w = synth.normal((kt, p.N), 0.02, synth.seed_of(12, i, 1), device, torch.bfloat16)
        y = torch.empty((S, p.N), dtype=torch.bfloat16, device=device)
        for _ in range(2):
            torch.mm(x, w, out=y)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(calls):
            torch.mm(x, w, out=y)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / calls
        flop = 2.0 * S * p.N * kt
        out[p.name] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
        flop_sum += flop
        ms_sum += ms
        del x, w, y
    torch.cuda.empty_cache()
    out["block_tflops"] = round(flop_sum / (ms_sum * 1e-3) / 1e12, 1)
    out["library"] = str(torch.backends.cuda.preferred_blas_library())
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on exactly one GPU; multi-GPU runs are not supported "
              "(the projection would shard by rows of x with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_linear_dynamic_amd as h3q
    from bit_linear_dynamic_amd import workloads as wl

    device = "cuda"
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=device)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_mib": args.calibrate_copy, "launches": 3}), flush=True)
        return
    S = args.S
    # the side sections: the block at S = 8192 and at S + 2 = 37728 (the canvas's second packed length,
    # whose first 37726 rows are the headline's input), and adapter switching at S = 16384
    side = not args.timed_only and S == wl.S_CANVAS
    S_alloc = wl.S_CANVAS_ALT if side else S
    print(f"bench: building the projections at S={S}", file=sys.stderr, flush=True)
    projs = build_block(S_alloc, device, args.proj)
    for d in projs:
        d["rows"] = {n: (d["x"][:n], d["y"][:n]) for n in {S, S_alloc, wl.S_MID, wl.S_SWITCH} if n <= S_alloc}
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        step(projs, stream, S)
    torch.cuda.synchronize()
    print(f"bench: warmup done, timing {args.loops} loops of {args.steps} steps", file=sys.stderr, flush=True)

    # headline: the median of the loops, nothing but the library's own launches on the stream
    ms_per_step, loops_ms = time_loops(lambda: step(projs, stream, S), args.steps, args.loops, stream)

    # per-kernel breakdown: one more loop with the library's HIP events around each launch
    h3q.h3q_timing_enable(True)
    for _ in range(args.steps):
        step(projs, stream, S)
    torch.cuda.synchronize()
    gemm_ms, gemm_n = h3q.h3q_timing_get(h3q.H3Q_KERNEL_GEMM)
    down_ms, down_n = h3q.h3q_timing_get(h3q.H3Q_KERNEL_LORA_DOWN)
    h3q.h3q_timing_enable(False)

    flops_step = sum(wl.effective_flops(S, d["p"]) for d in projs)
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    gemm_flops_launch = sum(2 * S * d["p"].N * (d["p"].K + d["p"].rank) for d in projs) / len(projs)
    gemm_avg_ms = gemm_ms / max(gemm_n, 1)
    achieved = gemm_flops_launch / (gemm_avg_ms * 1e-3) / 1e12

    # per-projection breakdown (separate, untimed-above pass with timing on)
    per_proj = {}
    for d in ([] if args.timed_only else projs):
        h3q.h3q_timing_enable(True)
        x, y = d["rows"][S]
        for _ in range(3):
            h3q.h3q_linear(x, d["pqs"], d["handle"], 1, 1.0, y=y)
        torch.cuda.synchronize()
        g, gn = h3q.h3q_timing_get(h3q.H3Q_KERNEL_GEMM)
        l, ln = h3q.h3q_timing_get(h3q.H3Q_KERNEL_LORA_DOWN)
        h3q.h3q_timing_enable(False)
        p = d["p"]
        per_proj[p.name] = {"gemm_ms": round(g / gn, 4), "lora_down_ms": round(l / ln, 4),
                            "gemm_tflops": round(2 * S * p.N * (p.K + p.rank) / (g / gn * 1e-3) / 1e12, 1)}

    # the QKV projection with the fused Q/K RMSNorm + rotary epilogue (48 heads of 128, 96 rotated)
    qk = None
    for d in projs:
        p = d["p"]
        if p.name != "qkv" or args.timed_only:
            continue
        from bit_linear_dynamic_amd import synth
        q_width = p.N // 3
        g = torch.ones(q_width, dtype=torch.float32, device=device)
        cos, sin = (t.to(device) for t in synth.rope_table(S, 96))
        x, y = d["rows"][S]
        h3q.h3q_linear_qk_norm_rope(x, d["pqs"], d["handle"], 1, 1.0, q_width, 96, 1e-6, g, g, cos, sin, y=y)
        torch.cuda.synchronize()
        h3q.h3q_timing_enable(True)
        for _ in range(3):
            h3q.h3q_linear_qk_norm_rope(x, d["pqs"], d["handle"], 1, 1.0, q_width, 96, 1e-6, g, g, cos, sin, y=y)
        torch.cuda.synchronize()
        gq, gqn = h3q.h3q_timing_get(h3q.H3Q_KERNEL_GEMM)
        h3q.h3q_timing_enable(False)
        plain = per_proj["qkv"]["gemm_ms"]
        qk = {"gemm_ms": round(gq / gqn, 4), "plain_gemm_ms": plain,
              "epilogue_overhead_pct": round(100.0 * (gq / gqn - plain) / plain, 2)}

    # the other workload configurations, same protocol
    cfg2 = block_side(projs, stream, wl.S_MID, args.steps, args.loops) if side else None
    cfg3alt = block_side(projs, stream, wl.S_CANVAS_ALT, args.steps, args.loops) if side else None
    cfg4 = switching(projs, stream, wl.S_SWITCH, max(1, args.steps // 2), args.loops) if side else None

    # the merged route (the update folded into the weight before quantizing) against the dynamic call
    mvd = None if args.timed_only else merged_vs_dynamic(projs, stream, S)
    adaln = None if args.timed_only else adaln_curve(stream, device)
    fusion = None if args.timed_only else producer_fusion(projs, stream, S)
    w4a4 = None if args.timed_only else w4a4_gate_up(projs, stream, S)
    ceiling = None if args.timed_only else mfma_ceiling(stream, device, achieved)
    small = None if args.timed_only else small_s_graph(device)
    library = None if args.timed_only else library_bf16_gemm(projs, S, device)

    cpu = None
    if not args.no_cpu:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(projs, S)

    line = {
        "metric": "effective TFLOP/s (+% bf16 MFMA peak) of W4+LoRA linear, S=37726",
        "only_projection": args.proj,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "loops": args.loops,
        "loops_ms_per_step": loops_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": "MiniMax-H3 DiT block, four W4+LoRA projections at packed sequence length S",
                   "S": S, "projections": {p.name: [p.N, p.K, p.rank] for p in wl.BLOCK},
                   "weights": "NVFP4 (E2M1 + E4M3/16 + fp32)", "lora": "bf16, rank=alpha, strength 1.0",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "gemm_w4_kernel<0, true>", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_ms": round(gemm_avg_ms, 4), "launches": gemm_n,
                     "flop_per_launch": gemm_flops_launch, "traffic": gemm_traffic(),
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE/WRITE_SIZE)"},
        "kernels_ms_per_step": {"gemm": round(gemm_ms / args.steps, 4), "lora_down": round(down_ms / args.steps, 4),
                                "note": "from one extra loop of the same steps with per-launch HIP events"},
        "cfg2_block_s8192": cfg2,
        "cfg3alt_s37728": cfg3alt,
        "cfg4_switching_s16384": cfg4,
        "per_projection": per_proj,
        "qkv_with_qk_norm_rope": qk,
        "merged_vs_dynamic": mvd,
        "adaln_curve": adaln,
        "mlp_producer_fusion": fusion,
        "w4a4_swiglu_gate_up": w4a4,
        "mfma_loop_ceiling": ceiling,
        "library_bf16_gemm": library,
        "small_s_latency": small,
        "cpu_baseline": cpu,
    }
    for d in projs:
        h3q.h3q_free_weight(d["handle"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
