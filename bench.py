#!/usr/bin/env python3
"""Benchmark of libmsr on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only a,b,...] [--no-cpu]

Headline (the JSON line's "value"): forward of the full gated multi-scale
retention layer (X W_Q/W_K/W_V, rotation, chunkwise retention, GroupNorm,
swish(X W_G) gate, W_O; bf16 with float32 accumulation) on batch 4 x 8192
tokens, d_model 4096, 16 heads, q/k head dim 256, v head dim 512, chunk 512
-- tokens per second, inputs and weights resident in HBM, W untimed warm-up
steps then exactly K timed steps between two stream synchronisations.  The
same line carries:

* roofline   -- the dominant kernel's achieved rate over the timed steps,
                from HIP events bracketing each of its launches (msr_trace)
                against the MI355X peak;
* chunkwise  -- the same for the chunkwise retention kernels of the step,
                alone and together (the core's share of the MFMA peak);
* kernels    -- every kernel of the step;
* decode     -- recurrent decode, batch 128, 16 heads of 256, fp32 state
                (512 MiB) prefilled from an 8192-token context, 512 timed
                steps: steps/s and fraction of HBM peak; also a 1024-token
                context for the length-independence check;
* layer_decode -- the whole layer's decode step at that shape, 512 steps;
* layer_b8_n2048 -- the layer at batch 8 x 2048, d_model 2048, 8 heads of
                256, chunk 256;
* long       -- chunkwise core (batch 2, 16384 tokens, 10 heads of 256,
                chunk 512) and a sequence-length sweep of chunkwise vs
                parallel form, plus that layer;
* cpu_baseline -- the float64 oracle timed on this host on a bounded sample
                of the headline workload.

There is one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 256 * 2.4e9 * 4096        # dense MFMA flop/s: 2516.6 TFLOP/s
PEAK_F32_MFMA = 157.3e12
PEAK_HBM = 8.0e12                      # bytes/s


# HBM bytes per launch of each kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over `bench.py --only <part>`,
# scaled by what the same counters read for a 1 GiB device-to-device copy
# (FETCH_SIZE x 2, WRITE_SIZE x 1).  Each figure holds only for the sources
# it was taken with: the sha256 prefix of those files is recorded, and a
# kernel whose sources have changed since reports null.
MEASURED_TRAFFIC = {  # (workload, kernel): (bytes per launch, sources, sha256[:16])
    ("block_bf16_b4_n8192", "k_gemm"): (7.450e+09, ('k_gemm.hip', 'msr_device.h'), "ada3023b46f5318f"),
    ("block_bf16_b4_n8192", "k_chunk_out"): (3.316e+09, ('k_chunk_o16.hip', 'msr_device.h'), "d363d9876734f0d8"),
    ("block_bf16_b4_n8192", "k_chunk_rscan"): (1.078e+09, ('k_chunk_rscan.hip', 'msr_device.h'), "f884352b01858490"),
    ("block_bf16_b4_n8192:core", "k_chunk_out"): (1.880e+09, ('k_chunk_o16.hip', 'msr_device.h'),
                                                  "d363d9876734f0d8"),
    ("block_bf16_b4_n8192:core", "k_chunk_rscan"): (1.078e+09, ('k_chunk_rscan.hip', 'msr_device.h'),
                                                    "f884352b01858490"),
    ("long_bf16_b2_n16384:core", "k_chunk_out"): (7.554e+08, ('k_chunk_o16.hip', 'msr_device.h'), "d363d9876734f0d8"),
    ("long_bf16_b2_n16384:core", "k_chunk_state"): (4.212e+08, ('k_chunk.hip', 'msr_device.h'), "6d4c12e791058fb3"),
    ("long_bf16_b2_n16384:core", "k_chunk_scan"): (1.678e+08, ('k_chunk.hip', 'msr_device.h'), "6d4c12e791058fb3"),
}
CSRC = os.path.join(ROOT, "linear_recurrence_sequence_amd", "csrc")


def measured_traffic(workload, kernel):
    import hashlib
    e = MEASURED_TRAFFIC.get((workload, kernel))
    if e is None:
        return None
    nbytes, files, digest = e
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return round(nbytes) if h.hexdigest()[:16] == digest else None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
def gpu_time(fn, steps, warmup):
    """Average seconds per call of fn over `steps` calls after `warmup`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e-3 / steps


def step_stats(fn, steps):
    """Median and minimum seconds of single calls of fn (an event pair around
    each call), from a pass after the timed region."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    return ts[len(ts) // 2], ts[0]


def traced(fn, steps):
    """Per-kernel (total s, launches) over `steps` calls, from HIP events the
    library records around each launch on its stream."""
    import torch
    import linear_recurrence_sequence_amd as msr
    torch.cuda.synchronize()
    msr.msr_trace_enable(True)
    for _ in range(steps):
        fn()
    tot = msr.trace_totals()
    msr.msr_trace_enable(False)
    return {k: (ms * 1e-3, n) for k, (ms, n) in tot.items()}


def roof(name, work_per_step, bound, trace, steps, launches_per_step=None, workload=None, bytes_per_step=None):
    """Roofline entry for one kernel: work_per_step is flops (mfma) or bytes
    (hbm) of algorithmic work in one step; traffic = measured HBM bytes per
    launch (see MEASURED_TRAFFIC) or None.  For a matrix-core kernel with
    its algorithmic bytes given, also the attainable rate min(peak, I x HBM
    peak), I = flops / bytes, and the fraction of it achieved."""
    t, n = trace[name]
    per_launch_t = t / n
    lps = n / steps if launches_per_step is None else launches_per_step
    per_launch_work = work_per_step / lps
    peak, unit = (PEAK_BF16, "TFLOP/s") if bound == "mfma" else (PEAK_HBM, "GB/s")
    scale = 1e12 if bound == "mfma" else 1e9
    ach = per_launch_work / per_launch_t
    r = {"kernel": name, "bound": bound, "achieved": round(ach / scale, 2), "peak": round(peak / scale, 1),
         "unit": unit, "frac": round(ach / peak, 4), "traffic": measured_traffic(workload, name),
         "avg_launch_us": round(per_launch_t * 1e6, 2), "launches_per_step": lps}
    if bound == "mfma" and bytes_per_step:
        inten = work_per_step / bytes_per_step
        att = min(peak, inten * PEAK_HBM)
        r.update({"intensity_flop_per_byte": round(inten, 1), "attainable": round(att / scale, 1),
                  "frac_of_attainable": round(ach / att, 4)})
    return r


def layer_flops(B, N, dm, H, dk, dv, C):
    proj = 2 * dm * (2 * H * dk + 2 * H * dv) + 2 * H * dv * dm
    core = H * (C * (dk + dv) + 4 * dk * dv)
    return B * N * proj, B * N * core


def make_layer(w, device_inputs):
    """Device tensors X, W_Q, W_K, W_V, W_G, W_O (bf16) for workload w."""
    import numpy as np
    import torch
    import workloads
    if not device_inputs:
        arrs = workloads.layer_inputs(w)
        return [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in arrs]
    s = 1.0 / math.sqrt(w.d_model)
    hk, hv = w.heads * w.d_k, w.heads * w.d_v
    shapes = [(w.batch, w.seqlen, w.d_model), (w.d_model, hk), (w.d_model, hk), (w.d_model, hv), (w.d_model, hv),
              (hv, w.d_model)]
    out = []
    for i, shp in enumerate(shapes):
        t = workloads.device_normal(shp, seed=1000 * (w.seed + 1) + i)
        out.append((t if i == 0 else t * s).to(torch.bfloat16))
    return out


def bench_layer(w, steps, warmup, device_inputs=False):
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    X, WQ, WK, WV, WG, WO = make_layer(w, device_inputs)
    g = workloads.gammas(w.heads)
    out = torch.empty_like(X)
    ws = torch.empty(msr.msr_layer_workspace_bytes(1, w.batch, w.seqlen, w.d_model, w.heads, w.d_k, w.d_v, w.chunk),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: msr.msr_layer_fwd(X, WQ, WK, WV, WG, WO, g, w.heads, w.d_k, w.d_v, w.chunk, rope_base=w.rope_base,
                                   gn_eps=1e-5, out=out, workspace=ws)
    t = gpu_time(fn, steps, warmup)
    med, mn = step_stats(fn, steps)
    tr = traced(fn, steps)
    proj, core = layer_flops(w.batch, w.seqlen, w.d_model, w.heads, w.d_k, w.d_v, w.chunk)
    B, N, H, dk, dv, C = w.batch, w.seqlen, w.heads, w.d_k, w.d_v, w.chunk
    nc = -(-N // C)
    es = 2
    M, dm, hk, hv = B * N, w.d_model, H * dk, H * dv
    ntot = 2 * hk + 2 * hv
    states = B * H * nc * dk * dv * es
    work = {  # algorithmic work per step: flops (mfma) or bytes (hbm); algorithmic bytes of the mfma kernels
        "k_gemm": (proj, "mfma", (M * dm + dm * ntot + M * ntot + M * hv + hv * dm + M * dm) * es),
        "k_chunk_out": (B * N * H * (C * (dk + dv) + 2 * dk * dv), "mfma", M * (ntot + hv) * es + states),
        "k_chunk_state": (B * N * H * 2 * dk * dv, "mfma", M * (hk + hv) * es + states),
        "k_chunk_scan": (2 * states, "hbm", None),     # read dR_i, write R_{i-1} (element type)
        # one pass: read K and V, write every R_{i-1}
        "k_chunk_rscan": (B * N * H * 2 * dk * dv, "mfma", M * (hk + hv) * es + states),
        "k_rope_table": (N * dk // 2 * 8, "hbm", None),
    }
    kern = {n: roof(n, wk, bd, tr, steps, workload=w.name, bytes_per_step=by) for n, (wk, bd, by) in work.items()
            if n in tr}
    del X, WQ, WK, WV, WG, WO, out, ws
    torch.cuda.empty_cache()
    res = {"s_per_step": t, "s_per_step_median": med, "s_per_step_min": mn, "tokens_per_s": B * N / t,
           "flops_per_step": proj + core,
           "tflops": (proj + core) / t / 1e12, "mfma_frac": (proj + core) / t / PEAK_BF16, "kernels": kern,
           "trace_s_per_step": {k: v[0] / steps for k, v in tr.items()},
           "chunkwise": chunkwise_summary(tr, steps, core, kern)}
    return res


CHUNK_KERNELS = ("k_chunk_state", "k_chunk_scan", "k_chunk_rscan", "k_chunk_out")


def chunkwise_summary(tr, steps, core_flops, kern):
    """The chunkwise retention kernels of a step together: the core's
    algorithmic flops (causal intra-chunk products, Q R and the state
    contributions) over their summed launch time, against the bf16 peak;
    and each kernel's own roofline entry."""
    t = sum(tr[n][0] for n in CHUNK_KERNELS if n in tr) / steps
    if t <= 0:
        return None
    ach = core_flops / t
    return {"bound": "mfma", "achieved": round(ach / 1e12, 2), "peak": round(PEAK_BF16 / 1e12, 1),
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16, 4), "us_per_step": round(t * 1e6, 2),
            "flops_per_step": core_flops, "kernels": {n: kern[n] for n in CHUNK_KERNELS if n in kern}}


def bench_core(B, N, H, d, C, steps, warmup, parallel=False, dv=None, rope_base=0.0, workload=None):
    """Chunkwise (or parallel) retention core on projected bf16 Q, K, V of
    [B, N, H, d] (V and O [B, N, H, dv]), rotated inside the call when
    rope_base > 0; algorithmic flops count the causal half of the
    intra-chunk products: per token and head C (d_k + d_v) + 4 d_k d_v
    (chunkwise), N (d_k + d_v) on average (parallel)."""
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    dk, dv = d, dv or d
    Q, K = (workloads.device_normal((B, N, H, dk), seed=7 + i, dtype=torch.bfloat16) for i in range(2))
    V = workloads.device_normal((B, N, H, dv), seed=9, dtype=torch.bfloat16)
    O = torch.empty_like(V)
    g = workloads.gammas(H)
    s = 1 / math.sqrt(dk)
    if parallel:
        wp = torch.empty(max(1, msr.msr_parallel_workspace_bytes(1, B, N, H, dk, dv, rope_base)), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: msr.msr_parallel_fwd(Q, K, V, g, qk_scale=s, rope_base=rope_base, O=O, workspace=wp)
        flops = B * N * H * N * (dk + dv)
    else:
        ws = torch.empty(msr.msr_chunkwise_workspace_bytes(1, B, N, H, dk, dv, C, rope_base), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: msr.msr_chunkwise_fwd(Q, K, V, g, C, qk_scale=s, rope_base=rope_base, O=O, workspace=ws)
        flops = B * N * H * (C * (dk + dv) + 4 * dk * dv)
    t = gpu_time(fn, steps, warmup)
    res = {"N": N, "s": t, "tokens_per_s": B * N / t, "tflops": flops / t / 1e12, "mfma_frac": flops / t / PEAK_BF16}
    if not parallel:
        tr = traced(fn, steps)
        nc = -(-N // C)
        states = B * H * nc * dk * dv * 2
        work = {
            # Q, K read, V read, O written, R_{i-1} read
            "k_chunk_out": (B * N * H * (C * (dk + dv) + 2 * dk * dv), "mfma",
                            B * N * H * (2 * dk + 2 * dv) * 2 + states),
            "k_chunk_state": (B * N * H * 2 * dk * dv, "mfma", B * N * H * (dk + dv) * 2 + states),
            "k_chunk_scan": (2 * states, "hbm", None),
            "k_chunk_rscan": (B * N * H * 2 * dk * dv, "mfma", B * N * H * (dk + dv) * 2 + states),
        }
        res["kernels"] = {n: roof(n, wk, bd, tr, steps, workload=workload, bytes_per_step=by)
                          for n, (wk, bd, by) in work.items() if n in tr}
        res["trace_us_per_step"] = {k: round(v[0] / steps * 1e6, 2) for k, v in tr.items()}
    return res


def bench_backward(B, N, H, d, C, steps, warmup):
    """Chunkwise backward (dQ, dK, dV, dS_in) at a core shape, bf16, no
    rotation; algorithmic flops = three chunkwise passes."""
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    Q, K, V, dO = (workloads.device_normal((B, N, H, d), seed=70 + i, dtype=torch.bfloat16) for i in range(4))
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dS_in = torch.empty((B, H, d, d), device="cuda")
    g = workloads.gammas(H)
    s = 1 / math.sqrt(d)
    ws = torch.empty(msr.msr_chunkwise_bwd_workspace_bytes(1, B, N, H, d, d, C, 0.0), dtype=torch.uint8,
                     device="cuda")
    fn = lambda: msr.msr_chunkwise_bwd(Q, K, V, dO, g, C, qk_scale=s, dS_in=dS_in, dQ=dQ, dK=dK, dV=dV,
                                       workspace=ws)
    flops = 3 * B * N * H * (C * 2 * d + 4 * d * d)
    t = gpu_time(fn, steps, warmup)
    tr = traced(fn, steps)
    # with the forward's per-chunk states kept (msr_chunkwise_fwd_save, outside the timed region)
    R = torch.empty(msr.msr_chunkwise_states_shape(B, N, H, d, d, C), dtype=torch.bfloat16, device="cuda")
    msr.msr_chunkwise_fwd_save(Q, K, V, g, C, R, qk_scale=s)
    fs = lambda: msr.msr_chunkwise_bwd_saved(Q, K, V, dO, g, C, R, qk_scale=s, dS_in=dS_in, dQ=dQ, dK=dK, dV=dV,
                                             workspace=ws)
    ts = gpu_time(fs, steps, warmup)
    res = {"batch": B, "seqlen": N, "heads": H, "d": d, "chunk": C, "ms_per_step": round(t * 1e3, 4),
           "tokens_per_s": round(B * N / t, 1), "tflops": round(flops / t / 1e12, 1),
           "mfma_frac": round(flops / t / PEAK_BF16, 4),
           "trace_ms_per_step": {k: round(v[0] / steps * 1e3, 4) for k, v in tr.items()},
           "saved_states_ms_per_step": round(ts * 1e3, 4), "saved_states_tokens_per_s": round(B * N / ts, 1)}
    del Q, K, V, dO, dQ, dK, dV, ws, R
    torch.cuda.empty_cache()
    return res


def bench_rglru(B, T, D, steps, warmup):
    """RG-LRU over a sequence (gate GEMM with sigmoid epilogue + float32
    scan), bf16, inputs of the seeded recipe drawn on the host once."""
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    x, Wa, ba, Wx, bx, lam = workloads.rglru_inputs(80, B, T, D, "bf16")
    cu = lambda a, dt=torch.bfloat16: torch.from_numpy(a).cuda().to(dt)
    X, WA, WX = cu(x), cu(Wa), cu(Wx)
    BA, BX, LAM = cu(ba, torch.float32), cu(bx, torch.float32), cu(lam, torch.float32)
    Y = torch.empty_like(X)
    hT = torch.empty((B, D), device="cuda")
    ws = torch.empty(msr.msr_rglru_workspace_bytes(1, B, T, D), dtype=torch.uint8, device="cuda")
    fn = lambda: msr.msr_rglru_fwd(X, WA, BA, WX, BX, LAM, h_last=hT, Y=Y, workspace=ws)
    t = gpu_time(fn, steps, warmup)
    tr = traced(fn, steps)
    M = B * T
    scan_bytes = M * D * 4 * 2            # x, r, i read once, y written once (bf16)
    res = {"workload": f"rglru_bf16_b{B}_n{T}_d{D}", "ms_per_step": round(t * 1e3, 4),
           "tokens_per_s": round(M / t, 1),
           "kernels": {"k_gemm": roof("k_gemm", 2 * M * 2 * D * D, "mfma", tr, steps, workload=f"rglru_bf16_b{B}_n{T}_d{D}"),
                       "k_rglru_scan": roof("k_rglru_scan", scan_bytes, "hbm", tr, steps,
                                            workload=f"rglru_bf16_b{B}_n{T}_d{D}")}}
    del X, WA, WX, Y, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(steps_timed, warmup):
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    w = workloads.WORKLOADS["decode_fp32_b128_h16"]
    B, H, d, C = w.batch, w.heads, w.d_k, w.chunk
    g = workloads.gammas(H)
    s = 1 / math.sqrt(d)
    out = {}
    for ctx in (w.context, 1024):
        S = torch.empty((B, H, d, d), device="cuda")
        sl = 16
        ws = torch.empty(msr.msr_chunkwise_workspace_bytes(0, sl, ctx, H, d, d, C, w.rope_base), dtype=torch.uint8,
                         device="cuda")
        for b0 in range(0, B, sl):  # prefill in batch slices (inputs drawn on the device, seeded)
            q, k, v = (workloads.device_normal((sl, ctx, H, d), seed=100000 * i + b0 + ctx) for i in range(1, 4))
            msr.msr_chunkwise_fwd(q, k, v, g, C, rope_base=w.rope_base, qk_scale=s, S_out=S[b0:b0 + sl],
                                  workspace=ws)
            del q, k, v
        del ws
        n = steps_timed if ctx == w.context else max(64, steps_timed // 8)
        qs, ks, vs = (workloads.device_normal((n, B, H, d), seed=200000 * i + ctx) for i in range(1, 4))
        o = torch.empty((B, H, d), device="cuda")
        Sw = S.clone()
        for t in range(warmup):
            msr.msr_recurrent_step(qs[t % n], ks[t % n], vs[t % n], Sw, g, pos=ctx, rope_base=w.rope_base,
                                   qk_scale=s, o=o)
        del Sw
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(n):
            msr.msr_recurrent_step(qs[t], ks[t], vs[t], S, g, pos=ctx + t, rope_base=w.rope_base, qk_scale=s, o=o)
        e1.record()
        torch.cuda.synchronize()
        ts = e0.elapsed_time(e1) * 1e-3 / n
        byts = B * H * (2 * d * d * 4 + 4 * d * 4)
        entry = {"context": ctx, "steps": n, "us_per_step": round(ts * 1e6, 2), "steps_per_s": round(1 / ts, 1),
                 "tokens_per_s": round(B / ts, 1), "GB_per_s": round(byts / ts / 1e9, 1),
                 "hbm_frac": round(byts / ts / PEAK_HBM, 4), "bytes_per_step": byts}
        if ctx == w.context:
            tr = traced(lambda: msr.msr_recurrent_step(qs[0], ks[0], vs[0], S, g, pos=ctx + n, rope_base=w.rope_base,
                                                       qk_scale=s, o=o), min(n, 128))
            entry["roofline"] = roof("k_recurrent_step", byts, "hbm", tr, min(n, 128), workload=w.name)
        out[str(ctx)] = entry
        del S, qs, ks, vs, o
        torch.cuda.empty_cache()
    a, b = out[str(w.context)]["us_per_step"], out["1024"]["us_per_step"]
    out["length_ratio_8192_vs_1024"] = round(a / b, 4)
    return out


def bench_layer_decode(n_steps, warmup):
    """Gated layer decode step at the decode workload's shape (batch 128,
    d_model 4096, 16 heads of 256; bf16 tokens and weights, float32 state):
    projections, rotation, state update, GroupNorm, gate, W_O per step.
    n_steps consecutive steps between two events (the rate), then the same
    steps with an event pair around each (the median step) and the host's
    issue time per step (wall time to enqueue the steps, before waiting)."""
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    w = workloads.WORKLOADS["decode_fp32_b128_h16"]
    B, dm, H, dk, dv = w.batch, w.d_model, w.heads, w.d_k, w.d_v
    g = workloads.gammas(H)
    s = dm ** -0.5
    W = [(workloads.device_normal(shp, seed=910 + i) * s).to(torch.bfloat16)
         for i, shp in enumerate([(dm, H * dk), (dm, H * dk), (dm, H * dv), (dm, H * dv)])]
    WO = (workloads.device_normal((H * dv, dm), seed=920) * (H * dv) ** -0.5).to(torch.bfloat16)
    S = workloads.device_normal((B, H, dk, dv), seed=930) * 0.5
    xs = workloads.device_normal((n_steps, B, dm), seed=940).to(torch.bfloat16)
    out = torch.empty((B, dm), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(msr.msr_layer_decode_workspace_bytes(1, B, dm, H, dk, dv), dtype=torch.uint8, device="cuda")
    step = lambda t: msr.msr_layer_decode_step(xs[t % n_steps], *W, WO, S, g, H, dk, dv, w.context + t,
                                               rope_base=w.rope_base, gn_eps=1e-5, out=out, workspace=ws)
    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h0 = time.perf_counter()
    for t in range(n_steps):
        step(t)
    host_issue = (time.perf_counter() - h0) / n_steps
    e1.record()
    torch.cuda.synchronize()
    ts = e0.elapsed_time(e1) * 1e-3 / n_steps
    med, mn = step_stats(lambda: step(0), n_steps)
    tr = traced(lambda: step(0), n_steps)
    wbytes = (dm * (2 * H * dk + 2 * H * dv) + H * dv * dm) * 2
    byts = B * H * dk * dv * 4 * 2 + wbytes + B * dm * 2 * 2
    ksum = sum(v[0] for v in tr.values()) / n_steps
    res = {"batch": B, "d_model": dm, "heads": H, "d_k": dk, "d_v": dv, "steps": n_steps,
           "us_per_step": round(ts * 1e6, 2), "us_per_step_median": round(med * 1e6, 2),
           "us_per_step_min": round(mn * 1e6, 2), "host_issue_us_per_step": round(host_issue * 1e6, 2),
           "kernel_sum_us_per_step": round(ksum * 1e6, 2),
           "steps_per_s": round(1 / ts, 1), "tokens_per_s": round(B / ts, 1),
           "GB_per_s": round(byts / ts / 1e9, 1), "hbm_frac": round(byts / ts / PEAK_HBM, 4), "bytes_per_step": byts,
           "trace_us_per_step": {k: round(v[0] / n_steps * 1e6, 2) for k, v in tr.items()}}
    del W, WO, S, xs, out, ws
    torch.cuda.empty_cache()
    return res


def bench_retnet_block(steps, warmup):
    """RetNet block (LayerNorm, the gated layer, residual, LayerNorm, gelu
    feed-forward network of width 2 d_model, residual) at the headline
    layer's shape, bf16."""
    import torch
    import linear_recurrence_sequence_amd as msr
    import workloads
    w = workloads.WORKLOADS["layer_bf16_b8_n2048"]
    F = 2 * w.d_model
    X, WQ, WK, WV, WG, WO = make_layer(w, True)
    s = w.d_model ** -0.5
    W1 = (workloads.device_normal((w.d_model, F), seed=950) * s).to(torch.bfloat16)
    W2 = (workloads.device_normal((F, w.d_model), seed=951) * F ** -0.5).to(torch.bfloat16)
    g = workloads.gammas(w.heads)
    out = torch.empty_like(X)
    ws = torch.empty(msr.msr_retnet_block_workspace_bytes(1, w.batch, w.seqlen, w.d_model, w.heads, w.d_k, w.d_v,
                                                          w.chunk, F), dtype=torch.uint8, device="cuda")
    fn = lambda: msr.msr_retnet_block_fwd(X, WQ, WK, WV, WG, WO, W1, W2, g, w.heads, w.d_k, w.d_v, w.chunk,
                                          rope_base=w.rope_base, out=out, workspace=ws)
    t = gpu_time(fn, steps, warmup)
    tr = traced(fn, steps)
    proj, core = layer_flops(w.batch, w.seqlen, w.d_model, w.heads, w.d_k, w.d_v, w.chunk)
    ffn = w.batch * w.seqlen * 2 * 2 * w.d_model * F
    fl = proj + core + ffn
    del X, WQ, WK, WV, WG, WO, W1, W2, out, ws
    torch.cuda.empty_cache()
    return {"d_ffn": F, "tokens_per_s": round(w.batch * w.seqlen / t, 1), "ms_per_step": round(t * 1e3, 3),
            "tflops": round(fl / t / 1e12, 1), "mfma_frac": round(fl / t / PEAK_BF16, 4),
            "trace_ms_per_step": {k: round(v[0] / steps * 1e3, 4) for k, v in tr.items()}}


def bench_copy(nbytes=1 << 30, reps=8):
    """A plain device-to-device copy of a known size: the calibration run for
    the FETCH_SIZE / WRITE_SIZE counters (each reads nbytes and writes nbytes
    per launch)."""
    import torch
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    t = gpu_time(lambda: dst.copy_(src), reps, 2)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": round(t * 1e6, 1),
            "GB_per_s": round(2 * nbytes / t / 1e9, 1)}


def cpu_baseline(budget_s=10.0):
    """The float64 oracle on a bounded sample of the headline workload:
    the whole layer on batch element 0 (8192 tokens; causal, so it is the
    exact first quarter of the batch), repeated until at least budget_s
    seconds of CPU work are done."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    w = workloads.WORKLOADS["block_bf16_b4_n8192"]
    # the workload's recipe drawn at batch 1: the same shapes and
    # distributions (the cost of the oracle does not depend on the values)
    X, WQ, WK, WV, WG, WO = workloads.layer_inputs(w, batch=1)
    g = workloads.gammas(w.heads)
    t0 = time.perf_counter()
    done = 0
    while True:
        oracle.msr_layer(X[0:1], WQ, WK, WV, WG, WO, g, w.heads, w.d_k, w.d_v, w.chunk, rope_base=w.rope_base,
                         eps=1e-5)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    t = time.perf_counter() - t0
    return {"value": round(done * w.seqlen / t, 1), "unit": "tokens/s", "cores": threads,
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{done} pass(es) of the whole layer over one batch element ({w.seqlen} tokens, the "
                      f"headline workload's recipe drawn at batch 1) of {w.name}, float64 numpy, {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="layer,decode,small,long,retnet,backward,rglru,cpu")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): this library has no "
              f"multi-GPU path (one process, one GPU).", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    parts = set(args.only.split(","))
    if args.no_cpu:
        parts.discard("cpu")
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} CUs={props.multi_processor_count}")

    w = workloads.WORKLOADS["block_bf16_b4_n8192"]
    line = {"metric": "MSR fwd tokens/s + %MFMA peak (chunkwise); decode steps/s + %HBM peak",
            "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded Gaussian inputs and random-init weights)",
            "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "d_model": w.d_model,
                       "heads": w.heads, "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk, "form": "chunkwise",
                       "step": "gated MSR layer forward"}}
    if "layer" in parts:
        log("layer", w.name)
        r = bench_layer(w, args.steps, args.warmup, device_inputs=True)
        line["value"] = round(r["tokens_per_s"], 1)
        line["ms_per_step"] = round(r["s_per_step"] * 1e3, 4)
        line["ms_per_step_median"] = round(r["s_per_step_median"] * 1e3, 4)   # single-call events, a pass after
        line["ms_per_step_min"] = round(r["s_per_step_min"] * 1e3, 4)
        line["mfma_frac"] = round(r["mfma_frac"], 4)
        line["tflops"] = round(r["tflops"], 1)
        k = r["kernels"]
        dom = max(k, key=lambda n: r["trace_s_per_step"].get(n, 0))
        line["roofline"] = {x: k[dom][x] for x in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
        line["roofline"]["kernel"] = dom
        line["chunkwise"] = r["chunkwise"]
        line["kernels"] = k
        line["trace_ms_per_step"] = {n: round(v * 1e3, 4) for n, v in r["trace_s_per_step"].items()}
        # the chunkwise core alone at this shape (projected Q, K, V; d_v = 512)
        bc = bench_core(w.batch, w.seqlen, w.heads, w.d_k, w.chunk, max(3, args.steps // 2), 2, dv=w.d_v,
                        workload=w.name + ":core")
        line["core_chunkwise"] = {
            "tokens_per_s": round(bc["tokens_per_s"], 1), "us_per_step": round(bc["s"] * 1e6, 1),
            "tflops": round(bc["tflops"], 1), "mfma_frac": round(bc["mfma_frac"], 4), "kernels": bc["kernels"]}
    if "decode" in parts:
        log("decode")
        line["decode"] = bench_decode(512, 16)
        log("layer decode")
        line["layer_decode"] = bench_layer_decode(512, 16)
    if "small" in parts:
        sw = workloads.WORKLOADS["layer_bf16_b8_n2048"]
        log("layer", sw.name)
        r = bench_layer(sw, args.steps, args.warmup)
        line["layer_b8_n2048"] = {"tokens_per_s": round(r["tokens_per_s"], 1), "mfma_frac": round(r["mfma_frac"], 4),
                                  "ms_per_step": round(r["s_per_step"] * 1e3, 4), "tflops": round(r["tflops"], 1),
                                  "chunkwise": r["chunkwise"], "kernels": r["kernels"]}
    if "long" in parts:
        log("long")
        lw = workloads.WORKLOADS["long_bf16_b2_n16384"]
        long = {"core_chunkwise": bench_core(lw.batch, lw.seqlen, lw.heads, lw.d_k, lw.chunk, args.steps,
                                             args.warmup, workload=lw.name + ":core"),
                "core_chunkwise_rotated": bench_core(lw.batch, lw.seqlen, lw.heads, lw.d_k, lw.chunk, args.steps,
                                                     args.warmup, rope_base=lw.rope_base)}
        sweep = []
        for N in (1024, 2048, 4096, 8192, 16384):
            c = bench_core(lw.batch, N, lw.heads, lw.d_k, lw.chunk, 5, 2)
            p = bench_core(lw.batch, N, lw.heads, lw.d_k, lw.chunk, 3, 1, parallel=True)
            sweep.append({"N": N, "chunkwise_us": round(c["s"] * 1e6, 1), "parallel_us": round(p["s"] * 1e6, 1),
                          "chunkwise_tflops": round(c["tflops"], 1), "parallel_tflops": round(p["tflops"], 1)})
        long["sweep"] = sweep
        lr = bench_layer(lw, max(3, args.steps // 4), 2, device_inputs=True)
        long["layer"] = {"tokens_per_s": round(lr["tokens_per_s"], 1), "mfma_frac": round(lr["mfma_frac"], 4),
                         "ms_per_step": round(lr["s_per_step"] * 1e3, 3), "chunkwise": lr["chunkwise"]}
        line["long"] = long
    # single cores for counter passes: the chunkwise and the parallel form at
    # the long workload's and the headline workload's shapes
    for tag, wname, par in (("core3", "long_bf16_b2_n16384", False), ("core5", "block_bf16_b4_n8192", False),
                            ("par3", "long_bf16_b2_n16384", True), ("par5", "block_bf16_b4_n8192", True)):
        if tag in parts:
            cw = workloads.WORKLOADS[wname]
            log(tag, cw.name)
            r = bench_core(cw.batch, cw.seqlen, cw.heads, cw.d_k, cw.chunk, args.steps, args.warmup, parallel=par,
                           dv=cw.d_v)
            line.setdefault("cores", {})[tag] = {
                "workload": cw.name, "form": "parallel" if par else "chunkwise", "us_per_step": round(r["s"] * 1e6, 1),
                "tflops": round(r["tflops"], 1), "mfma_frac": round(r["mfma_frac"], 4),
                "trace_us_per_step": r.get("trace_us_per_step")}
    if "retnet" in parts:
        log("retnet block")
        line["retnet_block"] = bench_retnet_block(max(3, args.steps // 2), 2)
    if "backward" in parts:
        log("backward")
        lw = workloads.WORKLOADS["long_bf16_b2_n16384"]
        line["backward"] = {
            "headline_core": bench_backward(w.batch, w.seqlen, w.heads, w.d_k, w.chunk, args.steps, args.warmup),
            "long_core": bench_backward(lw.batch, lw.seqlen, lw.heads, lw.d_k, lw.chunk, max(3, args.steps // 2), 2)}
    if "rglru" in parts:
        log("rglru")
        line["rglru"] = bench_rglru(8, 2048, 2048, args.steps, args.warmup)
    if "copy" in parts:
        log("copy calibration")
        line["copy_calibration"] = bench_copy()
    if "cpu" in parts:
        log("cpu baseline")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
