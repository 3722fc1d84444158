"""Parity at the full workload sizes, in the launch configuration bench.py
times, against the float64 oracle on sampled outputs it can compute: whole
batch elements for the layers and the long-sequence core, sampled (batch,
head) states and outputs for the decode step.  Properties that hold at any
size (chunkwise == parallel form on the GPU) cover the rest."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, first_token_bound, layer_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _msr():
    import linear_recurrence_sequence_amd as msr
    return msr


def _layer_check(name, batches):
    import torch
    msr = _msr()
    w = workloads.WORKLOADS[name]
    X, WQ, WK, WV, WG, WO = workloads.layer_inputs(w)
    g = workloads.gammas(w.heads)
    say("full layer", name)
    out = msr.msr_layer_fwd(*(dev(a, w.dtype) for a in (X, WQ, WK, WV, WG, WO)), g, w.heads, w.d_k, w.d_v, w.chunk,
                            rope_base=w.rope_base, gn_eps=1e-5)
    torch.cuda.synchronize()
    got = host(out)
    del out
    for b in batches:
        ref = oracle.msr_layer(X[b:b + 1], WQ, WK, WV, WG, WO, g, w.heads, w.d_k, w.d_v, w.chunk,
                               rope_base=w.rope_base, eps=1e-5)
        bound0 = first_token_bound(X[b:b + 1], WQ, WK, WV, WG, WO, w.heads, w.d_k, w.d_v, w.dtype, 1e-5)
        err, excluded = layer_err(got[b:b + 1], ref, bound0, w.dtype)
        print(f"{name} batch {b}: max rel err {err:.3e} (first-token rows excluded: {excluded}, "
              f"bound {bound0[0]:.2e})", flush=True)
        assert err < TOL[w.dtype]


def test_layer_b8_n2048_full():
    """bf16 layer, batch 8 x 2048 tokens, d_model 2048, 8 heads of 256, chunk 256."""
    _layer_check("layer_bf16_b8_n2048", [0, 7])


def test_layer_fp32_b1_n256_full():
    _layer_check("layer_fp32_b1_n256", [0])


def test_layer_long_b2_n16384_full():
    """bf16 layer, batch 2 x 16384 tokens, d_model 2560, 10 heads of 256,
    chunk 512 (the long-sequence workload's layer, as bench.py times it):
    batch element 1 against the oracle."""
    _layer_check("long_bf16_b2_n16384", [1])


def test_block_b4_n8192_full():
    """bf16 gated block, batch 4 x 8192 tokens, d_model 4096, 16 heads,
    q/k head dim 256, v head dim 512, chunk 512 (oracle on the last batch
    element: every chunk carry of an 8192-token sequence)."""
    _layer_check("block_bf16_b4_n8192", [3])


def test_long_core_chunkwise_vs_oracle_and_parallel():
    """Chunkwise core, batch 2 x 16384 tokens, 10 heads of 256, chunk 512:
    batch element 1 against the oracle per (batch, head), and the whole
    output against the GPU parallel form."""
    import torch
    msr = _msr()
    w = workloads.WORKLOADS["long_bf16_b2_n16384"]
    B, N, H, d, C = w.batch, w.seqlen, w.heads, w.d_k, w.chunk
    q, k, v = workloads.core_inputs(31, B, N, H, d, d, "bf16")
    g = workloads.gammas(H)
    s = 1 / math.sqrt(d)
    say("full long core")
    Qd, Kd, Vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    S_out = torch.empty((B, H, d, d), device="cuda")
    o_c = msr.msr_chunkwise_fwd(Qd, Kd, Vd, g, C, qk_scale=s, S_out=S_out)
    o_p = msr.msr_parallel_fwd(Qd, Kd, Vd, g, qk_scale=s)
    torch.cuda.synchronize()
    assert oracle.max_rel_err_per_head(host(o_c), host(o_p)) < TOL["bf16"]
    ref, Sref = oracle.retention_chunkwise(q[1:], k[1:], v[1:], g, C, s)
    err = oracle.max_rel_err_per_head(host(o_c)[1:], ref)
    err_p = oracle.max_rel_err_per_head(host(o_p)[1:], ref)
    print(f"long core batch 1: max rel err per head {err:.3e} (chunkwise), {err_p:.3e} (parallel)", flush=True)
    assert err < TOL["bf16"] and err_p < TOL["bf16"]
    assert oracle.max_rel_err(host(S_out)[1:], Sref) < 1e-2


def test_block_core_parallel_vs_chunkwise_and_oracle():
    """The block workload's core shape (batch 4 x 8192 tokens, 16 heads,
    d_k 256, d_v 512) through the parallel form -- one chunk of 64 row tiles
    on the paired 16-row output kernel, as bench.py times it -- against the
    chunkwise form everywhere and against the oracle on batch element 2."""
    import torch
    msr = _msr()
    w = workloads.WORKLOADS["block_bf16_b4_n8192"]
    B, N, H, dk, dv = w.batch, w.seqlen, w.heads, w.d_k, w.d_v
    q, k, v = workloads.core_inputs(33, B, N, H, dk, dv, "bf16")
    g = workloads.gammas(H)
    s = 1 / math.sqrt(dk)
    say("block core parallel vs chunkwise")
    Qd, Kd, Vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o_p = msr.msr_parallel_fwd(Qd, Kd, Vd, g, qk_scale=s)
    o_c = msr.msr_chunkwise_fwd(Qd, Kd, Vd, g, w.chunk, qk_scale=s)
    torch.cuda.synchronize()
    e_pc = oracle.max_rel_err_per_head(host(o_p), host(o_c))
    ref, _ = oracle.retention_chunkwise(q[2:3], k[2:3], v[2:3], g, w.chunk, s)
    e_p = oracle.max_rel_err_per_head(host(o_p)[2:3], ref)
    print(f"block core: parallel vs chunkwise {e_pc:.3e}, parallel vs oracle (batch 2) {e_p:.3e}", flush=True)
    assert e_pc < TOL["bf16"] and e_p < TOL["bf16"]


def test_parallel_dv256_4096_tokens_paired_tiles():
    """The parallel form at d_v 256 and 4096 tokens -- one chunk of 32 row
    tiles on the paired 16-row output kernel -- at the long workload's head
    shape (batch 2, 10 heads of 256): batch element 1 against the oracle,
    everything against the GPU chunkwise form (chunk 512)."""
    import torch
    msr = _msr()
    B, N, H, d = 2, 4096, 10, 256
    q, k, v = workloads.core_inputs(34, B, N, H, d, d, "bf16")
    g = workloads.gammas(H)
    s = 1 / math.sqrt(d)
    say("parallel d_v 256, 4096 tokens")
    Qd, Kd, Vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o_p = msr.msr_parallel_fwd(Qd, Kd, Vd, g, qk_scale=s)
    o_c = msr.msr_chunkwise_fwd(Qd, Kd, Vd, g, 512, qk_scale=s)
    torch.cuda.synchronize()
    e_pc = oracle.max_rel_err_per_head(host(o_p), host(o_c))
    ref, _ = oracle.retention_chunkwise(q[1:], k[1:], v[1:], g, 512, s)
    e_p = oracle.max_rel_err_per_head(host(o_p)[1:], ref)
    print(f"parallel d_v 256 N 4096: vs chunkwise {e_pc:.3e}, vs oracle (batch 1) {e_p:.3e}", flush=True)
    assert e_pc < TOL["bf16"] and e_p < TOL["bf16"]


def test_layer_b8_n2048_chunkwise_equals_parallel():
    """The bf16 b8 x 2048 workload's core shape through both forms on the
    GPU (the layer runs the chunkwise one), each against the oracle on
    batch elements 2 and 7, and against each other everywhere."""
    import torch
    msr = _msr()
    w = workloads.WORKLOADS["layer_bf16_b8_n2048"]
    q, k, v = workloads.core_inputs(32, w.batch, w.seqlen, w.heads, w.d_k, w.d_v, "bf16")
    g = workloads.gammas(w.heads)
    s = 1 / math.sqrt(w.d_k)
    say("b8n2048 chunkwise vs parallel")
    Qd, Kd, Vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o_c = msr.msr_chunkwise_fwd(Qd, Kd, Vd, g, w.chunk, rope_base=w.rope_base, qk_scale=s)
    o_p = msr.msr_parallel_fwd(Qd, Kd, Vd, g, rope_base=w.rope_base, qk_scale=s)
    torch.cuda.synchronize()
    assert oracle.max_rel_err_per_head(host(o_c), host(o_p)) < TOL["bf16"]
    for b in (2, 7):
        ref = oracle.retention_parallel(oracle.rotary(q[b:b + 1], 0, w.rope_base),
                                        oracle.rotary(k[b:b + 1], 0, w.rope_base), v[b:b + 1], g, s)
        e_c = oracle.max_rel_err_per_head(host(o_c)[b:b + 1], ref)
        e_p = oracle.max_rel_err_per_head(host(o_p)[b:b + 1], ref)
        print(f"b8n2048 core batch {b}: chunkwise {e_c:.3e}, parallel {e_p:.3e}", flush=True)
        assert e_c < TOL["bf16"] and e_p < TOL["bf16"]


def test_decode_full_state_sampled():
    """Decode workload: fp32 state [128, 16, 256, 256] prefilled by the
    chunkwise kernel (chunk 512) from an 8192-token context drawn on the
    device, then 3 decode steps at positions 8192..8194 -- sampled (batch,
    head) outputs and states against the oracle's own prefill and steps."""
    import torch
    msr = _msr()
    w = workloads.WORKLOADS["decode_fp32_b128_h16"]
    B, H, d, C, ctx = w.batch, w.heads, w.d_k, w.chunk, w.context
    g = workloads.gammas(H)
    s = 1 / math.sqrt(d)
    sl = 16
    S = torch.empty((B, H, d, d), device="cuda")
    ws = torch.empty(msr.msr_chunkwise_workspace_bytes(0, sl, ctx, H, d, d, C, w.rope_base), dtype=torch.uint8,
                     device="cuda")
    gen = lambda i, b0: workloads.device_normal((sl, ctx, H, d), seed=100000 * i + b0 + ctx)
    say("decode prefill")
    for b0 in range(0, B, sl):
        qc, kc, vc = (gen(i, b0) for i in range(1, 4))
        msr.msr_chunkwise_fwd(qc, kc, vc, g, C, rope_base=w.rope_base, qk_scale=s, S_out=S[b0:b0 + sl], workspace=ws)
        del qc, kc, vc
    steps = 3
    qs, ks, vs = (workloads.device_normal((steps, B, H, d), seed=200000 * i + ctx) for i in range(1, 4))
    outs = []
    say("decode steps")
    for t in range(steps):
        outs.append(msr.msr_recurrent_step(qs[t], ks[t], vs[t], S, g, pos=ctx + t, rope_base=w.rope_base,
                                           qk_scale=s).cpu().numpy())
    torch.cuda.synchronize()
    samples = [(0, 0), (0, 15), (77, 3), (127, 15)]
    for b, h in samples:
        b0 = (b // sl) * sl
        qc, kc, vc = (host(gen(i, b0)[b - b0:b - b0 + 1, :, h:h + 1]) for i in range(1, 4))
        qr, kr = oracle.rotary(qc, 0, w.rope_base), oracle.rotary(kc, 0, w.rope_base)
        _, Sref = oracle.retention_chunkwise(qr, kr, vc, g[h:h + 1], C, s)
        for t in range(steps):
            o_ref, Sref = oracle.recurrent_step(Sref, host(qs[t, b:b + 1, h:h + 1]), host(ks[t, b:b + 1, h:h + 1]),
                                                host(vs[t, b:b + 1, h:h + 1]), g[h:h + 1], s, pos=ctx + t,
                                                base=w.rope_base)
            err = oracle.max_rel_err(outs[t][b, h], o_ref[0, 0])
            assert err < TOL["f32"], (b, h, t, err)
        errS = oracle.max_rel_err(host(S[b, h]), Sref[0, 0])
        print(f"decode (b={b}, h={h}): state rel err {errS:.2e}", flush=True)
        assert errS < TOL["f32"]
