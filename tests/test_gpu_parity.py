"""GPU (HIP, gfx950) results against the float64 oracle on the same seeded
inputs, through the C ABI.  Small and ragged shapes spanning several tiles,
every supported head-dim combination, both dtypes."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, first_token_bound, layer_err, say

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (256, 256), (256, 512)]
GAMMAS = [1 - 2.0 ** -5, 0.5, 1.0, 1 - 2.0 ** -12, 0.0]


def _msr():
    import linear_recurrence_sequence_amd as msr
    return msr


def _gam(H):
    return np.array([GAMMAS[h % len(GAMMAS)] for h in range(H)])


# ------------------------------------------------------------- recurrent ---
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", DIMS)
def test_recurrent_steps(dtype, dk, dv):
    import torch
    msr = _msr()
    B, H, steps, pos0, base = 3, 5, 4, 1000, 10000.0
    rng = np.random.default_rng(7)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    q, k, v = workloads.core_inputs(8, B, steps, H, dk, dv, dtype)
    g = _gam(H)
    scale = 1 / math.sqrt(dk)
    S = torch.from_numpy(S0).cuda()
    Sref = S0.astype(np.float64)
    for t in range(steps):
        say("recurrent", dtype, dk, dv, "step", t)
        o = msr.msr_recurrent_step(dev(q[:, t], dtype), dev(k[:, t], dtype), dev(v[:, t], dtype), S, g,
                                   pos=pos0 + t, rope_base=base, qk_scale=scale)
        oref, Sref = oracle.recurrent_step(Sref, q[:, t], k[:, t], v[:, t], g, scale, pos=pos0 + t, base=base)
        torch.cuda.synchronize()
        assert oracle.max_rel_err_per_head(host(o)[:, None], oref[:, None]) < TOL[dtype]
    assert oracle.max_rel_err(host(S), Sref) < 1e-5


# ------------------------------------------------------------- chunkwise ---
# (the bf16 d_k 256 forms with a chunk that is a multiple of 128 run the
# 16-rows-per-wave output kernel: 130 leaves a second row tile with two rows,
# most of its waves without any; 777 / 384 three row tiles and a ragged chunk)
CHUNK_CASES = [(200, 64), (256, 128), (97, 32), (300, 96), (1, 32), (513, 256), (130, 128), (777, 384)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("N,chunk", CHUNK_CASES)
def test_chunkwise(dtype, dk, dv, N, chunk):
    import torch
    msr = _msr()
    B, H = 2, 3
    if dtype == "f32" and dv == 512:
        with pytest.raises(msr.MsrError, match="UNSUPPORTED"):
            q = torch.zeros((B, N, H, dk), device="cuda")
            msr.msr_chunkwise_fwd(q, q, torch.zeros((B, N, H, dv), device="cuda"), _gam(H), chunk)
        return
    q, k, v = workloads.core_inputs(11, B, N, H, dk, dv, dtype)
    S0 = np.random.default_rng(12).standard_normal((B, H, dk, dv)).astype(np.float32)
    g = np.array([0.9, 1 - 2.0 ** -5, 1 - 2.0 ** -12])
    scale, pos0, base = 1 / math.sqrt(dk), 5, 10000.0
    S_out = torch.empty((B, H, dk, dv), device="cuda")
    say("chunkwise", dtype, dk, dv, N, chunk)
    O = msr.msr_chunkwise_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, chunk, rope_base=base, pos0=pos0,
                              qk_scale=scale, S_in=torch.from_numpy(S0).cuda(), S_out=S_out)
    torch.cuda.synchronize()
    qr, kr = oracle.rotary(q, pos0, base), oracle.rotary(k, pos0, base)
    Oref, Sref = oracle.retention_chunkwise(qr, kr, v, g, chunk, scale, S0)
    assert oracle.max_rel_err_per_head(host(O), Oref) < TOL[dtype]
    assert oracle.max_rel_err(host(S_out), Sref) < (1e-4 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("dv,chunk", [(512, 512), (256, 256)])
def test_chunkwise_paired_tiles_ragged(dv, chunk):
    """Enough (batch, head, chunk) units that each workgroup of the 16-row
    output kernel walks several tiles, so that the backward-walked row tiles
    (key blocks from the diagonal down, Q R_{i-1} last with Q pre-scaled)
    run beside the forward-walked ones, with a ragged last chunk and an
    initial state: batch 4, 3000 tokens, 16 heads, d_k 256, bf16, no
    rotation; the last batch element against the oracle (outputs per head,
    final states)."""
    import torch
    msr = _msr()
    B, N, H, dk = 4, 3000, 16, 256
    q, k, v = workloads.core_inputs(71, B, N, H, dk, dv, "bf16")
    S0 = np.random.default_rng(72).standard_normal((B, H, dk, dv)).astype(np.float32)
    g = workloads.gammas(H)
    scale = 1 / math.sqrt(dk)
    S_out = torch.empty((B, H, dk, dv), device="cuda")
    say("chunkwise paired tiles, ragged", dv, chunk)
    O = msr.msr_chunkwise_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), g, chunk, qk_scale=scale,
                              S_in=torch.from_numpy(S0).cuda(), S_out=S_out)
    torch.cuda.synchronize()
    Oref, Sref = oracle.retention_chunkwise(q[3:], k[3:], v[3:], g, chunk, scale, S0[3:])
    err = oracle.max_rel_err_per_head(host(O)[3:], Oref)
    print(f"paired tiles d_v {dv} chunk {chunk}: max rel err per head {err:.3e}", flush=True)
    assert err < TOL["bf16"]
    assert oracle.max_rel_err(host(S_out)[3:], Sref) < 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunkwise_special_gammas_no_state(dtype):
    """gamma = 0, 0.5 and 1 (the degenerate decays), no initial state, no
    rotation, scale 1, ragged sequence."""
    import torch
    msr = _msr()
    B, N, H, d = 2, 161, 5, 64
    q, k, v = workloads.core_inputs(13, B, N, H, d, d, dtype)
    g = _gam(H)
    say("chunkwise-special", dtype)
    S_out = torch.empty((B, H, d, d), device="cuda")
    O = msr.msr_chunkwise_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, 64, S_out=S_out)
    torch.cuda.synchronize()
    Oref, Sref = oracle.retention_recurrent(q, k, v, g)
    assert oracle.max_rel_err_per_head(host(O), Oref) < TOL[dtype]
    assert oracle.max_rel_err(host(S_out), Sref) < (1e-4 if dtype == "f32" else 1e-2)


# Shapes with enough (batch, head) pairs for the one-pass state kernel (no
# rotation; every state tile walks the chunks in order): 256 x 128 and
# 128 x 128 tiles, d_k 128 and 256, ragged last chunks (also shorter than a
# key block), the degenerate decays.
STATE_WALK_CASES = [(256, 512, 4, 16, 1000, 256), (256, 256, 2, 24, 700, 128), (128, 128, 16, 12, 333, 64),
                    (256, 512, 2, 12, 260, 128)]


@pytest.mark.parametrize("dk,dv,B,H,N,chunk", STATE_WALK_CASES)
def test_chunkwise_state_walk(dk, dv, B, H, N, chunk):
    """bf16 msr_chunkwise_fwd_save with an initial state and the final
    state: the run takes the one-pass state kernel (no separate scan), and on
    sampled (batch, head) slices -- heads with gamma 1 - 2^-5, 0.5, 1, 0 --
    O, every kept chunk state R_{i-1} and S_out match the oracle."""
    import torch
    msr = _msr()
    q, k, v = workloads.core_inputs(17 + dk + dv, B, N, H, dk, dv, "bf16")
    S0 = np.random.default_rng(18).standard_normal((B, H, dk, dv)).astype(np.float32)
    g = _gam(H)
    scale = 1 / math.sqrt(dk)
    R = torch.empty(msr.msr_chunkwise_states_shape(B, N, H, dk, dv, chunk), dtype=torch.bfloat16, device="cuda")
    S_out = torch.empty((B, H, dk, dv), device="cuda")
    say("state walk", dk, dv, B, H, N, chunk)
    msr.msr_trace_enable(True)
    try:
        O = msr.msr_chunkwise_fwd_save(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), g, chunk, R, qk_scale=scale,
                                       S_in=torch.from_numpy(S0).cuda(), S_out=S_out)
        torch.cuda.synchronize()
        tot = msr.trace_totals()
    finally:
        msr.msr_trace_enable(False)
    assert "k_chunk_rscan" in tot and "k_chunk_scan" not in tot and "k_chunk_state" not in tot
    for b, h in ((0, 0), (B - 1, 1), (1, 2), (B // 2, 4), (B - 1, H - 1)):
        sl = lambda a: a[b:b + 1, :, h:h + 1]
        S0s = S0[b:b + 1, h:h + 1]
        Oref, Sref = oracle.retention_chunkwise(sl(q), sl(k), sl(v), g[h:h + 1], chunk, scale, S0s)
        assert oracle.max_rel_err_per_head(host(O[b:b + 1, :, h:h + 1]), Oref) < TOL["bf16"], (b, h)
        assert oracle.max_rel_err(host(S_out[b:b + 1, h:h + 1]), Sref) < 1e-2, (b, h)
        for i in range(R.shape[2]):
            c0 = i * chunk
            ref = S0s if c0 == 0 else oracle.retention_chunkwise(sl(q)[:, :c0], sl(k)[:, :c0], sl(v)[:, :c0],
                                                                 g[h:h + 1], chunk, scale, S0s)[1]
            got = np.swapaxes(host(R[b:b + 1, h:h + 1, i]), -1, -2)
            assert oracle.max_rel_err(got, ref) < 1e-2, (b, h, i)


# -------------------------------------------------------------- parallel ---
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("N", [1, 33, 200, 300])
def test_parallel(dtype, dk, dv, N):
    import torch
    msr = _msr()
    B, H = 2, 3
    q, k, v = workloads.core_inputs(14, B, N, H, dk, dv, dtype)
    g = np.array([0.97, 1.0, 0.5])
    if dtype == "f32" and dv == 512:
        # no float32 matrix-core kernel for 512-wide value heads: the call
        # fails with MSR_ERR_UNSUPPORTED (4) and launches nothing
        with pytest.raises(msr.MsrError) as ei:
            msr.msr_parallel_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, rope_base=500.0, pos0=3,
                                 qk_scale=0.25)
        assert ei.value.status == 4 and "float32" in str(ei.value)
        return
    say("parallel", dtype, dk, dv, N)
    O = msr.msr_parallel_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, rope_base=500.0, pos0=3,
                             qk_scale=0.25)
    torch.cuda.synchronize()
    Oref = oracle.retention_parallel(oracle.rotary(q, 3, 500.0), oracle.rotary(k, 3, 500.0), v, g, 0.25)
    # A one-token slice is a single score q.k; in bf16 the rotated q, k are
    # rounded to bf16 (matrix-core operands), so a score with heavy
    # cancellation carries ~2^-9 sqrt(sum (q_i k_i)^2) absolute error: such
    # slices are measured against the whole tensor instead.
    err = oracle.max_rel_err(host(O), Oref) if N == 1 else oracle.max_rel_err_per_head(host(O), Oref)
    assert err < TOL[dtype]


# ----------------------------------------------------------------- layer ---
def _layer(dtype, B, N, dm, H, dk, dv, chunk, seed):
    w = workloads.Workload("t", dtype, B, N, dm, H, dk, dv, chunk, seed=seed)
    return workloads.layer_inputs(w)


@pytest.mark.parametrize("dtype,B,N,dm,H,dk,dv,chunk", [
    ("f32", 1, 256, 256, 4, 64, 64, 64),         # the fp32 single-layer workload
    ("f32", 2, 150, 128, 2, 64, 64, 32),
    ("bf16", 2, 300, 256, 2, 128, 128, 128),
    ("bf16", 1, 200, 256, 2, 256, 512, 64),
    ("bf16", 2, 300, 256, 2, 256, 512, 128),     # GroupNorm + gate fused, 512-wide value heads
    ("bf16", 1, 260, 256, 3, 256, 256, 256),
    # sequences shorter than a projection wave's 128 rows: the rotation's
    # table row is then taken per row rather than from the wave's first one
    ("bf16", 4, 40, 256, 2, 128, 128, 32),
    ("f32", 3, 60, 128, 2, 64, 64, 32),
    # 100 tokens: the output projection (no epilogue option) runs on the
    # skinny direct-copy tiles, rows past the 100th clamped and not stored
    ("bf16", 1, 100, 256, 2, 128, 128, 32),
])
def test_layer(dtype, B, N, dm, H, dk, dv, chunk):
    import torch
    msr = _msr()
    X, WQ, WK, WV, WG, WO = _layer(dtype, B, N, dm, H, dk, dv, chunk, 0)
    g = workloads.gammas(H)
    say("layer", dtype, B, N, dm, H, dk, dv, chunk)
    out = msr.msr_layer_fwd(*(dev(a, dtype) for a in (X, WQ, WK, WV, WG, WO)), g, H, dk, dv, chunk,
                            rope_base=10000.0, gn_eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.msr_layer(X, WQ, WK, WV, WG, WO, g, H, dk, dv, chunk, rope_base=10000.0, eps=1e-5)
    bound0 = first_token_bound(X, WQ, WK, WV, WG, WO, H, dk, dv, dtype, 1e-5)
    err, excluded = layer_err(host(out), ref, bound0, dtype)
    print(f"layer {dtype} err {err:.2e}, excluded first-token rows {excluded}", flush=True)
    assert err < TOL[dtype]


def test_fp32_workload_three_forms():
    """The fp32 single-layer workload (batch 1, 256 tokens, d_model 256, 4
    heads of 64, chunk 64): the GPU parallel, chunkwise and recurrent forms on
    the layer's rotated projections all match the oracle, and each other."""
    import torch
    msr = _msr()
    w = workloads.WORKLOADS["layer_fp32_b1_n256"]
    X, WQ, WK, WV, WG, WO = workloads.layer_inputs(w)
    H, d = w.heads, w.d_k
    g = workloads.gammas(H)
    q = (X.astype(np.float64) @ WQ).reshape(1, w.seqlen, H, d).astype(np.float32)
    k = (X.astype(np.float64) @ WK).reshape(1, w.seqlen, H, d).astype(np.float32)
    v = (X.astype(np.float64) @ WV).reshape(1, w.seqlen, H, d).astype(np.float32)
    s = 1 / math.sqrt(d)
    say("fp32 workload three forms")
    Qd, Kd, Vd = dev(q, "f32"), dev(k, "f32"), dev(v, "f32")
    o_par = msr.msr_parallel_fwd(Qd, Kd, Vd, g, rope_base=w.rope_base, qk_scale=s)
    o_chk = msr.msr_chunkwise_fwd(Qd, Kd, Vd, g, w.chunk, rope_base=w.rope_base, qk_scale=s)
    S = torch.zeros((1, H, d, d), device="cuda")
    o_rec = torch.empty_like(o_par)
    for n in range(w.seqlen):
        o_rec[:, n] = msr.msr_recurrent_step(Qd[:, n].contiguous(), Kd[:, n].contiguous(), Vd[:, n].contiguous(),
                                             S, g, pos=n, rope_base=w.rope_base, qk_scale=s)
    torch.cuda.synchronize()
    ref = oracle.retention_parallel(oracle.rotary(q, 0, w.rope_base), oracle.rotary(k, 0, w.rope_base), v, g, s)
    for o in (o_par, o_chk, o_rec):
        assert oracle.max_rel_err_per_head(host(o), ref) < TOL["f32"]
    assert oracle.max_rel_err_per_head(host(o_chk), host(o_par)) < TOL["f32"]


# ----------------------------------------------------- continuation, misc --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_continuation_and_decode(dtype):
    """chunkwise over [0, M) -> S_out -> chunkwise over [M, N) with S_in and
    pos0 = M, then single recurrent steps: equal one oracle pass."""
    import torch
    msr = _msr()
    B, N, H, d, M, C = 2, 200, 2, 128, 130, 64
    q, k, v = workloads.core_inputs(15, B, N + 3, H, d, d, dtype)
    g = np.array([0.99, 1 - 2.0 ** -9])
    base, s = 10000.0, 1 / math.sqrt(d)
    say("split", dtype)
    S1 = torch.empty((B, H, d, d), device="cuda")
    S2 = torch.empty_like(S1)
    o1 = msr.msr_chunkwise_fwd(dev(q[:, :M], dtype), dev(k[:, :M], dtype), dev(v[:, :M], dtype), g, C,
                               rope_base=base, qk_scale=s, S_out=S1)
    o2 = msr.msr_chunkwise_fwd(dev(q[:, M:N], dtype), dev(k[:, M:N], dtype), dev(v[:, M:N], dtype), g, C,
                               rope_base=base, pos0=M, qk_scale=s, S_in=S1, S_out=S2)
    o3 = [msr.msr_recurrent_step(dev(q[:, n], dtype), dev(k[:, n], dtype), dev(v[:, n], dtype), S2, g, pos=n,
                                 rope_base=base, qk_scale=s) for n in range(N, N + 3)]
    torch.cuda.synchronize()
    ref, _ = oracle.retention_chunkwise(oracle.rotary(q, 0, base), oracle.rotary(k, 0, base), v, g, C, s)
    got = np.concatenate([host(o1), host(o2), np.stack([host(o) for o in o3], 1)], 1)
    assert oracle.max_rel_err_per_head(got, ref) < TOL[dtype]


def test_empty_sequence_passes_state_through():
    import torch
    msr = _msr()
    S0 = torch.randn((2, 3, 64, 64), device="cuda")
    S1 = torch.full_like(S0, 7.0)
    z = torch.empty((2, 0, 3, 64), device="cuda")
    msr.msr_chunkwise_fwd(z, z, z, [0.5, 0.6, 0.7], 32, S_in=S0, S_out=S1)
    torch.cuda.synchronize()
    assert torch.equal(S0, S1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic(dtype):
    """No atomics: two runs are bit-identical."""
    import torch
    msr = _msr()
    q, k, v = workloads.core_inputs(16, 2, 777, 4, 128, 128, dtype)
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    a = msr.msr_chunkwise_fwd(Q, K, V, _gam(4), 128, rope_base=10000.0)
    b = msr.msr_chunkwise_fwd(Q, K, V, _gam(4), 128, rope_base=10000.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
