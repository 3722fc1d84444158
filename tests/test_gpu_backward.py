"""Parity of the chunkwise backward (msr_chunkwise_bwd) against the float64
oracle's retention gradients (themselves pinned to finite differences of the
recurrent form): every supported head dim, ragged tails over several chunks,
initial state, final-state gradient and rotation, the degenerate decays, the
empty cases, and the headline core shape (batch 8, 2048 tokens, 8 heads of
256, bf16) on sampled (batch, head) slices."""

import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, say

pytestmark = pytest.mark.gpu

STATE_TOL = {"f32": 1e-4, "bf16": 1e-2}


def _msr():
    import linear_recurrence_sequence_amd as msr
    return msr


def _state_err(got, ref):
    """max over (batch, head) of the slice's max-abs-relative error."""
    return max(oracle.max_rel_err(got[b, h], ref[b, h]) for b in range(ref.shape[0]) for h in range(ref.shape[1]))


def _check(name, got, ref, tol):
    err = oracle.max_rel_err_per_head(got, ref)
    print(f"{name}: {err:.2e}", flush=True)
    assert np.all(np.isfinite(got)), name
    assert err < tol, (name, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,N,chunk", [(64, 200, 64), (64, 31, 32), (64, 400, 128), (128, 300, 128),
                                       (256, 257, 128), (256, 520, 256)])
def test_backward(dtype, d, N, chunk):
    import torch
    msr = _msr()
    B, H = 2, 3
    q, k, v = workloads.core_inputs(21 + d, B, N, H, d, d, dtype)
    rng = np.random.default_rng(22 + d)
    dO = workloads.normal(rng, (B, N, H, d), 1.0, dtype)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dS = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g = np.array([0.9, 1 - 2.0 ** -5, 1 - 2.0 ** -12])
    scale, pos0, base = 1 / math.sqrt(d), 5, 10000.0
    dS_in = torch.empty((B, H, d, d), device="cuda")
    say("backward", dtype, d, N, chunk)
    dQ, dK, dV = msr.msr_chunkwise_bwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(dO, dtype), g, chunk,
                                       rope_base=base, pos0=pos0, qk_scale=scale, S_in=torch.from_numpy(S0).cuda(),
                                       dS_out=torch.from_numpy(dS).cuda(), dS_in=dS_in)
    torch.cuda.synchronize()
    qr, kr = oracle.rotary(q, pos0, base), oracle.rotary(k, pos0, base)
    rq, rk, rv, rS = oracle.retention_grad(qr, kr, v, dO, g, scale, S0=S0, dS=dS)
    _check("dQ", host(dQ), oracle.rotary_adjoint(rq, pos0, base), TOL[dtype])
    _check("dK", host(dK), oracle.rotary_adjoint(rk, pos0, base), TOL[dtype])
    _check("dV", host(dV), rv, TOL[dtype])
    err = _state_err(host(dS_in), rS)
    print(f"dS_in: {err:.2e}", flush=True)
    assert err < STATE_TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk", [("f32", 64, 64), ("bf16", 64, 64), ("bf16", 256, 128)])
def test_backward_degenerate_decays_without_states(dtype, d, chunk):
    """gamma = 0, 0.5 and 1, no S_in, no dS_out, no rotation, scale 1,
    ragged sequence over several chunks (d 256: the 16-row output kernel's
    reversed passes); dS_in still returned."""
    import torch
    msr = _msr()
    B, N, H = 2, 161 if d == 64 else 300, 3
    q, k, v = workloads.core_inputs(31, B, N, H, d, d, dtype)
    dO = workloads.normal(np.random.default_rng(32), (B, N, H, d), 1.0, dtype)
    g = np.array([0.0, 0.5, 1.0])
    dS_in = torch.empty((B, H, d, d), device="cuda")
    say("backward degenerate", dtype, d, chunk)
    dQ, dK, dV = msr.msr_chunkwise_bwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(dO, dtype), g, chunk,
                                       dS_in=dS_in)
    torch.cuda.synchronize()
    rq, rk, rv, rS = oracle.retention_grad(q, k, v, dO, g, 1.0)
    for name, got, ref in (("dQ", dQ, rq), ("dK", dK, rk), ("dV", dV, rv)):
        _check(name, host(got), ref, TOL[dtype])
    got = host(dS_in)
    assert np.all(got[:, 0] == 0.0)                      # gamma = 0: no gradient reaches the initial state
    assert _state_err(got[:, 1:], rS[:, 1:]) < STATE_TOL[dtype]


def test_backward_empty_sequences():
    """seqlen = 0: dS_in = dS_out exactly (and zeros without dS_out); batch = 0
    is a no-op."""
    import torch
    msr = _msr()
    B, H, d = 3, 2, 64
    g = np.array([0.9, 0.99])
    dS = torch.randn((B, H, d, d), device="cuda")
    dS_in = torch.full((B, H, d, d), 7.0, device="cuda")
    e = torch.empty((B, 0, H, d), device="cuda")
    say("backward empty")
    msr.msr_chunkwise_bwd(e, e, e, e, g, 64, dS_out=dS, dS_in=dS_in)
    torch.cuda.synchronize()
    assert torch.equal(dS_in, dS)
    msr.msr_chunkwise_bwd(e, e, e, e, g, 64, dS_in=dS_in)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dS_in).item() == 0
    z = torch.empty((0, 5, H, d), device="cuda")
    msr.msr_chunkwise_bwd(z, z, z, z, g, 64)


@pytest.mark.slow
def test_backward_headline_core_shape_sampled():
    """Batch 8, 2048 tokens, 8 heads of 256, bf16, chunk 256, rotation, the
    heads' gammas 1 - 2^(-5-h), scale 1/16: (batch, head) slices (0, 0),
    (3, 5) and (7, 7) of dQ, dK, dV and dS_in against the oracle."""
    import torch
    msr = _msr()
    B, N, H, d, C = 8, 2048, 8, 256, 256
    g = workloads.gammas(H)
    say("backward headline core shape")
    q, k, v, dO = (workloads.device_normal((B, N, H, d), seed=900 + i).to(torch.bfloat16) for i in range(4))
    dS_in = torch.empty((B, H, d, d), device="cuda")
    dQ, dK, dV = msr.msr_chunkwise_bwd(q, k, v, dO, g, C, rope_base=1e4, qk_scale=1 / 16, dS_in=dS_in)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 5), (7, 7)):
        sl = lambda t: host(t[b:b + 1, :, h:h + 1])
        qs, ks = oracle.rotary(sl(q), 0, 1e4), oracle.rotary(sl(k), 0, 1e4)
        rq, rk, rv, rS = oracle.retention_grad(qs, ks, sl(v), sl(dO), g[h:h + 1], 1 / 16)
        _check(f"dQ[{b},{h}]", sl(dQ), oracle.rotary_adjoint(rq, 0, 1e4), TOL["bf16"])
        _check(f"dK[{b},{h}]", sl(dK), oracle.rotary_adjoint(rk, 0, 1e4), TOL["bf16"])
        _check(f"dV[{b},{h}]", sl(dV), rv, TOL["bf16"])
        assert oracle.max_rel_err(host(dS_in[b, h]), rS[0, 0]) < STATE_TOL["bf16"]


@pytest.mark.parametrize("dtype,d,N,chunk", [("bf16", 128, 300, 128), ("bf16", 64, 400, 128),
                                             ("bf16", 256, 520, 256), ("bf16", 64, 200, 64), ("f32", 64, 200, 64)])
def test_backward_with_saved_forward_states(dtype, d, N, chunk):
    """msr_chunkwise_fwd_save then msr_chunkwise_bwd_saved, with rotation and
    both seeds: O is msr_chunkwise_fwd's bit for bit, the kept states are
    the oracle's per-chunk starting states (of the rotated K), and the
    gradients match the oracle.  On the direct-copy path (bf16, chunk a
    multiple of 128) the dQ pass reads the kept states, so only the dV pass
    runs the state kernel; elsewhere they are not read."""
    import torch
    msr = _msr()
    B, H = 2, 3
    q, k, v = workloads.core_inputs(41 + d, B, N, H, d, d, dtype)
    rng = np.random.default_rng(42 + d)
    dO = workloads.normal(rng, (B, N, H, d), 1.0, dtype)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dS = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g = np.array([0.9, 1 - 2.0 ** -5, 1 - 2.0 ** -12])
    scale, pos0, base = 1 / math.sqrt(d), 3, 10000.0
    Q, K, V, S0d = dev(q, dtype), dev(k, dtype), dev(v, dtype), torch.from_numpy(S0).cuda()
    R = torch.empty(msr.msr_chunkwise_states_shape(B, N, H, d, d, chunk), dtype=Q.dtype, device="cuda")
    say("saved states", dtype, d, N, chunk)
    O_plain = msr.msr_chunkwise_fwd(Q, K, V, g, chunk, rope_base=base, pos0=pos0, qk_scale=scale, S_in=S0d)
    O = msr.msr_chunkwise_fwd_save(Q, K, V, g, chunk, R, rope_base=base, pos0=pos0, qk_scale=scale, S_in=S0d)
    torch.cuda.synchronize()
    assert torch.equal(O, O_plain)
    qr, kr = oracle.rotary(q, pos0, base), oracle.rotary(k, pos0, base)
    Rh = host(R)
    for i in range(R.shape[2]):
        c0 = i * chunk
        ref = S0 if c0 == 0 else oracle.retention_chunkwise(qr[:, :c0], kr[:, :c0], v[:, :c0], g, chunk, scale,
                                                            S0=S0)[1]
        err = _state_err(np.swapaxes(Rh[:, :, i], -1, -2), ref)
        assert err < STATE_TOL[dtype], (i, err)
    dS_in = torch.empty((B, H, d, d), device="cuda")
    msr.msr_trace_enable(True)
    try:
        dQ, dK, dV = msr.msr_chunkwise_bwd_saved(Q, K, V, dev(dO, dtype), g, chunk, R, rope_base=base, pos0=pos0,
                                                 qk_scale=scale, S_in=S0d, dS_out=torch.from_numpy(dS).cuda(),
                                                 dS_in=dS_in)
        torch.cuda.synchronize()
        launches = msr.trace_totals()["k_chunk_state"][1]
    finally:
        msr.msr_trace_enable(False)
    assert launches == (1 if dtype == "bf16" and chunk % 128 == 0 else 2)
    rq, rk, rv, rS = oracle.retention_grad(qr, kr, v, dO, g, scale, S0=S0, dS=dS)
    _check("dQ", host(dQ), oracle.rotary_adjoint(rq, pos0, base), TOL[dtype])
    _check("dK", host(dK), oracle.rotary_adjoint(rk, pos0, base), TOL[dtype])
    _check("dV", host(dV), rv, TOL[dtype])
    assert _state_err(host(dS_in), rS) < STATE_TOL[dtype]


@pytest.mark.slow
def test_saved_states_backward_headline_core_shape_sampled():
    """The kept-state path at the shape bench.py times it (batch 8, 2048
    tokens, 8 heads of 256, bf16, chunk 256, gammas 1 - 2^(-5-h), scale 1/16,
    no rotation): O of msr_chunkwise_fwd_save equals msr_chunkwise_fwd's,
    and (batch, head) slices (1, 2), (6, 7) of dQ, dK, dV and dS_in from
    msr_chunkwise_bwd_saved match the oracle."""
    import torch
    msr = _msr()
    B, N, H, d, C = 8, 2048, 8, 256, 256
    g = workloads.gammas(H)
    say("saved-state backward headline core shape")
    q, k, v, dO = (workloads.device_normal((B, N, H, d), seed=950 + i).to(torch.bfloat16) for i in range(4))
    R = torch.empty(msr.msr_chunkwise_states_shape(B, N, H, d, d, C), dtype=torch.bfloat16, device="cuda")
    O = msr.msr_chunkwise_fwd_save(q, k, v, g, C, R, qk_scale=1 / 16)
    assert torch.equal(O, msr.msr_chunkwise_fwd(q, k, v, g, C, qk_scale=1 / 16))
    dS_in = torch.empty((B, H, d, d), device="cuda")
    dQ, dK, dV = msr.msr_chunkwise_bwd_saved(q, k, v, dO, g, C, R, qk_scale=1 / 16, dS_in=dS_in)
    torch.cuda.synchronize()
    for b, h in ((1, 2), (6, 7)):
        sl = lambda t: host(t[b:b + 1, :, h:h + 1])
        rq, rk, rv, rS = oracle.retention_grad(sl(q), sl(k), sl(v), sl(dO), g[h:h + 1], 1 / 16)
        _check(f"dQ[{b},{h}]", sl(dQ), rq, TOL["bf16"])
        _check(f"dK[{b},{h}]", sl(dK), rk, TOL["bf16"])
        _check(f"dV[{b},{h}]", sl(dV), rv, TOL["bf16"])
        assert oracle.max_rel_err(host(dS_in[b, h]), rS[0, 0]) < STATE_TOL["bf16"]


@pytest.mark.parametrize("dtype,dk,dv,N,chunk", [("bf16", 256, 512, 200, 64), ("f32", 128, 128, 97, 32)])
def test_kept_states_of_the_forward(dtype, dk, dv, N, chunk):
    """msr_chunkwise_fwd_save's R_chunks = the oracle's state at the start of
    every chunk (transposed), also where d_k != d_v and for a ragged last
    chunk; O and S_out are msr_chunkwise_fwd's bit for bit."""
    import torch
    msr = _msr()
    B, H = 2, 2
    q, k, v = workloads.core_inputs(61 + dk, B, N, H, dk, dv, dtype)
    S0 = np.random.default_rng(62).standard_normal((B, H, dk, dv)).astype(np.float32)
    g = np.array([0.95, 1 - 2.0 ** -9])
    Q, K, V, S0d = dev(q, dtype), dev(k, dtype), dev(v, dtype), torch.from_numpy(S0).cuda()
    R = torch.empty(msr.msr_chunkwise_states_shape(B, N, H, dk, dv, chunk), dtype=Q.dtype, device="cuda")
    S1, S2 = (torch.empty((B, H, dk, dv), device="cuda") for _ in range(2))
    say("kept states", dtype, dk, dv, N, chunk)
    O1 = msr.msr_chunkwise_fwd(Q, K, V, g, chunk, qk_scale=0.1, S_in=S0d, S_out=S1)
    O2 = msr.msr_chunkwise_fwd_save(Q, K, V, g, chunk, R, qk_scale=0.1, S_in=S0d, S_out=S2)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)
    Rh = host(R)
    for i in range(R.shape[2]):
        c0 = i * chunk
        ref = S0 if c0 == 0 else oracle.retention_chunkwise(q[:, :c0], k[:, :c0], v[:, :c0], g, chunk, 0.1,
                                                            S0=S0)[1]
        err = _state_err(np.swapaxes(Rh[:, :, i], -1, -2), ref)
        assert err < STATE_TOL[dtype], (i, err)


def test_backward_one_pass_states_reversed_ragged_sampled():
    """Enough (batch, head) pairs for the one-pass state kernel in both of the
    backward's state computations (the dQ pass forward, the dV pass on the
    time-reversed sequence), with a ragged last chunk, both seeds and the
    rotation: batch 4, 700 tokens, 16 heads of 256, bf16, chunk 128; the
    library's trace shows the one-pass kernel twice and no chunk-parallel
    state kernel, and (batch, head) slices (0, 0), (2, 7), (3, 15) of dQ,
    dK, dV and dS_in match the oracle."""
    import torch
    msr = _msr()
    B, N, H, d, C = 4, 700, 16, 256, 128
    g = workloads.gammas(H)
    q, k, v = workloads.core_inputs(61, B, N, H, d, d, "bf16")
    rng = np.random.default_rng(62)
    dO = workloads.normal(rng, (B, N, H, d), 1.0, "bf16")
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dS = rng.standard_normal((B, H, d, d)).astype(np.float32)
    scale, pos0, base = 1 / math.sqrt(d), 7, 10000.0
    dS_in = torch.empty((B, H, d, d), device="cuda")
    say("backward one-pass states, reversed, ragged")
    msr.msr_trace_enable(True)
    try:
        dQ, dK, dV = msr.msr_chunkwise_bwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(dO, "bf16"), g, C,
                                           rope_base=base, pos0=pos0, qk_scale=scale,
                                           S_in=torch.from_numpy(S0).cuda(), dS_out=torch.from_numpy(dS).cuda(),
                                           dS_in=dS_in)
        torch.cuda.synchronize()
        tot = msr.trace_totals()
    finally:
        msr.msr_trace_enable(False)
    assert tot["k_chunk_rscan"][1] == 2 and "k_chunk_state" not in tot, tot
    for b, h in ((0, 0), (2, 7), (3, 15)):
        sl = lambda a: a[b:b + 1, :, h:h + 1]
        qs, ks = oracle.rotary(sl(q), pos0, base), oracle.rotary(sl(k), pos0, base)
        rq, rk, rv, rS = oracle.retention_grad(qs, ks, sl(v), sl(dO), g[h:h + 1], scale, S0=S0[b:b + 1, h:h + 1],
                                               dS=dS[b:b + 1, h:h + 1])
        _check(f"dQ[{b},{h}]", host(dQ)[b:b + 1, :, h:h + 1], oracle.rotary_adjoint(rq, pos0, base), TOL["bf16"])
        _check(f"dK[{b},{h}]", host(dK)[b:b + 1, :, h:h + 1], oracle.rotary_adjoint(rk, pos0, base), TOL["bf16"])
        _check(f"dV[{b},{h}]", host(dV)[b:b + 1, :, h:h + 1], rv, TOL["bf16"])
        assert oracle.max_rel_err(host(dS_in[b, h]), rS[0, 0]) < STATE_TOL["bf16"]
