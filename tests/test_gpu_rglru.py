"""Parity of the RG-LRU (msr_rglru_fwd: sigmoid-gate GEMM + float32 scan)
against the float64 oracle's RG-LRU (pinned to closed forms, exact gate
values, limits and split continuation): ragged lengths over several time
tiles, initial and final states, the empty sequence, and batch 8 x 2048
tokens x width 2048 in bf16 on sampled batch elements."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, say

pytestmark = pytest.mark.gpu

STATE_TOL = {"f32": 1e-4, "bf16": 2e-2}


def _msr():
    import linear_recurrence_sequence_amd as msr
    return msr


def _f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(2, 200, 128), (3, 65, 64), (1, 1, 256), (2, 1000, 192)])
def test_rglru(dtype, B, T, D):
    import torch
    msr = _msr()
    x, Wa, ba, Wx, bx, lam = workloads.rglru_inputs(60 + T, B, T, D, dtype)
    h0 = np.random.default_rng(61).standard_normal((B, D)).astype(np.float32)
    h_last = torch.empty((B, D), device="cuda")
    say("rglru", dtype, B, T, D)
    Y = msr.msr_rglru_fwd(dev(x, dtype), dev(Wa, dtype), _f32(ba), dev(Wx, dtype), _f32(bx), _f32(lam),
                          h0=_f32(h0), h_last=h_last)
    torch.cuda.synchronize()
    ref, refT = oracle.rglru(x, Wa, ba, Wx, bx, lam, 8.0, h0=h0)
    got = host(Y)
    err, errT = oracle.max_rel_err(got, ref), oracle.max_rel_err(host(h_last), refT)
    print(f"y err {err:.2e}, h_last err {errT:.2e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err < TOL[dtype] and errT < STATE_TOL[dtype]


def test_rglru_exact_gates_and_constant_input():
    """W = 0, b = 0, Lambda = 0: a_t = 1/16 exactly; a constant input gives
    the geometric series of the oracle pin (float32 path)."""
    import torch
    msr = _msr()
    B, T, D = 2, 300, 64
    u = np.random.default_rng(62).standard_normal((B, D)).astype(np.float32)
    x = np.repeat(u[:, None, :], T, axis=1)
    z, zb = np.zeros((D, D), np.float32), np.zeros(D, np.float32)
    say("rglru exact gates")
    Y = msr.msr_rglru_fwd(dev(x, "f32"), dev(z, "f32"), _f32(zb), dev(z, "f32"), _f32(zb), _f32(zb))
    torch.cuda.synchronize()
    ref, _ = oracle.rglru(x, z, zb, z, zb, zb, 8.0)
    assert oracle.max_rel_err(host(Y), ref) < 1e-5


def test_rglru_empty_sequence_copies_state():
    import torch
    msr = _msr()
    B, D = 3, 128
    h0 = torch.randn((B, D), device="cuda")
    hT = torch.full((B, D), 5.0, device="cuda")
    lam = torch.zeros(D, device="cuda")
    e = torch.empty((B, 0, D), device="cuda")
    say("rglru empty")
    msr.msr_rglru_fwd(e, None, None, None, None, lam, h0=h0, h_last=hT)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)
    msr.msr_rglru_fwd(e, None, None, None, None, lam, h_last=hT)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hT).item() == 0


@pytest.mark.slow
def test_rglru_full_shape_sampled():
    """Batch 8, 2048 tokens, width 2048, bf16: batch elements 0 and 6 of Y
    and of the last state against the oracle."""
    import torch
    msr = _msr()
    B, T, D = 8, 2048, 2048
    x, Wa, ba, Wx, bx, lam = workloads.rglru_inputs(70, B, T, D, "bf16")
    h_last = torch.empty((B, D), device="cuda")
    say("rglru full shape")
    Y = msr.msr_rglru_fwd(dev(x, "bf16"), dev(Wa, "bf16"), _f32(ba), dev(Wx, "bf16"), _f32(bx), _f32(lam),
                          h_last=h_last)
    torch.cuda.synchronize()
    for b in (0, 6):
        ref, refT = oracle.rglru(x[b:b + 1], Wa, ba, Wx, bx, lam, 8.0)
        err = oracle.max_rel_err(host(Y[b:b + 1]), ref)
        errT = oracle.max_rel_err(host(h_last[b:b + 1]), refT)
        print(f"batch {b}: y err {err:.2e}, h_last err {errT:.2e}", flush=True)
        assert err < TOL["bf16"] and errT < STATE_TOL["bf16"]
