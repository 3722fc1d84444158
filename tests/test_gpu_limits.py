"""Parity at the documented limits of the C ABI: the largest chunk (4096
tokens, with a ragged second chunk), the most heads (128), and a chunk
longer than the whole sequence, for the chunkwise form, the recurrent step
and the backward, against the float64 oracle."""

import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, say

pytestmark = pytest.mark.gpu


def _msr():
    import linear_recurrence_sequence_amd as msr
    return msr


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_largest_chunk_with_ragged_tail(dtype):
    import torch
    msr = _msr()
    B, N, H, d, C = 1, 4200, 2, 64, 4096
    q, k, v = workloads.core_inputs(91, B, N, H, d, d, dtype)
    g = np.array([1 - 2.0 ** -8, 1 - 2.0 ** -12])
    S_out = torch.empty((B, H, d, d), device="cuda")
    say("chunk 4096", dtype)
    O = msr.msr_chunkwise_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, C, qk_scale=1 / 8, S_out=S_out)
    torch.cuda.synchronize()
    ref, Sref = oracle.retention_chunkwise(q, k, v, g, C, 1 / 8)
    err = oracle.max_rel_err_per_head(host(O), ref)
    print(f"chunk 4096 {dtype}: {err:.2e}", flush=True)
    assert err < TOL[dtype]
    assert oracle.max_rel_err(host(S_out), Sref) < (1e-4 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_most_heads_and_chunk_longer_than_sequence(dtype):
    """128 heads (the maximum), 100 tokens with chunk 512: one short chunk;
    the gammas span the whole schedule 1 - 2^(-5-h) down to 1 - 2^-132 = 1
    in double, so the slowest heads do not decay at all."""
    import torch
    msr = _msr()
    B, N, H, d, C = 2, 100, 128, 64, 512
    q, k, v = workloads.core_inputs(92, B, N, H, d, d, dtype)
    g = workloads.gammas(H)
    say("128 heads", dtype)
    O = msr.msr_chunkwise_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, C, rope_base=1e4, qk_scale=1 / 8)
    torch.cuda.synchronize()
    ref = oracle.retention_parallel(oracle.rotary(q, 0, 1e4), oracle.rotary(k, 0, 1e4), v, g, 1 / 8)
    err = oracle.max_rel_err_per_head(host(O), ref)
    print(f"128 heads {dtype}: {err:.2e}", flush=True)
    assert err < TOL[dtype]


def test_recurrent_step_most_heads():
    import torch
    msr = _msr()
    B, H, d = 3, 128, 64
    rng = np.random.default_rng(93)
    q, k, v = (rng.standard_normal((B, H, d)).astype(np.float32) for _ in range(3))
    S = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g = workloads.gammas(H)
    Sd = torch.from_numpy(S).cuda()
    say("recurrent step 128 heads")
    o = msr.msr_recurrent_step(dev(q, "f32"), dev(k, "f32"), dev(v, "f32"), Sd, g, pos=77, rope_base=1e4,
                               qk_scale=1 / 8)
    torch.cuda.synchronize()
    ro, rS = oracle.recurrent_step(S, q, k, v, g, 1 / 8, pos=77, base=1e4)
    assert oracle.max_rel_err(host(o), ro) < TOL["f32"]
    assert oracle.max_rel_err(host(Sd), rS) < TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_largest_chunk(dtype):
    import torch
    msr = _msr()
    B, N, H, d, C = 1, 4200, 2, 64, 4096
    q, k, v = workloads.core_inputs(94, B, N, H, d, d, dtype)
    dO = workloads.normal(np.random.default_rng(95), (B, N, H, d), 1.0, dtype)
    g = np.array([1 - 2.0 ** -8, 1 - 2.0 ** -12])
    say("backward chunk 4096", dtype)
    dQ, dK, dV = msr.msr_chunkwise_bwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(dO, dtype), g, C,
                                       qk_scale=1 / 8)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.retention_grad(q, k, v, dO, g, 1 / 8)
    for name, got, ref in (("dQ", dQ, rq), ("dK", dK, rk), ("dV", dV, rv)):
        err = oracle.max_rel_err_per_head(host(got), ref)
        print(f"{name}: {err:.2e}", flush=True)
        assert err < TOL[dtype], name
