"""Parity of the gated MSR layer decode step (msr_layer_decode_step) against
the float64 oracle's layer decode step (itself pinned to the layer forward):
small shapes over every supported head-dim pair in both precisions, two
steps in a row on the same in-place state, and the full decode shape
(batch 128, d_model 4096, 16 heads of 256) on sampled batch rows."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, say

pytestmark = pytest.mark.gpu


def _msr():
    import linear_recurrence_sequence_amd as msr
    return msr


def _inputs(seed, B, dm, H, dk, dv, dtype, s_std=0.5):
    rng = np.random.default_rng(seed)
    n = lambda shape, std: workloads.normal(rng, shape, std, dtype)
    x = n((B, dm), 1.0)
    ws = dm ** -0.5
    WQ, WK = n((dm, H * dk), ws), n((dm, H * dk), ws)
    WV, WG = n((dm, H * dv), ws), n((dm, H * dv), ws)
    WO = n((H * dv, dm), (H * dv) ** -0.5)
    S = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * s_std
    return x, WQ, WK, WV, WG, WO, S


# the last case has more than 128 rows: its bf16 projections take the
# 256 x 256 direct-copy tiles with split-K instead of the 128 x 64 ones
CASES = [(3, 128, 2, 64, 64), (2, 256, 2, 128, 128), (4, 512, 2, 256, 256), (2, 256, 2, 256, 512),
         (200, 512, 2, 256, 256)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,dm,H,dk,dv", CASES)
def test_layer_decode_step(B, dm, H, dk, dv, dtype):
    import torch
    msr = _msr()
    x, WQ, WK, WV, WG, WO, S = _inputs(11 + dk + dv, B, dm, H, dk, dv, dtype)
    g = workloads.gammas(H)
    say("layer decode step", dtype, B, dm, H, dk, dv)
    Sd = torch.from_numpy(S).cuda()
    args = [dev(a, dtype) for a in (WQ, WK, WV, WG, WO)]
    ref_S = S.astype(np.float64)
    for t, pos in enumerate((1000, 1001)):                      # two steps on the same in-place state
        xt = x if t == 0 else np.ascontiguousarray(x[::-1])     # bf16-exact either way
        out = msr.msr_layer_decode_step(dev(xt, dtype), *args, Sd, g, H, dk, dv, pos, rope_base=1e4, gn_eps=1e-5)
        torch.cuda.synchronize()
        ref, ref_S = oracle.msr_layer_decode_step(xt, ref_S, WQ, WK, WV, WG, WO, g, H, dk, dv, pos, rope_base=1e4,
                                                  eps=1e-5)
        err = oracle.max_rel_err(host(out), ref)
        errS = oracle.max_rel_err(host(Sd), ref_S)
        print(f"step {t}: out err {err:.2e}, state err {errS:.2e}", flush=True)
        assert np.all(np.isfinite(host(out)))
        assert err < TOL[dtype], (t, err)
        assert errS < TOL[dtype], (t, errS)


def test_layer_decode_step_without_rotation_and_first_position():
    """rope_base <= 0 (no rotation) and pos = 0 from a zero state: the output
    is the single-token layer forward."""
    import torch
    msr = _msr()
    B, dm, H, dk, dv = 2, 128, 2, 64, 64
    x, WQ, WK, WV, WG, WO, _ = _inputs(5, B, dm, H, dk, dv, "f32")
    g = workloads.gammas(H)
    Sd = torch.zeros((B, H, dk, dv), device="cuda")
    out = msr.msr_layer_decode_step(dev(x, "f32"), *(dev(a, "f32") for a in (WQ, WK, WV, WG, WO)), Sd, g, H, dk, dv,
                                    0, rope_base=0.0, gn_eps=1e-5)
    ref = oracle.msr_layer(x[:, None], WQ, WK, WV, WG, WO, g, H, dk, dv, eps=1e-5, form="recurrent")[:, 0]
    assert oracle.max_rel_err(host(out), ref) < TOL["f32"]


@pytest.mark.slow
def test_layer_decode_step_full_shape_sampled():
    """Batch 128, d_model 4096, 16 heads of 256, bf16 weights and tokens, a
    float32 state drawn on the device, position 8192: batch rows 0, 77 and
    127 of the output and their states against the oracle."""
    import torch
    msr = _msr()
    B, dm, H, dk, dv = 128, 4096, 16, 256, 256
    g = workloads.gammas(H)
    say("layer decode step full shape")
    s = dm ** -0.5
    x = workloads.device_normal((B, dm), seed=801).to(torch.bfloat16)
    W = [(workloads.device_normal(shp, seed=810 + i) * s).to(torch.bfloat16)
         for i, shp in enumerate([(dm, H * dk), (dm, H * dk), (dm, H * dv), (dm, H * dv)])]
    WO = (workloads.device_normal((H * dv, dm), seed=820) * (H * dv) ** -0.5).to(torch.bfloat16)
    S = workloads.device_normal((B, H, dk, dv), seed=830) * 0.5
    rows = [0, 77, 127]
    S_rows = host(S[rows])
    out = msr.msr_layer_decode_step(x, *W, WO, S, g, H, dk, dv, 8192, rope_base=1e4, gn_eps=1e-5)
    torch.cuda.synchronize()
    ref, S_ref = oracle.msr_layer_decode_step(host(x[rows]), S_rows, *(host(w) for w in W), host(WO), g, H, dk, dv,
                                              8192, rope_base=1e4, eps=1e-5)
    err = oracle.max_rel_err(host(out[rows]), ref)
    errS = oracle.max_rel_err(host(S[rows]), S_ref)
    print(f"full shape: out err {err:.2e}, state err {errS:.2e}", flush=True)
    assert err < TOL["bf16"] and errS < TOL["bf16"]
