"""The allocation-free layer decode step (msr_layer_decode_step_noalloc,
static device scratch) against the layer decode step with a caller
workspace: the same outputs and states, on two calls in a row, the second
with a smaller batch, both through the C ABI; and against the float64
oracle."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, dev, host, say

pytestmark = pytest.mark.gpu


def test_noalloc_decode_step_matches_the_workspace_entry_point():
    import torch
    import linear_recurrence_sequence_amd as msr
    dm, H, dk, dv, dt = 512, 4, 256, 256, "bf16"
    rng = np.random.default_rng(91)
    W = [workloads.normal(rng, (dm, H * d), dm ** -0.5, dt) for d in (dk, dk, dv, dv)]
    WO = workloads.normal(rng, (H * dv, dm), (H * dv) ** -0.5, dt)
    g = workloads.gammas(H)
    Wd = [dev(w, dt) for w in W] + [dev(WO, dt)]
    for call, B in enumerate((48, 20)):              # the second call is smaller
        X = workloads.normal(rng, (B, dm), 1.0, dt)
        S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.5
        pos = 300 + call
        Xd = dev(X, dt)
        S_a = torch.from_numpy(S0).cuda()
        S_b = S_a.clone()
        out_a = torch.empty((B, dm), dtype=torch.bfloat16, device="cuda")
        out_b = torch.empty_like(out_a)
        ws = torch.empty(msr.msr_layer_decode_workspace_bytes(1, B, dm, H, dk, dv), dtype=torch.uint8,
                         device="cuda")
        say("noalloc decode step", call, B)
        msr.msr_layer_decode_step(Xd, *Wd, S_a, g, H, dk, dv, pos, out=out_a, workspace=ws)
        msr.msr_layer_decode_step_noalloc(Xd, *Wd, S_b, g, H, dk, dv, pos, out=out_b)
        torch.cuda.synchronize()
        # the same kernels in the same configuration: identical results
        assert torch.equal(out_a, out_b) and torch.equal(S_a, S_b)
        ref, Sref = oracle.msr_layer_decode_step(X, S0, *W, WO, g, H, dk, dv, pos, rope_base=10000.0, eps=1e-5)
        assert np.all(np.isfinite(host(out_b)))
        assert oracle.max_rel_err(host(out_b), ref) < TOL[dt]
        assert oracle.max_rel_err(host(S_b), Sref) < TOL[dt]
