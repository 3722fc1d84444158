"""Helpers of the GPU parity tests: host <-> device moves and tolerances."""
import numpy as np

# Bounds on max|gpu - ref| / max|ref| (per (batch, head) slice for raw
# retention outputs, per tensor after GroupNorm): float32 path and
# bf16-input / float32-accumulate path.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(x, dtype):
    """numpy float32 (bf16-exact for bf16) -> contiguous GPU tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch_dtype(dtype)).contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a fault)."""
    print("[case]", *a, flush=True)


def well_conditioned_rows(gn_var, eps, kappa=1000.0):
    """Rows (tokens) whose every head enters GroupNorm with variance >=
    kappa * eps.  Below that, the normalised output is decided by eps and a
    bf16 rounding of the single-score inputs (e.g. token 0, whose output is
    one term c v_0 with c = s q_0.k_0 near a cancellation) moves it by O(1):
    the method itself is ill-conditioned there.  gn_var: [B, N, H]."""
    import numpy as np
    return np.all(gn_var >= kappa * eps, axis=-1)


def layer_err(got, ref, gn_var, eps):
    """(max-abs-relative error over well-conditioned rows, fraction of rows
    excluded); every output must still be finite."""
    import numpy as np
    assert np.all(np.isfinite(got)), "non-finite layer output"
    ok = well_conditioned_rows(gn_var, eps)
    den = np.max(np.abs(ref))
    err = float(np.max(np.abs(got - ref)[ok]) / den) if ok.any() else 0.0
    return err, 1.0 - float(ok.mean())
