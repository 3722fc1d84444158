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
