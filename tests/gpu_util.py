"""Helpers of the GPU parity tests: host <-> device moves and tolerances."""
import math

import numpy as np

# Bounds on max|gpu - ref| / max|ref| (per (batch, head) slice for raw
# retention outputs, per tensor after GroupNorm): float32 path and
# bf16-input / float32-accumulate path.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# unit roundoff of the element type the projections are stored in
UNIT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8}


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


def first_token_bound(X, WQ, WK, WV, WG, WO, heads, d_k, d_v, dtype, eps, scale=None, rounded_input=False):
    """Bound, per batch element, on how far the rounding of the projections
    can move row 0 of the layer output.

    Token 0 (no initial state) is the one row whose retention output is a
    single term per head, o_0 = c v_0 with c = s q_0 . k_0 (the rotation at
    position 0 is the identity).  Its GroupNorm output is f(c) (v_0 -
    mean(v_0)) with f(c) = c / sqrt(c^2 var(v_0) + eps), so row 0 of the
    layer output is exactly sum_h f(c_h) e_h, e_h = (swish(g_h) (.) (v_0 -
    mean)) W_O[head h rows].  The library stores q_0 and k_0 in the element
    type after a float32 accumulation of d_model products: q_i' = q_i (1 +
    r_i) with |r_i| <= u (the type's unit roundoff) plus an accumulation
    error of standard deviation <= 2^-24 sqrt(d_model / 3) ||x (.) w_i||.
    Treating these 2 d_k rounding errors as independent with zero mean (the
    usual probabilistic rounding-error model), c' - c has standard deviation
    sigma <= s sqrt(sum_i (q_i k_i)^2 (2 u^2 / 3) + (accumulation terms)),
    and eta = 6 sigma bounds it.  f is monotone, so head h moves row 0 by at
    most max |f(c +- eta) - f(c)| max|e_h|.  Where c sits within eta of zero
    the sign of the head's output can flip: the method is ill-conditioned
    there, not the kernel.  rounded_input: X itself is a rounded result
    (the block's LayerNorm output), adding u^2/3 sum_j (x_j w_ji)^2 to the
    variance of each projection.  Returns [B] (summed over heads).
    """
    f64 = np.float64
    x = np.asarray(X, f64)[:, 0]                     # [B, d_model]
    B, dm = x.shape
    WQ, WK, WV, WG, WO = (np.asarray(w, f64) for w in (WQ, WK, WV, WG, WO))
    u = UNIT[dtype]
    s = 1.0 / math.sqrt(d_k) if scale is None else scale
    x2 = x * x
    q = (x @ WQ).reshape(B, heads, d_k)
    k = (x @ WK).reshape(B, heads, d_k)
    v = (x @ WV).reshape(B, heads, d_v)
    g = (x @ WG).reshape(B, heads, d_v)
    acc = 2.0 ** -48 * dm / 3.0                      # variance factor of a float32 accumulation
    if rounded_input:
        acc += u * u / 3.0
    var_q = u * u / 3.0 * q * q + acc * (x2 @ (WQ * WQ)).reshape(B, heads, d_k)
    var_k = u * u / 3.0 * k * k + acc * (x2 @ (WK * WK)).reshape(B, heads, d_k)
    c = s * np.sum(q * k, axis=-1)                   # [B, H]
    eta = 6.0 * s * np.sqrt(np.sum(k * k * var_q + q * q * var_k, axis=-1))
    dv = v - v.mean(axis=-1, keepdims=True)
    var = np.mean(dv ** 2, axis=-1)
    f = lambda t: t / np.sqrt(t * t * var + eps)
    df = np.maximum(np.abs(f(c + eta) - f(c)), np.abs(f(c) - f(c - eta)))
    sw = g / (1.0 + np.exp(-g))
    e = np.stack([(sw[:, h] * dv[:, h]) @ WO[h * d_v:(h + 1) * d_v] for h in range(heads)], axis=1)
    return np.sum(df * np.max(np.abs(e), axis=-1), axis=-1)


def layer_err(got, ref, bound0, dtype, row0_bound=True):
    """(max-abs-relative error, number of excluded rows).

    Row 0 of a batch element is left out of the comparison only when
    first_token_bound says the rounding of its single scores can move it by
    more than half the tolerance; it is then still required to be finite
    and (row0_bound) within that bound plus the tolerance.  No other row is
    ever left out, and on the float32 path none is."""
    assert np.all(np.isfinite(got)), "non-finite layer output"
    den = np.max(np.abs(ref))
    ok = np.ones(got.shape[:2], dtype=bool)
    excl = np.asarray(bound0) > 0.5 * TOL[dtype] * den
    ok[:, 0] = ~excl
    err = float(np.max(np.abs(got - ref)[ok]) / den)
    for b in np.nonzero(excl)[0] if row0_bound else ():
        dev0 = float(np.max(np.abs(got[b, 0] - ref[b, 0])))
        assert dev0 <= bound0[b] + TOL[dtype] * den, f"row 0 of batch element {b} moved {dev0} > bound {bound0[b]}"
    if dtype == "f32":
        assert not excl.any(), "the float32 path excludes no row"
    return err, int(excl.sum())
