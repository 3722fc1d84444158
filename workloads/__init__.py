"""Seeded synthetic inputs for the multi-scale retention (MSR) workloads.

This module is shared by the float64 oracle (``oracle/``), the tests and the
benchmark.  It holds *no* arithmetic of the method: only workload shapes, the
per-head decay values handed to both sides as inputs, and seeded random
generators.  Neither the oracle nor the HIP library is imported here.

Workloads (sizes as named; all inputs Gaussian, weights with variance
1/d_model, i.e. standard deviation d_model**-0.5):

* ``layer_fp32_b1_n256``  -- one MSR layer, fp32, batch 1, 256 tokens,
  d_model 256, 4 heads of 64, chunk 64.
* ``layer_bf16_b8_n2048`` -- one MSR layer, bf16, batch 8, 2048 tokens,
  d_model 2048, 8 heads of 256, chunk 256.
* ``long_bf16_b2_n16384`` -- long-sequence chunkwise MSR, bf16, batch 2,
  16384 tokens, d_model 2560, 10 heads of 256, chunk 512.
* ``decode_fp32_b128_h16`` -- recurrent decode, fp32 state [128,16,256,256]
  prefilled from an 8192-token context, 512 timed steps.
* ``block_bf16_b4_n8192`` -- gated MSR block, bf16, batch 4, 8192 tokens,
  d_model 4096, 16 heads, q/k head dim 256, v head dim 512, chunk 512.

RG-LRU inputs (``rglru_inputs``): x ~ N(0, 1); W_a, W_x ~ N(0, 1/width)
(LeCun normal, the Griffin page's initialisation); b_a, b_x ~ N(0, 1/4);
Lambda drawn so that a^c = sigma(Lambda)^c is uniform on [0.9, 0.999] (the
same page's initialisation of the recurrent weight), c = 8.

The per-head decay is gamma_h = 1 - 2**(-5-h); the pages give a different
fixed gamma to every head (RetNet page "Transformer取代者登場！微軟、清華剛推出
RetNet", section "門控多尺度 Retention") but their formula is stripped, so the
schedule is part of the workload definition.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "gammas", "round_bf16", "bf16_bits",
    "normal", "layer_inputs", "core_inputs", "device_normal", "rglru_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": the input/activation type
    batch: int
    seqlen: int
    d_model: int
    heads: int
    d_k: int
    d_v: int
    chunk: int
    rope_base: float = 10000.0
    seed: int = 0
    context: int = 0      # decode only: prefilled context length
    steps: int = 0        # decode only: timed decode steps

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


WORKLOADS = {
    w.name: w
    for w in [
        Workload("layer_fp32_b1_n256", "f32", 1, 256, 256, 4, 64, 64, 64),
        Workload("layer_bf16_b8_n2048", "bf16", 8, 2048, 2048, 8, 256, 256, 256),
        Workload("long_bf16_b2_n16384", "bf16", 2, 16384, 2560, 10, 256, 256, 512),
        Workload("decode_fp32_b128_h16", "f32", 128, 1, 4096, 16, 256, 256, 512,
                 context=8192, steps=512),
        Workload("block_bf16_b4_n8192", "bf16", 4, 8192, 4096, 16, 256, 512, 512),
    ]
}


def gammas(heads: int) -> np.ndarray:
    """Per-head decay gamma_h = 1 - 2**(-5-h), h = 0..heads-1, as float64."""
    return np.array([1.0 - 2.0 ** (-5 - h) for h in range(heads)], dtype=np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bf16.  Pure bit
    manipulation on the IEEE encoding; NaN/Inf are not expected in inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """Draw float64 N(0, std**2), cast to float32, then round to ``dtype``."""
    x = (rng.standard_normal(size=shape) * std).astype(np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def layer_inputs(w: Workload, batch: int | None = None, seqlen: int | None = None):
    """Inputs of one MSR layer: X, W_Q, W_K, W_V, W_G, W_O (float32 arrays,
    bf16-exact when ``w.dtype == 'bf16'``).

    Drawn from ``numpy.random.default_rng(w.seed)`` in the order X, W_Q, W_K,
    W_V, W_G, W_O.  X ~ N(0, 1); weights ~ N(0, 1/d_model).  Weights are
    row-major [in, out] so the layer computes X @ W.
    """
    b = w.batch if batch is None else batch
    n = w.seqlen if seqlen is None else seqlen
    rng = np.random.default_rng(w.seed)
    s = 1.0 / math.sqrt(w.d_model)
    hk, hv = w.heads * w.d_k, w.heads * w.d_v
    X = normal(rng, (b, n, w.d_model), 1.0, w.dtype)
    WQ = normal(rng, (w.d_model, hk), s, w.dtype)
    WK = normal(rng, (w.d_model, hk), s, w.dtype)
    WV = normal(rng, (w.d_model, hv), s, w.dtype)
    WG = normal(rng, (w.d_model, hv), s, w.dtype)
    WO = normal(rng, (hv, w.d_model), s, w.dtype)
    return X, WQ, WK, WV, WG, WO


def core_inputs(seed, batch, seqlen, heads, d_k, d_v, dtype="f32", std=1.0):
    """q, k, v of shape [batch, seqlen, heads, d] ~ N(0, std**2), drawn in
    the order q, k, v from ``default_rng(seed)`` (seed may be a list)."""
    rng = np.random.default_rng(seed)
    q = normal(rng, (batch, seqlen, heads, d_k), std, dtype)
    k = normal(rng, (batch, seqlen, heads, d_k), std, dtype)
    v = normal(rng, (batch, seqlen, heads, d_v), std, dtype)
    return q, k, v


def device_normal(shape, seed: int, device="cuda", dtype=None):
    """N(0, 1) float32 tensor drawn on ``device`` by torch's seeded generator.

    Used where numpy generation would take minutes (the 8192-token decode
    context: 3 x 4.3e9 values).  Slices are copied to the host for the oracle.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t if dtype is None else t.to(dtype)


def rglru_inputs(seed, batch, seqlen, width, dtype="f32", c=8.0):
    """x [batch, seqlen, width], W_a, W_x [width, width] (dtype-rounded),
    b_a, b_x, Lambda [width] (float32), drawn from ``default_rng(seed)`` in
    that order (x, W_a, b_a, W_x, b_x, then the uniform draw for Lambda).
    Lambda = logit(u^(1/c)) with u ~ U[0.9, 0.999], so sigma(Lambda)^c = u."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (batch, seqlen, width), 1.0, dtype)
    Wa = normal(rng, (width, width), width ** -0.5, dtype)
    ba = normal(rng, (width,), 0.5, "f32")
    Wx = normal(rng, (width, width), width ** -0.5, dtype)
    bx = normal(rng, (width,), 0.5, "f32")
    u = rng.uniform(0.9, 0.999, size=width)
    p = u ** (1.0 / c)
    lam = np.log(p / (1.0 - p)).astype(np.float32)
    return x, Wa, ba, Wx, bx, lam
