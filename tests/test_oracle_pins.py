"""Pins of the float64 oracle against facts fixed by the pages and by
mathematics, independent of the oracle's own formulas.

Pages: [RN-zh] = "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、速度快、
性能強（2）"; [RN-ru] = "Retentive Network: архитектурный прорыв или временный
успех?"; [RN-it] = "This article on AI proposes Retentive Networks (RetNet)
as a fundamental architecture for large language models ...".
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import expit

import oracle
from oracle.retention import decay_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def close(a, b, tol=1e-12):
    a, b = np.asarray(a, float), np.asarray(b, float)
    den = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / den <= tol


# ---------------------------------------------------------------- P1 -------
@pytest.mark.parametrize("gamma", [Fraction(0), Fraction(1, 2), Fraction(97, 100), Fraction(1)])
def test_parallel_equals_exact_bruteforce(gamma):
    """Eq. (5) evaluated in float64 equals the exact rational double loop
    o_n = sum_{m<=n} gamma^(n-m) (q_n . k_m) v_m on small integer inputs."""
    rng = np.random.default_rng(1)
    B, N, H, dk, dv = 2, 6, 2, 3, 2
    q = rng.integers(-3, 4, (B, N, H, dk))
    k = rng.integers(-3, 4, (B, N, H, dk))
    v = rng.integers(-3, 4, (B, N, H, dv))
    gam = [gamma, Fraction(1, 3)]
    exact = oracle.retention_bruteforce(q.tolist(), k.tolist(), v.tolist(), gam)
    exact = np.array(exact.tolist(), dtype=float)
    got = oracle.retention_parallel(q, k, v, np.array([float(g) for g in gam]))
    assert close(got, exact, 1e-13)


def test_chunkwise_ragged_equals_exact_bruteforce():
    """Eq. (7) with a ragged last chunk (N=7, B=3) against the exact double
    loop: catches an off-by-one in zeta, xi or the gamma^L carry."""
    rng = np.random.default_rng(2)
    B, N, H, dk, dv = 1, 7, 1, 2, 3
    q = rng.integers(-2, 3, (B, N, H, dk))
    k = rng.integers(-2, 3, (B, N, H, dk))
    v = rng.integers(-2, 3, (B, N, H, dv))
    exact = oracle.retention_bruteforce(q.tolist(), k.tolist(), v.tolist(), [Fraction(3, 4)], Fraction(1, 2))
    exact = np.array(exact.tolist(), dtype=float)
    for chunk in (1, 2, 3, 4, 7, 9):
        got, _ = oracle.retention_chunkwise(q, k, v, np.array([0.75]), chunk, 0.5)
        assert close(got, exact, 1e-13), chunk


# ---------------------------------------------------------------- P2 -------
def test_gamma_one_is_causal_linear_attention():
    """gamma = 1, no rotation, scale 1: retention is plain causal linear
    attention (the softmax-free attention of [RN-ru] / [RN-it]),
    o_n = q_n (sum_{m<=n} k_m^T v_m), computed here with a running sum."""
    B, N, H, dk, dv = 2, 9, 3, 4, 5
    q, k, v = rnd(3, B, N, H, dk), rnd(4, B, N, H, dk), rnd(5, B, N, H, dv)
    kv = np.cumsum(k[..., :, None] * v[..., None, :], axis=1)   # [B,N,H,dk,dv]
    lin = np.einsum("bnhi,bnhij->bnhj", q, kv)
    g = np.ones(H)
    assert close(oracle.retention_parallel(q, k, v, g), lin)
    assert close(oracle.retention_recurrent(q, k, v, g)[0], lin)
    assert close(oracle.retention_chunkwise(q, k, v, g, 4)[0], lin)


# ---------------------------------------------------------------- P3 -------
@settings(max_examples=40, deadline=None)
@given(
    N=st.integers(1, 24),
    extra=st.integers(0, 3),
    chunk_frac=st.floats(0.0, 1.0),
    dk=st.sampled_from([2, 4, 6]),
    dv=st.sampled_from([1, 3, 4]),
    H=st.integers(1, 3),
    seed=st.integers(0, 10_000),
    gsel=st.lists(st.sampled_from([0.0, 0.5, 1 - 2.0 ** -5, 1 - 2.0 ** -12, 1.0]), min_size=3, max_size=3),
    use_s0=st.booleans(),
)
def test_three_forms_agree(N, extra, chunk_frac, dk, dv, H, seed, gsel, use_s0):
    """The parallel, recurrent and chunkwise forms are one function ([RN-zh]
    sections 1)-3): Eq. (5) is derived from Eq. (6), Eq. (7) runs Eq. (5)
    inside chunks and Eq. (6) across them), for every chunk length
    1 <= B <= N + 3, ragged last chunks included, and with an initial state."""
    chunk = 1 + int(chunk_frac * (N + 2 + extra - 1))
    B = 2
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, dk))
    k = rng.standard_normal((B, N, H, dk))
    v = rng.standard_normal((B, N, H, dv))
    g = np.array(gsel[:H])
    s = 0.7
    S0 = rng.standard_normal((B, H, dk, dv)) if use_s0 else None
    o_r, S_r = oracle.retention_recurrent(q, k, v, g, s, S0)
    o_c, S_c = oracle.retention_chunkwise(q, k, v, g, chunk, s, S0)
    assert close(o_c, o_r, 1e-11)
    assert close(S_c, S_r, 1e-11)
    if S0 is None:
        assert close(oracle.retention_parallel(q, k, v, g, s), o_r, 1e-11)


def test_chunk_extremes_reduce_to_other_forms():
    """B = N is the parallel form; B = 1 is the recurrent form."""
    B, N, H, d = 1, 11, 2, 3
    q, k, v = rnd(6, B, N, H, d), rnd(7, B, N, H, d), rnd(8, B, N, H, d)
    g = np.array([0.9, 0.5])
    assert close(oracle.retention_chunkwise(q, k, v, g, N)[0], oracle.retention_parallel(q, k, v, g))
    assert close(oracle.retention_chunkwise(q, k, v, g, 1)[0], oracle.retention_recurrent(q, k, v, g)[0])


# ---------------------------------------------------------------- P4 -------
def test_gamma_zero_keeps_only_the_diagonal():
    """gamma = 0: D is the identity, so o_n = s (q_n . k_n) v_n."""
    B, N, H, dk, dv = 2, 7, 1, 3, 4
    q, k, v = rnd(9, B, N, H, dk), rnd(10, B, N, H, dk), rnd(11, B, N, H, dv)
    want = 0.3 * np.sum(q * k, axis=-1, keepdims=True) * v
    for got in (oracle.retention_parallel(q, k, v, [0.0], 0.3),
                oracle.retention_recurrent(q, k, v, [0.0], 0.3)[0],
                oracle.retention_chunkwise(q, k, v, [0.0], 3, 0.3)[0]):
        assert close(got, want)


# ---------------------------------------------------------------- P5 -------
def test_geometric_series_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "geometric_series.txt")) if not l.startswith("#")]
    for gamma in sorted({float(r[0]) for r in rows}):
        want = np.array([float(r[2]) for r in rows if float(r[0]) == gamma])
        N = len(want)
        one = np.ones((1, N, 1, 1))
        for got in (oracle.retention_parallel(one, one, one, [gamma])[0, :, 0, 0],
                    oracle.retention_recurrent(one, one, one, [gamma])[0][0, :, 0, 0],
                    oracle.retention_chunkwise(one, one, one, [gamma], 5)[0][0, :, 0, 0]):
            np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)


def test_decay_mask_entries():
    D = decay_mask(4, 0.5)
    assert D[3, 0] == 0.125 and D[0, 3] == 0.0 and D[2, 2] == 1.0 and D[2, 1] == 0.5


# ---------------------------------------------------------------- P6 -------
def test_split_sequence_continuation():
    """The state is the whole memory of the prefix ([RN-zh] Eq. (6)-(7)):
    chunkwise over [0, M) -> S_out -> chunkwise over [M, N) from S_in equals
    one pass; a prefill followed by single recurrent steps (with rotation at
    the absolute position) equals one pass over all tokens."""
    B, N, H, dk, dv, M = 2, 20, 2, 4, 3, 13
    g = np.array([0.8, 0.99])
    base = 100.0
    q0, k0, v = rnd(12, B, N, H, dk), rnd(13, B, N, H, dk), rnd(14, B, N, H, dv)
    q, k = oracle.rotary(q0, 0, base), oracle.rotary(k0, 0, base)
    full, S_full = oracle.retention_chunkwise(q, k, v, g, 4, 0.5)
    a, Sa = oracle.retention_chunkwise(q[:, :M], k[:, :M], v[:, :M], g, 4, 0.5)
    b, Sb = oracle.retention_chunkwise(q[:, M:], k[:, M:], v[:, M:], g, 4, 0.5, Sa)
    assert close(np.concatenate([a, b], 1), full) and close(Sb, S_full)
    # rotation of the continuation computed at its own offset
    q2 = oracle.rotary(q0[:, M:], M, base)
    assert close(q2, q[:, M:])
    # prefill M tokens, then decode the rest one token at a time
    S = Sa
    for n in range(M, N):
        o, S = oracle.recurrent_step(S, q0[:, n], k0[:, n], v[:, n], g, 0.5, pos=n, base=base)
        assert close(o, full[:, n])
    assert close(S, S_full)


# ---------------------------------------------------------------- P7 -------
def test_rotary_golden_and_properties():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "rotary_unit.txt")) if not l.startswith("#")]
    for base, d, j, p, c, s in rows:
        base, d, j, p, c, s = float(base), int(d), int(j), int(p), float(c), float(s)
        x = np.zeros((1, 1, 1, d))
        x[..., 2 * j] = 1.0
        y = oracle.rotary(x, p, base)
        assert abs(y[0, 0, 0, 2 * j] - c) < 1e-12 and abs(y[0, 0, 0, 2 * j + 1] - s) < 1e-12
        x2 = np.zeros((1, 1, 1, d))
        x2[..., 2 * j + 1] = 1.0                    # i * e^{i a} = (-sin a, cos a)
        y2 = oracle.rotary(x2, p, base)
        assert abs(y2[0, 0, 0, 2 * j] + s) < 1e-12 and abs(y2[0, 0, 0, 2 * j + 1] - c) < 1e-12
    x = rnd(15, 2, 9, 3, 8)
    y = oracle.rotary(x, 5, 10000.0)
    assert close(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.array_equal(oracle.rotary(x, 5, 0.0), x)


def test_rotation_is_relative():
    """With the same rotation on Q and K the scores depend on n - m only
    ([RN-zh] "Retention": xPos is a relative position embedding): shifting the
    absolute origin leaves the retention output unchanged."""
    B, N, H, d = 1, 10, 2, 6
    q, k, v = rnd(16, B, N, H, d), rnd(17, B, N, H, d), rnd(18, B, N, H, d)
    g = np.array([1.0, 0.9])
    outs = [oracle.retention_parallel(oracle.rotary(q, p0, 50.0), oracle.rotary(k, p0, 50.0), v, g)
            for p0 in (0, 3, 1000)]
    assert close(outs[1], outs[0], 1e-10) and close(outs[2], outs[0], 1e-10)
    assert not close(outs[0], oracle.retention_parallel(q, k, v, g), 1e-3)


# ---------------------------------------------------------------- P8/P9 ----
def test_groupnorm_scale_invariance_and_moments():
    O = rnd(19, 2, 5, 3, 16)
    alpha = np.exp(rnd(20, 2, 5, 3, 1))          # positive per-row factors
    y = oracle.group_norm_heads(O, 0.0)
    assert close(oracle.group_norm_heads(alpha * O, 0.0), y, 1e-12)
    np.testing.assert_allclose(y.mean(-1), 0.0, atol=1e-14)
    np.testing.assert_allclose(y.var(-1), 1.0, rtol=1e-12)
    # a constant row normalises to 0 when eps > 0
    assert np.all(oracle.group_norm_heads(np.ones((1, 1, 1, 4)), 1e-5) == 0.0)


def test_normalisation_tricks_leave_layer_unchanged():
    """[RN-zh] "Retention Score 歸一化": QK^T/sqrt(d), D~ and R~ do not change
    the layer output because GroupNorm is scale invariant (eps = 0)."""
    B, N, dm, H, dk, dv = 1, 12, 16, 2, 4, 6
    rng = np.random.default_rng(21)
    X = rng.standard_normal((B, N, dm))
    W = [rng.standard_normal(s) / 4 for s in ((dm, H * dk), (dm, H * dk), (dm, H * dv), (dm, H * dv), (H * dv, dm))]
    g = np.array([0.9, 0.6])
    plain = oracle.msr_layer(X, *W, g, H, dk, dv, rope_base=30.0, eps=0.0, form="parallel", scale=1.0)
    tricks = oracle.msr_layer(X, *W, g, H, dk, dv, rope_base=30.0, eps=0.0, normalized=True)
    assert close(tricks, plain, 1e-11)
    # at eps > 0 the deviation is small but not zero
    a = oracle.msr_layer(X, *W, g, H, dk, dv, rope_base=30.0, eps=1e-5, form="parallel", scale=1.0)
    assert close(a, plain, 1e-3)


# ---------------------------------------------------------------- P10 ------
def test_linearity_and_independence():
    B, N, H, dk, dv = 2, 8, 3, 4, 5
    q, k, v, v2 = rnd(22, B, N, H, dk), rnd(23, B, N, H, dk), rnd(24, B, N, H, dv), rnd(25, B, N, H, dv)
    g = np.array([0.5, 0.9, 1.0])
    f = lambda q, k, v: oracle.retention_chunkwise(q, k, v, g, 3)[0]
    assert close(f(q, k, 2 * v - v2), 2 * f(q, k, v) - f(q, k, v2))
    assert close(f(3 * q, k, v), 3 * f(q, k, v)) and close(f(q, -2 * k, v), -2 * f(q, k, v))
    # heads are independent: permuting heads (with their gamma) permutes outputs
    perm = [2, 0, 1]
    out_p = oracle.retention_chunkwise(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[perm], 3)[0]
    assert close(out_p, f(q, k, v)[:, :, perm])
    # batch rows are independent
    assert close(oracle.retention_chunkwise(q[1:], k[1:], v[1:], g, 3)[0], f(q, k, v)[1:])


# ---------------------------------------------------------------- P11 ------
def test_swish():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.swish(x), x * expit(x), rtol=1e-13, atol=1e-300)
    assert oracle.swish(0.0) == 0.0
    assert abs(oracle.swish(40.0) - 40.0) < 1e-12


# ---------------------------------------------------------------- layer ----
def _layer_case(seed, B=1, N=10, dm=12, H=3, dk=4, dv=4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((B, N, dm))
    W = [rng.standard_normal(s) / 3 for s in ((dm, H * dk), (dm, H * dk), (dm, H * dv), (dm, H * dv), (H * dv, dm))]
    return X, W, np.array([0.5, 0.8, 0.95][:H])


def test_layer_decomposes_over_heads():
    """Heads are contiguous column blocks of the projections and GroupNorm
    is per head, so the layer equals the sum over heads of one-head layers
    built from the matching weight slices ([RN-zh] Eq. (8))."""
    X, (WQ, WK, WV, WG, WO), g = _layer_case(26)
    H, dk, dv = 3, 4, 4
    full = oracle.msr_layer(X, WQ, WK, WV, WG, WO, g, H, dk, dv, chunk=3)
    acc = 0
    for h in range(H):
        sk, sv = slice(h * dk, (h + 1) * dk), slice(h * dv, (h + 1) * dv)
        acc = acc + oracle.msr_layer(X, WQ[:, sk], WK[:, sk], WV[:, sv], WG[:, sv], WO[sv, :], g[h:h + 1], 1, dk, dv, chunk=3)
    assert close(full, acc)


def test_layer_forms_agree_and_gate():
    X, W, g = _layer_case(27)
    outs = [oracle.msr_layer(X, *W, g, 3, 4, 4, chunk=c, form=f)
            for f, c in (("parallel", None), ("recurrent", None), ("chunkwise", 3), ("chunkwise", 4))]
    for o in outs[1:]:
        assert close(o, outs[0], 1e-11)
    WQ, WK, WV, WG, WO = W
    zero_gate = oracle.msr_layer(X, WQ, WK, WV, np.zeros_like(WG), WO, g, 3, 4, 4, chunk=3)
    assert np.all(zero_gate == 0.0)


def test_layer_rectangular_heads():
    """d_v != d_k and H*d_v != d_model (the block shape with v head dim 512):
    weight shapes follow the projections, W_O is [H*d_v, d_model]."""
    X, W, g = _layer_case(28, dm=8, H=2, dk=2, dv=6)
    o = oracle.msr_layer(X, *W, g[:2], 2, 2, 6, chunk=4)
    assert o.shape == (1, 10, 8)
    assert close(o, oracle.msr_layer(X, *W, g[:2], 2, 2, 6, form="recurrent"), 1e-11)


def test_error_measures():
    ref = np.zeros((1, 3, 2, 2))
    ref[0, :, 0] = 100.0
    ref[0, :, 1] = 1.0
    got = ref.copy()
    got[0, 0, 1, 0] += 0.05
    assert oracle.max_rel_err(got, ref) == pytest.approx(0.0005)
    assert oracle.max_rel_err_per_head(got, ref) == pytest.approx(0.05)


def test_layer_gn_var_output_is_the_groupnorm_input_variance():
    """return_gn_var returns the per-(token, head) variance that the
    GroupNorm divides by: normalising by it reproduces a zero-mean, unit-
    variance row (eps = 0)."""
    X, W, g = _layer_case(29)
    out, gv = oracle.msr_layer(X, *W, g, 3, 4, 4, chunk=3, eps=0.0, return_gn_var=True)
    assert close(out, oracle.msr_layer(X, *W, g, 3, 4, 4, chunk=3, eps=0.0))
    assert gv.shape == (1, 10, 3) and np.all(gv > 0)


def test_layer_decode_steps_reproduce_the_layer_forward():
    """Decoding a sequence token by token with the layer decode step from a
    zero state (positions 0, 1, ...) gives the rows of the full-sequence
    layer forward in the parallel form -- rotation at each absolute
    position, the state update order of Eq. (6), GroupNorm and gate per
    token -- and the final state equals the recurrent form's.  A second
    batch element starts from a non-zero state: its steps equal the layer
    forward of the same tokens with that state as the chunkwise form's
    initial state."""
    rng = np.random.default_rng(17)
    B, N, dm, H, dk, dv = 2, 9, 16, 2, 4, 6
    X = rng.standard_normal((B, N, dm))
    WQ, WK = (rng.standard_normal((dm, H * dk)) / 4 for _ in range(2))
    WV, WG = (rng.standard_normal((dm, H * dv)) / 4 for _ in range(2))
    WO = rng.standard_normal((H * dv, dm)) / 4
    g = np.array([0.9, 0.6])
    ref = oracle.msr_layer(X, WQ, WK, WV, WG, WO, g, H, dk, dv, form="parallel", eps=1e-5)
    S = np.zeros((B, H, dk, dv))
    for n in range(N):
        out, S = oracle.msr_layer_decode_step(X[:, n], S, WQ, WK, WV, WG, WO, g, H, dk, dv, pos=n, eps=1e-5)
        assert np.max(np.abs(out - ref[:, n])) < 1e-12
    q = oracle.rotary((X @ WQ).reshape(B, N, H, dk), 0, 1e4)
    k = oracle.rotary((X @ WK).reshape(B, N, H, dk), 0, 1e4)
    v = (X @ WV).reshape(B, N, H, dv)
    _, S_rec = oracle.retention_recurrent(q, k, v, g, 1 / np.sqrt(dk))
    assert np.max(np.abs(S - S_rec)) < 1e-12
    # continuation from a non-zero state: 4 more tokens at positions N..N+3
    X2 = rng.standard_normal((B, 4, dm))
    S2 = S.copy()
    outs = []
    for n in range(4):
        out, S2 = oracle.msr_layer_decode_step(X2[:, n], S2, WQ, WK, WV, WG, WO, g, H, dk, dv, pos=N + n, eps=1e-5)
        outs.append(out)
    q2 = oracle.rotary((X2 @ WQ).reshape(B, 4, H, dk), N, 1e4)
    k2 = oracle.rotary((X2 @ WK).reshape(B, 4, H, dk), N, 1e4)
    v2 = (X2 @ WV).reshape(B, 4, H, dv)
    o2, _ = oracle.retention_chunkwise(q2, k2, v2, g, 2, 1 / np.sqrt(dk), S0=S)
    y2 = oracle.group_norm_heads(o2, 1e-5).reshape(B, 4, H * dv)
    ref2 = (oracle.swish(X2 @ WG) * y2) @ WO
    assert np.max(np.abs(np.stack(outs, axis=1) - ref2)) < 1e-12


def test_layer_norm_moments_and_invariance():
    """LayerNorm output rows have mean 0 and (at eps = 0) variance 1, and
    LN(a x + b) = LN(x) for a > 0 and any shift b, row by row."""
    rng = np.random.default_rng(21)
    X = rng.standard_normal((3, 5, 12)) * 3 + 1
    Y = oracle.layer_norm(X, 0.0)
    assert np.max(np.abs(Y.mean(axis=-1))) < 1e-12
    assert np.max(np.abs((Y ** 2).mean(axis=-1) - 1)) < 1e-12
    a = rng.uniform(0.1, 10, (3, 5, 1))
    b = rng.standard_normal((3, 5, 1))
    assert np.max(np.abs(oracle.layer_norm(a * X + b, 0.0) - Y)) < 1e-12
    # eps shrinks the output by sqrt(var / (var + eps))
    var = X.var(axis=-1, keepdims=True)
    assert np.max(np.abs(oracle.layer_norm(X, 0.5) - Y * np.sqrt(var / (var + 0.5)))) < 1e-12


def test_gelu_closed_forms():
    """gelu(x) = x Phi(x): gelu(0) = 0, gelu(x) - gelu(-x) = x, gelu(1) =
    Phi(1) = 0.841344746068542948..., gelu(-1) = Phi(1) - 1, and gelu(x) ->
    x (resp. 0) for large positive (negative) x."""
    x = np.linspace(-6, 6, 101)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    assert np.max(np.abs(oracle.gelu(x) - oracle.gelu(-x) - x)) < 1e-12
    phi1 = 0.841344746068542948585232545632
    assert abs(oracle.gelu(np.array([1.0]))[0] - phi1) < 1e-15
    assert abs(oracle.gelu(np.array([-1.0]))[0] - (phi1 - 1.0)) < 1e-15
    assert abs(oracle.gelu(np.array([12.0]))[0] - 12.0) < 1e-12
    assert abs(oracle.gelu(np.array([-12.0]))[0]) < 1e-12


def test_retnet_block_wiring():
    """The block's residual wiring: with W_1 = 0 the feed-forward branch
    vanishes and out = MSR(LN(X)) + X; with W_O = 0 the layer's branch
    vanishes and out = X + gelu(LN(X) W_1) W_2; with both, out = X."""
    rng = np.random.default_rng(22)
    B, N, dm, H, dk, dv, F = 2, 7, 16, 2, 4, 4, 24
    X = rng.standard_normal((B, N, dm))
    WQ, WK = (rng.standard_normal((dm, H * dk)) / 4 for _ in range(2))
    WV, WG = (rng.standard_normal((dm, H * dv)) / 4 for _ in range(2))
    WO = rng.standard_normal((H * dv, dm)) / 4
    W1 = rng.standard_normal((dm, F)) / 4
    W2 = rng.standard_normal((F, dm)) / 4
    g = np.array([0.9, 0.5])
    Z1, ZO = np.zeros_like(W1), np.zeros_like(WO)
    msr_x = oracle.msr_layer(oracle.layer_norm(X, 1e-5), WQ, WK, WV, WG, WO, g, H, dk, dv, form="parallel")
    got = oracle.retnet_block(X, WQ, WK, WV, WG, WO, Z1, W2, g, H, dk, dv, chunk=3)
    assert np.max(np.abs(got - (msr_x + X))) < 1e-12
    got = oracle.retnet_block(X, WQ, WK, WV, WG, ZO, W1, W2, g, H, dk, dv, chunk=3)
    ffn = oracle.gelu(oracle.layer_norm(X, 1e-5) @ W1) @ W2
    assert np.max(np.abs(got - (X + ffn))) < 1e-12
    got = oracle.retnet_block(X, WQ, WK, WV, WG, ZO, Z1, W2, g, H, dk, dv, chunk=3)
    assert np.max(np.abs(got - X)) < 1e-15


# --------------------------------------------------------------------------
# Gradients (training with the parallel and chunkwise forms)
# --------------------------------------------------------------------------
def _loss(q, k, v, S0, dO, dS, gamma, scale):
    O, S = oracle.retention_recurrent(q, k, v, gamma, scale, S0=S0)
    return float(np.sum(dO * O) + np.sum(dS * S))


def test_retention_grad_matches_finite_differences():
    """Every entry of dQ, dK, dV, dS0 against a central difference of the
    recurrent form's loss <dO, O> + <dS, S_last>.  The loss is linear in
    each single entry, so the difference is exact up to rounding; gamma = 0
    and gamma = 1 heads are included."""
    rng = np.random.default_rng(41)
    B, N, H, dk, dv = 2, 5, 3, 3, 2
    gamma = np.array([0.9, 0.0, 1.0])
    scale = 0.7
    q, k = rng.standard_normal((B, N, H, dk)), rng.standard_normal((B, N, H, dk))
    v, dO = rng.standard_normal((B, N, H, dv)), rng.standard_normal((B, N, H, dv))
    S0, dS = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, H, dk, dv))
    grads = oracle.retention_grad(q, k, v, dO, gamma, scale, S0=S0, dS=dS)
    args = [q, k, v, S0]
    eps = 1e-3
    for which, g in enumerate(grads):
        x = args[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(*args, dO, dS, gamma, scale)
            x[idx] = old - eps
            lm = _loss(*args, dO, dS, gamma, scale)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-9, atol=1e-9, err_msg=f"gradient {which}")


def test_retention_grad_without_state_terms():
    """S0 = None and dS = None are zeros: the gradients equal those with
    explicit zero states, and dS0 is then scale * (Q (.) xi)^T dO alone, a
    sum that the recurrent form's loss also yields by differences in S0."""
    rng = np.random.default_rng(42)
    B, N, H, dk, dv = 1, 4, 2, 2, 3
    gamma = np.array([0.5, 0.8])
    q, k = rng.standard_normal((B, N, H, dk)), rng.standard_normal((B, N, H, dk))
    v, dO = rng.standard_normal((B, N, H, dv)), rng.standard_normal((B, N, H, dv))
    z = np.zeros((B, H, dk, dv))
    a = oracle.retention_grad(q, k, v, dO, gamma, 1.3)
    b = oracle.retention_grad(q, k, v, dO, gamma, 1.3, S0=z, dS=z)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # entry (0, 1, 1, 2) of dS0 by difference
    e = np.zeros_like(z)
    e[0, 1, 1, 2] = 1.0
    fd = (_loss(q, k, v, e, dO, z, gamma, 1.3) - _loss(q, k, v, -e, dO, z, gamma, 1.3)) / 2
    assert abs(a[3][0, 1, 1, 2] - fd) < 1e-12


def test_retention_grad_sequence_split():
    """Carried-state semantics: the gradients of a sequence equal those of
    its two halves, the second half started from the first half's last
    state, and the first half receiving the second half's dS0 as dS."""
    rng = np.random.default_rng(43)
    B, N, H, dk, dv, n1 = 2, 9, 2, 3, 4, 4
    gamma = np.array([0.95, 0.6])
    q, k = rng.standard_normal((B, N, H, dk)), rng.standard_normal((B, N, H, dk))
    v, dO = rng.standard_normal((B, N, H, dv)), rng.standard_normal((B, N, H, dv))
    S0, dS = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, H, dk, dv))
    full = oracle.retention_grad(q, k, v, dO, gamma, 0.5, S0=S0, dS=dS)
    _, S_mid = oracle.retention_recurrent(q[:, :n1], k[:, :n1], v[:, :n1], gamma, 0.5, S0=S0)
    second = oracle.retention_grad(q[:, n1:], k[:, n1:], v[:, n1:], dO[:, n1:], gamma, 0.5, S0=S_mid, dS=dS)
    first = oracle.retention_grad(q[:, :n1], k[:, :n1], v[:, :n1], dO[:, :n1], gamma, 0.5, S0=S0, dS=second[3])
    for i in range(3):
        np.testing.assert_allclose(np.concatenate([first[i], second[i]], axis=1), full[i], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(first[3], full[3], rtol=1e-12, atol=1e-12)


def test_rotary_adjoint_is_the_inverse_rotation():
    rng = np.random.default_rng(44)
    x, y = rng.standard_normal((2, 7, 3, 8)), rng.standard_normal((2, 7, 3, 8))
    for base, pos0 in ((10000.0, 0), (10000.0, 4000), (50.0, 3), (0.0, 9)):
        rx = oracle.rotary(x, pos0, base)
        assert abs(np.sum(rx * y) - np.sum(x * oracle.rotary_adjoint(y, pos0, base))) < 1e-10
        np.testing.assert_allclose(oracle.rotary_adjoint(rx, pos0, base), x, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# RG-LRU ([GR-zh] section "實門線性循環單元 (RG-LRU)")
# --------------------------------------------------------------------------
def _zero_gates(D):
    z = np.zeros((D, D))
    return z, np.zeros(D), z.copy(), np.zeros(D)


def test_log_sigmoid():
    z = np.array([-3.0, -0.5, 0.0, 0.7, 4.0])
    np.testing.assert_allclose(oracle.log_sigmoid(z), np.log(1.0 / (1.0 + np.exp(-z))), rtol=1e-14)
    assert oracle.log_sigmoid(np.array([-800.0]))[0] == -800.0
    big = oracle.log_sigmoid(np.array([800.0]))[0]
    assert big <= 0.0 and big > -1e-300


def test_rglru_geometric_closed_form():
    """W = 0, b = 0 give r = i = 1/2; Lambda = 0 gives a = 1/2, so with c = 8
    a_t = (1/2)^4 = 1/16 and the gain is sqrt(1 - 1/256).  A constant input
    u then gives h_t = a^(t+1) h0 + gain (u/2) (1 - a^(t+1)) / (1 - a)."""
    rng = np.random.default_rng(51)
    B, T, D = 2, 40, 8
    u = rng.standard_normal((B, D))
    x = np.repeat(u[:, None, :], T, axis=1)
    h0 = rng.standard_normal((B, D))
    y, hT = oracle.rglru(x, *_zero_gates(D), np.zeros(D), 8.0, h0=h0)
    a, gain = 1.0 / 16.0, math.sqrt(1.0 - 1.0 / 256.0)
    t = np.arange(T)[None, :, None]
    ref = a ** (t + 1) * h0[:, None, :] + gain * (u[:, None, :] / 2) * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(hT, y[:, -1])


def test_rglru_gate_orientation_exact_values():
    """One weight W_a[j, k] = ln 3 and x_j = 1 make r_k = sigma(ln 3) = 3/4
    (applied as x @ W_a; the transposed product would gate channel j
    instead); with Lambda = 0, a_k = (1/2)^(8 * 3/4) = 1/64, i = 1/2, and
    one step from h0 = 0 gives y_k = sqrt(1 - 1/4096) * x_k / 2, while the
    other channels keep a = 1/16."""
    D, j, k = 6, 1, 4
    Wa, ba, Wx, bx = _zero_gates(D)
    Wa[j, k] = math.log(3.0)
    x = np.zeros((1, 1, D))
    x[0, 0, j], x[0, 0, k], x[0, 0, 0] = 1.0, 2.0, -3.0
    y, _ = oracle.rglru(x, Wa, ba, Wx, bx, np.zeros(D), 8.0)
    assert abs(y[0, 0, k] - math.sqrt(4095.0) / 64.0) < 1e-14
    g16 = math.sqrt(1.0 - 1.0 / 256.0)
    assert abs(y[0, 0, j] - g16 * 0.5) < 1e-14
    assert abs(y[0, 0, 0] - g16 * -1.5) < 1e-14
    assert np.all(y[0, 0, [2, 3, 5]] == 0.0)


def test_rglru_limits_and_log_space():
    """a -> 0 (Lambda very negative): no memory, y = i x.  a -> 1 (Lambda
    very positive): the state is kept, y = h0.  Lambda = 45: a_t rounds to
    1 in float64, but the log-space gain is sqrt(8 e^-45) (since
    log sigma(45) = -e^-45 to 20 digits and 1 - a^2 = -2 * 4 * log sigma(45)
    to first order)."""
    rng = np.random.default_rng(52)
    B, T, D = 2, 9, 5
    x = rng.standard_normal((B, T, D))
    h0 = rng.standard_normal((B, D))
    y, _ = oracle.rglru(x, *_zero_gates(D), np.full(D, -60.0), 8.0, h0=h0)
    np.testing.assert_allclose(y, 0.5 * x, rtol=1e-13, atol=1e-15)
    y, hT = oracle.rglru(x, *_zero_gates(D), np.full(D, 40.0), 8.0, h0=h0)
    np.testing.assert_allclose(y, np.repeat(h0[:, None], T, axis=1), rtol=0, atol=1e-7)
    y, _ = oracle.rglru(np.ones((1, 1, 1)), *_zero_gates(1), np.array([45.0]), 8.0)
    assert abs(y[0, 0, 0] / (0.5 * math.sqrt(8.0) * math.exp(-22.5)) - 1.0) < 1e-12


def test_rglru_split_continuation():
    """Running the second half from the first half's last state gives the
    full sequence's outputs and last state."""
    rng = np.random.default_rng(53)
    B, T, D, t1 = 2, 17, 6, 7
    x = rng.standard_normal((B, T, D))
    Wa, Wx = rng.standard_normal((D, D)) / math.sqrt(D), rng.standard_normal((D, D)) / math.sqrt(D)
    ba, bx, lam = rng.standard_normal(D), rng.standard_normal(D), rng.standard_normal(D) * 3
    h0 = rng.standard_normal((B, D))
    y, hT = oracle.rglru(x, Wa, ba, Wx, bx, lam, 8.0, h0=h0)
    y1, h1 = oracle.rglru(x[:, :t1], Wa, ba, Wx, bx, lam, 8.0, h0=h0)
    y2, h2 = oracle.rglru(x[:, t1:], Wa, ba, Wx, bx, lam, 8.0, h0=h1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(h2, hT, rtol=1e-14, atol=1e-15)


def test_rglru_input_recipe():
    """The generated Lambda puts sigma(Lambda)^8 on [0.9, 0.999]."""
    import workloads
    *_, lam = workloads.rglru_inputs(5, 1, 2, 512)
    ac = np.exp(8.0 * oracle.log_sigmoid(lam.astype(np.float64)))
    assert ac.min() >= 0.9 - 1e-6 and ac.max() <= 0.999 + 1e-6
    assert 0.93 < ac.mean() < 0.97


# ------------------------------------------------------- Eq. (8), by hand --
# A two-token, two-head layer small enough to work out on paper ([RN-zh]
# "門控多尺度 Retention", Eq. (8): Y = GroupNorm_h(Concat_h head_h),
# MSR(X) = (swish(X W_G) (.) Y) W_O).  X is the 2 x 2 identity, so row n of
# each weight matrix is token n's projection; head h owns columns 2h, 2h+1.
# No rotation, score scale s = 1/sqrt(d_k) = 1/sqrt(2), eps = 1/2,
# gamma = (1/2, 1/4).
#
#   token 0: q = (1, 0 | 1, 1)   k = (1, 0 | 1, 1)   v = (2, 0 | 1, 3)   g = (1, -1 | 0, 2)
#   token 1: q = (1, 1 | 2, 0)   k = (1, 1 | 1, 1)   v = (0, 4 | -1, 1)  g = (2, 0 | -2, 1)
#
# Retention, o_n = s sum_{m <= n} gamma^(n-m) (q_n . k_m) v_m:
#   head 0: o_0 = s (2, 0);   o_1 = s [ 1/2 * 1 * (2, 0) + 2 * (0, 4) ] = s (1, 8)
#   head 1: o_0 = s 2 (1, 3) = s (2, 6);   o_1 = s [ 1/4 * 2 * (1, 3) + 2 * (-1, 1) ] = s (-3/2, 7/2)
# GroupNorm of a pair (a, b): deviations +-(a - b)/2, variance ((a - b)/2)^2,
#   y = (a - b)/2 / sqrt(((a - b)/2)^2 + eps) * (1, -1):
#   head 0, token 0: (a-b)/2 = s,       var 1/2   -> y = (1, -1) / sqrt(2)
#   head 0, token 1: (a-b)/2 = -7s/2,   var 49/8  -> y = (-7, 7) / sqrt(53)
#   head 1, token 0: (a-b)/2 = -2s,     var 2     -> y = (-2, 2) / sqrt(5)
#   head 1, token 1: (a-b)/2 = -5s/2,   var 25/8  -> y = (-5, 5) / sqrt(29)
# Gate z = swish(g) (.) y, then out = z W_O with W_O rows (1,0), (0,1), (1,1), (0,-1):
#   out_n = (z0 + z2, z1 + z2 - z3).
_EQ8_W = {
    "WQ": [[1, 0, 1, 1], [1, 1, 2, 0]],
    "WK": [[1, 0, 1, 1], [1, 1, 1, 1]],
    "WV": [[2, 0, 1, 3], [0, 4, -1, 1]],
    "WG": [[1, -1, 0, 2], [2, 0, -2, 1]],
    "WO": [[1, 0], [0, 1], [1, 1], [0, -1]],
}
_EQ8_GAMMA = np.array([0.5, 0.25])


def _sw(x):
    return x / (1.0 + math.exp(-x))


def _eq8_by_hand():
    r2, r5, r29, r53 = math.sqrt(2), math.sqrt(5), math.sqrt(29), math.sqrt(53)
    z0 = [_sw(1) / r2, _sw(-1) * (-1 / r2), _sw(0) * (-2 / r5), _sw(2) * (2 / r5)]
    z1 = [_sw(2) * (-7 / r53), _sw(0) * (7 / r53), _sw(-2) * (-5 / r29), _sw(1) * (5 / r29)]
    out = [[z[0] + z[2], z[1] + z[2] - z[3]] for z in (z0, z1)]
    # state after both tokens, S_h = gamma_h k_0^T v_0 + k_1^T v_1
    S = [[[0.5 * 2 + 0, 0 + 4], [0 + 0, 0 + 4]],
         [[0.25 * 1 - 1, 0.25 * 3 + 1], [0.25 * 1 - 1, 0.25 * 3 + 1]]]
    return np.array([out]), np.array([S])


def _eq8_weights():
    return [np.array(_EQ8_W[n], dtype=np.float64) for n in ("WQ", "WK", "WV", "WG", "WO")]


def test_layer_composition_by_hand():
    """oracle.msr_layer (all three retention forms) and two decode steps of
    oracle.msr_layer_decode_step equal the hand-derived values above."""
    want, S_want = _eq8_by_hand()
    X = np.eye(2)[None]
    W = _eq8_weights()
    for form, chunk in (("parallel", None), ("recurrent", None), ("chunkwise", 1), ("chunkwise", 2)):
        got = oracle.msr_layer(X, *W, _EQ8_GAMMA, 2, 2, 2, chunk=chunk, rope_base=0.0, eps=0.5, form=form)
        assert np.max(np.abs(got - want)) < 1e-14, form
    S = np.zeros((1, 2, 2, 2))
    for n in range(2):
        out, S = oracle.msr_layer_decode_step(X[:, n], S, *W, _EQ8_GAMMA, 2, 2, 2, pos=n, rope_base=0.0, eps=0.5)
        assert np.max(np.abs(out - want[:, n])) < 1e-14
    assert np.max(np.abs(S - S_want)) < 1e-15


def test_layer_composition_pin_rejects_misreadings():
    """The hand-derived value separates Eq. (8) from plausible misreadings
    of it, each built here from the oracle's own parts: the gate applied
    before the GroupNorm, swish taken of the normalised heads instead of the
    gate branch, no swish, a sigmoid gate, one GroupNorm over all heads, and
    the heads' rows of W_O exchanged."""
    want, _ = _eq8_by_hand()
    X = np.eye(2)[None]
    WQ, WK, WV, WG, WO = _eq8_weights()
    s = 1 / math.sqrt(2)
    q = (X @ WQ).reshape(1, 2, 2, 2)
    k = (X @ WK).reshape(1, 2, 2, 2)
    v = (X @ WV).reshape(1, 2, 2, 2)
    g = X @ WG
    o = oracle.retention_parallel(q, k, v, _EQ8_GAMMA, s)
    gn = lambda t: oracle.group_norm_heads(t, 0.5).reshape(1, 2, 4)
    wrong = {
        "gate before GroupNorm": gn(oracle.swish(g).reshape(1, 2, 2, 2) * o) @ WO,
        "swish of the heads": (g * oracle.swish(gn(o))) @ WO,
        "no swish": (g * gn(o)) @ WO,
        "sigmoid gate": ((1 / (1 + np.exp(-g))) * gn(o)) @ WO,
        "one group": (oracle.swish(g) * oracle.group_norm_heads(o.reshape(1, 2, 1, 4), 0.5).reshape(1, 2, 4)) @ WO,
        "heads swapped in W_O": (oracle.swish(g) * gn(o)) @ WO[[2, 3, 0, 1]],
    }
    right = (oracle.swish(g) * gn(o)) @ WO
    assert np.max(np.abs(right - want)) < 1e-14
    for name, val in wrong.items():
        assert np.max(np.abs(val - want)) > 1e-2, name
