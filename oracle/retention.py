"""Float64 reference implementation of retention and the gated MSR layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, float64,
no blocking or fusion beyond what each definition states.

Pages cited (titles as printed on them):

* [RN-zh]  "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、速度快、
  性能強（2）" -- the RetNet method section.  Its displayed equations are
  stripped by the extraction; each function below states the definition it
  implements in words and names the equation number the page refers to.
* [RN-ja]  "[論文レビュー] Retentive Network: A Successor to Transformer for
  Large Language Models" -- abstract and method bullets.
* [RN-ru]  "Retentive Network: архитектурный прорыв или временный успех?" --
  decay-masked causal mask, per-head gamma, chunkwise recursion.
* [GR-zh]  "Griffin ：將門控線性循環與局部注意力混合以實現高效的語言模型" --
  section "實門線性循環單元 (RG-LRU)": the gated diagonal recurrence.

Tensor layout everywhere: [batch, seqlen, heads, head_dim] (token-major, the
natural output of X @ W).  gamma is a float64 array with one value per head.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


# --------------------------------------------------------------------------
# Relative-position rotation (xPos / rotary)
# --------------------------------------------------------------------------
def rotary(x, pos0: int = 0, base: float = 10000.0):
    """Rotate interleaved pairs of ``x`` [B, N, H, d] by position.

    [RN-zh] section "Retention", Eq. (3)-(4): diagonalising the state matrix
    gives the factor e^{i n theta} on Q_n (and its conjugate on K_m) so the
    score depends on the relative position n - m (the page calls it xPos).
    Real form: pair j = (x[2j], x[2j+1]) read as the complex number
    x[2j] + i x[2j+1] is multiplied by e^{i p theta_j}, with p = pos0 + n and
    theta_j = base^(-2j/d).  The same rotation is applied to Q and to K.
    ``base <= 0`` means no rotation.
    """
    x = _f64(x)
    if base is None or base <= 0:
        return x.copy()
    B, N, H, d = x.shape
    if d % 2:
        raise ValueError("rotary needs an even head dimension")
    j = np.arange(d // 2, dtype=F64)
    theta = base ** (-2.0 * j / d)                       # [d/2]
    p = (pos0 + np.arange(N, dtype=F64))[:, None]        # [N, 1]
    ang = p * theta[None, :]                             # [N, d/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# --------------------------------------------------------------------------
# Decay mask and the three forms of retention
# --------------------------------------------------------------------------
def decay_mask(N: int, gamma: float):
    """D[n, m] = gamma^(n-m) for n >= m, else 0.

    [RN-zh] section "1) Retention 的並行表征", Eq. (5); [RN-ru] "Causal Mask
    с затуханием".  gamma = 0 gives the identity (0^0 = 1 on the diagonal).
    """
    n = np.arange(N)
    diff = n[:, None] - n[None, :]
    D = np.zeros((N, N), dtype=F64)
    low = diff >= 0
    D[low] = np.power(F64(gamma), diff[low].astype(F64))
    return D


def retention_parallel(q, k, v, gamma, scale: float = 1.0):
    """Parallel form: O = ((Q K^T) * scale  (.)  D) V per (batch, head).

    [RN-zh] section "1) Retention 的並行表征", Eq. (5), Fig. 3a.
    q, k: [B, N, H, dk]; v: [B, N, H, dv]; gamma: [H].  Returns [B, N, H, dv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, _ = q.shape
    out = np.zeros(v.shape, dtype=F64)
    for h in range(H):
        D = decay_mask(N, float(gamma[h]))
        for b in range(B):
            scores = (q[b, :, h, :] @ k[b, :, h, :].T) * scale
            out[b, :, h, :] = (scores * D) @ v[b, :, h, :]
    return out


def retention_recurrent(q, k, v, gamma, scale: float = 1.0, S0=None):
    """Recurrent form, token by token.

    [RN-zh] section "2) Retention 的循環表征", Eq. (6), Fig. 3b:
    S_n = gamma * S_{n-1} + K_n^T V_n, then o_n = scale * Q_n S_n (the state is
    updated before it is read, so token n sees itself with weight gamma^0).
    S0: optional initial state [B, H, dk, dv] (zeros if None).
    Returns (O [B, N, H, dv], S_final [B, H, dk, dv]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv), dtype=F64) if S0 is None else _f64(S0).copy()
    g = _f64(gamma)[None, :, None, None]
    out = np.zeros((B, N, H, dv), dtype=F64)
    for n in range(N):
        S = g * S + k[:, n, :, :, None] * v[:, n, :, None, :]
        out[:, n] = scale * np.einsum("bhi,bhij->bhj", q[:, n], S)
    return out, S


def retention_chunkwise(q, k, v, gamma, chunk: int, scale: float = 1.0, S0=None):
    """Chunkwise recurrent form.

    [RN-zh] section "3) Retention 分塊循環表征", Eq. (7); [RN-ru]
    "Chunk-wise рекурсия": inside a chunk the parallel form (Eq. 5) is used,
    across chunks the state is passed on as in the recurrent form (Eq. 6).
    Chunks are the contiguous slices [i*B, (i+1)*B); the last one may be short
    (length L).  With rows t, s indexed from 0 inside the chunk:

      O_[i] = ((Q_[i] K_[i]^T) * scale (.) D_L) V_[i]
              + scale * (Q_[i] R_{i-1}) (.) xi,     xi_t   = gamma^(t+1)
      R_i   = gamma^L R_{i-1} + K_[i]^T (V_[i] (.) zeta),  zeta_s = gamma^(L-1-s)

    R_{-1} = S0 (zeros if None).  Returns (O, R_last).
    """
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, dk = q.shape
    dv = v.shape[-1]
    R = np.zeros((B, H, dk, dv), dtype=F64) if S0 is None else _f64(S0).copy()
    out = np.zeros((B, N, H, dv), dtype=F64)
    for c0 in range(0, N, chunk):
        L = min(chunk, N - c0)
        qc, kc, vc = q[:, c0:c0 + L], k[:, c0:c0 + L], v[:, c0:c0 + L]
        for h in range(H):
            gam = F64(gamma[h])
            D = decay_mask(L, gam)
            t = np.arange(L, dtype=F64)
            xi = np.power(gam, t + 1.0)                  # [L]
            zeta = np.power(gam, L - 1.0 - t)            # [L]
            for b in range(B):
                Qb, Kb, Vb = qc[b, :, h], kc[b, :, h], vc[b, :, h]
                inner = ((Qb @ Kb.T) * scale * D) @ Vb
                cross = scale * (Qb @ R[b, h]) * xi[:, None]
                out[b, c0:c0 + L, h] = inner + cross
                R[b, h] = np.power(gam, L) * R[b, h] + Kb.T @ (Vb * zeta[:, None])
    return out, R


def retention_bruteforce(q, k, v, gamma, scale=1.0):
    """Scalar double loop, exact in rational arithmetic when the inputs are
    Fractions or integers (tiny inputs only).

    o[b,n,h,:] = sum_{m <= n} gamma^(n-m) * scale * (q_n . k_m) * v_m.
    Nested Python lists or numpy object arrays of shape [B, N, H, d].
    """
    q = np.asarray(q, dtype=object)
    k = np.asarray(k, dtype=object)
    v = np.asarray(v, dtype=object)
    B, N, H, dk = q.shape
    dv = v.shape[-1]
    out = np.empty((B, N, H, dv), dtype=object)
    for b in range(B):
        for h in range(H):
            g = gamma[h]
            for n in range(N):
                acc = [0] * dv
                for m in range(n + 1):
                    dot = 0
                    for i in range(dk):
                        dot += q[b, n, h, i] * k[b, m, h, i]
                    w = (g ** (n - m)) * scale * dot
                    for j in range(dv):
                        acc[j] += w * v[b, m, h, j]
                out[b, n, h, :] = acc
    return out


def retention_parallel_normalized(q, k, v, gamma):
    """Parallel form with the three normalisation factors of [RN-zh] section
    "Retention Score 歸一化":

      1. scores Q K^T / sqrt(dk);
      2. D~[n, m] = D[n, m] / sqrt(sum_{i<=n} D[n, i]);
      3. R = (Q K^T / sqrt(dk)) (.) D~, R~[n, m] = R[n, m] / max(|sum_{i<=n} R[n, i]|, 1).

    Output R~ V.  The page prints only the first factor; factors 2 and 3 are
    the reading stated here (both are positive per-row factors, so GroupNorm
    removes them exactly).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, dk = q.shape
    out = np.zeros(v.shape, dtype=F64)
    for h in range(H):
        D = decay_mask(N, float(gamma[h]))
        Dn = D / np.sqrt(D.sum(axis=1, keepdims=True))
        for b in range(B):
            R = (q[b, :, h] @ k[b, :, h].T) / math.sqrt(dk) * Dn
            R = R / np.maximum(np.abs(R.sum(axis=1, keepdims=True)), 1.0)
            out[b, :, h] = R @ v[b, :, h]
    return out


def recurrent_step(S, q, k, v, gamma, scale=1.0, pos=None, base=0.0):
    """One decode step of Eq. (6) for every (batch, head).

    S: [B, H, dk, dv]; q, k: [B, H, dk]; v: [B, H, dv].  When ``base > 0``
    q and k are first rotated at absolute position ``pos``.
    Returns (o [B, H, dv], S_new).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if base is not None and base > 0:
        q = rotary(q[:, None], pos, base)[:, 0]
        k = rotary(k[:, None], pos, base)[:, 0]
    g = _f64(gamma)[None, :, None, None]
    S_new = g * _f64(S) + k[..., :, None] * v[..., None, :]
    o = scale * np.einsum("bhi,bhij->bhj", q, S_new)
    return o, S_new


# --------------------------------------------------------------------------
# GroupNorm, swish gate, the gated MSR layer
# --------------------------------------------------------------------------
def group_norm_heads(O, eps: float):
    """GroupNorm with one group per head ([RN-zh] "門控多尺度 Retention":
    each head's output is normalised on its own because heads with different
    gamma have different variance).  Statistics per (token, head) over the
    head's d_v channels, biased variance, identity affine.
    """
    O = _f64(O)
    mu = O.mean(axis=-1, keepdims=True)
    var = ((O - mu) ** 2).mean(axis=-1, keepdims=True)
    return (O - mu) / np.sqrt(var + eps)


def swish(x):
    """swish(x) = x * sigmoid(x) (beta = 1)."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def msr_layer(X, WQ, WK, WV, WG, WO, gamma, heads, d_k, d_v, chunk=None,
              rope_base=10000.0, eps=1e-5, form="chunkwise", normalized=False,
              scale=None, return_gn_var=False):
    """Gated multi-scale retention layer, [RN-zh] "門控多尺度 Retention", Eq. (8):

      Q^ = X W_Q, K^ = X W_K, V = X W_V (heads = contiguous column blocks)
      Q, K = rotary(Q^), rotary(K^) at positions 0..N-1
      head_h = Retention_h(Q, K, V) with gamma_h, score scale 1/sqrt(d_k)
      Y = GroupNorm_h(Concat_h head_h)
      MSR(X) = (swish(X W_G) (.) Y) W_O

    X: [B, N, d_model]; W_Q, W_K: [d_model, H*d_k]; W_V, W_G: [d_model, H*d_v];
    W_O: [H*d_v, d_model].  ``form`` picks the retention form
    ("parallel", "recurrent", "chunkwise"); ``normalized=True`` uses the
    three score-normalisation factors instead (parallel form).
    ``return_gn_var=True`` also returns the biased variance of every
    (token, head) group entering the GroupNorm, [B, N, H] (how strongly eps
    weighs on that group's normalisation).
    """
    X = _f64(X)
    B, N, _ = X.shape
    q = (X @ _f64(WQ)).reshape(B, N, heads, d_k)
    k = (X @ _f64(WK)).reshape(B, N, heads, d_k)
    v = (X @ _f64(WV)).reshape(B, N, heads, d_v)
    g = X @ _f64(WG)
    q = rotary(q, 0, rope_base)
    k = rotary(k, 0, rope_base)
    s = 1.0 / math.sqrt(d_k) if scale is None else scale
    if normalized:
        o = retention_parallel_normalized(q, k, v, gamma)
    elif form == "parallel":
        o = retention_parallel(q, k, v, gamma, s)
    elif form == "recurrent":
        o, _ = retention_recurrent(q, k, v, gamma, s)
    elif form == "chunkwise":
        o, _ = retention_chunkwise(q, k, v, gamma, chunk or N, s)
    else:
        raise ValueError(form)
    y = group_norm_heads(o, eps).reshape(B, N, heads * d_v)
    out = (swish(g) * y) @ _f64(WO)
    if return_gn_var:
        return out, o.var(axis=-1)
    return out


def msr_layer_decode_step(x, S, WQ, WK, WV, WG, WO, gamma, heads, d_k, d_v, pos,
                          rope_base=10000.0, eps=1e-5, scale=None):
    """One decode step of the gated MSR layer: Eq. (8) with the recurrent
    form of retention, Eq. (6) ([RN-zh] "2) Retention 的循環表征" and
    "門控多尺度 Retention"), for one new token per sequence:

      q^, k^, v, g = x W_Q, x W_K, x W_V, x W_G         (x: [B, d_model])
      q, k = rotary(q^), rotary(k^) at absolute position ``pos``
      S <- gamma_h S + k^T v ;  o = scale * q S           (per head)
      out = (swish(g) (.) GroupNorm_h(o)) W_O

    S: [B, H, d_k, d_v] (the state after the tokens before ``pos``).
    Returns (out [B, d_model], S_new).
    """
    x = _f64(x)
    B = x.shape[0]
    q = (x @ _f64(WQ)).reshape(B, heads, d_k)
    k = (x @ _f64(WK)).reshape(B, heads, d_k)
    v = (x @ _f64(WV)).reshape(B, heads, d_v)
    g = x @ _f64(WG)
    s = 1.0 / math.sqrt(d_k) if scale is None else scale
    o, S_new = recurrent_step(S, q, k, v, gamma, s, pos=pos, base=rope_base)
    y = group_norm_heads(o, eps).reshape(B, heads * d_v)
    return (swish(g) * y) @ _f64(WO), S_new


# --------------------------------------------------------------------------
# The RetNet block around the layer
# --------------------------------------------------------------------------
def layer_norm(X, eps: float):
    """LayerNorm over the last axis ([RN-zh] "Retention 網路總體結構" names
    LayerNorm [BKH16]): biased variance, identity affine (no parameters are
    given), (x - mean) / sqrt(var + eps)."""
    X = _f64(X)
    mu = X.mean(axis=-1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=-1, keepdims=True)
    return (X - mu) / np.sqrt(var + eps)


def gelu(x):
    """gelu(x) = x * Phi(x), Phi the standard normal distribution function
    (the exact, erf form)."""
    from scipy.special import erf
    x = _f64(x)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def retnet_block(X, WQ, WK, WV, WG, WO, W1, W2, gamma, heads, d_k, d_v, chunk=None,
                 rope_base=10000.0, gn_eps=1e-5, ln_eps=1e-5):
    """One RetNet block ([RN-zh] "Retention 網路總體結構"): the layer of
    Eq. (8) and the feed-forward network FFN(X) = gelu(X W_1) W_2, each
    behind a LayerNorm and with a residual connection:

      Y   = MSR(LN(X)) + X
      out = FFN(LN(Y)) + Y

    X: [B, N, d_model]; W_1: [d_model, d_ffn]; W_2: [d_ffn, d_model]; the
    layer's weights as in msr_layer.
    """
    X = _f64(X)
    Y = msr_layer(layer_norm(X, ln_eps), WQ, WK, WV, WG, WO, gamma, heads, d_k, d_v, chunk,
                  rope_base=rope_base, eps=gn_eps) + X
    return gelu(layer_norm(Y, ln_eps) @ _f64(W1)) @ _f64(W2) + Y


# --------------------------------------------------------------------------
# Gradients of retention (training)
# --------------------------------------------------------------------------
def rotary_adjoint(x, pos0: int = 0, base: float = 10000.0):
    """Adjoint (= inverse) of ``rotary``: every interleaved pair is
    multiplied by e^{-i p theta_j} instead of e^{+i p theta_j}, so a
    gradient with respect to the rotated Q or K becomes the gradient with
    respect to the unrotated one.  ``base <= 0`` means no rotation."""
    x = _f64(x)
    if base is None or base <= 0:
        return x.copy()
    B, N, H, d = x.shape
    j = np.arange(d // 2, dtype=F64)
    theta = base ** (-2.0 * j / d)
    ang = (pos0 + np.arange(N, dtype=F64))[:, None] * theta[None, :]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c + xo * s
    out[..., 1::2] = -xe * s + xo * c
    return out


def retention_grad(q, k, v, dO, gamma, scale: float = 1.0, S0=None, dS=None):
    """Gradients of retention for training.  [RN-zh] "Retention 網路總體結構"
    trains with the parallel (Eq. 5) and chunkwise (Eq. 7) forms, which both
    compute, per (batch, head) with initial state S0 (zeros if None):

      S_n = gamma^(n+1) S0 + sum_{m <= n} gamma^(n-m) k_m^T v_m   (Eq. 6 unrolled)
      o_n = scale * q_n S_n,     S_last = S_{N-1}

    For the loss L = <dO, O> + <dS, S_last> (dS: gradient arriving at the
    last state, zeros if None) the gradients, written with the decay mask D
    of Eq. (5), xi_n = gamma^(n+1), zeta_m = gamma^(N-1-m) and A = (dO V^T) (.) D:

      dQ  = scale * A K + scale * xi (.) (dO S0^T)
      dK  = scale * A^T Q + zeta (.) (V dS^T)
      dV  = scale * ((Q K^T) (.) D)^T dO + zeta (.) (K dS)
      dS0 = scale * (Q (.) xi)^T dO + gamma^N dS

    q, k: [B, N, H, dk]; v, dO: [B, N, H, dv]; S0, dS: [B, H, dk, dv].
    Returns (dq, dk, dv, dS0).
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, N, H, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv), dtype=F64) if S0 is None else _f64(S0)
    dS = np.zeros((B, H, dk, dv), dtype=F64) if dS is None else _f64(dS)
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dS0 = np.zeros((B, H, dk, dv), dtype=F64)
    t = np.arange(N, dtype=F64)
    for h in range(H):
        gam = F64(gamma[h])
        D = decay_mask(N, gam)
        xi = np.power(gam, t + 1.0)[:, None]
        zeta = np.power(gam, N - 1.0 - t)[:, None]
        for b in range(B):
            Q, K, V, G = q[b, :, h], k[b, :, h], v[b, :, h], dO[b, :, h]
            A = (G @ V.T) * D
            dq[b, :, h] = scale * (A @ K) + scale * xi * (G @ S0[b, h].T)
            dkk[b, :, h] = scale * (A.T @ Q) + zeta * (V @ dS[b, h].T)
            dvv[b, :, h] = scale * (((Q @ K.T) * D).T @ G) + zeta * (K @ dS[b, h])
            dS0[b, h] = scale * ((Q * xi).T @ G) + np.power(gam, N) * dS[b, h]
    return dq, dkk, dvv, dS0


# --------------------------------------------------------------------------
# RG-LRU: the gated diagonal linear recurrence of Griffin
# --------------------------------------------------------------------------
def log_sigmoid(z):
    """log(sigma(z)) = -log(1 + e^(-z)), evaluated without overflow."""
    z = _f64(z)
    return -(np.maximum(-z, 0.0) + np.log1p(np.exp(-np.abs(z))))


def rglru(x, Wa, ba, Wx, bx, Lam, c: float = 8.0, h0=None):
    """Real-gated linear recurrent unit, [GR-zh] section "實門線性循環單元
    (RG-LRU)" (page "Griffin"):

      r_t = sigma(x_t W_a + b_a)            recurrence gate
      i_t = sigma(x_t W_x + b_x)            input gate
      a_t = a^(c r_t),  a = sigma(Lambda)   (diagonal, per channel)
      h_t = a_t (.) h_{t-1} + sqrt(1 - a_t^2) (.) (i_t (.) x_t)
      y_t = h_t

    a^(c r_t) is formed in log space, log a_t = c r_t log sigma(Lambda), and
    1 - a_t^2 = -expm1(2 log a_t), so neither loses precision as a_t -> 1.
    x: [B, T, D]; W_a, W_x: [D, D] (applied as x @ W); b_a, b_x, Lambda: [D];
    h0: [B, D] (zeros if None).  Returns (y [B, T, D], h_T [B, D]).
    """
    x = _f64(x)
    B, T, D = x.shape
    r = 1.0 / (1.0 + np.exp(-(x @ _f64(Wa) + _f64(ba))))
    i = 1.0 / (1.0 + np.exp(-(x @ _f64(Wx) + _f64(bx))))
    log_a = c * r * log_sigmoid(Lam)                       # [B, T, D]
    a = np.exp(log_a)
    gain = np.sqrt(-np.expm1(2.0 * log_a))
    h = np.zeros((B, D), dtype=F64) if h0 is None else _f64(h0).copy()
    y = np.empty((B, T, D), dtype=F64)
    for t in range(T):
        h = a[:, t] * h + gain[:, t] * (i[:, t] * x[:, t])
        y[:, t] = h
    return y, h


# --------------------------------------------------------------------------
# Error measures
# --------------------------------------------------------------------------
def max_rel_err(got, ref):
    """max|got - ref| / max|ref| over the whole tensor."""
    got, ref = _f64(got), _f64(ref)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def max_rel_err_per_head(got, ref):
    """max over (batch, head) slices of max|got - ref| / max|ref| for raw
    retention outputs [B, N, H, d] (heads differ in scale by an order of
    magnitude, so a tensor-wide denominator would hide the small ones)."""
    got, ref = _f64(got), _f64(ref)
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[2]):
            worst = max(worst, max_rel_err(got[b, :, h], ref[b, :, h]))
    return worst


def exact_fraction(x):
    """Helper for the rational brute force: Fraction of a float, exactly."""
    return Fraction(x)
