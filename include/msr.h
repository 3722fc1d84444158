/*
 * msr.h -- C ABI of libmsr: multi-scale retention (MSR) on AMD Instinct
 * MI355X (gfx950).
 *
 * Pages cited:
 *   [RN-zh] "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、速度快、
 *           性能強（2）" -- the RetNet method: retention in three forms
 *           (sections "1) Retention 的並行表征" Eq. (5), "2) Retention 的循環
 *           表征" Eq. (6), "3) Retention 分塊循環表征" Eq. (7)), the gated
 *           multi-scale layer (section "門控多尺度 Retention", Eq. (8)) and the
 *           score normalisation (section "Retention Score 歸一化").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.   Activations are token-major [batch, seqlen, heads, head_dim],
 *           head_dim fastest (exactly what X @ W produces).  Weights are
 *           row-major [in, out] so the layer computes X @ W.  The recurrent
 *           state S is [batch, heads, d_k, d_v] float32, d_v fastest.
 * dtype.    MSR_F32: float32 everywhere.  MSR_BF16: bfloat16 inputs and
 *           outputs, float32 accumulation; the state S is always float32.
 * gamma.    Host array of `heads` doubles, 0 <= gamma_h <= 1, the per-head
 *           decay.  Powers of gamma are formed on the device as
 *           exp2(k * log2(gamma_h)) from log2(gamma_h) computed on the host
 *           in double precision.
 * Rotation. rope_base > 0 rotates interleaved pairs (x[2j], x[2j+1]) of Q
 *           and K by the angle p * theta_j, theta_j = rope_base^(-2j/d_k),
 *           p = absolute token position ([RN-zh] section "Retention",
 *           Eq. (3)-(4), xPos).  rope_base <= 0: no rotation.
 * Memory.   Every pointer except `gamma` is device memory allocated by the
 *           caller; the library allocates nothing and, apart from the
 *           opt-in msr_trace_* diagnostics and the static scratch of
 *           msr_layer_decode_step_noalloc, keeps no mutable global state
 *           (it is thread safe; that one entry point is not, per GPU).  Outputs must not alias
 *           inputs, except S of msr_recurrent_step and
 *           msr_layer_decode_step, which is updated in place.
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call
 *           only enqueues work and returns without synchronising.
 * Errors.   All arguments are validated on the host before anything is
 *           launched; on error nothing is enqueued and a status is returned
 *           (never an abort).  msr_last_error() gives a human-readable
 *           reason for the last failure on the calling thread.  A launch
 *           failure reported by the HIP runtime maps to MSR_ERR_HIP.
 * Supported head dims (else MSR_ERR_UNSUPPORTED): (d_k, d_v) in
 *           {(64,64), (128,128), (256,256), (256,512)}, the last one in
 *           bf16 only except for msr_recurrent_step; heads <= 128; chunk a
 *           positive multiple of 32, at most 4096; batch * seqlen < 2^31;
 *           heads * (2 d_k + 2 d_v) * 4096 < 2^31.
 */
#ifndef MSR_H
#define MSR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSR_OK = 0,
  MSR_ERR_NULL = 1,         /* a required pointer is NULL */
  MSR_ERR_SHAPE = 2,        /* negative / inconsistent sizes */
  MSR_ERR_DTYPE = 3,        /* unknown dtype */
  MSR_ERR_UNSUPPORTED = 4,  /* valid but not implemented (head dim, chunk) */
  MSR_ERR_WORKSPACE = 5,    /* workspace missing or too small */
  MSR_ERR_HIP = 6,          /* the HIP runtime reported an error */
  /* range markers, never returned: any int32 is a valid value of the type */
  MSR_STATUS_RANGE_MIN_ = -2147483647 - 1,
  MSR_STATUS_RANGE_MAX_ = 2147483647
} msr_status;

/* The two range markers are not dtypes (they are rejected as
 * MSR_ERR_DTYPE); they give the enum the full int32 range, so that any
 * integer a caller passes is a valid value of the type and can be checked
 * (in C++ a value outside an enum's range is undefined behaviour). */
typedef enum {
  MSR_F32 = 0,
  MSR_BF16 = 1,
  MSR_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  MSR_DTYPE_RANGE_MAX_ = 2147483647
} msr_dtype;

typedef struct {
  int32_t batch, seqlen, heads, d_k, d_v;
} msr_dims;

/* Parallel form, [RN-zh] Eq. (5):
 *   O = ((Q K^T) * qk_scale  (.)  D) V,  D[n,m] = gamma_h^(n-m) (n >= m), else 0,
 * per (batch, head), with Q, K rotated at positions pos0 + n when
 * rope_base > 0.  Q, K: [batch, seqlen, heads, d_k]; V, O: [.., d_v].
 * Workspace: msr_parallel_workspace_bytes() bytes (0 when rope_base <= 0). */
msr_status msr_parallel_fwd(msr_dtype dtype, msr_dims dims, const double* gamma,
                            float rope_base, int64_t pos0, float qk_scale,
                            const void* Q, const void* K, const void* V, void* O,
                            void* workspace, size_t ws_bytes, void* stream);
size_t msr_parallel_workspace_bytes(msr_dtype dtype, msr_dims dims, float rope_base);

/* Chunkwise recurrent form, [RN-zh] Eq. (7).  Contiguous chunks of `chunk`
 * tokens (the last may be short, length L); t, s index rows inside a chunk:
 *   O_[i] = ((Q_[i] K_[i]^T) * qk_scale (.) D) V_[i]
 *           + qk_scale * (Q_[i] R_{i-1}) (.) xi,       xi_t   = gamma^(t+1)
 *   R_i   = gamma^L R_{i-1} + K_[i]^T (V_[i] (.) zeta), zeta_s = gamma^(L-1-s)
 * R_{-1} = S_in (NULL: zeros); S_out (nullable) receives the last R.  The
 * state is carried across chunks in float32.  S_in/S_out:
 * [batch, heads, d_k, d_v] float32; S_out may not alias S_in.  pos0 is the
 * absolute position of token 0 (the rotation of a continued sequence).
 * Workspace: msr_chunkwise_workspace_bytes() bytes. */
msr_status msr_chunkwise_fwd(msr_dtype dtype, msr_dims dims, int32_t chunk,
                             const double* gamma, float rope_base, int64_t pos0,
                             float qk_scale, const void* Q, const void* K,
                             const void* V, const float* S_in, float* S_out,
                             void* O, void* workspace, size_t ws_bytes,
                             void* stream);
size_t msr_chunkwise_workspace_bytes(msr_dtype dtype, msr_dims dims, int32_t chunk,
                                     float rope_base);

/* msr_chunkwise_fwd that also keeps, for msr_chunkwise_bwd_saved, the state
 * each chunk starts from ([RN-zh] Eq. (7): R_{i-1}, with R_{-1} = S_in or
 * zeros): R_chunks [batch, heads, ceil(seqlen / chunk), d_v, d_k] (dtype,
 * caller-owned device memory, non-NULL unless there are no tokens) receives
 * R_{i-1}^T of every chunk i, the states of the rotated K when rope_base >
 * 0.  Costs nothing extra: the forward computes these states in any case
 * and writes them there instead of into the workspace.  Arguments,
 * workspace and errors otherwise as msr_chunkwise_fwd. */
msr_status msr_chunkwise_fwd_save(msr_dtype dtype, msr_dims dims, int32_t chunk,
                                  const double* gamma, float rope_base, int64_t pos0,
                                  float qk_scale, const void* Q, const void* K,
                                  const void* V, const float* S_in, float* S_out,
                                  void* R_chunks, void* O, void* workspace,
                                  size_t ws_bytes, void* stream);

/* Backward of the chunkwise (equivalently parallel) form, for training
 * ([RN-zh] section "Retention 網路總體結構": training runs the parallel
 * form, Eq. (5), and the chunkwise form, Eq. (7)).  With Q, K rotated as in
 * msr_chunkwise_fwd, S_n = gamma^(n+1) S_in + sum_{m<=n} gamma^(n-m) k_m^T v_m
 * and o_n = qk_scale q_n S_n, it returns the gradients of
 * L = <dO, O> + <dS_out, S_last>, per (batch, head), D as in Eq. (5),
 * xi_n = gamma^(n+1), zeta_m = gamma^(seqlen-1-m), A = (dO V^T) (.) D:
 *   dQ    = qk_scale A K + qk_scale xi (.) (dO S_in^T)   (then rotated back)
 *   dK    = qk_scale A^T Q + zeta (.) (V dS_out^T)       (then rotated back)
 *   dV    = qk_scale ((Q K^T) (.) D)^T dO + zeta (.) (K dS_out)
 *   dS_in = qk_scale (Q (.) xi)^T dO + gamma^seqlen dS_out
 * Q, K, dQ, dK: [batch, seqlen, heads, d_k]; V, dO, dV: [.., d_v] (dtype);
 * S_in, dS_out (nullable: zeros) and dS_in (nullable: not computed):
 * [batch, heads, d_k, d_v] float32.  Q, K are the unrotated inputs when
 * rope_base > 0 and dQ, dK the gradients with respect to them.  Needs
 * d_k == d_v; with dS_out, |qk_scale| * gamma_h >= 2^-60 for every head
 * (else MSR_ERR_UNSUPPORTED).  dS_in may alias dS_out but not S_in.  The
 * gradient state runs backwards through the sequence in float32 chunk by
 * chunk.  Workspace: msr_chunkwise_bwd_workspace_bytes() bytes. */
msr_status msr_chunkwise_bwd(msr_dtype dtype, msr_dims dims, int32_t chunk,
                             const double* gamma, float rope_base, int64_t pos0,
                             float qk_scale, const void* Q, const void* K,
                             const void* V, const void* dO, const float* S_in,
                             const float* dS_out, void* dQ, void* dK, void* dV,
                             float* dS_in, void* workspace, size_t ws_bytes,
                             void* stream);
size_t msr_chunkwise_bwd_workspace_bytes(msr_dtype dtype, msr_dims dims, int32_t chunk,
                                         float rope_base);

/* msr_chunkwise_bwd given the forward's per-chunk states R_chunks, as
 * msr_chunkwise_fwd_save left them for the same dtype, dims, chunk, gamma,
 * rope_base, pos0, Q, K, V and S_in (not checked; read only).  The dQ term
 * is the causal retention of (dO, V, K) seeded with S_in^T, whose per-chunk
 * states are exactly those transposed (sums of v^T k against k^T v), so it
 * reads them instead of recomputing them -- on the bf16 path with d_k ==
 * d_v in {64, 128, 256} and chunk a multiple of 128; elsewhere R_chunks is
 * not read and the result is that of msr_chunkwise_bwd.  Arguments,
 * workspace and errors otherwise as msr_chunkwise_bwd; R_chunks must be
 * non-NULL unless there are no tokens. */
msr_status msr_chunkwise_bwd_saved(msr_dtype dtype, msr_dims dims, int32_t chunk,
                                   const double* gamma, float rope_base, int64_t pos0,
                                   float qk_scale, const void* Q, const void* K,
                                   const void* V, const void* dO, const float* S_in,
                                   const float* dS_out, const void* R_chunks, void* dQ,
                                   void* dK, void* dV, float* dS_in, void* workspace,
                                   size_t ws_bytes, void* stream);

/* RG-LRU, the gated diagonal linear recurrence of the page "Griffin ：將門控
 * 線性循環與局部注意力混合以實現高效的語言模型", section "實門線性循環單元
 * (RG-LRU)", per batch element and channel:
 *   r_t = sigmoid(x_t W_a + b_a),  i_t = sigmoid(x_t W_x + b_x)
 *   a_t = a^(c r_t), a = sigmoid(Lambda), formed in log space:
 *         log a_t = c r_t log sigmoid(Lambda), 1 - a_t^2 = -expm1(2 log a_t)
 *   h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i_t x_t),  y_t = h_t
 * X, Y: [batch, seqlen, width] (dtype); W_a, W_x: [width, width] (dtype,
 * applied as x @ W); b_a, b_x, Lambda: [width] float32; h0 (nullable:
 * zeros) and h_last (nullable) [batch, width] float32, h_last may not
 * alias h0.  The gates are stored in the workspace in dtype; the recurrence
 * runs in float32.  width must be a multiple of 64; c > 0 (the page uses 8).
 * Workspace: msr_rglru_workspace_bytes() bytes. */
msr_status msr_rglru_fwd(msr_dtype dtype, int32_t batch, int32_t seqlen,
                         int32_t width, float c, const void* X, const void* W_a,
                         const float* b_a, const void* W_x, const float* b_x,
                         const float* Lambda, const float* h0, float* h_last,
                         void* Y, void* workspace, size_t ws_bytes, void* stream);
size_t msr_rglru_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t seqlen,
                                 int32_t width);

/* Recurrent form, one decode step, [RN-zh] Eq. (6), for every (batch, head):
 *   S <- gamma_h S + k^T v ;  o = qk_scale * q S   (S updated in place)
 * q, k: [batch, heads, d_k]; v, o: [batch, heads, d_v] (dtype); S:
 * [batch, heads, d_k, d_v] float32.  q and k are rotated at position `pos`
 * when rope_base > 0.  No workspace. */
msr_status msr_recurrent_step(msr_dtype dtype, int32_t batch, int32_t heads,
                              int32_t d_k, int32_t d_v, const double* gamma,
                              float rope_base, int64_t pos, float qk_scale,
                              const void* q, const void* k, const void* v,
                              float* S, void* o, void* stream);

/* Gated multi-scale retention layer, [RN-zh] Eq. (8):
 *   Q^ = X W_Q, K^ = X W_K, V = X W_V, G = X W_G   (head h = column block h)
 *   Q, K = rotation of Q^, K^ at positions 0..seqlen-1 (rope_base > 0)
 *   head_h = chunkwise retention (chunk, gamma_h, score scale 1/sqrt(d_k))
 *   Y = GroupNorm per (token, head) over d_v, biased variance, eps = gn_eps,
 *       identity affine
 *   out = (swish(G) (.) Y) W_O,  swish(x) = x * sigmoid(x)
 * X: [batch, seqlen, d_model]; W_Q, W_K: [d_model, heads*d_k];
 * W_V, W_G: [d_model, heads*d_v]; W_O: [heads*d_v, d_model];
 * out: [batch, seqlen, d_model].  d_model must be a multiple of 64.
 * Workspace: msr_layer_workspace_bytes() bytes. */
msr_status msr_layer_fwd(msr_dtype dtype, int32_t batch, int32_t seqlen,
                         int32_t d_model, int32_t heads, int32_t d_k, int32_t d_v,
                         int32_t chunk, const double* gamma, float rope_base,
                         float gn_eps, const void* X, const void* W_Q,
                         const void* W_K, const void* W_V, const void* W_G,
                         const void* W_O, void* out, void* workspace,
                         size_t ws_bytes, void* stream);
size_t msr_layer_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t seqlen,
                                 int32_t d_model, int32_t heads, int32_t d_k,
                                 int32_t d_v, int32_t chunk);

/* One RetNet block around the layer, [RN-zh] section "Retention 網路總體結構":
 * the layer of Eq. (8) and the feed-forward network FFN(X) = gelu(X W_1) W_2,
 * each behind a LayerNorm and with a residual connection (pre-LayerNorm):
 *   Y   = MSR(LN(X)) + X
 *   out = FFN(LN(Y)) + Y
 * LN: per token over d_model, biased variance, identity affine, ln_eps;
 * gelu(x) = x Phi(x) (erf form).  X, out: [batch, seqlen, d_model]; the
 * layer's weights as in msr_layer_fwd; W_1: [d_model, d_ffn]; W_2:
 * [d_ffn, d_model].  Y and the hidden rows are kept in the element type.
 * d_model (at most 8192) and d_ffn must be multiples of 64.
 * Workspace: msr_retnet_block_workspace_bytes() bytes. */
msr_status msr_retnet_block_fwd(msr_dtype dtype, int32_t batch, int32_t seqlen,
                                int32_t d_model, int32_t heads, int32_t d_k, int32_t d_v,
                                int32_t chunk, int32_t d_ffn, const double* gamma,
                                float rope_base, float gn_eps, float ln_eps,
                                const void* X, const void* W_Q, const void* W_K,
                                const void* W_V, const void* W_G, const void* W_O,
                                const void* W_1, const void* W_2, void* out,
                                void* workspace, size_t ws_bytes, void* stream);
size_t msr_retnet_block_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t seqlen,
                                        int32_t d_model, int32_t heads, int32_t d_k,
                                        int32_t d_v, int32_t chunk, int32_t d_ffn);

/* One decode step of the gated MSR layer: Eq. (8) of [RN-zh] with the
 * recurrent form of retention, Eq. (6), for one new token per sequence:
 *   q^, k^, v, g = x W_Q, x W_K, x W_V, x W_G
 *   q, k = q^, k^ rotated at absolute position `pos` (rope_base <= 0: none)
 *   S <- gamma_h S + k^T v ;  o = (q S) / sqrt(d_k)        (per head)
 *   out = (swish(g) (.) GroupNorm_h(o)) W_O
 * X: [batch, d_model] (the new token of each sequence); weights as in
 * msr_layer_fwd; S: [batch, heads, d_k, d_v] float32, the state after the
 * tokens before `pos`, updated in place; out: [batch, d_model].  `pos` is
 * the number of tokens the state has absorbed (>= 0).  The retention output
 * stays float32 up to the GroupNorm.  d_model must be a multiple of 64.
 * Workspace: msr_layer_decode_workspace_bytes() bytes. */
msr_status msr_layer_decode_step(msr_dtype dtype, int32_t batch, int32_t d_model,
                                 int32_t heads, int32_t d_k, int32_t d_v,
                                 const double* gamma, float rope_base, float gn_eps,
                                 int64_t pos, const void* X, const void* W_Q,
                                 const void* W_K, const void* W_V, const void* W_G,
                                 const void* W_O, float* S, void* out,
                                 void* workspace, size_t ws_bytes, void* stream);
size_t msr_layer_decode_workspace_bytes(msr_dtype dtype, int32_t batch,
                                        int32_t d_model, int32_t heads,
                                        int32_t d_k, int32_t d_v);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * msr_layer_decode_step with its workspace in a static device array of
 * msr_layer_decode_noalloc_max_bytes() bytes (64 MiB) that each GPU holds
 * from the time the library is loaded on it until the process ends.  Same
 * arguments and results as msr_layer_decode_step, without the workspace;
 * the array of the current device is used (the stream must belong to it).
 * It allocates nothing and calls no allocating routine; the first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress).
 * Returns MSR_ERR_WORKSPACE, before anything is enqueued, when the step
 * needs more than the array holds (msr_layer_decode_workspace_bytes() >
 * msr_layer_decode_noalloc_max_bytes(), e.g. batch 256 at d_model 4096 with
 * 16 heads of 256).  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (several streams, several host threads) race. */
msr_status msr_layer_decode_step_noalloc(msr_dtype dtype, int32_t batch, int32_t d_model,
                                         int32_t heads, int32_t d_k, int32_t d_v,
                                         const double* gamma, float rope_base, float gn_eps,
                                         int64_t pos, const void* X, const void* W_Q,
                                         const void* W_K, const void* W_V, const void* W_G,
                                         const void* W_O, float* S, void* out, void* stream);
size_t msr_layer_decode_noalloc_max_bytes(void);

/* Diagnostics for benchmarks: per-kernel timing with HIP events.
 * msr_trace_enable(1) clears earlier totals and from then on brackets every
 * kernel the library launches with an event pair recorded on that launch's
 * stream; msr_trace_enable(0) stops (and clears).  msr_trace_count() waits
 * for all recorded events, folds them into per-kernel totals and returns the
 * number of distinct kernels; msr_trace_get(i, ...) returns the i-th kernel's
 * name (valid until the next msr_trace_* call), total milliseconds and launch
 * count (MSR_ERR_SHAPE for i out of range).  Process-wide state, not thread
 * safe; never enable it in a caller that must not synchronise. */
void msr_trace_enable(int32_t on);
int32_t msr_trace_count(void);
msr_status msr_trace_get(int32_t i, const char** name, double* total_ms, int64_t* launches);

/* Name of a status code. */
const char* msr_status_str(msr_status s);
/* Reason for the last non-OK status returned on the calling thread. */
const char* msr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MSR_H */
