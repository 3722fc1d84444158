// libmsr C ABI: argument validation, workspace layout and dispatch.
// The operations and their arguments are documented in include/msr.h.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/msr.h"
#include "msr_launch.h"

using namespace msr;

namespace {

thread_local std::string g_last_error;

msr_status fail(msr_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
msr_status fail(msr_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

msr_status ok() {
  g_last_error.clear();
  return MSR_OK;
}

msr_status from_hip(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MSR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
size_t elt_size(msr_dtype d) { return d == MSR_BF16 ? 2 : 4; }

bool dims_supported(int dk, int dv) {
  return (dk == 64 && dv == 64) || (dk == 128 && dv == 128) || (dk == 256 && dv == 256) ||
         (dk == 256 && dv == 512);
}

msr_status check_dtype(msr_dtype d) {
  if (d != MSR_F32 && d != MSR_BF16) return fail(MSR_ERR_DTYPE, "unknown dtype %d", (int)d);
  return MSR_OK;
}

msr_status check_heads(int32_t batch, int32_t seqlen, int32_t heads, int32_t dk, int32_t dv) {
  if (batch < 0 || seqlen < 0 || heads <= 0 || dk <= 0 || dv <= 0)
    return fail(MSR_ERR_SHAPE, "invalid sizes batch=%d seqlen=%d heads=%d d_k=%d d_v=%d", batch, seqlen, heads, dk,
                dv);
  if (heads > kMaxHeads) return fail(MSR_ERR_UNSUPPORTED, "heads=%d exceeds %d", heads, kMaxHeads);
  if (!dims_supported(dk, dv))
    return fail(MSR_ERR_UNSUPPORTED, "(d_k, d_v) = (%d, %d) has no kernel; supported: (64,64) (128,128) (256,256) "
                "(256,512)", dk, dv);
  const int64_t tokens = (int64_t)batch * seqlen;
  if (tokens > (int64_t)INT32_MAX) return fail(MSR_ERR_UNSUPPORTED, "batch*seqlen exceeds 2^31-1");
  // in-chunk offsets are 32-bit: a chunk of rows of the widest token stride
  // (the fused projection buffer) must stay below 2^31 elements
  if ((int64_t)heads * (2 * dk + 2 * dv) * 4096 > (int64_t)INT32_MAX)
    return fail(MSR_ERR_UNSUPPORTED, "heads*(2 d_k + 2 d_v) too large");
  return MSR_OK;
}

// The matrix-core (chunkwise / parallel / layer) kernels have no float32
// variant for 512-wide value heads: its accumulators and tiles do not fit.
msr_status check_matrix_dims(msr_dtype dt, int dv) {
  if (dt == MSR_F32 && dv > 256)
    return fail(MSR_ERR_UNSUPPORTED, "d_v = %d has no float32 chunkwise/parallel kernel (bf16 only)", dv);
  return MSR_OK;
}

msr_status check_gamma(const double* gamma, int heads) {
  if (!gamma) return fail(MSR_ERR_NULL, "gamma is NULL");
  for (int h = 0; h < heads; ++h)
    if (!(gamma[h] >= 0.0 && gamma[h] <= 1.0))
      return fail(MSR_ERR_SHAPE, "gamma[%d] = %g is outside [0, 1]", h, gamma[h]);
  return MSR_OK;
}

msr_status check_chunk(int32_t chunk) {
  if (chunk <= 0) return fail(MSR_ERR_SHAPE, "chunk = %d must be positive", chunk);
  if (chunk % 32) return fail(MSR_ERR_UNSUPPORTED, "chunk = %d is not a multiple of 32", chunk);
  if (chunk > 4096) return fail(MSR_ERR_UNSUPPORTED, "chunk = %d exceeds 4096", chunk);
  return MSR_OK;
}

HeadTab make_tab(const double* gamma, int heads, int chunk, int seqlen) {
  HeadTab t;
  std::memset(&t, 0, sizeof t);
  int last = seqlen > 0 && chunk > 0 ? seqlen - ((seqlen - 1) / chunk) * chunk : 0;
  for (int h = 0; h < heads; ++h) {
    const double g = gamma[h];
    t.lg2[h] = g > 0.0 ? (float)std::log2(g) : -INFINITY;
    t.gchunk[h] = (float)std::pow(g, (double)chunk);
    t.glast[h] = (float)std::pow(g, (double)last);
    t.gam[h] = (float)g;
  }
  return t;
}

struct ChunkWs {
  size_t qr = 0, kr = 0, tab = 0, dr = 0, rx = 0, total = 0;
};

ChunkWs chunk_ws_layout(msr_dtype dt, const msr_dims& d, int32_t chunk, bool rope, bool with_state) {
  ChunkWs w;
  const size_t es = elt_size(dt);
  const size_t tok = (size_t)d.batch * d.seqlen;
  size_t off = 0;
  if (rope) {
    w.qr = off; off += align_up(tok * d.heads * d.d_k * es);
    w.kr = off; off += align_up(tok * d.heads * d.d_k * es);
    w.tab = off; off += align_up((size_t)d.seqlen * (d.d_k / 2) * sizeof(float2));
  }
  if (with_state) {
    const size_t nc = chunk > 0 ? ((size_t)d.seqlen + chunk - 1) / chunk : 0;
    const size_t st = (size_t)d.batch * d.heads * nc * d.d_k * d.d_v;
    w.dr = off; off += align_up(st * es);
    w.rx = w.dr;   // the scan overwrites each chunk's contribution with R_{i-1}
  }
  w.total = off;
  return w;
}

// Chunkwise backward: the retention passes' chunk workspace (shared, the
// passes run one after another), the rotated Q and K, the four reversed
// inputs and the two state seeds.
struct BwdWs {
  ChunkWs cw;
  size_t chunk = 0, sin_t = 0, dso = 0, total = 0;
};
BwdWs bwd_ws_layout(msr_dtype dt, const msr_dims& d, int32_t chunk, bool rope) {
  BwdWs w;
  const size_t state = (size_t)d.batch * d.heads * d.d_k * d.d_v * sizeof(float);
  w.cw = chunk_ws_layout(dt, d, chunk, rope, true);
  size_t off = 0;
  w.chunk = off; off += align_up(w.cw.total);
  w.sin_t = off; off += align_up(state);
  w.dso = off; off += align_up(state);
  w.total = off;
  return w;
}

struct LayerWs {
  size_t qkvg = 0, z = 0, tab = 0, chunk = 0, total = 0;
  ChunkWs cw;
};
LayerWs layer_ws_layout(msr_dtype dt, int32_t batch, int32_t seqlen, int32_t d_model, int32_t heads, int32_t dk,
                        int32_t dv, int32_t chunk) {
  (void)d_model;
  LayerWs w;
  const size_t es = elt_size(dt);
  const size_t M = (size_t)batch * seqlen;
  const size_t ntot = (size_t)heads * (2 * dk + 2 * dv);
  size_t off = 0;
  w.qkvg = off; off += align_up(M * ntot * es);
  w.z = off; off += align_up(M * heads * dv * es);
  w.tab = off; off += align_up((size_t)seqlen * (dk / 2) * sizeof(float2));
  msr_dims d{batch, seqlen, heads, dk, dv};
  w.cw = chunk_ws_layout(dt, d, chunk, false, true);
  w.chunk = off; off += w.cw.total;
  w.total = off;
  return w;
}

template <class P> P* at(void* base, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(base) + off); }

}  // namespace

struct DecodeWs {
  size_t qkvg = 0, o = 0, z = 0, part = 0, total = 0;
  int split_qkvg = 1, split_o = 1;
};
// Few rows (one per sequence): the projections split K over several
// workgroups (float32 partials) so that the weight stream covers the CUs.
DecodeWs decode_ws_layout(msr_dtype dt, int32_t batch, int32_t d_model, int32_t heads, int32_t dk, int32_t dv) {
  DecodeWs w;
  const size_t es = elt_size(dt);
  const int ntot = heads * (2 * dk + 2 * dv), hv = heads * dv;
  if (batch <= 256) {
    const Elt e = dt == MSR_BF16 ? kBF16 : kF32;
    w.split_qkvg = gemm_splits(e, batch, ntot, d_model);
    w.split_o = gemm_splits(e, batch, d_model, hv);
  }
  const size_t part = std::max((size_t)(w.split_qkvg > 1 ? w.split_qkvg : 0) * batch * ntot,
                               (size_t)(w.split_o > 1 ? w.split_o : 0) * batch * d_model);
  size_t off = 0;
  w.qkvg = off; off += align_up((size_t)batch * ntot * es);
  w.o = off; off += align_up((size_t)batch * hv * sizeof(float));
  w.z = off; off += align_up((size_t)batch * hv * es);
  w.part = off; off += align_up(part * sizeof(float));
  w.total = off;
  return w;
}

// RetNet block: the layer's workspace, then LN output, Y, and the
// feed-forward hidden rows.
struct BlockWs {
  LayerWs lw;
  size_t layer = 0, h = 0, y = 0, f = 0, total = 0;
};
BlockWs block_ws_layout(msr_dtype dt, int32_t batch, int32_t seqlen, int32_t d_model, int32_t heads, int32_t dk,
                        int32_t dv, int32_t chunk, int32_t d_ffn) {
  BlockWs w;
  const size_t es = elt_size(dt);
  const size_t M = (size_t)batch * seqlen;
  w.lw = layer_ws_layout(dt, batch, seqlen, d_model, heads, dk, dv, chunk);
  size_t off = 0;
  w.layer = off; off += align_up(w.lw.total);
  w.h = off; off += align_up(M * d_model * es);
  w.y = off; off += align_up(M * d_model * es);
  w.f = off; off += align_up(M * (size_t)d_ffn * es);
  w.total = off;
  return w;
}

// The layer's launches on validated arguments; the output projection adds
// `resid` ([M, d_model], nullable) in its epilogue.
static msr_status layer_launch(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t d_model, int32_t heads,
                               int32_t d_k, int32_t d_v, int32_t chunk, const double* gamma, float rope_base,
                               float gn_eps, const void* X, const void* W_Q, const void* W_K, const void* W_V,
                               const void* W_G, const void* W_O, void* out, const void* resid, const LayerWs& w,
                               void* workspace, void* stream) {
  const int64_t M = (int64_t)batch * seqlen;
  hipStream_t st = (hipStream_t)stream;
  const Elt e = dtype == MSR_BF16 ? kBF16 : kF32;
  const size_t es = elt_size(dtype);
  const int hk = heads * d_k, hv = heads * d_v;
  const int ntot = 2 * hk + 2 * hv;
  char* qkvg = at<char>(workspace, w.qkvg);
  char* z = at<char>(workspace, w.z);
  float2* tab = at<float2>(workspace, w.tab);
  void* cws = at<void>(workspace, w.chunk);
  const bool rope = rope_base > 0.f;

  // 1. (cos, sin) table of the positions 0..seqlen-1
  hipError_t err = rope ? launch_rope_table(tab, seqlen, d_k, 0, rope_base, st) : hipSuccess;
  // 2. [Q | K | V | G] = X [W_Q | W_K | W_V | W_G], Q and K rotated in the epilogue
  GemmB bq{};
  bq.ptr[0] = W_Q; bq.ptr[1] = W_K; bq.ptr[2] = W_V; bq.ptr[3] = W_G;
  bq.ld[0] = hk; bq.ld[1] = hk; bq.ld[2] = hv; bq.ld[3] = hv;
  bq.start[0] = 0; bq.start[1] = hk; bq.start[2] = 2 * hk; bq.start[3] = 2 * hk + hv;
  bq.rope_segs = rope ? 2 : 0;
  bq.rope_d = d_k;
  bq.seqlen = seqlen;
  bq.rope_tab = tab;
  if (err == hipSuccess) err = launch_gemm(e, X, d_model, bq, qkvg, ntot, (int)M, ntot, d_model, st);
  if (err != hipSuccess) return from_hip(err, "msr_layer_fwd(projections)");
  // 3. chunkwise retention + per-head GroupNorm + swish gate -> Z
  ChunkArgs a{};
  a.elt = e;
  a.d_k = d_k; a.d_v = d_v; a.batch = batch; a.seqlen = seqlen; a.heads = heads;
  a.chunk = chunk;
  a.Q = qkvg; a.ldq = ntot;
  a.K = qkvg + (size_t)hk * es; a.ldk = ntot;
  a.V = qkvg + (size_t)2 * hk * es; a.ldv = ntot;
  a.G = qkvg + (size_t)(2 * hk + hv) * es; a.ldg = ntot;
  a.O = z; a.ldo = hv;
  a.scale = 1.0f / std::sqrt((float)d_k);
  a.eps = gn_eps;
  a.fuse_gn_gate = true;
  a.dR = at<void>(cws, w.cw.dr);
  a.Rx = at<void>(cws, w.cw.rx);
  const HeadTab htab = make_tab(gamma, heads, chunk, seqlen);
  err = launch_chunkwise(a, htab, st);
  if (err != hipSuccess) return from_hip(err, "msr_layer_fwd(retention)");
  // 4. out = Z W_O
  GemmB bo{};
  bo.ptr[0] = W_O; bo.ld[0] = d_model;
  bo.start[0] = 0; bo.start[1] = bo.start[2] = bo.start[3] = INT32_MAX;
  bo.resid = resid; bo.ldr = d_model;
  err = launch_gemm(e, z, hv, bo, out, d_model, (int)M, d_model, hv, st);
  return from_hip(err, "msr_layer_fwd(output projection)");
}

extern "C" {

const char* msr_status_str(msr_status s) {
  switch (s) {
    case MSR_OK: return "MSR_OK";
    case MSR_ERR_NULL: return "MSR_ERR_NULL";
    case MSR_ERR_SHAPE: return "MSR_ERR_SHAPE";
    case MSR_ERR_DTYPE: return "MSR_ERR_DTYPE";
    case MSR_ERR_UNSUPPORTED: return "MSR_ERR_UNSUPPORTED";
    case MSR_ERR_WORKSPACE: return "MSR_ERR_WORKSPACE";
    case MSR_ERR_HIP: return "MSR_ERR_HIP";
    default: break;
  }
  return "MSR_ERR_UNKNOWN";
}

const char* msr_last_error(void) { return g_last_error.c_str(); }

size_t msr_chunkwise_workspace_bytes(msr_dtype dtype, msr_dims dims, int32_t chunk, float rope_base) {
  if (dims.batch < 0 || dims.seqlen < 0 || dims.heads <= 0 || dims.d_k <= 0 || dims.d_v <= 0 || chunk <= 0) return 0;
  return chunk_ws_layout(dtype, dims, chunk, rope_base > 0.f, true).total;
}

size_t msr_parallel_workspace_bytes(msr_dtype dtype, msr_dims dims, float rope_base) {
  if (dims.batch < 0 || dims.seqlen < 0 || dims.heads <= 0 || dims.d_k <= 0 || dims.d_v <= 0) return 0;
  return chunk_ws_layout(dtype, dims, 0, rope_base > 0.f, false).total;
}

// The (cos, sin) table of positions pos0 .. pos0 + seqlen - 1 into the
// workspace, and rotated copies of Q and K (either may be null: not rotated
// here) into it; *Qo / *Ko then point at the copies.
static msr_status rotate_qk(msr_dtype dtype, const msr_dims& d, float rope_base, int64_t pos0, const void* Q,
                            const void* K, void* ws, const ChunkWs& w, hipStream_t st, const void** Qo,
                            const void** Ko) {
  const Elt e = dtype == MSR_BF16 ? kBF16 : kF32;
  float2* tab = at<float2>(ws, w.tab);
  const int64_t ld = (int64_t)d.heads * d.d_k;
  const int rows = d.batch * d.seqlen;
  hipError_t err = launch_rope_table(tab, d.seqlen, d.d_k, pos0, rope_base, st);
  if (err == hipSuccess && Q)
    err = launch_rope_apply(e, Q, ld, at<void>(ws, w.qr), ld, rows, d.seqlen, d.heads, d.d_k, tab, st);
  if (err == hipSuccess && K)
    err = launch_rope_apply(e, K, ld, at<void>(ws, w.kr), ld, rows, d.seqlen, d.heads, d.d_k, tab, st);
  if (Q) *Qo = at<void>(ws, w.qr);
  if (K) *Ko = at<void>(ws, w.kr);
  return from_hip(err, "rotation");
}

msr_status msr_parallel_fwd(msr_dtype dtype, msr_dims d, const double* gamma, float rope_base, int64_t pos0,
                            float qk_scale, const void* Q, const void* K, const void* V, void* O, void* workspace,
                            size_t ws_bytes, void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(d.batch, d.seqlen, d.heads, d.d_k, d.d_v))) return s;
  if ((s = check_matrix_dims(dtype, d.d_v))) return s;
  if ((s = check_gamma(gamma, d.heads))) return s;
  if (pos0 < 0) return fail(MSR_ERR_SHAPE, "pos0 = %lld is negative", (long long)pos0);
  const size_t tok = (size_t)d.batch * d.seqlen;
  if (tok == 0) return ok();
  if (!Q || !K || !V || !O) return fail(MSR_ERR_NULL, "Q, K, V and O must be non-NULL");
  const bool rope = rope_base > 0.f;
  const ChunkWs w = chunk_ws_layout(dtype, d, 0, rope, false);
  if (w.total > 0 && (!workspace || ws_bytes < w.total))
    return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total, workspace ? ws_bytes : 0);
  hipStream_t st = (hipStream_t)stream;
  ChunkArgs a{};
  a.elt = dtype == MSR_BF16 ? kBF16 : kF32;
  a.d_k = d.d_k; a.d_v = d.d_v; a.batch = d.batch; a.seqlen = d.seqlen; a.heads = d.heads;
  a.ldq = a.ldk = (int64_t)d.heads * d.d_k;
  a.ldv = a.ldo = (int64_t)d.heads * d.d_v;
  if (rope) {
    // K rotated by a pass (no state kernel stages it here); Q by the output
    // kernel as it loads it where that kernel can, else by the pass too
    const int tpc = (d.seqlen + 127) / 128;
    const bool q_in_kernel = chunk_out_rotates_q(a.elt, d.d_k, d.d_v, tpc * 128) &&
                             !(a.elt == kBF16 && d.d_v <= 256);
    if ((s = rotate_qk(dtype, d, rope_base, pos0, q_in_kernel ? nullptr : Q, K, workspace, w, st, &Q, &K))) return s;
    if (q_in_kernel) a.q_rope_tab = at<float2>(workspace, w.tab);
  }
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.scale = qk_scale;
  const HeadTab tab = make_tab(gamma, d.heads, 0, d.seqlen);
  return from_hip(launch_parallel(a, tab, st), "msr_parallel_fwd");
}

// R_chunks (nullable): where the per-chunk states R_{i-1}^T go (else the workspace)
static msr_status chunkwise_fwd(msr_dtype dtype, msr_dims d, int32_t chunk, const double* gamma, float rope_base,
                                int64_t pos0, float qk_scale, const void* Q, const void* K, const void* V,
                                const float* S_in, float* S_out, void* R_chunks, void* O, void* workspace,
                                size_t ws_bytes, void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(d.batch, d.seqlen, d.heads, d.d_k, d.d_v))) return s;
  if ((s = check_matrix_dims(dtype, d.d_v))) return s;
  if ((s = check_chunk(chunk))) return s;
  if ((s = check_gamma(gamma, d.heads))) return s;
  if (pos0 < 0) return fail(MSR_ERR_SHAPE, "pos0 = %lld is negative", (long long)pos0);
  if (S_out && S_out == S_in) return fail(MSR_ERR_SHAPE, "S_out may not alias S_in");
  hipStream_t st = (hipStream_t)stream;
  const size_t tok = (size_t)d.batch * d.seqlen;
  if (d.batch == 0) return ok();
  if (d.seqlen == 0) {  // no tokens: the state passes through unchanged
    if (!S_out) return ok();
    HeadScale one;
    std::fill(one.c, one.c + kMaxHeads, 1.0f);
    return from_hip(launch_state_xform(S_in, S_out, d.batch * d.heads, d.heads, d.d_k, d.d_v, false, one, st),
                    "msr_chunkwise_fwd(seqlen=0)");
  }
  if (!Q || !K || !V || !O) return fail(MSR_ERR_NULL, "Q, K, V and O must be non-NULL");
  const bool rope = rope_base > 0.f;
  const ChunkWs w = chunk_ws_layout(dtype, d, chunk, rope, true);
  if (!workspace || ws_bytes < w.total)
    return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total, workspace ? ws_bytes : 0);
  (void)tok;
  ChunkArgs a{};
  a.elt = dtype == MSR_BF16 ? kBF16 : kF32;
  if (rope) {
    // K is rotated by the state kernel as it stages it (which writes the
    // rotated rows for the output kernel), Q by the output kernel as it
    // loads it -- or, for the one output kernel that cannot, by a pass
    const bool q_in_kernel = chunk_out_rotates_q(a.elt, d.d_k, d.d_v, chunk);
    if ((s = rotate_qk(dtype, d, rope_base, pos0, q_in_kernel ? nullptr : Q, nullptr, workspace, w, st, &Q,
                       nullptr)))
      return s;
    const float2* tab = at<float2>(workspace, w.tab);
    if (q_in_kernel) a.q_rope_tab = tab;
    a.k_rope_tab = tab;
    a.k_rot = at<void>(workspace, w.kr);
    a.ld_k_rot = (int64_t)d.heads * d.d_k;
  }
  a.d_k = d.d_k; a.d_v = d.d_v; a.batch = d.batch; a.seqlen = d.seqlen; a.heads = d.heads;
  a.chunk = chunk;
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.ldq = a.ldk = (int64_t)d.heads * d.d_k;
  a.ldv = a.ldo = (int64_t)d.heads * d.d_v;
  a.scale = qk_scale;
  a.S_in = S_in; a.S_out = S_out;
  // the state kernel's contributions and the scan's R_{i-1} share one buffer
  a.dR = a.Rx = R_chunks ? R_chunks : at<void>(workspace, w.rx);
  const HeadTab tab = make_tab(gamma, d.heads, chunk, d.seqlen);
  return from_hip(launch_chunkwise(a, tab, st), "msr_chunkwise_fwd");
}

msr_status msr_chunkwise_fwd(msr_dtype dtype, msr_dims d, int32_t chunk, const double* gamma, float rope_base,
                             int64_t pos0, float qk_scale, const void* Q, const void* K, const void* V,
                             const float* S_in, float* S_out, void* O, void* workspace, size_t ws_bytes,
                             void* stream) {
  return chunkwise_fwd(dtype, d, chunk, gamma, rope_base, pos0, qk_scale, Q, K, V, S_in, S_out, nullptr, O,
                       workspace, ws_bytes, stream);
}

msr_status msr_chunkwise_fwd_save(msr_dtype dtype, msr_dims d, int32_t chunk, const double* gamma, float rope_base,
                                  int64_t pos0, float qk_scale, const void* Q, const void* K, const void* V,
                                  const float* S_in, float* S_out, void* R_chunks, void* O, void* workspace,
                                  size_t ws_bytes, void* stream) {
  if (!R_chunks && d.batch > 0 && d.seqlen > 0) return fail(MSR_ERR_NULL, "R_chunks must be non-NULL");
  return chunkwise_fwd(dtype, d, chunk, gamma, rope_base, pos0, qk_scale, Q, K, V, S_in, S_out, R_chunks, O,
                       workspace, ws_bytes, stream);
}

size_t msr_chunkwise_bwd_workspace_bytes(msr_dtype dtype, msr_dims dims, int32_t chunk, float rope_base) {
  if (dims.batch < 0 || dims.seqlen < 0 || dims.heads <= 0 || dims.d_k <= 0 || dims.d_v <= 0 || chunk <= 0) return 0;
  return bwd_ws_layout(dtype, dims, chunk, rope_base > 0.f).total;
}

// dQ is the causal retention of (dO, V, K) seeded with S_in^T; dV and dK are
// the causal retentions of (rev K, rev Q, rev dO) and (rev V, rev dO, rev Q)
// on the time-reversed sequence, seeded with dS_out / (scale gamma) and its
// transpose (the dK pass's per-chunk states are the dV pass's transposed),
// whose output kernels write their rows back in forward time order;
// dS_in = scale gamma times the last state of the dV pass.
// R_chunks (nullable): the forward's per-chunk states R_{i-1}^T, which are the
// dQ pass's states R_{i-1} themselves; read in place by the direct-copy
// output kernel, ignored elsewhere (the dQ pass computes its own)
static msr_status chunkwise_bwd(msr_dtype dtype, msr_dims d, int32_t chunk, const double* gamma, float rope_base,
                                int64_t pos0, float qk_scale, const void* Q, const void* K, const void* V,
                                const void* dO, const float* S_in, const float* dS_out, const void* R_chunks,
                                void* dQ, void* dK, void* dV, float* dS_in, void* workspace, size_t ws_bytes,
                                void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(d.batch, d.seqlen, d.heads, d.d_k, d.d_v))) return s;
  if (d.d_k != d.d_v)
    return fail(MSR_ERR_UNSUPPORTED, "the backward needs d_k == d_v (got %d, %d): its dQ and dK passes swap them",
                d.d_k, d.d_v);
  if ((s = check_matrix_dims(dtype, d.d_v))) return s;
  if ((s = check_chunk(chunk))) return s;
  if ((s = check_gamma(gamma, d.heads))) return s;
  if (pos0 < 0) return fail(MSR_ERR_SHAPE, "pos0 = %lld is negative", (long long)pos0);
  if (dS_in && dS_in == S_in) return fail(MSR_ERR_SHAPE, "dS_in may not alias S_in");
  if (dS_out && d.batch > 0 && d.seqlen > 0)
    for (int h = 0; h < d.heads; ++h)
      if (!(std::fabs((double)qk_scale) * gamma[h] >= 0x1p-60))
        return fail(MSR_ERR_UNSUPPORTED,
                    "dS_out needs |qk_scale| * gamma_h >= 2^-60 (head %d: gamma %g, scale %g): it seeds the "
                    "reversed passes divided by qk_scale * gamma_h", h, gamma[h], (double)qk_scale);
  if (d.batch == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  const int nbh = d.batch * d.heads;
  HeadScale hs;
  if (d.seqlen == 0) {  // no tokens: dS_in = dS_out
    if (!dS_in) return ok();
    std::fill(hs.c, hs.c + kMaxHeads, 1.0f);
    return from_hip(launch_state_xform(dS_out, dS_in, nbh, d.heads, d.d_k, d.d_v, false, hs, st),
                    "msr_chunkwise_bwd(seqlen=0)");
  }
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV)
    return fail(MSR_ERR_NULL, "Q, K, V, dO, dQ, dK and dV must be non-NULL");
  const bool rope = rope_base > 0.f;
  const BwdWs w = bwd_ws_layout(dtype, d, chunk, rope);
  if (!workspace || ws_bytes < w.total)
    return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total, workspace ? ws_bytes : 0);
  void* cws = at<void>(workspace, w.chunk);
  if (rope && (s = rotate_qk(dtype, d, rope_base, pos0, Q, K, cws, w.cw, st, &Q, &K))) return s;
  const Elt e = dtype == MSR_BF16 ? kBF16 : kF32;
  const int64_t ld = (int64_t)d.heads * d.d_k;   // d_k == d_v: one token stride for every tensor
  const HeadTab tab = make_tab(gamma, d.heads, chunk, d.seqlen);
  float* sin_t = at<float>(workspace, w.sin_t);
  float* dso = at<float>(workspace, w.dso);
  hipError_t err = hipSuccess;
  // state seeds
  std::fill(hs.c, hs.c + kMaxHeads, 1.0f);
  const bool direct = chunk_out_direct(e, d.d_k, d.d_v, chunk);
  const bool saved = R_chunks && direct;          // the dQ pass reads the forward's states
  if (S_in && !saved) err = launch_state_xform(S_in, sin_t, nbh, d.heads, d.d_v, d.d_k, true, hs, st);
  if (dS_out && err == hipSuccess) {
    for (int h = 0; h < d.heads; ++h) hs.c[h] = (float)(1.0 / ((double)qk_scale * gamma[h]));
    err = launch_state_xform(dS_out, dso, nbh, d.heads, d.d_k, d.d_v, false, hs, st);
  }
  if (err != hipSuccess) return from_hip(err, "msr_chunkwise_bwd(state seeds)");
  // dS_in = s gamma_h * the dV pass's last state, scaled as the scan writes it
  float ds_scale[kMaxHeads];
  for (int h = 0; h < d.heads; ++h) ds_scale[h] = (float)((double)qk_scale * gamma[h]);
  // rev: the pass runs on the time-reversed sequence, reading its Q, K, V
  // rows backwards and writing its output rows back in forward order
  auto pass = [&](const void* q, const void* k, const void* v, void* o, const float* sin, float* sout, bool rev,
                  bool reuse = false, bool seeded = false, bool rx_kv = false, const void* rx = nullptr) {
    ChunkArgs a{};
    a.elt = e;
    a.d_k = d.d_k; a.d_v = d.d_v; a.batch = d.batch; a.seqlen = d.seqlen; a.heads = d.heads;
    a.chunk = chunk;
    a.Q = q; a.K = k; a.V = v; a.O = o;
    a.ldq = a.ldk = a.ldv = a.ldo = ld;
    a.scale = qk_scale;
    a.S_in = sin; a.S_out = sout;
    a.sout_scale = sout ? ds_scale : nullptr;
    a.dR = at<void>(cws, w.cw.dr);
    a.Rx = rx ? const_cast<void*>(rx) : at<void>(cws, w.cw.rx);   // a given rx is only read
    a.rev_out = rev;
    a.rev_in = rev;
    a.reuse_rx = reuse;
    a.reuse_seeded = seeded;
    a.rx_kv = rx_kv;
    return launch_chunkwise(a, tab, st);
  };
  // the 16-rows-per-wave output kernel (d_k = d_v = 256) reads each chunk's
  // state in the layout the scans write; the direct-copy kernel of the
  // other dims also reads it transposed
  const bool o16 = chunk_out_o16(e, d.d_k, d.d_v, chunk);
  const int NC = (d.seqlen + chunk - 1) / chunk;
  // dQ = causal retention of (dO, V, K) from S_in^T; its per-chunk states
  // are the forward's transposed (sums of V^T K against K^T V, seeded with
  // S_in^T against S_in)
  if (saved && o16) {
    err = launch_transpose_blocks_to(e, R_chunks, at<void>(cws, w.cw.rx), d.d_k, (int64_t)nbh * NC, st);
    if (err == hipSuccess) err = pass(dO, V, K, dQ, nullptr, nullptr, false, true, S_in != nullptr);
  } else if (saved) {
    err = pass(dO, V, K, dQ, nullptr, nullptr, false, true, S_in != nullptr, true, R_chunks);
  } else {
    err = pass(dO, V, K, dQ, S_in ? sin_t : nullptr, nullptr, false);
  }
  if (err != hipSuccess) return from_hip(err, "msr_chunkwise_bwd(dQ)");
  // dV = causal retention of (rev K, rev Q, rev dO), its rows written back in
  // forward time order; its last state gives dS_in
  err = pass(K, Q, dO, dV, dS_out ? dso : nullptr, dS_in, true);
  if (err != hipSuccess) return from_hip(err, "msr_chunkwise_bwd(dV)");
  // dK = causal retention of (rev V, rev dO, rev Q), rows in forward order.
  // Its state is the transpose of the dV pass's, chunk by chunk (the sum of
  // rev dO^T rev Q against rev Q^T rev dO, seeded with dS_out^T against
  // dS_out), so it reuses those per-chunk states: the direct-copy output
  // kernel of d_k <= 128 reads them as they are (with the transposing LDS
  // read), the others after an in-place transpose.
  const bool rx_kv = direct && !o16;
  if (!rx_kv) {
    err = launch_transpose_blocks(e, at<void>(cws, w.cw.rx), d.d_k, (int64_t)nbh * NC, st);
    if (err != hipSuccess) return from_hip(err, "msr_chunkwise_bwd(state transpose)");
  }
  err = pass(V, dO, Q, dK, nullptr, nullptr, true, true, dS_out != nullptr, rx_kv);
  if (err != hipSuccess) return from_hip(err, "msr_chunkwise_bwd(dK)");
  if (rope) {  // gradients with respect to the unrotated Q and K
    const float2* rtab = at<float2>(cws, w.cw.tab);
    const int rows = d.batch * d.seqlen;
    err = launch_rope_apply(e, dQ, ld, dQ, ld, rows, d.seqlen, d.heads, d.d_k, rtab, st, true);
    if (err == hipSuccess) err = launch_rope_apply(e, dK, ld, dK, ld, rows, d.seqlen, d.heads, d.d_k, rtab, st, true);
    if (err != hipSuccess) return from_hip(err, "msr_chunkwise_bwd(rotation)");
  }
  return ok();
}

msr_status msr_chunkwise_bwd(msr_dtype dtype, msr_dims d, int32_t chunk, const double* gamma, float rope_base,
                             int64_t pos0, float qk_scale, const void* Q, const void* K, const void* V,
                             const void* dO, const float* S_in, const float* dS_out, void* dQ, void* dK, void* dV,
                             float* dS_in, void* workspace, size_t ws_bytes, void* stream) {
  return chunkwise_bwd(dtype, d, chunk, gamma, rope_base, pos0, qk_scale, Q, K, V, dO, S_in, dS_out, nullptr, dQ,
                       dK, dV, dS_in, workspace, ws_bytes, stream);
}

msr_status msr_chunkwise_bwd_saved(msr_dtype dtype, msr_dims d, int32_t chunk, const double* gamma, float rope_base,
                                   int64_t pos0, float qk_scale, const void* Q, const void* K, const void* V,
                                   const void* dO, const float* S_in, const float* dS_out, const void* R_chunks,
                                   void* dQ, void* dK, void* dV, float* dS_in, void* workspace, size_t ws_bytes,
                                   void* stream) {
  if (!R_chunks && d.batch > 0 && d.seqlen > 0) return fail(MSR_ERR_NULL, "R_chunks must be non-NULL");
  return chunkwise_bwd(dtype, d, chunk, gamma, rope_base, pos0, qk_scale, Q, K, V, dO, S_in, dS_out, R_chunks, dQ,
                       dK, dV, dS_in, workspace, ws_bytes, stream);
}

size_t msr_rglru_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t width) {
  if (check_dtype(dtype) || batch < 0 || seqlen < 0 || width <= 0) return 0;
  return align_up((size_t)batch * seqlen * 2 * width * elt_size(dtype));
}

msr_status msr_rglru_fwd(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t width, float c, const void* X,
                         const void* W_a, const float* b_a, const void* W_x, const float* b_x, const float* Lambda,
                         const float* h0, float* h_last, void* Y, void* workspace, size_t ws_bytes, void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if (batch < 0 || seqlen < 0 || width <= 0)
    return fail(MSR_ERR_SHAPE, "invalid sizes batch=%d seqlen=%d width=%d", batch, seqlen, width);
  if (width % 64) return fail(MSR_ERR_UNSUPPORTED, "width = %d is not a multiple of 64", width);
  if (!(c > 0.f) || !std::isfinite(c)) return fail(MSR_ERR_SHAPE, "c = %g must be positive and finite", (double)c);
  const int64_t M = (int64_t)batch * seqlen;
  if (M > (int64_t)INT32_MAX) return fail(MSR_ERR_UNSUPPORTED, "batch*seqlen exceeds 2^31-1");
  if ((int64_t)2 * width * 4096 > (int64_t)INT32_MAX) return fail(MSR_ERR_UNSUPPORTED, "width too large");
  if (h_last && h_last == h0) return fail(MSR_ERR_SHAPE, "h_last may not alias h0");
  if (batch == 0) return ok();
  if (!Lambda) return fail(MSR_ERR_NULL, "Lambda must be non-NULL");
  hipStream_t st = (hipStream_t)stream;
  const Elt e = dtype == MSR_BF16 ? kBF16 : kF32;
  if (M > 0) {
    if (!X || !W_a || !b_a || !W_x || !b_x || !Y)
      return fail(MSR_ERR_NULL, "X, W_a, b_a, W_x, b_x and Y must be non-NULL");
    const size_t need = msr_rglru_workspace_bytes(dtype, batch, seqlen, width);
    if (!workspace || ws_bytes < need)
      return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? ws_bytes : 0);
    // [r | i] = sigmoid(X [W_a | W_x] + [b_a | b_x])
    GemmB bg{};
    bg.ptr[0] = W_a; bg.ptr[1] = W_x;
    bg.ld[0] = bg.ld[1] = width;
    bg.start[0] = 0; bg.start[1] = width; bg.start[2] = bg.start[3] = INT32_MAX;
    bg.bias[0] = b_a; bg.bias[1] = b_x;
    bg.act = 2;
    hipError_t err = launch_gemm(e, X, width, bg, workspace, 2 * width, (int)M, 2 * width, width, st);
    if (err != hipSuccess) return from_hip(err, "msr_rglru_fwd(gates)");
  }
  // seqlen == 0 runs the scan too: it copies h0 (or zeros) to h_last
  return from_hip(launch_rglru_scan(e, X, width, workspace, 2 * width, Lambda, c, h0, h_last, Y, width, batch, seqlen,
                                    width, st),
                  "msr_rglru_fwd(scan)");
}

msr_status msr_recurrent_step(msr_dtype dtype, int32_t batch, int32_t heads, int32_t d_k, int32_t d_v,
                              const double* gamma, float rope_base, int64_t pos, float qk_scale, const void* q,
                              const void* k, const void* v, float* S, void* o, void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(batch, 1, heads, d_k, d_v))) return s;
  if ((s = check_gamma(gamma, heads))) return s;
  if (pos < 0) return fail(MSR_ERR_SHAPE, "pos = %lld is negative", (long long)pos);
  if (batch == 0) return ok();
  if (!q || !k || !v || !S || !o) return fail(MSR_ERR_NULL, "q, k, v, S and o must be non-NULL");
  if ((int64_t)batch * heads > (int64_t)INT32_MAX) return fail(MSR_ERR_UNSUPPORTED, "batch*heads too large");
  const HeadTab tab = make_tab(gamma, heads, 1, 1);
  const StepIO io{q, (int64_t)heads * d_k, k, (int64_t)heads * d_k, v, (int64_t)heads * d_v,
                  o, (int64_t)heads * d_v, false};
  return from_hip(launch_recurrent_step(dtype == MSR_BF16 ? kBF16 : kF32, d_k, d_v, batch, heads, io, S, qk_scale,
                                        pos, rope_base, tab, (hipStream_t)stream),
                  "msr_recurrent_step");
}

// ---------------------------------------------------------------------------
// Layer decode step: Eq. (8) with the recurrent form for one token per
// sequence.  Workspace: [Q | K | V | G] rows, float32 retention outputs, Z.
// ---------------------------------------------------------------------------

size_t msr_layer_decode_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t d_model, int32_t heads, int32_t d_k,
                                        int32_t d_v) {
  (void)d_model;
  if (check_dtype(dtype) || check_heads(batch, 1, heads, d_k, d_v) || batch == 0) return 0;
  if (d_model <= 0 || d_model % 64) return 0;
  return decode_ws_layout(dtype, batch, d_model, heads, d_k, d_v).total;
}

// Validation shared by the two layer decode step entry points.
static msr_status decode_check(msr_dtype dtype, int32_t batch, int32_t d_model, int32_t heads, int32_t d_k,
                               int32_t d_v, const double* gamma, float gn_eps, int64_t pos) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(batch, 1, heads, d_k, d_v))) return s;
  if ((s = check_gamma(gamma, heads))) return s;
  if (d_model <= 0) return fail(MSR_ERR_SHAPE, "d_model = %d must be positive", d_model);
  if (d_model % 64) return fail(MSR_ERR_UNSUPPORTED, "d_model = %d is not a multiple of 64", d_model);
  if (!(gn_eps >= 0.f)) return fail(MSR_ERR_SHAPE, "gn_eps must be >= 0");
  if (pos < 0) return fail(MSR_ERR_SHAPE, "pos = %lld is negative", (long long)pos);
  if ((int64_t)batch * heads > (int64_t)INT32_MAX) return fail(MSR_ERR_UNSUPPORTED, "batch*heads too large");
  return MSR_OK;
}

// The layer decode step's launches on validated arguments and a workspace
// of the layout decode_ws_layout gives.
static msr_status decode_launch(msr_dtype dtype, int32_t batch, int32_t d_model, int32_t heads, int32_t d_k,
                                int32_t d_v, const double* gamma, float rope_base, float gn_eps, int64_t pos,
                                const void* X, const void* W_Q, const void* W_K, const void* W_V, const void* W_G,
                                const void* W_O, float* S, void* out, const DecodeWs& w, void* workspace,
                                void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const Elt e = dtype == MSR_BF16 ? kBF16 : kF32;
  const size_t es = elt_size(dtype);
  const int hk = heads * d_k, hv = heads * d_v;
  const int ntot = 2 * hk + 2 * hv;
  char* qkvg = at<char>(workspace, w.qkvg);
  float* o = at<float>(workspace, w.o);
  char* z = at<char>(workspace, w.z);
  // 1. [q | k | v | g] = x [W_Q | W_K | W_V | W_G]
  GemmB bq{};
  bq.ptr[0] = W_Q; bq.ptr[1] = W_K; bq.ptr[2] = W_V; bq.ptr[3] = W_G;
  bq.ld[0] = hk; bq.ld[1] = hk; bq.ld[2] = hv; bq.ld[3] = hv;
  bq.start[0] = 0; bq.start[1] = hk; bq.start[2] = 2 * hk; bq.start[3] = 2 * hk + hv;
  bq.rope_segs = 0;
  float* part = at<float>(workspace, w.part);
  hipError_t err = w.split_qkvg > 1
                       ? launch_gemm_splitk(e, X, d_model, bq, qkvg, ntot, batch, ntot, d_model, w.split_qkvg, part, st)
                       : launch_gemm(e, X, d_model, bq, qkvg, ntot, batch, ntot, d_model, st);
  if (err != hipSuccess) return from_hip(err, "msr_layer_decode_step(projections)");
  // 2. q, k rotated at pos; S <- gamma S + k^T v; o = q S / sqrt(d_k) (float32)
  const HeadTab tab = make_tab(gamma, heads, 1, 1);
  const StepIO io{qkvg, ntot, qkvg + (size_t)hk * es, ntot, qkvg + (size_t)2 * hk * es, ntot, o, hv, true};
  err = launch_recurrent_step(e, d_k, d_v, batch, heads, io, S, 1.0f / std::sqrt((float)d_k), pos, rope_base, tab,
                              st);
  if (err != hipSuccess) return from_hip(err, "msr_layer_decode_step(recurrent step)");
  // 3. z = swish(g) (.) GroupNorm_h(o)
  err = launch_gn_gate(e, d_v, batch, heads, o, hv, qkvg + (size_t)(2 * hk + hv) * es, ntot, z, hv, gn_eps, st);
  if (err != hipSuccess) return from_hip(err, "msr_layer_decode_step(group norm, gate)");
  // 4. out = z W_O
  GemmB bo{};
  bo.ptr[0] = W_O; bo.ld[0] = d_model;
  bo.start[0] = 0; bo.start[1] = bo.start[2] = bo.start[3] = INT32_MAX;
  err = w.split_o > 1 ? launch_gemm_splitk(e, z, hv, bo, out, d_model, batch, d_model, hv, w.split_o, part, st)
                      : launch_gemm(e, z, hv, bo, out, d_model, batch, d_model, hv, st);
  return from_hip(err, "msr_layer_decode_step(output projection)");
}

msr_status msr_layer_decode_step(msr_dtype dtype, int32_t batch, int32_t d_model, int32_t heads, int32_t d_k,
                                 int32_t d_v, const double* gamma, float rope_base, float gn_eps, int64_t pos,
                                 const void* X, const void* W_Q, const void* W_K, const void* W_V, const void* W_G,
                                 const void* W_O, float* S, void* out, void* workspace, size_t ws_bytes,
                                 void* stream) {
  msr_status s;
  if ((s = decode_check(dtype, batch, d_model, heads, d_k, d_v, gamma, gn_eps, pos))) return s;
  if (batch == 0) return ok();
  if (!X || !W_Q || !W_K || !W_V || !W_G || !W_O || !S || !out)
    return fail(MSR_ERR_NULL, "X, W_Q, W_K, W_V, W_G, W_O, S and out must be non-NULL");
  const DecodeWs w = decode_ws_layout(dtype, batch, d_model, heads, d_k, d_v);
  if (!workspace || ws_bytes < w.total)
    return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total, workspace ? ws_bytes : 0);
  return decode_launch(dtype, batch, d_model, heads, d_k, d_v, gamma, rope_base, gn_eps, pos, X, W_Q, W_K, W_V, W_G,
                       W_O, S, out, w, workspace, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free layer decode step: the same launches on a workspace in a
// file-scope device array.  Each GPU holds its own copy of `scratch` from the
// moment the library's code object is loaded on it until the process ends;
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept.  In host code the array's name is only a
// stand-in, never a device address: only that looked-up pointer is passed to
// kernels.  Every call on a GPU reuses that GPU's array (nothing in it has to
// start at zero: each call writes every element it later reads), so calls
// that overlap on one GPU race.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

msr_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "msr_layer_decode_step_noalloc(current device)");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MSR_ERR_UNSUPPORTED, "device %d is beyond the %d the static scratch is kept for", dev, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return from_hip(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                               "msr_layer_decode_step_noalloc(scratch address)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSR_OK;
}
}  // namespace

extern "C" {

size_t msr_layer_decode_noalloc_max_bytes(void) { return kScratchBytes; }

msr_status msr_layer_decode_step_noalloc(msr_dtype dtype, int32_t batch, int32_t d_model, int32_t heads,
                                         int32_t d_k, int32_t d_v, const double* gamma, float rope_base,
                                         float gn_eps, int64_t pos, const void* X, const void* W_Q, const void* W_K,
                                         const void* W_V, const void* W_G, const void* W_O, float* S, void* out,
                                         void* stream) {
  msr_status s;
  if ((s = decode_check(dtype, batch, d_model, heads, d_k, d_v, gamma, gn_eps, pos))) return s;
  if (batch == 0) return ok();
  if (!X || !W_Q || !W_K || !W_V || !W_G || !W_O || !S || !out)
    return fail(MSR_ERR_NULL, "X, W_Q, W_K, W_V, W_G, W_O, S and out must be non-NULL");
  const DecodeWs w = decode_ws_layout(dtype, batch, d_model, heads, d_k, d_v);
  if (w.total > kScratchBytes)
    return fail(MSR_ERR_WORKSPACE, "this step needs %zu bytes of scratch; the static scratch holds %zu "
                "(msr_layer_decode_step takes a caller workspace of any size)", w.total, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws))) return s;
  return decode_launch(dtype, batch, d_model, heads, d_k, d_v, gamma, rope_base, gn_eps, pos, X, W_Q, W_K, W_V, W_G,
                       W_O, S, out, w, ws, stream);
}

size_t msr_layer_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t d_model, int32_t heads,
                                 int32_t d_k, int32_t d_v, int32_t chunk) {
  if (batch < 0 || seqlen < 0 || d_model <= 0 || heads <= 0 || d_k <= 0 || d_v <= 0 || chunk <= 0) return 0;
  return layer_ws_layout(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk).total;
}

msr_status msr_layer_fwd(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t d_model, int32_t heads, int32_t d_k,
                         int32_t d_v, int32_t chunk, const double* gamma, float rope_base, float gn_eps,
                         const void* X, const void* W_Q, const void* W_K, const void* W_V, const void* W_G,
                         const void* W_O, void* out, void* workspace, size_t ws_bytes, void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(batch, seqlen, heads, d_k, d_v))) return s;
  if ((s = check_matrix_dims(dtype, d_v))) return s;
  if ((s = check_chunk(chunk))) return s;
  if ((s = check_gamma(gamma, heads))) return s;
  if (d_model <= 0) return fail(MSR_ERR_SHAPE, "d_model = %d must be positive", d_model);
  if (d_model % 64) return fail(MSR_ERR_UNSUPPORTED, "d_model = %d is not a multiple of 64", d_model);
  if (!(gn_eps >= 0.f)) return fail(MSR_ERR_SHAPE, "gn_eps must be >= 0");
  const int64_t M = (int64_t)batch * seqlen;
  if (M == 0) return ok();
  if (!X || !W_Q || !W_K || !W_V || !W_G || !W_O || !out)
    return fail(MSR_ERR_NULL, "X, W_Q, W_K, W_V, W_G, W_O and out must be non-NULL");
  const LayerWs w = layer_ws_layout(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk);
  if (!workspace || ws_bytes < w.total)
    return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total, workspace ? ws_bytes : 0);
  return layer_launch(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk, gamma, rope_base, gn_eps, X, W_Q, W_K,
                      W_V, W_G, W_O, out, nullptr, w, workspace, stream);
}

size_t msr_retnet_block_workspace_bytes(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t d_model,
                                        int32_t heads, int32_t d_k, int32_t d_v, int32_t chunk, int32_t d_ffn) {
  if (check_dtype(dtype) || check_heads(batch, seqlen, heads, d_k, d_v) || check_chunk(chunk)) return 0;
  if ((int64_t)batch * seqlen == 0 || d_model <= 0 || d_ffn <= 0) return 0;
  return block_ws_layout(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk, d_ffn).total;
}

msr_status msr_retnet_block_fwd(msr_dtype dtype, int32_t batch, int32_t seqlen, int32_t d_model, int32_t heads,
                                int32_t d_k, int32_t d_v, int32_t chunk, int32_t d_ffn, const double* gamma,
                                float rope_base, float gn_eps, float ln_eps, const void* X, const void* W_Q,
                                const void* W_K, const void* W_V, const void* W_G, const void* W_O,
                                const void* W_1, const void* W_2, void* out, void* workspace, size_t ws_bytes,
                                void* stream) {
  msr_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_heads(batch, seqlen, heads, d_k, d_v))) return s;
  if ((s = check_matrix_dims(dtype, d_v))) return s;
  if ((s = check_chunk(chunk))) return s;
  if ((s = check_gamma(gamma, heads))) return s;
  if (d_model <= 0 || d_ffn <= 0) return fail(MSR_ERR_SHAPE, "d_model = %d and d_ffn = %d must be positive", d_model, d_ffn);
  if (d_model % 64 || d_ffn % 64)
    return fail(MSR_ERR_UNSUPPORTED, "d_model = %d and d_ffn = %d must be multiples of 64", d_model, d_ffn);
  if (d_model > 8192) return fail(MSR_ERR_UNSUPPORTED, "d_model = %d is above 8192", d_model);
  if (!(gn_eps >= 0.f) || !(ln_eps >= 0.f)) return fail(MSR_ERR_SHAPE, "gn_eps and ln_eps must be >= 0");
  const int64_t M = (int64_t)batch * seqlen;
  if (M == 0) return ok();
  if (!X || !W_Q || !W_K || !W_V || !W_G || !W_O || !W_1 || !W_2 || !out)
    return fail(MSR_ERR_NULL, "X, the seven weights and out must be non-NULL");
  if (M * (int64_t)d_ffn > (int64_t)INT32_MAX * 8) return fail(MSR_ERR_UNSUPPORTED, "batch*seqlen*d_ffn too large");
  const BlockWs w = block_ws_layout(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk, d_ffn);
  if (!workspace || ws_bytes < w.total)
    return fail(MSR_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total, workspace ? ws_bytes : 0);
  hipStream_t st = (hipStream_t)stream;
  const Elt e = dtype == MSR_BF16 ? kBF16 : kF32;
  void* H = at<void>(workspace, w.h);
  void* Y = at<void>(workspace, w.y);
  void* F = at<void>(workspace, w.f);
  // Y = MSR(LN(X)) + X
  hipError_t err = launch_layer_norm(e, X, d_model, H, d_model, (int)M, d_model, ln_eps, st);
  if (err != hipSuccess) return from_hip(err, "msr_retnet_block_fwd(layer norm)");
  s = layer_launch(dtype, batch, seqlen, d_model, heads, d_k, d_v, chunk, gamma, rope_base, gn_eps, H, W_Q, W_K, W_V,
                   W_G, W_O, Y, X, w.lw, at<void>(workspace, w.layer), stream);
  if (s != MSR_OK) return s;
  // out = gelu(LN(Y) W_1) W_2 + Y
  err = launch_layer_norm(e, Y, d_model, H, d_model, (int)M, d_model, ln_eps, st);
  if (err != hipSuccess) return from_hip(err, "msr_retnet_block_fwd(layer norm)");
  GemmB b1{};
  b1.ptr[0] = W_1; b1.ld[0] = d_ffn;
  b1.start[0] = 0; b1.start[1] = b1.start[2] = b1.start[3] = INT32_MAX;
  b1.act = 1;
  err = launch_gemm(e, H, d_model, b1, F, d_ffn, (int)M, d_ffn, d_model, st);
  if (err != hipSuccess) return from_hip(err, "msr_retnet_block_fwd(W_1)");
  GemmB b2{};
  b2.ptr[0] = W_2; b2.ld[0] = d_model;
  b2.start[0] = 0; b2.start[1] = b2.start[2] = b2.start[3] = INT32_MAX;
  b2.resid = Y; b2.ldr = d_model;
  err = launch_gemm(e, F, d_ffn, b2, out, d_model, (int)M, d_model, d_ffn, st);
  return from_hip(err, "msr_retnet_block_fwd(W_2)");
}

}  // extern "C"
