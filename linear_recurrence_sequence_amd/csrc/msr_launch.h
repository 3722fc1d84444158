// Host-side launchers of the libmsr kernels (internal; the public ABI is
// include/msr.h).  Every launcher only enqueues on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msr_device.h"

namespace msr {

enum Elt { kF32 = 0, kBF16 = 1 };

// Brackets one kernel launch with HIP events on its stream while tracing is
// enabled (msr_trace_enable); a no-op otherwise.
class TraceScope {
 public:
  TraceScope(const char* name, hipStream_t stream);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_{}, stop_{};
  bool active_ = false;
};

struct ChunkArgs {
  Elt elt;
  int d_k, d_v;
  int batch, seqlen, heads;
  int chunk;                 // tokens per chunk (multiple of 32)
  const void* Q; int64_t ldq;   // token stride in elements
  const void* K; int64_t ldk;
  const void* V; int64_t ldv;
  void* O; int64_t ldo;
  const void* G; int64_t ldg;   // gate (only with fused GroupNorm + gate)
  float scale, eps;
  bool fuse_gn_gate;
  const float* S_in; float* S_out;
  const float* sout_scale;   // host array [heads]: S_out = sout_scale[h] * final state (null: factor 1)
  void* dR;                  // [B, H, NC, d_v, d_k] elt: each chunk's own state contribution
  void* Rx;                  // [B, H, NC, d_v, d_k] elt: R_{i-1} per chunk (aliases dR)
  bool rev_out;              // write output row t of each sequence to row seqlen-1-t
  bool rev_in;               // read Q, K, V row t of each sequence from row seqlen-1-t
  // Rx already holds every chunk's R_{i-1} (state and scan kernels skipped);
  // reuse_seeded: chunk 0's R_{-1} is a seed (else zero)
  bool reuse_rx, reuse_seeded;
  // with reuse_rx, on the direct-copy path only (chunk_out_direct): Rx
  // holds each chunk's R_{i-1} itself, [d_k rows][d_v cols], instead of its
  // transpose
  bool rx_kv;
  // (cos, sin) table [seqlen][d_k / 2] of the positions of the sequence's
  // rows: the output kernel rotates Q with it as it loads Q (only where
  // chunk_out_o16 holds; K must then already be rotated); null: Q as given
  const float2* q_rope_tab;
  // (cos, sin) table of the rows' positions for K (forward passes only):
  // the state kernel rotates the K rows it stages with it and writes them
  // to k_rot (row stride ld_k_rot), which the output kernel then reads in
  // place of K; null: K as given
  const float2* k_rope_tab;
  void* k_rot; int64_t ld_k_rot;
};

// Whether the forward output kernel for these dims and chunk rotates Q
// itself from ChunkArgs::q_rope_tab (all but the bf16 direct-copy kernel
// of d_v <= 256).
bool chunk_out_rotates_q(Elt elt, int d_k, int d_v, int chunk);

// Whether the chunkwise form of these dims and chunk runs the bf16
// direct-copy output kernel (the one that can read Rx as R_{i-1} itself).
bool chunk_out_direct(Elt elt, int d_k, int d_v, int chunk);

// Whether the forward output kernel with 16 query rows per wave runs these
// dims and chunk (bf16, d_k 256, d_v 256 or 512, chunk a multiple of 128).
bool chunk_out_o16(Elt elt, int d_k, int d_v, int chunk);
// That kernel: the chunkwise form's outputs (state: Rx holds R_{i-1}^T per
// chunk) or the parallel form's (one chunk of chunk = TPC * 128 rows); with
// rev_in (and rev_out) set, those of the time-reversed sequence (no fused
// GroupNorm or rotation).
hipError_t launch_out_o16(const ChunkArgs& a, bool state, int chunk, int NC, int TPC, int has_sin,
                          const HeadTab& tab, hipStream_t stream);

// Chunkwise retention: state contributions, fp32 scan, outputs.
hipError_t launch_chunkwise(const ChunkArgs& a, const HeadTab& tab, hipStream_t stream);
// Parallel form: one "chunk" spanning the whole sequence, no state.
hipError_t launch_parallel(const ChunkArgs& a, const HeadTab& tab, hipStream_t stream);

// One decode step: S <- gamma S + k^T v; o = scale q S (q, k rotated at pos).
// Operands of a decode step: one row per batch element (head h at column
// h * d of the row), row strides in elements; o is float32 when o_f32.
struct StepIO {
  const void* q; int64_t ldq;
  const void* k; int64_t ldk;
  const void* v; int64_t ldv;
  void* o; int64_t ldo;
  bool o_f32;
};
hipError_t launch_recurrent_step(Elt elt, int d_k, int d_v, int batch, int heads, const StepIO& io, float* S,
                                 float scale, int64_t pos, float base, const HeadTab& tab, hipStream_t stream);
// z = swish(g) (.) GroupNorm_h(o) per (batch element, head) over d_v; o float32.
hipError_t launch_gn_gate(Elt elt, int d_v, int batch, int heads, const float* o, int64_t ldo, const void* g,
                          int64_t ldg, void* z, int64_t ldz, float eps, hipStream_t stream);

// RG-LRU scan over gates already formed: G = [r | i], [batch*seqlen, 2*width]
// (row stride ldg), X and Y [batch*seqlen, width] (row strides ldx, ldy),
// lam [width] float32, h0 / hT [batch, width] float32 (nullable).  width a
// multiple of 64.
hipError_t launch_rglru_scan(Elt elt, const void* X, int64_t ldx, const void* G, int64_t ldg, const float* lam,
                             float c, const float* h0, float* hT, void* Y, int64_t ldy, int batch, int seqlen,
                             int width, hipStream_t stream);

// In-place transpose of nblocks contiguous d x d blocks of elt (d a multiple
// of 64 for bf16, of 32 for float32).
hipError_t launch_transpose_blocks(Elt elt, void* base, int d, int64_t nblocks, hipStream_t stream);
// The same from src to dst (disjoint, or equal for the in-place transpose).
hipError_t launch_transpose_blocks_to(Elt elt, const void* src, void* dst, int d, int64_t nblocks, hipStream_t stream);
// Per-head factors of launch_state_xform.
struct HeadScale {
  float c[kMaxHeads];
};
// Every chunk's R_{i-1} (Rx, [B, H, NC, d_v, d_k]) and the final state in
// one kernel that walks the chunks of each state tile in order (bf16,
// (d_k, d_v) in {(128, 128), (256, 256), (256, 512)}, chunk a multiple of
// 64, enough (batch, head) pairs bh; K as given; rev_in: the time-reversed
// sequence).
bool chunk_rscan_ok(Elt elt, int dk, int dv, int chunk, int bh);
hipError_t launch_chunk_rscan(const ChunkArgs& a, const HeadTab& tab, const HeadScale& so, hipStream_t st);
// dst[bh] (rows x cols float32) = c[bh % heads] * (transpose ? src[bh]^T :
// src[bh]) for bh < nbh; src == nullptr writes zeros; dst may equal src
// only without transpose.  rows and cols multiples of 32.
hipError_t launch_state_xform(const float* src, float* dst, int nbh, int heads, int rows, int cols, bool transpose,
                              const HeadScale& hs, hipStream_t stream);

// cos/sin table: tab[n * (d/2) + j] = (cos, sin)((pos0 + n) * theta_j),
// theta_j = base^(-2j/d), n = 0..npos-1.
hipError_t launch_rope_table(float2* tab, int npos, int d, int64_t pos0, float base,
                             hipStream_t stream);
// Rotate the first d columns of every head of a [rows, heads * d] block
// (rows = batch * seqlen tokens, token n = row % seqlen) from src to dst
// (dst may equal src).  Strides in elements.
// inverse: rotate by the negative angle (the adjoint, for gradients).
hipError_t launch_rope_apply(Elt elt, const void* src, int64_t lds, void* dst, int64_t ldd,
                             int rows, int seqlen, int heads, int d, const float2* tab,
                             hipStream_t stream, bool inverse = false);

// B operand of launch_gemm: up to four column segments, segment s covering
// output columns [start[s], start[s+1]) (start[0] = 0, unused entries set to
// INT_MAX), each a row-major [K, width] block at ptr[s] with row stride
// ld[s] (elements; multiples of 8).  The first rope_segs segments get the
// rotation epilogue with head dim rope_d and table rope_tab ([seqlen][rope_d/2]
// (cos, sin)); output row m is token m % seqlen.
struct GemmB {
  const void* ptr[4];
  int64_t ld[4];
  int start[4];
  int rope_segs, rope_d, seqlen;
  const float2* rope_tab;
  // split-K: when set, workgroup z of the launch's z dimension sums K rows
  // [z K_s, (z + 1) K_s) and stores float32 partials to part + z M N (no
  // rotation); launch_gemm_splitk adds them up.
  float* part;
  // epilogue: C = act(A B + bias) + resid, act = gelu when act == 1 and
  // sigmoid when act == 2 (after any rotation), bias[s] a float32 vector
  // over segment s's columns (nullable), resid an [M, N] matrix with row
  // stride ldr (nullable).  Not with split-K.
  const float* bias[4];
  int act;
  const void* resid;
  int64_t ldr;
};

// C[M, N] = A[M, K] * B[K, N] (row-major A and B segments), fp32
// accumulation, C (row stride ldc) in elt.  K must be a multiple of 64.
hipError_t launch_gemm(Elt elt, const void* A, int64_t lda, const GemmB& b, void* C, int64_t ldc, int M, int N,
                       int K, hipStream_t stream);
// The same product for few rows (M <= 256): the K range split over
// `splits` workgroups per output tile (K a multiple of 64 * splits), float32
// partials in `part` ([splits, M, N]), then summed and rounded once into C.
hipError_t launch_gemm_splitk(Elt elt, const void* A, int64_t lda, const GemmB& b, void* C, int64_t ldc, int M,
                              int N, int K, int splits, float* part, hipStream_t stream);
// How many K splits launch_gemm_splitk should use for an M x N x K product.
int gemm_splits(Elt elt, int M, int N, int K);
// Row-wise LayerNorm over d columns (biased variance, identity affine):
// Y = (X - mean) / sqrt(var + eps); d a multiple of 8, at most 8192.
hipError_t launch_layer_norm(Elt elt, const void* X, int64_t ldx, void* Y, int64_t ldy, int rows, int d, float eps,
                             hipStream_t stream);

}  // namespace msr
