// RG-LRU scan for gfx950: the gated diagonal linear recurrence of the page
// "Griffin ：將門控線性循環與局部注意力混合以實現高效的語言模型", section
// "實門線性循環單元 (RG-LRU)":
//
//   a_t = a^(c r_t), a = sigma(Lambda)   (per channel; formed in log space)
//   h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i_t x_t),   y_t = h_t
//
// with the gates r_t, i_t already computed (sigmoid epilogue of the gate
// projection GEMM).  The recurrence is elementwise and HBM-bound: every
// input is read once and every output written once.
//
// One workgroup of NW waves per (batch element, 64 channels); lane = channel,
// so each load or store of a time step is one coalesced row segment.  Time
// runs in tiles of NW * S steps: wave w takes steps [w S, (w + 1) S) of the
// tile, forms a_t and b_t = sqrt(1 - a_t^2) i_t x_t for them, and folds them
// into the affine map h -> A h + B of its segment.  The NW maps are combined
// through LDS with the carry from the previous tile (a float32 scan over
// segments), each wave replays its steps from its own start state and writes
// y, and the carry moves on.  The next tile's inputs are loaded before the
// current tile is processed.
#include "msr_launch.h"

namespace msr {

namespace {

__device__ __forceinline__ void st_f(bf16* p, float v) { *p = (bf16)v; }
__device__ __forceinline__ void st_f(float* p, float v) { *p = v; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 1 - 2^(2 l2) for l2 <= 0, i.e. -expm1(z) with z = 2 l2 ln 2, without the
// cancellation of 1 - a^2 as a -> 1: the Taylor series of -expm1 through z^6
// for |z| < 1/4 (truncation below 1e-7 relative), else 1 - a^2 directly
// (there a^2 <= e^(-1/4), so no digits cancel).
__device__ __forceinline__ float one_minus_a2(float l2, float a) {
  const float z = l2 * (2.f * kLn2);
  float p = fmaf(z, 1.f / 720.f, 1.f / 120.f);
  p = fmaf(z, p, 1.f / 24.f);
  p = fmaf(z, p, 1.f / 6.f);
  p = fmaf(z, p, 0.5f);
  p = fmaf(z, p, 1.f);
  return z > -0.25f ? -z * p : fmaf(-a, a, 1.f);
}

}  // namespace

template <class T, int NW, int S>
__global__ __launch_bounds__(64 * NW) void k_rglru_scan(const T* __restrict__ X, int64_t ldx, const T* __restrict__ G,
                                                        int64_t ldg, const float* __restrict__ lam, float c,
                                                        const float* __restrict__ h0, float* __restrict__ hT,
                                                        T* __restrict__ Y, int64_t ldy, int seqlen, int width) {
  __shared__ float segA[2][NW][64], segB[2][NW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = width / 64;
  const int b = blockIdx.x / nblk;
  const int c0 = (blockIdx.x % nblk) * 64;
  const int ch = c0 + lane;
  // log2 a^c = c log2 sigma(Lambda), log sigma(z) = -(max(-z, 0) + log1p(e^-|z|))
  const float L = lam[ch];
  const float l2ac = -c * (fmaxf(-L, 0.f) + log1pf(expf(-fabsf(L)))) * kLog2e;
  float carry = h0 ? h0[(size_t)b * width + ch] : 0.f;
  // wave-uniform row bases: the per-step row offset is scalar arithmetic and
  // each access adds only the lane's channel
  const size_t row0 = (size_t)b * seqlen;
  const T* xb = X + row0 * ldx + c0;
  const T* rb = G + row0 * ldg + c0;
  const T* ib = rb + width;
  T* yb = Y + row0 * ldy + c0;

  // raw inputs of the current and the next tile, converted where used so
  // that no load has to complete before the next one is issued; rows past
  // the end re-read the last row (its steps are masked to the identity)
  using R = RawElt<T>;
  typename R::type cx[S], cr[S], ci[S], nx[S], nr[S], ni[S];
  auto load = [&](int t0, typename R::type* vx, typename R::type* vr, typename R::type* vi) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = min(t0 + wave * S + s, seqlen - 1);   // uniform
      vx[s] = R::load(xb + (int64_t)t * ldx + lane);
      vr[s] = R::load(rb + (int64_t)t * ldg + lane);
      vi[s] = R::load(ib + (int64_t)t * ldg + lane);
    }
  };
  if (seqlen > 0) load(0, cx, cr, ci);
  int it = 0;
  for (int t0 = 0; t0 < seqlen; t0 += NW * S, ++it) {
    const bool more = t0 + NW * S < seqlen;
    if (more) load(t0 + NW * S, nx, nr, ni);
    float a[S], bb[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bool ok = t0 + wave * S + s < seqlen;
      const float l2 = R::value(cr[s]) * l2ac;        // log2 a_t
      const float at = __builtin_amdgcn_exp2f(l2);
      const float gain = __builtin_amdgcn_sqrtf(one_minus_a2(l2, at));
      a[s] = ok ? at : 1.f;                           // steps past the end are the identity
      bb[s] = ok ? gain * (R::value(ci[s]) * R::value(cx[s])) : 0.f;
    }
    float A = 1.f, B = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      A *= a[s];
      B = fmaf(a[s], B, bb[s]);
    }
    const int p = it & 1;
    segA[p][wave][lane] = A;
    segB[p][wave][lane] = B;
    __syncthreads();
    float h = carry, next = carry;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float Aw = segA[p][w][lane], Bw = segB[p][w][lane];
      if (w < wave) h = fmaf(Aw, h, Bw);
      next = fmaf(Aw, next, Bw);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = t0 + wave * S + s;
      h = fmaf(a[s], h, bb[s]);
      if (t < seqlen) st_f(yb + (int64_t)t * ldy + lane, h);
    }
    carry = next;
    if (more) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        cx[s] = nx[s];
        cr[s] = nr[s];
        ci[s] = ni[s];
      }
    }
  }
  if (hT && wave == 0) hT[(size_t)b * width + ch] = carry;
}

hipError_t launch_rglru_scan(Elt elt, const void* X, int64_t ldx, const void* G, int64_t ldg, const float* lam,
                             float c, const float* h0, float* hT, void* Y, int64_t ldy, int batch, int seqlen,
                             int width, hipStream_t st) {
  if (width % 64) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)batch * (width / 64);
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  constexpr int NW = 16, S = 8;   // 16 waves x 8 steps: the fastest of a sweep at batch 8 x 2048 x 2048
  TraceScope ts("k_rglru_scan", st);
  if (elt == kBF16)
    hipLaunchKernelGGL((k_rglru_scan<bf16, NW, S>), dim3((unsigned)blocks), dim3(64 * NW), 0, st, (const bf16*)X,
                       ldx, (const bf16*)G, ldg, lam, c, h0, hT, (bf16*)Y, ldy, seqlen, width);
  else
    hipLaunchKernelGGL((k_rglru_scan<float, NW, S>), dim3((unsigned)blocks), dim3(64 * NW), 0, st, (const float*)X,
                       ldx, (const float*)G, ldg, lam, c, h0, hT, (float*)Y, ldy, seqlen, width);
  return hipGetLastError();
}

}  // namespace msr
