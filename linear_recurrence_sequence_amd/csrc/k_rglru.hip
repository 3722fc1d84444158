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

__device__ __forceinline__ float ld_f(const bf16* p) { return (float)*p; }
__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ void st_f(bf16* p, float v) { *p = (bf16)v; }
__device__ __forceinline__ void st_f(float* p, float v) { *p = v; }

}  // namespace

template <class T, int NW, int S>
__global__ __launch_bounds__(64 * NW) void k_rglru_scan(const T* __restrict__ X, int64_t ldx, const T* __restrict__ G,
                                                        int64_t ldg, const float* __restrict__ lam, float c,
                                                        const float* __restrict__ h0, float* __restrict__ hT,
                                                        T* __restrict__ Y, int64_t ldy, int seqlen, int width) {
  __shared__ float segA[2][NW][64], segB[2][NW][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nblk = width / 64;
  const int b = blockIdx.x / nblk;
  const int ch = (blockIdx.x % nblk) * 64 + lane;
  // log a^c = c log sigma(Lambda), log sigma(z) = -(max(-z, 0) + log1p(e^-|z|))
  const float L = lam[ch];
  const float la_c = -c * (fmaxf(-L, 0.f) + log1pf(expf(-fabsf(L))));
  float carry = h0 ? h0[(size_t)b * width + ch] : 0.f;
  const size_t row0 = (size_t)b * seqlen;
  const T* xp = X + ch;
  const T* rp = G + ch;
  const T* ip = G + width + ch;
  T* yp = Y + ch;

  float nx[S], nr[S], ni[S];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = t0 + wave * S + s;
      const bool ok = t < seqlen;
      const size_t row = row0 + (ok ? t : 0);
      nx[s] = ok ? ld_f(xp + row * ldx) : 0.f;
      nr[s] = ok ? ld_f(rp + row * ldg) : 0.f;
      ni[s] = ok ? ld_f(ip + row * ldg) : 0.f;
    }
  };
  load_tile(0);
  int it = 0;
  for (int t0 = 0; t0 < seqlen; t0 += NW * S, ++it) {
    float a[S], bb[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bool ok = t0 + wave * S + s < seqlen;
      const float la = nr[s] * la_c;                  // log a_t
      const float gain = sqrtf(-expm1f(2.f * la));    // sqrt(1 - a_t^2)
      a[s] = ok ? expf(la) : 1.f;                     // steps past the end are the identity
      bb[s] = ok ? gain * (ni[s] * nx[s]) : 0.f;
    }
    if (t0 + NW * S < seqlen) load_tile(t0 + NW * S);
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
      if (t < seqlen) st_f(yp + (row0 + t) * ldy, h);
    }
    carry = next;
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
  constexpr int NW = 8, S = 8;
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
