// Pieces of the RetNet block around the gated MSR layer for gfx950.
//
// [RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、速度快、
// 性能強（2）", section "Retention 網路總體結構": the layer and a feed-forward
// network FFN(X) = gelu(X W_1) W_2 are stacked, each behind a LayerNorm
// [BKH16] and with a residual connection.  The feed-forward network and the
// residual additions run in the GEMM epilogue (k_gemm.hip); this file holds
// the LayerNorm.
#include "msr_launch.h"

namespace msr {

// One workgroup (256 threads) per row; each thread holds VPT groups of 8
// consecutive columns in registers (16-byte loads and stores), so the row
// is read once: mean, then the biased variance of the centred values, then
// (x - mean) / sqrt(var + eps) with identity affine.
template <class T, int VPT>
__global__ __launch_bounds__(256) void k_layer_norm(const T* __restrict__ X, int64_t ldx, T* __restrict__ Y,
                                                    int64_t ldy, int d, float eps) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* xr = X + (size_t)blockIdx.x * ldx;
  T* yr = Y + (size_t)blockIdx.x * ldy;
  const int groups = d / 8;
  float v[VPT][8];
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int gi = tid + 256 * u;
    if (gi < groups) {
      Row8<T> r;
      load_row8(r, xr + 8 * gi, true);
      unpack_row8(v[u], r);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[u][e];
    }
  }
  auto block_sum = [&](float x, int slot) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    if (lane == 0) red[slot][wave] = x;
    __syncthreads();
    return red[slot][0] + red[slot][1] + red[slot][2] + red[slot][3];
  };
  const float mu = block_sum(s, 0) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int gi = tid + 256 * u;
    if (gi < groups) {
#pragma unroll
      for (int e = 0; e < 8; ++e) q += (v[u][e] - mu) * (v[u][e] - mu);
    }
  }
  const float rs = rsqrtf(block_sum(q, 1) / (float)d + eps);
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int gi = tid + 256 * u;
    if (gi < groups) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[u][e] - mu) * rs;
      Row8<T> r;
      pack_row8(r, o);
      store_row8(yr + 8 * gi, r);
    }
  }
}

hipError_t launch_layer_norm(Elt elt, const void* X, int64_t ldx, void* Y, int64_t ldy, int rows, int d, float eps,
                             hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (d % 8 || d > 8 * 256 * 4) return hipErrorInvalidValue;
  TraceScope ts("k_layer_norm", st);
  const int vpt = (d / 8 + 255) / 256;
#define MSR_LN(T, V)                                                                                          \
  if (vpt <= V) {                                                                                             \
    hipLaunchKernelGGL((k_layer_norm<T, V>), dim3(rows), dim3(256), 0, st, (const T*)X, ldx, (T*)Y, ldy, d, eps); \
    return hipGetLastError();                                                                                 \
  }
  if (elt == kBF16) {
    MSR_LN(bf16, 1) MSR_LN(bf16, 2) MSR_LN(bf16, 4)
  } else {
    MSR_LN(float, 1) MSR_LN(float, 2) MSR_LN(float, 4)
  }
#undef MSR_LN
  return hipErrorInvalidValue;
}

}  // namespace msr
