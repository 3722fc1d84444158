// Pieces of the chunkwise backward that are not retention passes: in-place
// transposes of the per-chunk states, and per-head scaled copies or
// transposes of float32 states.
//
// The gradients of retention ([RN-zh] "Retention 網路總體結構": training runs
// the parallel and chunkwise forms) are retentions themselves: dQ is the
// causal retention of (dO, V, K), and dK, dV are anti-causal retentions,
// which become causal ones on the time-reversed sequence.  The passes run on
// the chunkwise kernels (k_chunk.hip, which can read their input rows
// backwards and write their output rows back in forward order); this file
// supplies the state seeds and transposes.
#include "msr_launch.h"

namespace msr {

namespace {
// Four consecutive elements as floats (8-byte bf16 or 16-byte f32 accesses).
__device__ __forceinline__ void load4(float* v, const bf16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
}
__device__ __forceinline__ void load4(float* v, const float* p) {
  const float4 w = *reinterpret_cast<const float4*>(p);
  v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
}
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
}  // namespace

// Transpose of nblocks contiguous d x d blocks from src to dst, in place
// when they are equal: workgroup (block, tile pair I <= J) reads tiles
// (I, J) and (J, I) through LDS and writes each one transposed into the
// other's place.  Workgroups touch disjoint tile pairs, and each reads both
// tiles before writing.  Tiles are TT x TT with TT elements = 128 bytes (64
// for bf16, 32 for float32), so each row segment is a whole L2 line and no
// line is shared with another workgroup (on another XCD).
template <class T, int TT>
__global__ __launch_bounds__(256) void k_transpose_blocks(const T* src, T* dst, int d, int npairs) {
  __shared__ float ta[TT][TT + 1], tb[TT][TT + 1];
  const int nt = d / TT;
  const int64_t blk = blockIdx.x / npairs;
  int pr = blockIdx.x % npairs, I = 0;
  while (pr >= nt - I) {   // row-major upper triangle of the tile grid
    pr -= nt - I;
    ++I;
  }
  const int J = I + pr;
  const T* m = src + blk * d * d;
  T* o = dst + blk * d * d;
  // each thread moves 4 consecutive elements of a tile row at a time: TT / 4
  // threads per row, 1024 / TT rows per pass
  constexpr int TPR = TT / 4, RPP = 256 / TPR, NP = TT / RPP;
  const int r = threadIdx.x / TPR, c4 = (threadIdx.x % TPR) * 4;
  float x[NP][4], y[NP][4];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    load4(x[p], m + (size_t)(TT * I + r + RPP * p) * d + TT * J + c4);
    load4(y[p], m + (size_t)(TT * J + r + RPP * p) * d + TT * I + c4);
  }
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ta[r + RPP * p][c4 + e] = x[p][e];
      tb[r + RPP * p][c4 + e] = y[p][e];
    }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[p][e] = ta[c4 + e][r + RPP * p];
      y[p][e] = tb[c4 + e][r + RPP * p];
    }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    store4(o + (size_t)(TT * J + r + RPP * p) * d + TT * I + c4, x[p]);   // tile (I, J) transposed into (J, I)
    if (I != J) store4(o + (size_t)(TT * I + r + RPP * p) * d + TT * J + c4, y[p]);
  }
}

hipError_t launch_transpose_blocks_to(Elt elt, const void* src, void* dst, int d, int64_t nblocks, hipStream_t st) {
  const int TT = elt == kBF16 ? 64 : 32;
  if (d % TT || d <= 0) return hipErrorInvalidValue;
  const int nt = d / TT, npairs = nt * (nt + 1) / 2;
  const int64_t wgs = nblocks * npairs;
  if (wgs == 0) return hipSuccess;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  TraceScope ts("k_transpose_blocks", st);
  if (elt == kBF16)
    hipLaunchKernelGGL((k_transpose_blocks<bf16, 64>), dim3((unsigned)wgs), dim3(256), 0, st, (const bf16*)src,
                       (bf16*)dst, d, npairs);
  else
    hipLaunchKernelGGL((k_transpose_blocks<float, 32>), dim3((unsigned)wgs), dim3(256), 0, st, (const float*)src,
                       (float*)dst, d, npairs);
  return hipGetLastError();
}
hipError_t launch_transpose_blocks(Elt elt, void* base, int d, int64_t nblocks, hipStream_t st) {
  return launch_transpose_blocks_to(elt, base, base, d, nblocks, st);
}

// dst[bh] (rows x cols) = c_h * src[bh] or c_h * src[bh]^T (src cols x rows),
// h = bh % heads; src == nullptr writes zeros.  32 x 32 tiles through LDS
// so that both the reads and the writes of a transpose are row-contiguous.
__global__ __launch_bounds__(256) void k_state_xform(const float* __restrict__ src, float* dst, int heads, int rows,
                                                     int cols, int transpose, HeadScale hs) {
  __shared__ float tile[32][33];
  const int tc = cols / 32, tiles = (rows / 32) * tc;
  const int bh = blockIdx.x / tiles, tile_id = blockIdx.x % tiles;
  const int r0 = (tile_id / tc) * 32, c0 = (tile_id % tc) * 32;
  const float c = hs.c[bh % heads];
  const size_t base = (size_t)bh * rows * cols;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  if (!src) {
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[base + (size_t)(r0 + ty + 8 * k) * cols + c0 + tx] = 0.f;
    return;
  }
  if (!transpose) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t o = base + (size_t)(r0 + ty + 8 * k) * cols + c0 + tx;
      dst[o] = c * src[o];
    }
    return;
  }
  // src is [cols][rows]: read the (c0, r0) tile row-contiguously, write transposed
#pragma unroll
  for (int k = 0; k < 4; ++k) tile[ty + 8 * k][tx] = src[base + (size_t)(c0 + ty + 8 * k) * rows + r0 + tx];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) dst[base + (size_t)(r0 + ty + 8 * k) * cols + c0 + tx] = c * tile[tx][ty + 8 * k];
}

hipError_t launch_state_xform(const float* src, float* dst, int bh, int heads, int rows, int cols, bool transpose,
                              const HeadScale& hs, hipStream_t st) {
  if (rows % 32 || cols % 32 || heads < 1 || heads > kMaxHeads) return hipErrorInvalidValue;
  if (transpose && src == dst) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)bh * (rows / 32) * (cols / 32);
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  TraceScope ts("k_state_xform", st);
  hipLaunchKernelGGL(k_state_xform, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, heads, rows, cols,
                     transpose ? 1 : 0, hs);
  return hipGetLastError();
}

}  // namespace msr
