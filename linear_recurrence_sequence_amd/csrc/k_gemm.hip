// Projection GEMMs of the gated MSR layer on the gfx950 matrix cores.
//
// [RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、速度快、
// 性能強（2）", section "門控多尺度 Retention", Eq. (8): the layer projects X with
// W_Q, W_K, W_V, W_G and the gated, normalised heads with W_O.
//
// C[M, N] = A[M, K] * Bt[N, K]^T with both operands K-contiguous (the weights
// are transposed once per call into that layout).  bf16: 256x256 output tile
// per workgroup, 4 waves of 128x128 (16 accumulator tiles of 32x32 each), a
// 64-deep K slab double-buffered in LDS (2 x 72 KiB) with the next slab's
// global loads in flight during the current slab's matrix-core work.  f32:
// 128x128 tile, 32-deep slab.
#include "msr_launch.h"

namespace msr {

template <class T, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void k_gemm_nt(const T* __restrict__ A, int64_t lda, const T* __restrict__ Bt,
                                                 int64_t ldb, T* __restrict__ C, int64_t ldc, int M, int N, int K) {
  constexpr int EPU = 16 / (int)sizeof(T);    // elements per 16-byte unit
  constexpr int LDS_LD = BK + EPU;            // padded row (16 bytes)
  constexpr int TM = BM / 64, TN = BN / 64;   // 32x32 tiles per wave per dim
  constexpr int UPR = BK / EPU;               // units per row
  constexpr int AU = BM * UPR / 256, BU = BN * UPR / 256;
  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * LDS_LD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  uint4 ra[AU], rb[BU];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int idx = tid + 256 * u, row = idx / UPR, c = idx % UPR;
      const int gm = m0 + row;
      ra[u] = gm < M ? *reinterpret_cast<const uint4*>(A + (size_t)gm * lda + k0 + c * EPU) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int idx = tid + 256 * u, row = idx / UPR, c = idx % UPR;
      const int gn = n0 + row;
      rb[u] = gn < N ? *reinterpret_cast<const uint4*>(Bt + (size_t)gn * ldb + k0 + c * EPU) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    T* s = smem[buf];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int idx = tid + 256 * u, row = idx / UPR, c = idx % UPR;
      *reinterpret_cast<uint4*>(s + row * LDS_LD + c * EPU) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int idx = tid + 256 * u, row = idx / UPR, c = idx % UPR;
      *reinterpret_cast<uint4*>(s + (BM + row) * LDS_LD + c * EPU) = rb[u];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const T* sA = smem[kt & 1];
    const T* sB = sA + BM * LDS_LD;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      Frag<T> af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = load_frag(sA + (wm * (BM / 2) + 32 * i + lr) * LDS_LD + 16 * s + 8 * hh);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = load_frag(sB + (wn * (BN / 2) + 32 * j + lr) * LDS_LD + 16 * s + 8 * hh);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma16(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + 32 * j + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < M) C[(size_t)row * ldc + col] = (T)acc[i][j][r];
      }
    }
}

hipError_t launch_gemm_nt(Elt elt, const void* A, int64_t lda, const void* Bt, int64_t ldb, void* C, int64_t ldc,
                          int M, int N, int K, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  TraceScope ts("k_gemm_nt", st);
  if (elt == kBF16) {
    dim3 grid((N + 255) / 256, (M + 255) / 256);
    hipLaunchKernelGGL((k_gemm_nt<bf16, 256, 256, 64>), grid, dim3(256), 0, st, (const bf16*)A, lda,
                       (const bf16*)Bt, ldb, (bf16*)C, ldc, M, N, K);
  } else {
    dim3 grid((N + 127) / 128, (M + 127) / 128);
    hipLaunchKernelGGL((k_gemm_nt<float, 128, 128, 32>), grid, dim3(256), 0, st, (const float*)A, lda,
                       (const float*)Bt, ldb, (float*)C, ldc, M, N, K);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 64x64-tile transpose through LDS.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, int64_t lds, T* __restrict__ dst,
                                                   int64_t ldd, int rows, int cols) {
  __shared__ T t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) t[i][tx] = src[(size_t)r * lds + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * ldd + r] = t[tx][i];
  }
}

hipError_t launch_transpose(Elt elt, const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols,
                            hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  TraceScope ts("k_transpose", st);
  if (elt == kBF16)
    hipLaunchKernelGGL(k_transpose<bf16>, grid, dim3(256), 0, st, (const bf16*)src, lds, (bf16*)dst, ldd, rows, cols);
  else
    hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, st, (const float*)src, lds, (float*)dst, ldd, rows,
                       cols);
  return hipGetLastError();
}

}  // namespace msr
