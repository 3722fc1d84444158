// Chunkwise and parallel retention kernels for gfx950.
//
// Method ([RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、
// 速度快、性能強（2）", section "3) Retention 分塊循環表征", Eq. (7)): with
// chunks of B tokens (the last may be short, length L) and t, s the row
// index inside a chunk,
//   O_[i] = ((Q_[i] K_[i]^T) * scale (.) D) V_[i] + scale * (Q_[i] R_{i-1}) (.) xi,
//   R_i   = gamma^L R_{i-1} + K_[i]^T (V_[i] (.) zeta),
//   D[t,s] = gamma^(t-s) (t >= s), xi_t = gamma^(t+1), zeta_s = gamma^(L-1-s).
// The parallel form (section "1) Retention 的並行表征", Eq. (5)) is the same
// output kernel with one chunk spanning the sequence and no state.
//
// Three kernels per call:
//   k_chunk_state : dR_i^T = (V_[i] (.) zeta)^T K_[i]   (matrix cores, one
//                   workgroup per (batch, head, chunk, 128x128 state tile))
//   k_chunk_scan  : R_i = gamma^L R_{i-1} + dR_i in float32, writing the
//                   exclusive prefix R_{i-1} per chunk (as the input type)
//   k_chunk_out   : per 128-row tile: Q R_{i-1} (.) xi, then the causal,
//                   decay-weighted intra-chunk product, then either O or the
//                   fused per-head GroupNorm + swish gate.
// States are stored transposed, [d_v][d_k] (d_k contiguous), because that is
// the layout the matrix-core B operand of Q R wants.
#include "msr_launch.h"

namespace msr {

template <class T> constexpr int pad16() { return 16 / (int)sizeof(T); }

// ---------------------------------------------------------------------------
// k_chunk_state
// ---------------------------------------------------------------------------
template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void k_chunk_state(const T* __restrict__ K, const T* __restrict__ V,
                                                     int64_t ldk, int64_t ldv, float* __restrict__ dR,
                                                     int N, int H, int chunk, int NC, HeadTab tab) {
  constexpr int TS = (DK >= 128 && DV >= 128) ? 128 : 64;  // state tile edge
  constexpr int WT = TS / 64;                              // 32x32 tiles per wave per dim
  constexpr int KB = 64;                                   // keys per stage
  constexpr int LDT = KB + pad16<T>();
  __shared__ __attribute__((aligned(16))) T sV[TS * LDT];  // (V (.) zeta)^T : [dv][key]
  __shared__ __attribute__((aligned(16))) T sK[TS * LDT];  // K^T           : [dk][key]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int ci = blockIdx.x % NC;
  const int bh = blockIdx.x / NC;
  const int h = bh % H, b = bh / H;
  constexpr int NTV = DV / TS;
  const int tv = blockIdx.y % NTV, tk = blockIdx.y / NTV;
  const int c0 = ci * chunk;
  const int L = min(chunk, N - c0);
  const float lg2 = tab.lg2[h];
  const int wr = (wave >> 1) * 32 * WT;
  const int wc = (wave & 1) * 32 * WT;
  const size_t tok0 = (size_t)b * N + c0;

  f32x16 acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = (f32x16){};

  constexpr int CG = TS / 8;                  // 8-column groups per row
  constexpr int UNITS = (KB / 4) * CG;        // 4-key x 8-column units
  for (int kb = 0; kb < L; kb += KB) {
    for (int u = tid; u < UNITS; u += 256) {
      const int kg = u / CG, cg = u % CG;
      Row8<T> rk[4], rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 4 * kg + i;
        const bool ok = key < L;
        const size_t tok = tok0 + (ok ? key : 0);
        load_row8(rk[i], K + tok * ldk + (size_t)h * DK + tk * TS + 8 * cg, ok);
        load_row8(rv[i], V + tok * ldv + (size_t)h * DV + tv * TS + 8 * cg, ok);
        if (ok) scale_row8(rv[i], gpow(L - 1 - key, lg2));
      }
      store_transposed4x8(sK + (8 * cg) * LDT + 4 * kg, LDT, rk);
      store_transposed4x8(sV + (8 * cg) * LDT + 4 * kg, LDT, rv);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KB / 16; ++s) {
      Frag<T> a[WT], bb[WT];
#pragma unroll
      for (int i = 0; i < WT; ++i) a[i] = load_frag(sV + (wr + 32 * i + lr) * LDT + 16 * s + 8 * hh);
#pragma unroll
      for (int j = 0; j < WT; ++j) bb[j] = load_frag(sK + (wc + 32 * j + lr) * LDT + 16 * s + 8 * hh);
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) mma16(acc[i][j], a[i], bb[j]);
    }
    __syncthreads();
  }

  float* out = dR + ((size_t)bh * NC + ci) * DV * DK;
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tv * TS + wr + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int col = tk * TS + wc + 32 * j + lr;
        out[(size_t)row * DK + col] = acc[i][j][r];
      }
}

// ---------------------------------------------------------------------------
// k_chunk_scan: float32 carry across chunks, 64x64 state tile per workgroup.
// dR and Rx may alias (float32 path): each element is read before it is
// overwritten by the same thread, so no __restrict__ on them.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store16(float* p, const float* x) {
#pragma unroll
  for (int e = 0; e < 16; e += 4) *reinterpret_cast<f32x4*>(p + e) = (f32x4){x[e], x[e + 1], x[e + 2], x[e + 3]};
}
__device__ __forceinline__ void store16(bf16* p, const float* x) {
  uint4 a = make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
  uint4 b = make_uint4(pack_bf16(x[8], x[9]), pack_bf16(x[10], x[11]), pack_bf16(x[12], x[13]), pack_bf16(x[14], x[15]));
  *reinterpret_cast<uint4*>(p) = a;
  *reinterpret_cast<uint4*>(p + 8) = b;
}
__device__ __forceinline__ void load16(float* x, const float* p) {
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p + e);
    x[e] = v[0]; x[e + 1] = v[1]; x[e + 2] = v[2]; x[e + 3] = v[3];
  }
}

template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void k_chunk_scan(const float* dR, T* Rx, const float* __restrict__ S_in,
                                                    float* __restrict__ S_out, int H, int NC, HeadTab tab) {
  constexpr int NTV = DV / 64;
  constexpr int NT = NTV * (DK / 64);
  const int bh = blockIdx.x / NT, tile = blockIdx.x % NT;
  const int h = bh % H;
  const int tv = tile % NTV, tk = tile / NTV;
  const int tid = threadIdx.x;
  const int row = tid >> 2;         // d_v index inside the tile
  const int col = (tid & 3) * 16;   // first of 16 d_k indices inside the tile
  __shared__ float sT[64][65];

  float R[16];
  if (S_in != nullptr) {
    // S_in is [dk][dv]; stage the 64x64 tile and read it transposed.
    const float* src = S_in + (size_t)bh * DK * DV + (size_t)(tk * 64 + row) * DV + tv * 64 + col;
#pragma unroll
    for (int e = 0; e < 16; ++e) sT[row][col + e] = src[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) R[e] = sT[col + e][row];
    __syncthreads();
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) R[e] = 0.f;
  }

  const size_t cstride = (size_t)DV * DK;
  const size_t off = (size_t)bh * NC * cstride + (size_t)(tv * 64 + row) * DK + tk * 64 + col;
  const float* src = dR + off;
  T* dst = Rx + off;
  const float gB = tab.gchunk[h], gL = tab.glast[h];
  float d[16], dn[16];
  load16(d, src);
  for (int ci = 0; ci < NC; ++ci) {
    if (ci + 1 < NC) load16(dn, src + (size_t)(ci + 1) * cstride);
    store16(dst + (size_t)ci * cstride, R);
    const float g = (ci == NC - 1) ? gL : gB;
#pragma unroll
    for (int e = 0; e < 16; ++e) R[e] = fmaf(g, R[e], d[e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) d[e] = dn[e];
  }

  if (S_out != nullptr) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sT[col + e][row] = R[e];
    __syncthreads();
    float* o = S_out + (size_t)bh * DK * DV + (size_t)(tk * 64 + row) * DV + tv * 64 + col;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = sT[row][col + e];
  }
}

// ---------------------------------------------------------------------------
// k_chunk_out
// ---------------------------------------------------------------------------
template <class T, int DK, int DV>
struct OutSmem {
  // Q stays in registers unless the accumulators of a 512-wide row need them.
  static constexpr bool QREG = DV <= 256;
  static constexpr int KB = 32;                       // keys per stage
  static constexpr int LDK = DK + pad16<T>();
  static constexpr int LDV = KB + pad16<T>();
  static constexpr int SK = sizeof(T) == 2 ? 64 : 32;  // d_k rows of R per stage
  static constexpr int LDR = SK + pad16<T>();
  static constexpr int intra = (KB * LDK + DV * LDV) * (int)sizeof(T);
  static constexpr int inter = DV * LDR * (int)sizeof(T);
  static constexpr int qtile = QREG ? 0 : 128 * LDK * (int)sizeof(T);
  static constexpr int bytes = (intra > inter ? intra : inter) + qtile;
};

template <class T, int DK, int DV, bool STATE, bool GN>
__global__ __launch_bounds__(256) void k_chunk_out(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int64_t ldq, int64_t ldk,
    int64_t ldv, const T* __restrict__ Rx, const T* __restrict__ G, int64_t ldg, T* __restrict__ O,
    int64_t ldo, int BH, int N, int H, int chunk, int NC, int TPC, int RT, float scale, float eps,
    HeadTab tab) {
  using SM = OutSmem<T, DK, DV>;
  constexpr int KB = SM::KB, LDK = SM::LDK, LDV = SM::LDV, SK = SM::SK, LDR = SM::LDR;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::bytes];

  const int nthr = blockDim.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  // Heavy row tiles (late in their chunk) are scheduled first.
  const int per = NC * BH;
  const int li = TPC - 1 - (int)(blockIdx.x / per);
  const int rem = blockIdx.x % per;
  const int ci = rem / BH, bh = rem % BH;
  const int h = bh % H, b = bh / H;
  const int c0 = ci * chunk;
  const int r0 = c0 + li * RT;
  if (r0 >= N) return;
  const int q0 = r0 + 32 * wave;
  const float lg2 = tab.lg2[h];
  const size_t tokb = (size_t)b * N;

  // This wave's 32 query rows as matrix-core fragments: element t of lane
  // half hh of fragment s is column 16 s + 8 hh + t of query row q0 + lr.
  // The same registers serve as the B operand of K Q^T and as the A operand
  // of Q R.  For 512-wide value heads they live in LDS instead.
  constexpr bool QREG = SM::QREG;
  Frag<T> qf[QREG ? DK / 16 : 1];
  T* sQ = reinterpret_cast<T*>(smem + (SM::bytes - SM::qtile)) + (32 * wave) * LDK;
  {
    const int q = q0 + lr;
    const bool ok = q < N;
    const T* p = Q + (tokb + (ok ? q : 0)) * ldq + (size_t)h * DK + 8 * hh;
    if constexpr (QREG) {
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) qf[s] = ok ? load_frag(p + 16 * s) : zero_frag<T>();
    } else {
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) {
        Row8<T> r;
        load_row8(r, p + 16 * s, ok);
        store_row8(sQ + lr * LDK + 16 * s + 8 * hh, r);
      }
    }
  }
  auto qfrag = [&](int s) -> Frag<T> {
    if constexpr (QREG) return qf[s];
    else return load_frag(sQ + lr * LDK + 16 * s + 8 * hh);
  };

  f32x16 acc[DV / 32];
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) acc[j] = (f32x16){};

  if constexpr (STATE) {
    // acc = (xs (.) Q) R_{i-1}, xs_t = scale * xi_t for row t inside the
    // chunk.  In the A-operand layout a lane holds one query row (lr), so the
    // row factor is one scalar per lane folded into the Q fragment.
    // R_{i-1} is stored [dv][dk].
    const float xs = scale * gpow(q0 - c0 + lr + 1, lg2);
    T* sR = reinterpret_cast<T*>(smem);
    const T* Rt = Rx + ((size_t)bh * NC + ci) * DV * DK;
    if constexpr (!QREG) __syncthreads();  // Q tile visible (rows are per wave, but be safe)
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += SK) {
      for (int u = tid; u < DV * SK / 8; u += nthr) {
        const int row = u / (SK / 8), c8 = u % (SK / 8);
        Row8<T> r;
        load_row8(r, Rt + (size_t)row * DK + k0 + 8 * c8, true);
        store_row8(sR + row * LDR + 8 * c8, r);
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < SK / 16; ++s) {
        Frag<T> qa = qfrag(k0 / 16 + s);
#pragma unroll
        for (int t = 0; t < 8; ++t) qa.v[t] = (T)((float)qa.v[t] * xs);
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) {
          Frag<T> bfr = load_frag(sR + (32 * j + lr) * LDR + 16 * s + 8 * hh);
          mma16(acc[j], qa, bfr);
        }
      }
      __syncthreads();
    }
  }

  // Decay factors of a 32x32 score tile (lane lr = query offset, register r
  // = key offset kk = 8 (r/4) + 4 hh + r%4):
  //   diagonal tile:  dd[r] = scale * gamma^(lr - kk) for lr >= kk, else 0;
  //   tile kb < q0 :  scale * gamma^(q0-kb-31) * ab[r],
  //                   ab[r] = gamma^lr * gamma^(31 - kk)   (all exponents >= 0).
  float dd[16], ab[16];
  {
    const float glr = gpow(lr, lg2);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int dlt = lr - kk;
      dd[r] = dlt >= 0 ? scale * gpow(dlt, lg2) : 0.f;
      ab[r] = glr * gpow(31 - kk, lg2);
    }
  }

  T* sK = reinterpret_cast<T*>(smem);
  T* sVt = sK + KB * LDK;
  const int kend = min(r0 + RT, N);
  for (int kb = c0; kb < kend; kb += KB) {
    // K block row-major [key][dk]
    for (int u = tid; u < KB * (DK / 8); u += nthr) {
      const int row = u / (DK / 8), c8 = u % (DK / 8);
      const int key = kb + row;
      Row8<T> r;
      load_row8(r, K + (tokb + (key < N ? key : 0)) * ldk + (size_t)h * DK + 8 * c8, key < N);
      store_row8(sK + row * LDK + 8 * c8, r);
    }
    // V block transposed [dv][key]
    for (int u = tid; u < (KB / 4) * (DV / 8); u += nthr) {
      const int kg = u / (DV / 8), cg = u % (DV / 8);
      Row8<T> rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 4 * kg + i;
        load_row8(rv[i], V + (tokb + (key < N ? key : 0)) * ldv + (size_t)h * DV + 8 * cg, key < N);
      }
      store_transposed4x8(sVt + (8 * cg) * LDV + 4 * kg, LDV, rv);
    }
    __syncthreads();
    if (kb <= q0 && q0 < N) {
      f32x16 st = (f32x16){};
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) {
        Frag<T> a = load_frag(sK + lr * LDK + 16 * s + 8 * hh);
        mma16(st, a, qfrag(s));
      }
      float p[16];
      if (kb == q0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = st[r] * dd[r];
      } else {
        const float c = scale * gpow(q0 - kb - 31, lg2);
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = st[r] * (c * ab[r]);
      }
      const Frag<T> pa0 = frag_from<T>(p), pa1 = frag_from<T>(p + 8);
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) {
        const T* vr = sVt + (32 * j + lr) * LDV + 4 * hh;
        mma16(acc[j], pa0, load_frag2(vr, vr + 8));
        mma16(acc[j], pa1, load_frag2(vr + 16, vr + 24));
      }
    }
    __syncthreads();
  }

  // Epilogue.  Lane owns column 32 j + lr of rows q0 + 8 (r/4) + 4 hh + r%4.
  if constexpr (GN) {
    float mu[16], rs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) s += acc[j][r];
      mu[r] = half_wave_sum(s) * (1.0f / DV);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) {
        const float dlt = acc[j][r] - mu[r];
        s += dlt * dlt;
      }
      rs[r] = rsqrtf(half_wave_sum(s) * (1.0f / DV) + eps);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (q < N) {
        const T* gp = G + (tokb + q) * ldg + (size_t)h * DV + lr;
        T* op = O + (tokb + q) * ldo + (size_t)h * DV + lr;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) {
          const float g = (float)gp[32 * j];
          const float sw = g / (1.0f + __expf(-g));
          op[32 * j] = (T)(sw * (acc[j][r] - mu[r]) * rs[r]);
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (q < N) {
        T* op = O + (tokb + q) * ldo + (size_t)h * DV + lr;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) op[32 * j] = (T)acc[j][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int row_tile(int chunk) {
  if (chunk % 128 == 0) return 128;
  if (chunk % 64 == 0) return 64;
  return 32;
}

template <class T, int DK, int DV>
static hipError_t run_chunkwise(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  const int B = a.batch, N = a.seqlen, H = a.heads, C = a.chunk;
  const int NC = (N + C - 1) / C;
  const int BH = B * H;
  constexpr int TS = (DK >= 128 && DV >= 128) ? 128 : 64;
  {
    TraceScope ts("k_chunk_state", st);
    dim3 grid(BH * NC, (DV / TS) * (DK / TS));
    hipLaunchKernelGGL((k_chunk_state<T, DK, DV>), grid, dim3(256), 0, st, (const T*)a.K, (const T*)a.V,
                       a.ldk, a.ldv, a.dR, N, H, C, NC, tab);
  }
  {
    TraceScope ts("k_chunk_scan", st);
    dim3 grid(BH * (DV / 64) * (DK / 64));
    hipLaunchKernelGGL((k_chunk_scan<T, DK, DV>), grid, dim3(256), 0, st, (const float*)a.dR, (T*)a.Rx,
                       a.S_in, a.S_out, H, NC, tab);
  }
  {
    TraceScope ts("k_chunk_out", st);
    const int RT = row_tile(C);
    const int TPC = C / RT;
    dim3 grid(TPC * NC * BH);
    dim3 block(RT * 2);  // RT / 32 waves of 64 lanes
    if (a.fuse_gn_gate)
      hipLaunchKernelGGL((k_chunk_out<T, DK, DV, true, true>), grid, block, 0, st, (const T*)a.Q, (const T*)a.K,
                         (const T*)a.V, a.ldq, a.ldk, a.ldv, (const T*)a.Rx, (const T*)a.G, a.ldg, (T*)a.O,
                         a.ldo, BH, N, H, C, NC, TPC, RT, a.scale, a.eps, tab);
    else
      hipLaunchKernelGGL((k_chunk_out<T, DK, DV, true, false>), grid, block, 0, st, (const T*)a.Q,
                         (const T*)a.K, (const T*)a.V, a.ldq, a.ldk, a.ldv, (const T*)a.Rx, (const T*)nullptr,
                         (int64_t)0, (T*)a.O, a.ldo, BH, N, H, C, NC, TPC, RT, a.scale, a.eps, tab);
  }
  return hipGetLastError();
}

template <class T, int DK, int DV>
static hipError_t run_parallel(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  const int B = a.batch, N = a.seqlen, H = a.heads;
  const int BH = B * H;
  constexpr int RT = 128;
  const int TPC = (N + RT - 1) / RT;
  dim3 grid(TPC * BH);
  TraceScope ts("k_chunk_out", st);
  if (a.fuse_gn_gate)
    hipLaunchKernelGGL((k_chunk_out<T, DK, DV, false, true>), grid, dim3(256), 0, st, (const T*)a.Q,
                       (const T*)a.K, (const T*)a.V, a.ldq, a.ldk, a.ldv, (const T*)nullptr, (const T*)a.G,
                       a.ldg, (T*)a.O, a.ldo, BH, N, H, TPC * RT, 1, TPC, RT, a.scale, a.eps, tab);
  else
    hipLaunchKernelGGL((k_chunk_out<T, DK, DV, false, false>), grid, dim3(256), 0, st, (const T*)a.Q,
                       (const T*)a.K, (const T*)a.V, a.ldq, a.ldk, a.ldv, (const T*)nullptr, (const T*)nullptr,
                       (int64_t)0, (T*)a.O, a.ldo, BH, N, H, TPC * RT, 1, TPC, RT, a.scale, a.eps, tab);
  return hipGetLastError();
}

#define MSR_DISPATCH_DIMS(FN, T, ...)                                           \
  if (a.d_k == 64 && a.d_v == 64) return FN<T, 64, 64>(__VA_ARGS__);            \
  if (a.d_k == 128 && a.d_v == 128) return FN<T, 128, 128>(__VA_ARGS__);        \
  if (a.d_k == 256 && a.d_v == 256) return FN<T, 256, 256>(__VA_ARGS__);

hipError_t launch_chunkwise(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  if (a.elt == kBF16) {
    MSR_DISPATCH_DIMS(run_chunkwise, bf16, a, tab, st)
    if (a.d_k == 256 && a.d_v == 512) return run_chunkwise<bf16, 256, 512>(a, tab, st);
  } else {
    MSR_DISPATCH_DIMS(run_chunkwise, float, a, tab, st)
  }
  return hipErrorInvalidValue;
}

hipError_t launch_parallel(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  if (a.elt == kBF16) {
    MSR_DISPATCH_DIMS(run_parallel, bf16, a, tab, st)
    if (a.d_k == 256 && a.d_v == 512) return run_parallel<bf16, 256, 512>(a, tab, st);
  } else {
    MSR_DISPATCH_DIMS(run_parallel, float, a, tab, st)
  }
  return hipErrorInvalidValue;
}

}  // namespace msr
