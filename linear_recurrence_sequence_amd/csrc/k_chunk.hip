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
//                   workgroup per (batch, head, chunk, state tile); stored
//                   in the input type)
//   k_chunk_scan  : R_i = gamma^L R_{i-1} + dR_i carried in float32, writing
//                   the exclusive prefix R_{i-1} per chunk over dR_i
//   k_chunk_out   : per row tile: Q R_{i-1} (.) xi, then the causal,
//                   decay-weighted intra-chunk product, then either O or the
//                   fused per-head GroupNorm + swish gate.
// States are stored transposed, [d_v][d_k] (d_k contiguous), because that is
// the layout the matrix-core B operand of Q R wants.
#include "msr_launch.h"

namespace msr {

template <class T> constexpr int pad16() { return 16 / (int)sizeof(T); }

// ---------------------------------------------------------------------------
// k_chunk_state
// One workgroup per (batch, head, chunk, TS x TS state tile), 4 waves of
// (TS/2) x (TS/2).  K and zeta-weighted V are staged row-major ([key][col],
// one key per row, plain 16-byte copies) and read as fragments with the
// transposing LDS read.  The kernel is bound by reading K and V and writing
// dR, so it keeps LDS small (about 40 KiB) for three workgroups per CU
// rather than double-buffering.
// ---------------------------------------------------------------------------
template <class T, int DK, int DV>
struct StateCfg {
  static constexpr int TS = (DK >= 128 && DV >= 128) ? 128 : 64;  // state tile edge
  static constexpr int WT = TS / 64;                              // 32x32 tiles per wave per dim
  static constexpr int KB = sizeof(T) == 2 ? 64 : 32;             // keys per stage
  static constexpr int LDT = TS + rm_pad<T>();
  static constexpr int UNITS = KB * (TS / 8);                     // 8-element rows per operand
  static constexpr int UPT = (UNITS + 255) / 256;
  static constexpr int STAGE = 2 * KB * LDT;                      // elements (V then K)
};

// With a (cos, sin) table (forward only), the K rows are rotated as they
// are staged ([RN-zh] section "Retention", Eq. (3)-(4)) and the tiles with
// tv == 0 (which together stage every K column once) also write the rotated
// rows to Krot, for the output kernel.
template <class T, int DK, int DV, bool RV>
__global__ __launch_bounds__(256) void k_chunk_state(const T* __restrict__ K, const T* __restrict__ V,
                                                     int64_t ldk, int64_t ldv, T* __restrict__ dR,
                                                     int BH, int N, int H, int chunk, int NC, HeadTab tab,
                                                     const float2* __restrict__ rtab, T* __restrict__ Krot,
                                                     int64_t ldkr) {
  constexpr bool rev_in = RV;                        // read the sequence backwards
  using C = StateCfg<T, DK, DV>;
  constexpr int TS = C::TS, WT = C::WT, KB = C::KB, LDT = C::LDT, UNITS = C::UNITS, UPT = C::UPT;
  __shared__ __attribute__((aligned(16))) T smem[C::STAGE];
  T* sV = smem;
  T* sK = smem + KB * LDT;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  // block id -> (batch-head-chunk unit, state tile): the tiles of a unit
  // are 8 block ids apart, so they run on one XCD and share K and V in its L2
  constexpr int NTV = DV / TS, NTT = NTV * (DK / TS);
  const int xg = blockIdx.x & 7, yg = blockIdx.x >> 3;
  const int tile = yg % NTT, unit = (yg / NTT) * 8 + xg;
  if (unit >= BH * NC) return;
  const int ci = unit % NC;
  const int bh = unit / NC;
  const int h = bh % H, b = bh / H;
  const int tv = tile % NTV, tk = tile / NTV;
  const int c0 = ci * chunk;
  const int L = min(chunk, N - c0);
  const float lg2 = tab.lg2[h];
  const int wr = (wave >> 1) * 32 * WT;
  const int wc = (wave & 1) * 32 * WT;
  // uniform bases + small per-thread offsets; keys past the chunk end are
  // clamped to a valid row and get zeta = 0, so they add nothing.  With
  // rev_in key kc of the chunk is row N - 1 - c0 - kc: the base is the
  // chunk's lowest row and the offset L - 1 - kc.
  const size_t tok0 = (size_t)b * N + (rev_in ? N - c0 - L : c0);
  const T* Kb = K + (size_t)h * DK + tk * TS + tok0 * ldk;
  const T* Vb = V + (size_t)h * DV + tv * TS + tok0 * ldv;

  f32x16 acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = (f32x16){};

  for (int kb = 0; kb < L; kb += KB) {
#pragma unroll
    for (int q = 0; q < UPT; ++q) {
      const int u = tid + 256 * q;
      const int key = u / (TS / 8), c8 = u % (TS / 8);
      if (UNITS % 256 == 0 || u < UNITS) {
        const int kk = kb + key;
        const int kc = min(kk, L - 1), kr = rev_in ? L - 1 - kc : kc;
        Row8<T> rk, rv;
        load_row8(rk, Kb + (uint32_t)(kr * (int)ldk + 8 * c8), true);
        load_row8(rv, Vb + (uint32_t)(kr * (int)ldv + 8 * c8), true);
        if (rtab != nullptr) {                         // uniform
          rotate_row8(rk, rtab + (size_t)(c0 + kr) * (DK / 2) + (tk * TS + 8 * c8) / 2);
          if (tv == 0 && kk < L)
            store_row8(Krot + ((size_t)b * N + c0 + kr) * ldkr + (size_t)h * DK + tk * TS + 8 * c8, rk);
        }
        scale_row8(rv, kk < L ? gpow(L - 1 - kk, lg2) : 0.f);
        store_row8(sK + key * LDT + 8 * c8, rk);
        store_row8(sV + key * LDT + 8 * c8, rv);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KB / 16; ++s) {
      Frag<T> a[WT], bb[WT];
#pragma unroll
      for (int i = 0; i < WT; ++i) a[i] = load_frag_rm<KMAP_CONTIG>(sV + 16 * s * LDT + wr + 32 * i, LDT);
#pragma unroll
      for (int j = 0; j < WT; ++j) bb[j] = load_frag_rm<KMAP_CONTIG>(sK + 16 * s * LDT + wc + 32 * j, LDT);
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) mma16(acc[i][j], a[i], bb[j]);
    }
    __syncthreads();
  }

  T* out = dR + ((size_t)bh * NC + ci) * DV * DK;
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tv * TS + wr + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int col = tk * TS + wc + 32 * j + lr;
        out[(size_t)row * DK + col] = (T)acc[i][j][r];
      }
}

// ---------------------------------------------------------------------------
// k_chunk_scan: float32 carry across chunks, one state tile per workgroup.
// dR and Rx alias: each element is read (chunks ahead) before the same
// thread overwrites it, so no __restrict__ on them.
// ---------------------------------------------------------------------------
// E consecutive elements (E = 4 or 16) as loaded, not yet converted to float.
template <class T, int E> struct RawN;
template <int E> struct RawN<bf16, E> { uint32_t w[E / 2]; };
template <int E> struct RawN<float, E> { f32x4 x[E / 4]; };
template <int E>
__device__ __forceinline__ RawN<bf16, E> load_raw(const bf16* p) {
  RawN<bf16, E> r;
  if constexpr (E == 16) {
    const uint4 a = *reinterpret_cast<const uint4*>(p), b = *reinterpret_cast<const uint4*>(p + 8);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w; r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
  } else {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    r.w[0] = a.x; r.w[1] = a.y;
  }
  return r;
}
template <int E>
__device__ __forceinline__ RawN<float, E> load_raw(const float* p) {
  RawN<float, E> r;
#pragma unroll
  for (int i = 0; i < E / 4; ++i) r.x[i] = *reinterpret_cast<const f32x4*>(p + 4 * i);
  return r;
}
template <int E>
__device__ __forceinline__ void unpack_raw(float* x, const RawN<bf16, E>& r) {
#pragma unroll
  for (int i = 0; i < E / 2; ++i) { x[2 * i] = bf16_lo(r.w[i]); x[2 * i + 1] = bf16_hi(r.w[i]); }
}
template <int E>
__device__ __forceinline__ void unpack_raw(float* x, const RawN<float, E>& r) {
#pragma unroll
  for (int i = 0; i < E / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = r.x[i][e];
}
template <int E>
__device__ __forceinline__ void store_n(float* p, const float* x) {
#pragma unroll
  for (int e = 0; e < E; e += 4) *reinterpret_cast<f32x4*>(p + e) = (f32x4){x[e], x[e + 1], x[e + 2], x[e + 3]};
}
template <int E>
__device__ __forceinline__ void store_n(bf16* p, const float* x) {
  uint32_t w[E / 2];
#pragma unroll
  for (int i = 0; i < E / 2; ++i) w[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
  if constexpr (E == 16) {
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(p + 8) = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  }
}

// TR x TC state tile per workgroup (d_v rows x d_k columns): 64 x 64 (16
// elements per thread), or, for shapes with few (batch, head) pairs, 16 x 64
// (four times the workgroups, 4 elements per thread).  Every row segment a
// thread group reads or writes is 128 bytes (bf16), a whole L2 line, so no
// line is shared with a neighbouring tile's workgroup on another XCD.
template <class T, int DK, int DV, int TR, int TC>
__global__ __launch_bounds__(256) void k_chunk_scan(const T* dR, T* Rx, const float* __restrict__ S_in,
                                                    float* __restrict__ S_out, int H, int NC, HeadTab tab,
                                                    HeadScale so) {
  constexpr int E = TR * TC / 256;   // elements per thread
  constexpr int NTV = DV / TR;
  constexpr int NT = NTV * (DK / TC);
  static_assert(E >= 4 && TC % E == 0 && 256 % (TC / E) == 0, "whole rows per thread group");
  const int bh = blockIdx.x / NT, tile = blockIdx.x % NT;
  const int h = bh % H;
  const int tv = tile % NTV, tk = tile / NTV;
  const int tid = threadIdx.x;
  const int row = tid / (TC / E);       // d_v index inside the tile
  const int col = (tid % (TC / E)) * E; // first of E d_k indices inside the tile
  __shared__ float sT[TC][TR + 1];      // the tile as [d_k][d_v] (the float32 states' layout)

  float R[E];
  if (S_in != nullptr) {
    // S_in is [dk][dv]: stage the tile in that order, read it transposed
    const float* src = S_in + (size_t)bh * DK * DV + (size_t)(tk * TC) * DV + tv * TR;
    for (int i = tid; i < TR * TC; i += 256) sT[i / TR][i % TR] = src[(size_t)(i / TR) * DV + i % TR];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) R[e] = sT[col + e][row];
    __syncthreads();
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) R[e] = 0.f;
  }

  const size_t cstride = (size_t)DV * DK;
  const size_t off = (size_t)bh * NC * cstride + (size_t)(tv * TR + row) * DK + tk * TC + col;
  const T* src = dR + off;
  T* dst = Rx + off;
  const float gB = tab.gchunk[h], gL = tab.glast[h];
  // Contributions of the next PF chunks in flight (8 with the 16 x 64 tiles,
  // whose loads are 8 bytes per lane), kept raw (unconverted) in a
  // statically indexed ring: converting right after the load would make the
  // load complete at once.  Chunk ci's slot is reloaded with chunk ci + PF
  // right after it has been read.  The reloads are unconditional, clamped to
  // the last chunk (a re-read whose value is never used), so no slot has to
  // be kept across a branch; chunk NC - 1 is loaded before it is written.
  constexpr int PF = E == 4 ? 8 : 4;
  RawN<T, E> ring[PF];
  // (issued in slot order, as in the loop, so that the wait counts at the
  // loop head are the steady-state ones)
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    ring[u] = load_raw<E>(src + (size_t)min(u, NC - 1) * cstride);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int c0 = 0; c0 < NC; c0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int ci = c0 + u;
      float d[E];
      unpack_raw<E>(d, ring[u]);
      ring[u] = load_raw<E>(src + (size_t)min(ci + PF, NC - 1) * cstride);
      if (ci < NC) {
        store_n<E>(dst + (size_t)ci * cstride, R);
        const float g = (ci == NC - 1) ? gL : gB;
#pragma unroll
        for (int e = 0; e < E; ++e) R[e] = fmaf(g, R[e], d[e]);
      }
    }
  }

  if (S_out != nullptr) {
#pragma unroll
    for (int e = 0; e < E; ++e) sT[col + e][row] = R[e];
    __syncthreads();
    float* o = S_out + (size_t)bh * DK * DV + (size_t)(tk * TC) * DV + tv * TR;
    const float c = so.c[h];
    for (int i = tid; i < TR * TC; i += 256) o[(size_t)(i / TR) * DV + i % TR] = c * sT[i / TR][i % TR];
  }
}

// ---------------------------------------------------------------------------
// k_chunk_out
// One workgroup per (batch, head, chunk, row tile of 32*NW query rows); each
// wave owns 32 query rows and the full d_v width of their outputs (the
// accumulators), and keeps its Q rows in registers as matrix-core fragments.
// Stages, in order: the d_k slabs of R_{i-1} (Q R), then the key blocks of
// the chunk up to the tile's last row (causal, decay-weighted Q K^T, then
// P V).  bf16 with 4 waves runs them as a two-stage pipeline: the next
// stage's global loads are in flight in registers while the matrix cores
// work on the current stage in LDS, then land in the other LDS buffer.
// ---------------------------------------------------------------------------
template <class T, int DK, int DV, int NW>
struct OutCfg {
  static constexpr int NT = 64 * NW;                               // threads
  static constexpr bool PIPE = sizeof(T) == 2 && NW == 4;
  static constexpr int KB = (sizeof(T) == 4 || DV > 256) ? 32 : 64; // keys per stage
  static constexpr int SK = KB;                                    // d_k rows of R per stage
  static constexpr int PAD = pad16<T>();
  static constexpr int LDK = DK + PAD;                             // K block: [key][dk]
  static constexpr int LDV = DV + rm_pad<T>();                     // V block: [key][dv]
  static constexpr int LDR = SK + PAD;                             // R^T slab: [dv][dk]
  static constexpr int KV = KB * LDK + KB * LDV;
  static constexpr int RS = DV * LDR;
  static constexpr int STAGE = KV > RS ? KV : RS;                  // elements per stage
  static constexpr int NBUF = PIPE ? 2 : 1;
  static constexpr int NR = DK / SK;                               // R slabs
  // register staging (Row8 units per thread)
  static constexpr int KU = (KB * (DK / 8) + NT - 1) / NT;         // K rows
  static constexpr int VU = (KB * (DV / 8) + NT - 1) / NT;         // V rows
  static constexpr int RU = (DV * (SK / 8) + NT - 1) / NT;         // R slab rows
  static constexpr int PRE = (KU + VU) > RU ? (KU + VU) : RU;
};

template <class T, int DK, int DV, int NW, bool STATE, bool GN>
__global__ __launch_bounds__(64 * NW) void k_chunk_out(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int64_t ldq, int64_t ldk,
    int64_t ldv, const T* __restrict__ Rx, int has_sin, const T* __restrict__ G, int64_t ldg, T* __restrict__ O,
    int64_t ldo, int BH, int N, int H, int chunk, int NC, int TPC, float scale, float eps, HeadTab tab, int rev,
    const float2* __restrict__ qtab) {
  // rev bit 0: output row t to row N - 1 - t; bit 1: Q, K, V row t from row N - 1 - t
  // qtab: (cos, sin) table of the rows' positions; Q is rotated as it is
  // loaded (forward only)
  const bool rev_o = rev & 1, rev_i = rev & 2;
  using C = OutCfg<T, DK, DV, NW>;
  constexpr int NT = C::NT, KB = C::KB, SK = C::SK, LDK = C::LDK, LDV = C::LDV, LDR = C::LDR;
  constexpr int RT = 32 * NW;
  __shared__ __attribute__((aligned(16))) T smem[C::NBUF * C::STAGE];

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

  // Query rows as fragments: element t of lane half hh of fragment s is
  // column 16 s + 8 hh + t of query row q0 + lr.  They are the B operand of
  // K Q^T and (times xs) the A operand of Q R.
  Frag<T> qf[DK / 16];
  {
    // rows past the end are clamped (their outputs are never stored)
    const int qr = min(q0 + lr, N - 1);
    const T* p = Q + (tokb + (rev_i ? N - 1 - qr : qr)) * ldq + (size_t)h * DK + 8 * hh;
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) qf[s] = load_frag(p + 16 * s);
    if (qtab != nullptr) {                           // uniform; element t is column 16 s + 8 hh + t
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) rotate_frag(qf[s], qtab + (size_t)qr * (DK / 2) + 8 * s + 4 * hh);
    }
  }
  f32x16 acc[DV / 32];
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) acc[j] = (f32x16){};

  // ---- staging ----
  Row8<T> pre[C::PRE];
  const T* Rt = STATE ? Rx + ((size_t)bh * NC + ci) * DV * DK : nullptr;
  // Keys past the end of the sequence are clamped to the last row: they are
  // in the future of every stored query, so their P entries are exactly 0.
  const T* Kh = K + (size_t)h * DK + tokb * ldk;
  const T* Vh = V + (size_t)h * DV + tokb * ldv;
  auto load_R = [&](int k0) {
#pragma unroll
    for (int u = 0; u < C::RU; ++u) {
      const int idx = min(tid + NT * u, DV * (SK / 8) - 1);
      const int row = idx / (SK / 8), c8 = idx % (SK / 8);
      load_row8(pre[u], Rt + k0 + row * DK + 8 * c8, true);
    }
  };
  auto store_R = [&](T* sR) {
#pragma unroll
    for (int u = 0; u < C::RU; ++u) {
      const int idx = tid + NT * u;
      if (idx >= DV * (SK / 8)) break;
      const int row = idx / (SK / 8), c8 = idx % (SK / 8);
      store_row8(sR + row * LDR + 8 * c8, pre[u]);
    }
  };
  // 32-bit per-thread offsets inside a KB-row block (row < KB, so
  // row * stride fits easily); the block base is a uniform 64-bit pointer.
  const int ldk32 = (int)ldk, ldv32 = (int)ldv;
  // With rev_i, key kb + r is row N - 1 - kb - r: the block's base is its
  // lowest row, N - 1 - kb - lim, and key r sits lim - r rows above it.
  auto load_KV = [&](int kb) {
    const int lim = min(KB - 1, N - 1 - kb);
    const int base = rev_i ? N - 1 - kb - lim : kb;
    const T* Kk = Kh + (size_t)base * ldk;
    const T* Vk = Vh + (size_t)base * ldv;
    auto orow = [&](int row) { return rev_i ? lim - min(row, lim) : min(row, lim); };
#pragma unroll
    for (int u = 0; u < C::KU; ++u) {
      const int idx = min(tid + NT * u, KB * (DK / 8) - 1);
      const int row = idx / (DK / 8), c8 = idx % (DK / 8);
      load_row8(pre[u], Kk + (uint32_t)(orow(row) * ldk32 + 8 * c8), true);
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
      const int idx = min(tid + NT * u, KB * (DV / 8) - 1);
      const int row = idx / (DV / 8), c8 = idx % (DV / 8);
      load_row8(pre[C::KU + u], Vk + (uint32_t)(orow(row) * ldv32 + 8 * c8), true);
    }
  };
  auto store_KV = [&](T* sK) {
    T* sV = sK + KB * LDK;
#pragma unroll
    for (int u = 0; u < C::KU; ++u) {
      const int idx = tid + NT * u;
      if (idx >= KB * (DK / 8)) break;
      const int row = idx / (DK / 8), c8 = idx % (DK / 8);
      store_row8(sK + row * LDK + 8 * c8, pre[u]);
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
      const int idx = tid + NT * u;
      if (idx >= KB * (DV / 8)) break;
      const int row = idx / (DV / 8), c8 = idx % (DV / 8);
      store_row8(sV + row * LDV + 8 * c8, pre[C::KU + u]);
    }
  };
  auto buf = [&](int i) { return smem + (C::PIPE ? (i & 1) : 0) * C::STAGE; };

  // ---- compute ----
  // rows scaled by xs = scale * xi_t = scale * gamma^(t+1), t = row inside the chunk
  const float xs = scale * gpow(q0 - c0 + lr + 1, lg2);
  auto compute_R = [&](const T* sR, int slab) {
#pragma unroll
    for (int s = 0; s < SK / 16; ++s) {
      Frag<T> qa = qf[slab * (SK / 16) + s];
#pragma unroll
      for (int t = 0; t < 8; ++t) qa.v[t] = (T)((float)qa.v[t] * xs);
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) mma16(acc[j], qa, load_frag(sR + (32 * j + lr) * LDR + 16 * s + 8 * hh));
    }
  };
  // Decay of a 32x32 score tile (lane lr = query offset, register r = key
  // offset kk = 8 (r/4) + 4 hh + r%4): diagonal tile dd[r] = scale *
  // gamma^(lr-kk) (lr >= kk, else 0); a tile ks < q0 uses scale *
  // gamma^(q0-ks-31) * ab[r], ab[r] = gamma^lr gamma^(31-kk) (exponents >= 0).
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
  auto compute_KV = [&](const T* sK, int kb) {
    const T* sV = sK + KB * LDK;
#pragma unroll
    for (int u = 0; u < KB / 32; ++u) {
      const int ks = kb + 32 * u;
      if (ks > q0 || q0 >= N) continue;  // wave-uniform: keys all in this wave's future
      f32x16 st = (f32x16){};
#pragma unroll
      for (int s = 0; s < DK / 16; ++s) mma16(st, load_frag(sK + (32 * u + lr) * LDK + 16 * s + 8 * hh), qf[s]);
      float p[16];
      if (ks == q0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = st[r] * dd[r];
      } else {
        const float c = scale * gpow(q0 - ks - 31, lg2);
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = st[r] * (c * ab[r]);
      }
      const Frag<T> pa0 = frag_from<T>(p), pa1 = frag_from<T>(p + 8);
      // P's element t of lane half hh is key 8 (t/4) + 4 hh + t%4 of each
      // 16-key step: the V fragment is read in that (KMAP_ACC) order.
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) {
        const T* vr = sV + (32 * u) * LDV + 32 * j;
        mma16(acc[j], pa0, load_frag_rm<KMAP_ACC>(vr, LDV));
        mma16(acc[j], pa1, load_frag_rm<KMAP_ACC>(vr + 16 * LDV, LDV));
      }
    }
  };

  // ---- the pipeline ----
  const bool inter = STATE && (ci > 0 || has_sin);
  const int kend = min(r0 + RT, N);
  const int nkb = (kend - c0 + KB - 1) / KB;
  int stage = 0;
  if constexpr (C::PIPE) {
    if (inter) load_R(0); else load_KV(c0);
    if (inter) store_R(buf(0)); else store_KV(buf(0));
    __syncthreads();
  }
  if (inter) {
#pragma unroll
    for (int sl = 0; sl < C::NR; ++sl, ++stage) {
      if constexpr (C::PIPE) {
        if (sl + 1 < C::NR) load_R((sl + 1) * SK);
        else if (nkb > 0) load_KV(c0);
        compute_R(buf(stage), sl);
        if (sl + 1 < C::NR) store_R(buf(stage + 1));
        else if (nkb > 0) store_KV(buf(stage + 1));
      } else {
        load_R(sl * SK);
        store_R(buf(0));
        __syncthreads();
        compute_R(buf(0), sl);
      }
      __syncthreads();
    }
  }
  for (int i = 0; i < nkb; ++i, ++stage) {
    const int kb = c0 + i * KB;
    if constexpr (C::PIPE) {
      if (i + 1 < nkb) load_KV(kb + KB);
      compute_KV(buf(stage), kb);
      if (i + 1 < nkb) store_KV(buf(stage + 1));
    } else {
      load_KV(kb);
      store_KV(buf(0));
      __syncthreads();
      compute_KV(buf(0), kb);
    }
    __syncthreads();
  }

  // ---- epilogue: lane owns column 32 j + lr of rows q0 + 8 (r/4) + 4 hh + r%4 ----
  if constexpr (GN && DV > 256) {
    // d_v = 512 (every register in use): the normalised rows go through
    // LDS, 8 rows of this wave per pass (accumulator registers 4 p .. 4 p + 3),
    // so that each lane then takes one 8-column chunk of each row -- 16-byte
    // gate loads, the next pass's in flight during the current one, and
    // 16-byte stores.  The staging rows are the wave's own (in-order LDS
    // operations, a compiler fence between the phases).
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
    constexpr int SLD = DV + 4;                    // staged row stride (floats)
    constexpr int CH = 8 * (DV / 8) / 64;          // 8-column chunks per lane per pass
    static_assert(NW * 8 * SLD * 4 <= C::NBUF * C::STAGE * (int)sizeof(T), "staging fits in the stage buffers");
    __syncthreads();                               // every wave is done with the stage buffers
    float* stg = reinterpret_cast<float*>(smem) + wave * 8 * SLD;
    Row8<T> gv[2][CH];
    auto gload = [&](int p, int buf) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int c = lane + 64 * k, rr = c / (DV / 8), c8 = c % (DV / 8);
        const int q = min(q0 + 8 * p + rr, N - 1);
        load_row8(gv[buf][k], G + (tokb + q) * ldg + (size_t)h * DV + 8 * c8, true);
      }
    };
    gload(0, 0);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p + 1 < 4) gload(p + 1, (p + 1) & 1);
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int r = 4 * p + rq;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) stg[(4 * hh + rq) * SLD + 32 * j + lr] = (acc[j][r] - mu[r]) * rs[r];
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int c = lane + 64 * k, rr = c / (DV / 8), c8 = c % (DV / 8);
        const int q = q0 + 8 * p + rr;
        const f32x4 y0 = *reinterpret_cast<const f32x4*>(stg + rr * SLD + 8 * c8);
        const f32x4 y1 = *reinterpret_cast<const f32x4*>(stg + rr * SLD + 8 * c8 + 4);
        float g[8], z[8];
        unpack_row8(g, gv[p & 1][k]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[e] = swish_fast(g[e]) * y0[e];
          z[4 + e] = swish_fast(g[4 + e]) * y1[e];
        }
        Row8<T> o;
        pack_row8(o, z);
        if (q < N) store_row8(O + (tokb + (rev_o ? N - 1 - q : q)) * ldo + (size_t)h * DV + 8 * c8, o);
      }
      asm volatile("" ::: "memory");
    }
  } else if constexpr (GN) {
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
    // gate values RB rows at a time (raw, rows past the end clamped and never
    // stored): one round trip per RB rows instead of one per row
    constexpr int RB = DV <= 256 ? 16 : 4;
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RB) {
      typename RawElt<T>::type graw[RB][DV / 32];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int r = r0 + rr;
        const int q = min(q0 + 8 * (r >> 2) + 4 * hh + (r & 3), N - 1);
        const T* gp = G + (tokb + q) * ldg + (size_t)h * DV + lr;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) graw[rr][j] = RawElt<T>::load(gp + 32 * j);
      }
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int r = r0 + rr;
        const int q = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (q < N) {
          T* op = O + (tokb + (rev_o ? N - 1 - q : q)) * ldo + (size_t)h * DV + lr;
#pragma unroll
          for (int j = 0; j < DV / 32; ++j) {
            const float sw = swish_fast(RawElt<T>::value(graw[rr][j]));
            op[32 * j] = (T)(sw * (acc[j][r] - mu[r]) * rs[r]);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (q < N) {
        T* op = O + (tokb + (rev_o ? N - 1 - q : q)) * ldo + (size_t)h * DV + lr;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) op[32 * j] = (T)acc[j][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_chunk_dl: the bf16 output kernel with direct-to-LDS staging.
// One workgroup per (batch, head, chunk, 128-row tile), 4 waves of 32 query
// rows; each wave keeps its Q rows in registers and accumulates the full
// d_v width of its outputs.  The stages -- d_k slabs of R_{i-1}, then
// 32-key blocks of K and V up to the tile's last row -- stream through a
// ring of NS LDS slots filled by direct copies with NS - 1 stages in
// flight, so global latency overlaps the matrix-core work.
// Key blocks are software-pipelined across stages: while a wave computes
// S^T = K Q^T of block j it runs P_{j-1} V_{j-1} of the previous block, two
// independent matrix-core streams; so key stage j carries K of block j and
// V of block j - 1, and one more stage carries the last V.  Fragment reads
// run two steps ahead.
// LDS tiles are padded, in units of 16-byte slots, so that every fragment
// address is one base register plus an immediate offset and reads are
// free of bank conflicts: K and R^T rows (read row-wise, 16 rows at a time
// at the same chunk) get an odd stride in slots; V rows (read with the
// transposing read, 4 rows x 4 chunks per half-wave) a stride of 4 slots
// mod 16.  A direct copy fills 64 consecutive slots, so lanes that land on
// a pad slot copy a harmless duplicate.
// The two tiles of a chunk are dispatched to the same XCD (block ids 8
// apart) so the second reads K and V from that XCD's L2.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct DlCfg {
  static constexpr int NT = 256, RT = 128;
  static constexpr int KB = 32;                                   // keys per KV stage
  static constexpr int SK = DV <= 256 ? (DK < 64 ? DK : 64) : 32; // d_k columns per R stage
  static constexpr int CPK = DK / 8, CPV = DV / 8, CPR = SK / 8;  // 16-byte chunks per row
  static constexpr int SPK = CPK + 1, SPV = CPV + 4, SPR = CPR + 1; // padded strides (slots)
  static constexpr int r64(int x) { return (x + 63) / 64 * 64; }
  static constexpr int r4(int x) { return (x + 3) / 4 * 4; }
  static constexpr int KSL = r64(KB * SPK), VSL = r64(KB * SPV), RSL = r64(DV * SPR);  // slots
  static constexpr int IK = KSL / 64, IKV = r4((KSL + VSL) / 64), IR = r4(RSL / 64);    // 1 KiB copies
  static constexpr int LPW_KV = IKV / 4, LPW_R = IR / 4;          // copies per wave per stage
  static constexpr int STG = (IKV > IR ? IKV : IR) * 512;         // elements per ring slot
  static constexpr int NS = (150 * 1024) / (STG * 2) >= 4 ? 4 : (150 * 1024) / (STG * 2);
  static constexpr int AHEAD = NS - 1;
  static_assert(NS == 4 && AHEAD == 3, "four ring slots, three stages in flight");
  static_assert(LPW_KV == LPW_R, "equal copy counts per stage");
  // R_{i-1} itself ([d_k][d_v]) as the slab: SK rows of the V tile's stride
  static constexpr int RSLT = r64(SK * SPV);
  static_assert(RSLT / 64 <= 4 * LPW_KV, "a row slab fits the stage's copies");
};

template <int DK, int DV, bool STATE, bool GN, bool RV, bool RS>
__global__ __launch_bounds__(256) void k_chunk_dl(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, int64_t ldq, int64_t ldk,
    int64_t ldv, const bf16* __restrict__ Rx, int has_sin, const bf16* __restrict__ G, int64_t ldg,
    bf16* __restrict__ O, int64_t ldo, int BH, int N, int H, int chunk, int NC, int TPC, float scale, float eps,
    HeadTab tab, int rev) {
  // rev bit 0: output row t to row N - 1 - t; RV: Q, K, V row t from row N - 1 - t;
  // RS: Rx holds R_{i-1} itself ([DK][DV] per chunk) rather than its transpose
  const bool rev_o = rev & 1;
  constexpr bool rev_i = RV;
  using C = DlCfg<DK, DV>;
  constexpr int KB = C::KB, SK = C::SK, NS = C::NS, AHEAD = C::AHEAD, RT = C::RT;
  constexpr int CPK = C::CPK, CPV = C::CPV, CPR = C::CPR;
  __shared__ __attribute__((aligned(1024))) bf16 smem[NS * C::STG];
  (void)CPK; (void)CPV; (void)CPR;

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // block id -> (chunk unit, tile): units 8 apart in block id share an XCD;
  // a unit's tiles are consecutive groups of 8, heaviest first.
  const int U = NC * BH;
  const int xg = blockIdx.x & 7, yg = blockIdx.x >> 3;
  const int li = TPC - 1 - yg % TPC;
  const int unit = (yg / TPC) * 8 + xg;
  if (unit >= U) return;
  const int ci = unit / BH, bh = unit % BH;
  const int h = bh % H, b = bh / H;
  const int c0 = ci * chunk;
  const int r0 = c0 + li * RT;
  if (r0 >= N) return;
  const int q0 = r0 + 32 * wave;
  const bool active = q0 < N;                      // wave-uniform
  const float lg2 = tab.lg2[h];
  const size_t tokb = (size_t)b * N;

  // ---- stage list: nR slabs of R_{i-1}, then nKV key blocks ----
  const bool inter = STATE && (ci > 0 || has_sin);
  const int nR = inter ? DK / SK : 0;
  const int kend = min(r0 + RT, N);
  const int nKV = (kend - c0 + KB - 1) / KB;
  const int nst = nR + nKV + 1;                    // key stage j holds K of block j and V of block j - 1
  const bf16* Rt = STATE ? Rx + ((size_t)bh * NC + ci) * DV * DK : nullptr;
  const bf16* Kh = K + (size_t)h * DK + tokb * ldk;
  const bf16* Vh = V + (size_t)h * DV + tokb * ldv;
  const int ldk32 = (int)ldk, ldv32 = (int)ldv;
  auto slot = [&](int idx) { return smem + (idx % NS) * C::STG; };

  // Copies of stage idx by this wave: instruction ii fills slots
  // 64 ii .. 64 ii + 63 of the slot; slot u of a tile is row u / stride,
  // chunk u % stride (pad slots and slots past the tile copy chunk 0 of row
  // 0).  Keys past the end are clamped to the last row: they are in the
  // future of every stored query, so they get weight 0.  lim: the block's
  // last valid key (KB - 1 for a whole block); with rev_i key r of a block
  // is lim - r rows above the block's base (its lowest row).
  auto kv_off = [&](int t, int lim) -> uint32_t {
    const int ii = wave * C::LPW_KV + t;
    if (ii < C::IK) {
      const int u = ii * 64 + lane, row = u / C::SPK, c = u % C::SPK;
      const int r = rev_i ? lim - min(row, lim) : min(row, lim);
      return row < KB && c < CPK ? (uint32_t)((r * ldk32 + 8 * c) * 2) : 0u;
    }
    const int u = (ii - C::IK) * 64 + lane, row = u / C::SPV, c = u % C::SPV;
    const int r = rev_i ? lim - min(row, lim) : min(row, lim);
    return row < KB && c < CPV ? (uint32_t)((r * ldv32 + 8 * c) * 2) : 0u;
  };
  // Per-lane byte offsets of this wave's copies: they do not depend on the
  // stage, so they are computed once (only the sequence's last, partial key
  // block needs the clamp, computed when it comes).
  uint32_t okv[C::LPW_KV], orr[C::LPW_R];
#pragma unroll
  for (int t = 0; t < C::LPW_KV; ++t) okv[t] = kv_off(t, KB - 1);
#pragma unroll
  for (int t = 0; t < C::LPW_R; ++t) {
    const int u = (wave * C::LPW_R + t) * 64 + lane;
    if (RS) {                                      // rows of R_{i-1}: SK x DV, stride SPV
      const int row = u / C::SPV, c = u % C::SPV;
      orr[t] = row < SK && c < CPV ? (uint32_t)((row * DV + 8 * c) * 2) : 0u;
    } else {                                       // rows of R^T: DV x SK, stride SPR
      const int row = u / C::SPR, c = u % C::SPR;
      orr[t] = row < DV && c < CPR ? (uint32_t)((row * DK + 8 * c) * 2) : 0u;
    }
  }
  // The copies of one stage: wave-uniform source bases and LDS slot, and
  // this lane's offsets.  Stages past the last one copy the last stage
  // again into the free slot (unused), so that every stage issues the same
  // number of copies and the waits are fixed.
  struct Cp { const bf16* src[2]; bf16* dst; uint32_t off[C::LPW_KV]; };
  auto prep = [&](int g, Cp& c) {
    const int idx = min(g, nst - 1);
    c.dst = slot(g) + wave * C::LPW_KV * 512;
    if (idx < nR) {
      c.src[0] = c.src[1] = Rt + idx * SK * (RS ? DV : 1);
#pragma unroll
      for (int t = 0; t < C::LPW_KV; ++t) c.off[t] = orr[t];
    } else {
      // K of block j and V of block j - 1 (the first stage copies V of
      // block 0 and the last K of block nKV - 1 again: unused)
      const int j = idx - nR;
      const int kbk = c0 + min(j, nKV - 1) * KB, kbv = c0 + max(j - 1, 0) * KB;
      const int limk = min(KB - 1, N - 1 - kbk), limv = min(KB - 1, N - 1 - kbv);
      c.src[0] = Kh + (size_t)(rev_i ? N - 1 - kbk - limk : kbk) * ldk;
      c.src[1] = Vh + (size_t)(rev_i ? N - 1 - kbv - limv : kbv) * ldv;
      if (kbk + KB <= N) {                       // whole blocks (V's block is never later than K's)
#pragma unroll
        for (int t = 0; t < C::LPW_KV; ++t) c.off[t] = okv[t];
      } else {
#pragma unroll
        for (int t = 0; t < C::LPW_KV; ++t) c.off[t] = kv_off(t, wave * C::LPW_KV + t < C::IK ? limk : limv);
      }
    }
  };
  // copy t of the prepared stage (K part for the first IK copies of a key stage)
  auto cp = [&](const Cp& c, int t) {
    const int ii = wave * C::LPW_KV + t;         // wave-uniform
    copy16_to_lds(ii < C::IK ? c.src[0] : c.src[1], c.off[t], lds_addr(c.dst + t * 512));
  };
  {
    Cp c;
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) {
      prep(a, c);
#pragma unroll
      for (int t = 0; t < C::LPW_KV; ++t) cp(c, t);
    }
  }
  // Q rows as fragments (column 16 s + 8 hh + t of query row q0 + lr; rows
  // past the end clamped, never stored).
  Frag<bf16> qf[DK / 16];
  {
    const int qr = min(q0 + lr, N - 1);
    const bf16* p = Q + (tokb + (rev_i ? N - 1 - qr : qr)) * ldq + (size_t)h * DK + 8 * hh;
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) qf[s] = load_frag(p + 16 * s);
  }

  f32x16 acc[DV / 32];
#pragma unroll
  for (int j = 0; j < DV / 32; ++j) acc[j] = (f32x16){};

  // ---- Q R_{i-1} slab: acc[j] += Q[:, slab] R^T[32 j .., slab]^T; the rows
  // are scaled by scale * xi once all slabs are in (they come first) ----
  constexpr int NJ = DV / 32;
  const int g4 = lane >> 4, i4 = lane & 15, cq = g4 & 1, jj4 = i4 >> 2, q4 = i4 & 3;
  auto compute_R = [&](const bf16* sR, const Frag<bf16>* qs, const Cp& cn) {
    constexpr int T = (SK / 16) * NJ;
    static_assert(T >= C::LPW_KV, "one copy per step at most");
    const bf16* rb0 = sR + lr * (8 * C::SPR) + 8 * hh;
    // RS: the transposing read of V, on slab rows 16 s + 8 hh + 4 pp + jj4
    // (the Q fragment's column order), chunk 4 j + 2 cq + q4 / 2
    const bf16* rt0 = sR + (8 * hh + jj4) * (8 * C::SPV) + 8 * (2 * cq + (q4 >> 1)) + 4 * (q4 & 1);
    auto rd = [&](int t) {
      const int s = t / NJ, j = t % NJ;            // R^T row 32 j + lr, chunk 2 s + hh
      if constexpr (RS) {
        Frag<bf16> f;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const bf16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(const lds_char*)(rt0 + (16 * s + 4 * pp) * (8 * C::SPV) +
                                                                            32 * j));
#pragma unroll
          for (int e = 0; e < 4; ++e) f.v[4 * pp + e] = r4[e];
        }
        return f;
      } else {
        return load_frag(rb0 + j * (32 * 8 * C::SPR) + 16 * s);
      }
    };
    Frag<bf16> rb[3];
    rb[0] = rd(0);
    if (T > 1) rb[1] = rd(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (t + 2 < T) rb[(t + 2) % 3] = rd(t + 2);
      mma16(acc[t % NJ], qs[t / NJ], rb[t % 3]);
      if (t < C::LPW_KV) cp(cn, t);              // next stages' copies between the MFMAs
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      if (t + 2 < T) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, RS ? 2 : 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // acc rows (register r: query q0 + kk(r)) times scale * xi_t = scale * gamma^(t + 1)
  auto scale_rows_xi = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = scale * gpow(q0 - c0 + 8 * (r >> 2) + 4 * hh + (r & 3) + 1, lg2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j][r] *= x;
    }
  };

  // ---- key blocks ----
  // S^T = K Q^T: lane = query q0 + lr, register r = key kb + kk(r).
  // P V uses the accumulator as the A operand; V fragments are read in that
  // key order (transposing read).
  constexpr int NSS = DK / 16, NPV = DV / 16, TKV = NSS > NPV ? NSS : NPV;
  const int kofs = lr * (8 * C::SPK) + 8 * hh;    // K: row lr, chunk 2 t + hh
  const int vofs = (4 * hh + jj4) * (8 * C::SPV) + 8 * (2 * cq + (q4 >> 1)) + 4 * (q4 & 1);
  auto rdK = [&](const bf16* sK, int t) { return load_frag(sK + kofs + 16 * t); };
  // V: rows 16 s2 + 8 pp + 4 hh + jj4, chunk 4 j + 2 cq + q4 / 2 (+ 4 elements for odd q4)
  auto rdV = [&](const bf16* sV, int t) {
    const int j = t >> 1, s2 = t & 1;
    Frag<bf16> f;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const bf16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(const lds_char*)(sV + vofs + (16 * s2 + 8 * pp) * (8 * C::SPV) +
                                                                        32 * j));
#pragma unroll
      for (int e = 0; e < 4; ++e) f.v[4 * pp + e] = r4[e];
    }
    return f;
  };
  // One pipelined key step: S^T of the block in slot sK and P V of the
  // pending block (P in pa, V in slot sVp), then P of the new block.  Every
  // wave runs both matrix-core streams on every step -- P is zero for a
  // block in the wave's future and when nothing is pending -- so there is a
  // single code path for the accumulators; the waves meet at every stage
  // and each has its own SIMD, so the idle ones cost no time.
  Frag<bf16> pa[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) pa[0].v[e] = pa[1].v[e] = (bf16)0.0f;
  float wm[16];                                    // gamma^(27 - m_r), m_r = 8 (r/4) + r%4 (wave-uniform)
#pragma unroll
  for (int r = 0; r < 16; ++r)
    wm[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gpow(27 - (8 * (r >> 2) + (r & 3)), lg2))));
  static_assert(NSS >= 2 && NPV >= 4, "pipelined key step");
  static_assert(NSS >= C::LPW_KV, "one copy per step at most");
  auto kv_step = [&](const bf16* sK, const bf16* sVp, int kb, bool now, const Cp& cn) {
    constexpr int H1 = NPV / 2;                    // P V steps in region A
    f32x16 st = (f32x16){};
    Frag<bf16> kq[3], vq[3];
    kq[0] = rdK(sK, 0);
    kq[1] = rdK(sK, 1);
    vq[0] = rdV(sVp, 0);
    vq[1] = rdV(sVp, 1);
    __builtin_amdgcn_sched_barrier(0);
    // region A: every S^T step, the first half of P V, reads two steps ahead
#pragma unroll
    for (int t = 0; t < NSS; ++t) {
      if (t + 2 < NSS) kq[(t + 2) % 3] = rdK(sK, t + 2);
      mma16(st, kq[t % 3], qf[t]);
      if (t < C::LPW_KV) cp(cn, t);              // next stages' copies between the MFMAs
      if (t < H1) {
        if (t + 2 < NPV) vq[(t + 2) % 3] = rdV(sVp, t + 2);
        mma16(acc[t >> 1], pa[t & 1], vq[t % 3]);
      }
    }
#pragma unroll
    for (int t = 0; t < NSS; ++t) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      if (t + 2 < NSS) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      if (t < H1) {
        if (t + 2 < NPV) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // region B: the rest of P V with the decay of the new block between its
    // MFMAs.  D[query, key] = gamma^(query - key) for key <= query, with
    // query - key = n0 - m_r; off the diagonal block n0 >= 28 and
    // gamma^(n0 - m_r) = u * w_r, u = gamma^(n0 - 27), w_r = gamma^(27 - m_r)
    // (both exponents >= 0).
    const int n0 = q0 - kb + lr - 4 * hh;
    const float u = now ? scale * gpow(n0 - 27, lg2) : 0.0f;
    float p[16];
#pragma unroll
    for (int t = H1; t < NPV; ++t) {
      if (t + 2 < NPV) vq[(t + 2) % 3] = rdV(sVp, t + 2);
      mma16(acc[t >> 1], pa[t & 1], vq[t % 3]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = st[r] * (u * wm[r]);
#pragma unroll
    for (int t = H1; t < NPV; ++t) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      if (t + 2 < NPV) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, 6, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kb == q0) {                                // the diagonal block: key <= query only
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 - (8 * (r >> 2) + (r & 3));
        float e = exp2f((float)max(n, 0) * lg2);
        e = n == 0 ? 1.0f : e;
        p[r] = (now && n >= 0) ? st[r] * scale * e : 0.0f;
      }
    }
    pa[0] = frag_from<bf16>(p);
    pa[1] = frag_from<bf16>(p + 8);
  };

  // Make the compiler retire the Q loads here (together with the copies
  // issued before them, which complete first): a wait for them left inside
  // the loop would drain the copies in flight on every stage.
#pragma unroll
  for (int s = 0; s < DK / 16; ++s) asm volatile("" ::"v"(qf[s].v));
  // wait for stage idx's copies, then prepare those of stage idx + AHEAD
  // into the slot of stage idx - 1, which every wave is past; they are
  // issued between the MFMAs of stage idx
  // (the copies of the two stages after idx may stay in flight)
  Cp cn;
  auto advance = [&](int idx) {
    copies_wait_barrier<2 * C::LPW_KV>();
    prep(idx + AHEAD, cn);
  };
  // R slabs, then the rows scaled by scale * xi (outside both loops: VALU
  // work on the accumulators inside a loop would keep them out of the
  // accumulation registers there), then the key stages.
  int idx = 0;
  for (; idx < nR; ++idx) {
    advance(idx);
    // the slab's Q fragments, picked with static indices only (a dynamic
    // index would move qf to scratch memory)
    Frag<bf16> qs[SK / 16];
#pragma unroll
    for (int s2 = 0; s2 < SK / 16; ++s2) qs[s2] = qf[s2];
    static_for<DK / SK>([&](auto sl) {
      if (decltype(sl)::value > 0 && idx == decltype(sl)::value) {
#pragma unroll
        for (int s2 = 0; s2 < SK / 16; ++s2) qs[s2] = qf[decltype(sl)::value * (SK / 16) + s2];
      }
    });
    compute_R(slot(idx), qs, cn);
  }
  if (nR > 0) scale_rows_xi();
  for (; idx < nst; ++idx) {
    advance(idx);
    const int j = idx - nR;
    const int kb = c0 + j * KB;
    const bool now = j < nKV && active && kb <= q0;   // wave-uniform
    // S of block j (discarded when not now) and P_{j-1} V_{j-1} (P = 0 on
    // the first key stage)
    kv_step(slot(idx), slot(idx) + C::KSL * 8, kb, now, cn);
  }
  copies_wait_barrier<0>();                        // no copy may land after the workgroup ends

  // ---- epilogue: lane owns column 32 j + lr of rows q0 + 8 (r/4) + 4 hh + r%4 ----
  if (!active) return;
  if constexpr (GN) {
    // the gate values of all 16 rows first (raw, rows past the end clamped
    // to the last row and never stored): one round trip, overlapped with the
    // row statistics, instead of one per row
    typename RawElt<bf16>::type graw[16][DV / 32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = min(q0 + 8 * (r >> 2) + 4 * hh + (r & 3), N - 1);
      const bf16* gp = G + (tokb + qq) * ldg + (size_t)h * DV + lr;
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) graw[r][j] = RawElt<bf16>::load(gp + 32 * j);
    }
    float mu[16], rs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) sum += acc[j][r];
      mu[r] = half_wave_sum(sum) * (1.0f / DV);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < DV / 32; ++j) {
        const float dlt = acc[j][r] - mu[r];
        sum += dlt * dlt;
      }
      rs[r] = rsqrtf(half_wave_sum(sum) * (1.0f / DV) + eps);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (qq < N) {
        bf16* op = O + (tokb + (rev_o ? N - 1 - qq : qq)) * ldo + (size_t)h * DV + lr;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) {
          const float sw = swish_fast(RawElt<bf16>::value(graw[r][j]));
          op[32 * j] = (bf16)(sw * (acc[j][r] - mu[r]) * rs[r]);
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (qq < N) {
        bf16* op = O + (tokb + (rev_o ? N - 1 - qq : qq)) * ldo + (size_t)h * DV + lr;
#pragma unroll
        for (int j = 0; j < DV / 32; ++j) op[32 * j] = (bf16)acc[j][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <int DK, int DV, bool STATE>
static void launch_dl(const ChunkArgs& a, int chunk, int NC, int TPC, int has_sin, const HeadTab& tab,
                      hipStream_t st) {
  const int BH = a.batch * a.heads;
  const int U = NC * BH;
  dim3 grid(((U + 7) / 8) * 8 * TPC);
  // the reversed reads (the backward's passes: no fused GroupNorm) are a
  // compile-time variant, so the forward kernels carry none of their logic
  if (a.fuse_gn_gate)
    hipLaunchKernelGGL((k_chunk_dl<DK, DV, STATE, true, false, false>), grid, dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx, has_sin,
                       (const bf16*)a.G, a.ldg, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC, a.scale,
                       a.eps, tab, a.rev_out ? 1 : 0);
  else if (STATE && a.rx_kv && !a.rev_in)
    hipLaunchKernelGGL((k_chunk_dl<DK, DV, STATE, false, false, STATE>), grid, dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx, has_sin,
                       (const bf16*)nullptr, (int64_t)0, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC,
                       a.scale, a.eps, tab, a.rev_out ? 1 : 0);
  else if (STATE && a.rx_kv)
    hipLaunchKernelGGL((k_chunk_dl<DK, DV, STATE, false, true, STATE>), grid, dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx, has_sin,
                       (const bf16*)nullptr, (int64_t)0, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC,
                       a.scale, a.eps, tab, a.rev_out ? 1 : 0);
  else if (a.rev_in)
    hipLaunchKernelGGL((k_chunk_dl<DK, DV, STATE, false, true, false>), grid, dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx, has_sin,
                       (const bf16*)nullptr, (int64_t)0, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC,
                       a.scale, a.eps, tab, a.rev_out ? 1 : 0);
  else
    hipLaunchKernelGGL((k_chunk_dl<DK, DV, STATE, false, false, false>), grid, dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx, has_sin,
                       (const bf16*)nullptr, (int64_t)0, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC,
                       a.scale, a.eps, tab, a.rev_out ? 1 : 0);
}

template <class T, int DK, int DV, int NW, bool STATE>
static void launch_out(const ChunkArgs& a, int chunk, int NC, int TPC, int has_sin, const HeadTab& tab,
                       hipStream_t st) {
  const int BH = a.batch * a.heads;
  dim3 grid(TPC * NC * BH);
  if (a.fuse_gn_gate)
    hipLaunchKernelGGL((k_chunk_out<T, DK, DV, NW, STATE, true>), grid, dim3(64 * NW), 0, st, (const T*)a.Q,
                       (const T*)a.K, (const T*)a.V, a.ldq, a.ldk, a.ldv, (const T*)a.Rx, has_sin, (const T*)a.G,
                       a.ldg, (T*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC, a.scale, a.eps, tab,
                       (a.rev_out ? 1 : 0) | (a.rev_in ? 2 : 0), a.q_rope_tab);
  else
    hipLaunchKernelGGL((k_chunk_out<T, DK, DV, NW, STATE, false>), grid, dim3(64 * NW), 0, st, (const T*)a.Q,
                       (const T*)a.K, (const T*)a.V, a.ldq, a.ldk, a.ldv, (const T*)a.Rx, has_sin,
                       (const T*)nullptr, (int64_t)0, (T*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC,
                       a.scale, a.eps, tab, (a.rev_out ? 1 : 0) | (a.rev_in ? 2 : 0), a.q_rope_tab);
}

template <class T, int DK, int DV>
static hipError_t run_chunkwise(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  const int B = a.batch, N = a.seqlen, H = a.heads, Cn = a.chunk;
  const int NC = (N + Cn - 1) / Cn;
  const int BH = B * H;
  constexpr int TS = StateCfg<T, DK, DV>::TS;
  HeadScale so;
  for (int h = 0; h < H; ++h) so.c[h] = a.sout_scale ? a.sout_scale[h] : 1.0f;
  if (!a.reuse_rx && !a.k_rope_tab && chunk_rscan_ok(a.elt, DK, DV, Cn, BH)) {
    // every chunk's R_{i-1} in one pass over the keys
    TraceScope ts("k_chunk_rscan", st);
    const hipError_t err = launch_chunk_rscan(a, tab, so, st);
    if (err != hipSuccess) return err;
  } else if (!a.reuse_rx) {
  {
    TraceScope ts("k_chunk_state", st);
    dim3 grid(((BH * NC + 7) / 8) * 8 * (DV / TS) * (DK / TS));
    if (a.rev_in)
      hipLaunchKernelGGL((k_chunk_state<T, DK, DV, true>), grid, dim3(256), 0, st, (const T*)a.K, (const T*)a.V,
                         a.ldk, a.ldv, (T*)a.dR, BH, N, H, Cn, NC, tab, (const float2*)nullptr, (T*)nullptr,
                         (int64_t)0);
    else
      hipLaunchKernelGGL((k_chunk_state<T, DK, DV, false>), grid, dim3(256), 0, st, (const T*)a.K, (const T*)a.V,
                         a.ldk, a.ldv, (T*)a.dR, BH, N, H, Cn, NC, tab, a.k_rope_tab, (T*)a.k_rot, a.ld_k_rot);
  }
  {
    TraceScope ts("k_chunk_scan", st);
    // few (batch, head) pairs (one long sequence per head): 16 x 64 tiles, so
    // that enough workgroups walk the chunks
    if (DK >= 64 && DV >= 64 && BH * (DV / 64) * (DK / 64) >= 1024) {
      dim3 grid(BH * (DV / 64) * (DK / 64));
      hipLaunchKernelGGL((k_chunk_scan<T, DK, DV, 64, 64>), grid, dim3(256), 0, st, (const T*)a.dR, (T*)a.Rx,
                         a.S_in, a.S_out, H, NC, tab, so);
    } else {
      dim3 grid(BH * (DV / 16) * (DK / 64));
      hipLaunchKernelGGL((k_chunk_scan<T, DK, DV, 16, 64>), grid, dim3(256), 0, st, (const T*)a.dR, (T*)a.Rx,
                         a.S_in, a.S_out, H, NC, tab, so);
    }
  }
  }
  {
    TraceScope ts("k_chunk_out", st);
    const int has_sin = a.reuse_rx ? (int)a.reuse_seeded : (int)(a.S_in != nullptr);
    ChunkArgs ao = a;                                // the output kernel reads the rotated K rows
    if (a.k_rope_tab) { ao.K = a.k_rot; ao.ldk = a.ld_k_rot; }
    // (reversed reads come with reversed writes: the backward's passes,
    // which rotate Q and K beforehand)
    if (chunk_out_o16(a.elt, DK, DV, Cn) && a.rev_in == a.rev_out && !a.rx_kv && !(a.rev_in && a.q_rope_tab))
      return launch_out_o16(ao, true, Cn, NC, Cn / 128, has_sin, tab, st);
    if constexpr (sizeof(T) == 2 && DV <= 256) {
      if (Cn % 128 == 0) {
        if (a.q_rope_tab) return hipErrorInvalidValue;   // this kernel does not rotate Q
        launch_dl<DK, DV, true>(ao, Cn, NC, Cn / 128, has_sin, tab, st);
        return hipGetLastError();
      }
    }
    if (Cn % 128 == 0)
      launch_out<T, DK, DV, 4, true>(ao, Cn, NC, Cn / 128, has_sin, tab, st);
    else
      launch_out<T, DK, DV, 1, true>(ao, Cn, NC, Cn / 32, has_sin, tab, st);
  }
  return hipGetLastError();
}

template <class T, int DK, int DV>
static hipError_t run_parallel(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  const int TPC = (a.seqlen + 127) / 128;
  TraceScope ts("k_chunk_out", st);
  // the 16-rows-per-wave kernel for the 512-wide value heads, and for d_v
  // 256 up to 32 row tiles (4096 tokens): longer single chunks are mostly
  // matrix-core steps, where the 32-row kernel of d_v <= 256 is the faster
  // one (at d_v 256, b2 x 10 heads: 41 / 82 / 274 us against 46 / 97 / 281 us
  // at 1024 / 2048 / 4096 tokens, 3554 against 3111 us at 16384)
  if (chunk_out_o16(a.elt, DK, DV, TPC * 128) && (DV > 256 || TPC <= 32) && !a.rev_in && !a.rev_out)
    return launch_out_o16(a, false, TPC * 128, 1, TPC, 0, tab, st);
  if (a.q_rope_tab && sizeof(T) == 2 && DV <= 256) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2 && DV <= 256)
    launch_dl<DK, DV, false>(a, TPC * 128, 1, TPC, 0, tab, st);
  else
    launch_out<T, DK, DV, 4, false>(a, TPC * 128, 1, TPC, 0, tab, st);
  return hipGetLastError();
}

#define MSR_DISPATCH_DIMS(FN, T, ...)                                           \
  if (a.d_k == 64 && a.d_v == 64) return FN<T, 64, 64>(__VA_ARGS__);            \
  if (a.d_k == 128 && a.d_v == 128) return FN<T, 128, 128>(__VA_ARGS__);        \
  if (a.d_k == 256 && a.d_v == 256) return FN<T, 256, 256>(__VA_ARGS__);

bool chunk_out_rotates_q(Elt elt, int d_k, int d_v, int chunk) {
  if (chunk_out_o16(elt, d_k, d_v, chunk)) return true;
  return !(elt == kBF16 && d_v <= 256 && chunk % 128 == 0);
}

bool chunk_out_direct(Elt elt, int d_k, int d_v, int chunk) {
  const bool dims = (d_k == 64 && d_v == 64) || (d_k == 128 && d_v == 128) || (d_k == 256 && d_v == 256);
  return elt == kBF16 && dims && chunk % 128 == 0;
}

hipError_t launch_chunkwise(const ChunkArgs& a, const HeadTab& tab, hipStream_t st) {
  if (a.fuse_gn_gate && a.rev_in) return hipErrorInvalidValue;   // no reversed variant of the fused epilogue
  // R_{i-1} itself in Rx: only stored states (no scan writing the transpose),
  // read by the direct-copy output kernel
  if (a.rx_kv && !(a.reuse_rx && !a.fuse_gn_gate && chunk_out_direct(a.elt, a.d_k, a.d_v, a.chunk)))
    return hipErrorInvalidValue;
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
