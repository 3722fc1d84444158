// Per-chunk states of chunkwise retention in one pass, bf16, on the gfx950
// matrix cores.
//
// Method ([RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、
// 速度快、性能強（2）", section "3) Retention 分塊循環表征", Eq. (7)): with chunks
// of B tokens (the last may be short, length L) and s the key index inside
// a chunk,
//   R_i = gamma^L R_{i-1} + K_[i]^T (V_[i] (.) zeta),  zeta_s = gamma^(L-1-s),
// R_{-1} = the initial state (or zero).  The output kernel needs every
// R_{i-1}; they are stored transposed, [d_v][d_k] per chunk, in bf16.  The
// reversed variant (REV, the backward's anti-causal passes) runs on the
// time-reversed sequence: key t is read from row N - 1 - t.
//
// One workgroup (8 waves, two per SIMD) owns a TK x TV tile of the state of one (batch,
// head) and walks its chunks in order with the tile in float32 matrix-core
// accumulators: before a chunk's first key block it stores the tile as that
// chunk's R_{i-1}, multiplies it by gamma^L, then adds the chunk's keys.  The
// state never goes through memory in between (the two-kernel form writes
// each chunk's own contribution and reads it back for the scan).  The tiles
// of one (batch, head) run on one XCD (workgroup ids 8 apart), so the K rows
// they all read come from HBM once and from that XCD's L2 after.
//
// Key blocks of 32 keys (K columns of the tile, then V columns) stream into
// a ring of LDS slots (144 KiB) by direct global->LDS copies, all but two
// slots in flight; each block's V rows are scaled by zeta in place (every
// thread a few 16-byte pieces) while the matrix cores work on the block
// before it, and the matrix cores read both operands with the transposing
// LDS read.  One barrier per block.  The product is computed as
// R^T-tile-transposed, i.e. D[dk][dv] = sum_keys K[key][dk] V[key][dv], so
// the A operand is K (d_k rows of 32) and the B operand V.  Rows are stored
// unpadded; 16-byte chunk c of row r sits at c ^ swz(r) with swz(r) = 4 (r &
// 3) (rows of 256 bytes or more) or 4 ((r >> 1) & 1) (128-byte rows), so
// that the four key rows one transposing read serves fall on four different
// 64-byte bank groups.
#include "msr_launch.h"

namespace msr {

namespace {

template <int TK, int TV>
struct RsCfg {
  // keys per block: 64 where four slots of them fit with the staging area
  // (fewer, longer blocks: the fixed cost per block is a barrier and the
  // fragment-read latency), else 32
  static constexpr int KB = TK * TV <= 128 * 128 ? 64 : 32;
  static constexpr int CPK = TK / 8, CPV = TV / 8;     // 16-byte chunks per K / V row of the tile
  static constexpr int KCH = KB * CPK, VCH = KB * CPV; // chunks per block
  static constexpr int NCP = (KCH + VCH) / 64;         // 1 KiB copies per block
  static constexpr int NWV = 8;                        // waves: 4 along d_k x 2 along d_v, two per SIMD
  static constexpr int CPW = NCP / NWV;                // copies per wave
  static constexpr int STG = NCP * 1024;               // bytes per ring slot
  // ring slots: one block being multiplied, one being scaled, the rest in
  // flight (a deeper ring measured slower)
  static constexpr int NS = 4;
  static constexpr int WTM = TK / 128, WTN = TV / 64;  // 32x32 tiles per wave (d_k, d_v)
  static constexpr int VPT = VCH / (64 * NWV);         // V chunks per thread in the scaling pass
  static_assert(NCP % NWV == 0 && KCH % 64 == 0 && VCH % (64 * NWV) == 0 && WTM >= 1, "whole copies per wave");
  static_assert(CPK >= 16 && CPV >= 8, "rows of at least 256 (K) and 128 (V) bytes");
  // staging of the state tile on its way out: per wave one 32-row (d_v)
  // slice of its TK / 4 d_k columns at a time, rows padded by 16 bytes
  static constexpr int SROW = TK / 2 + 16;             // bytes per staged row
  static constexpr int SWAVE = 32 * SROW;              // bytes per wave
  static_assert(NS >= 3 && NS * STG + NWV * SWAVE <= 160 * 1024, "ring and staging fit in LDS");
};

template <int CPR>
__device__ __forceinline__ uint32_t rs_swz(uint32_t r) {
  return CPR >= 16 ? 4u * (r & 3u) : 4u * ((r >> 1) & 1u);
}

__device__ __forceinline__ const void* rs_uniform(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef uint32_t rs_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) rs_u32x4 lds_u32x4_t;
typedef uint32_t rs_u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) rs_u32x2 lds_u32x2_t;

}  // namespace

template <int DK, int DV, int TK, int TV, bool REV>
__global__ __launch_bounds__(512) void k_chunk_rscan(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                     int64_t ldk, int64_t ldv, bf16* __restrict__ Rx,
                                                     const float* __restrict__ S_in, float* __restrict__ S_out,
                                                     HeadScale so, int BH, int N, int H, int chunk, int NC,
                                                     HeadTab tab) {
  using C = RsCfg<TK, TV>;
  constexpr int KB = C::KB, NS = C::NS, CPW = C::CPW, WTM = C::WTM, WTN = C::WTN;
  constexpr int CPK = C::CPK, CPV = C::CPV, KCH = C::KCH;
  __shared__ __attribute__((aligned(1024))) char smem[NS * C::STG + C::NWV * C::SWAVE];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;           // wave's d_k quarter, d_v half of the tile
  constexpr int NTV = DV / TV, NT = NTV * (DK / TK);
  const int xg = blockIdx.x & 7, yg = blockIdx.x >> 3;
  const int tile = yg % NT, bh = (yg / NT) * 8 + xg;
  if (bh >= BH) return;                              // uniform
  const int tv = tile % NTV, tk = tile / NTV;
  const int h = bh % H, b = bh / H;
  const float lg2f = fmaxf(tab.lg2[h], -1.0e30f);    // log2(0) = -inf made finite: 0^0 = 1, 0^n = 0
  const int NB = (N + KB - 1) / KB;                  // key blocks of the sequence

  const bf16* Kb = K + (size_t)b * N * ldk + (size_t)h * DK + tk * TK;
  const bf16* Vb = V + (size_t)b * N * ldv + (size_t)h * DV + tv * TV;

  // ---- copies: copy t of this wave fills 16-byte slots 64 (CPW wave + t) +
  // lane of a block, K's chunks first.  Per lane, the key row and the byte
  // offset of the source chunk in it (rows past the sequence end are
  // clamped to its last row; their zeta is 0). ----
  uint32_t crow[CPW], ccol[CPW];
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int idx = wave * CPW + t;                  // uniform
    if (idx < KCH / 64) {
      const uint32_t s = (uint32_t)(idx * 64 + lane), r = s / CPK, pc = s % CPK;
      crow[t] = r;
      ccol[t] = 16u * (pc ^ rs_swz<CPK>(r));
    } else {
      const uint32_t s = (uint32_t)((idx - KCH / 64) * 64 + lane), r = s / CPV, pc = s % CPV;
      crow[t] = r;
      ccol[t] = 16u * (pc ^ rs_swz<CPV>(r));
    }
  }
  // (reversed: key kb + r of the block is row N - 1 - kb - r, i.e. lim - r
  // rows after the block's lowest row in memory)
  auto issue = [&](int n) {                          // copies of key block n (clamped) into its slot
    const int nb = min(n, NB - 1), kb = nb * KB;
    const uint32_t lim = (uint32_t)min(KB - 1, N - 1 - kb);
    const uint32_t row0 = (uint32_t)(REV ? N - 1 - kb - (int)lim : kb);
    const uint32_t slot = (uint32_t)(uintptr_t)(lds + (n % NS) * C::STG);
#pragma unroll
    for (int t = 0; t < CPW; ++t) {
      const int idx = wave * CPW + t;
      const bool isk = idx < KCH / 64;
      const uint32_t ld = (uint32_t)(isk ? ldk : ldv);
      // 32 x 32-bit row products, and the lane's row (< 64) times the byte
      // stride on the 24-bit multiplier (strides stay below 2^20 bytes)
      const bf16* base = (isk ? Kb : Vb) + (uint64_t)row0 * ld;
      const uint32_t r = REV ? lim - min(crow[t], lim) : min(crow[t], lim);
      copy16_to_lds(rs_uniform(base), __umul24(r, 2u * ld) + ccol[t],
                    __builtin_amdgcn_readfirstlane(slot + (uint32_t)idx * 1024u));
    }
  };

  // ---- accumulators: tile (i, j) of this wave holds, in lane lr + 32 hh,
  // register r, D[dkw + 32 i + 8 (r / 4) + 4 hh + r % 4][dvw + 32 j + lr] ----
  f32x16 acc[WTM][WTN];
  const int dkw = tk * TK + wm * (TK / 4), dvw = tv * TV + wn * (TV / 2);
  if (S_in != nullptr) {                             // S_in [dk][dv] float32
    const float* sp = S_in + (size_t)bh * DK * DV;
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] = sp[(size_t)(dkw + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3)) * DV + dvw + 32 * j + lr];
  } else {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j) acc[i][j] = (f32x16){};
  }

  // transposing-read offsets (bytes within a slot) of this lane: key row
  // 8 hh + 4 p + jr of a 16-key step, columns 16 c + 4 q of a 32-column
  // group (lane = 32 hh + 16 c + 4 jr + q), swizzled by the row (which
  // only depends on jr)
  const int c16 = (lane >> 4) & 1, jr = (lane >> 2) & 3, q4 = lane & 3;
  const uint32_t kswz = rs_swz<CPK>((uint32_t)jr), vswz = rs_swz<CPV>((uint32_t)jr);
  uint32_t ka[WTM], vb[WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
    ka[i] = (uint32_t)((8 * hh + jr) * (TK * 2)) +
            16u * ((((uint32_t)(wm * (TK / 4) + 32 * i) >> 3) ^ kswz) + 2 * c16 + (q4 >> 1)) + 8u * (q4 & 1);
#pragma unroll
  for (int j = 0; j < WTN; ++j)
    vb[j] = (uint32_t)(KCH * 16) + (uint32_t)((8 * hh + jr) * (TV * 2)) +
            16u * ((((uint32_t)(wn * (TV / 2) + 32 * j) >> 3) ^ vswz) + 2 * c16 + (q4 >> 1)) + 8u * (q4 & 1);

  // scale block m's V rows by zeta_s = gamma^(L - 1 - s) in place (s = key
  // index in its chunk; keys past the sequence end: 0)
  auto scale_v = [&](int m, int c0) {               // c0: first key of block m's chunk
    const int kb = m * KB, L = min(chunk, N - c0);
    lds_char* sl = lds + (m % NS) * C::STG;
#pragma unroll
    for (int v = 0; v < C::VPT; ++v) {
      const int s = tid + 64 * C::NWV * v, r = s / CPV;
      const float z = kb + r < N ? __builtin_amdgcn_exp2f((float)(L - 1 - (kb - c0 + r)) * lg2f) : 0.0f;
      lds_u32x4_t* p = (lds_u32x4_t*)(sl + KCH * 16 + 16 * s);
      rs_u32x4 w = *p;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16(bf16_lo(w[e]) * z, bf16_hi(w[e]) * z);
      *p = w;
    }
  };

  // Pipeline: blocks 0 .. NS - 2 in flight, block 0 scaled; then per block
  // n one barrier, after which block n is scaled (by every wave), block
  // n + 1 has landed and every wave is done with block n - 1, whose slot
  // takes block n + NS - 1.  Block n's products then run while block n + 1
  // is scaled.
#pragma unroll
  for (int a = 0; a < NS - 1; ++a) issue(a);
  copies_wait_barrier<(NS - 2) * CPW>();
  scale_v(0, 0);

  // chunk index and first key of the current block, stepped (a chunk is a
  // whole number of blocks) rather than divided per block
  int ci = 0, c0 = 0;
  for (int n = 0; n < NB; ++n) {
    const int kb = n * KB;
    if (kb == c0 + chunk) { ++ci; c0 += chunk; }     // uniform
    lds_char* sl = lds + (n % NS) * C::STG;
    copies_wait_barrier<(NS - 3) * CPW>();
    issue(n + NS - 1);

    // a chunk's first block: the tile is R_{ci-1}; store it, then decay it
    // by gamma^L of this chunk
    if (kb == c0) {                                  // uniform
      // Rx[dv][dk] rows: each 32-column d_v tile j of the wave goes through
      // its staging area ([32 dv][TK / 4 dk] bf16), then out as whole
      // 16-byte pieces of TK-byte row segments
      bf16* rp = Rx + ((size_t)bh * NC + ci) * DV * DK;
      lds_char* stg = lds + NS * C::STG + wave * C::SWAVE;
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            rs_u32x2 w;
            w[0] = pack_bf16(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]);
            w[1] = pack_bf16(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
            *(lds_u32x2_t*)(stg + lr * C::SROW + 2 * (32 * i + 8 * r4 + 4 * hh)) = w;
          }
        asm volatile("" ::: "memory");
        constexpr int CPR = TK / 32;                 // 16-byte pieces per staged row
#pragma unroll
        for (int u = 0; u < 32 * CPR / 64; ++u) {
          const int id = lane + 64 * u, row = id / CPR, pc = id % CPR;
          const rs_u32x4 w = *(const lds_u32x4_t*)(stg + row * C::SROW + 16 * pc);
          *reinterpret_cast<rs_u32x4*>(rp + (size_t)(dvw + 32 * j + row) * DK + dkw + 8 * pc) = w;
        }
        asm volatile("" ::: "memory");
      }
      const float gL = ci == NC - 1 ? tab.glast[h] : tab.gchunk[h];
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= gL;
    }

    // acc[i][j] += K[keys][dk tile i]^T V[keys][dv tile j] over the block's
    // 16-key steps, with block n + 1's scaling after the first
#pragma unroll
    for (int ks = 0; ks < KB / 16; ++ks) {
      Frag<bf16> af[WTM], bfr[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const bf16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)(sl + ka[i] + (16 * ks + 4 * p) * (TK * 2)));
#pragma unroll
          for (int e = 0; e < 4; ++e) af[i].v[4 * p + e] = r4[e];
        }
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const bf16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)(sl + vb[j] + (16 * ks + 4 * p) * (TV * 2)));
#pragma unroll
          for (int e = 0; e < 4; ++e) bfr[j].v[4 * p + e] = r4[e];
        }
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) mma16(acc[i][j], af[i], bfr[j]);
      if (ks == 0 && n + 1 < NB) scale_v(n + 1, kb + KB == c0 + chunk ? c0 + chunk : c0);   // uniform
    }
  }

  if (S_out != nullptr) {                            // final state R_{NC-1}, [dk][dv] float32, times c_h
    float* op = S_out + (size_t)bh * DK * DV;
    const float c = so.c[h];
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          op[(size_t)(dkw + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3)) * DV + dvw + 32 * j + lr] = c * acc[i][j][r];
  }
  copies_wait_barrier<0>();                          // no copy may land after the workgroup ends
}

// Shapes with enough (batch, head) pairs for about 200 workgroups of
// 128 x 128 tiles or larger; with fewer, each workgroup's walk over the
// chunks is long and serial, and the two-kernel form (state kernel parallel
// over chunks, then the scan) is the faster one.
bool chunk_rscan_ok(Elt elt, int dk, int dv, int chunk, int bh) {
  return elt == kBF16 && ((dk == 128 && dv == 128) || (dk == 256 && (dv == 256 || dv == 512))) &&
         chunk % 64 == 0 && bh * (dk / 128) * (dv / 128) >= 192;
}

template <int DK, int DV, int TK, int TV>
static void launch_rs_t(const ChunkArgs& a, int NC, const HeadTab& tab, const HeadScale& so, hipStream_t st) {
  const int BH = a.batch * a.heads;
  constexpr int NT = (DK / TK) * (DV / TV);
  dim3 grid(((BH + 7) / 8) * 8 * NT);
  if (a.rev_in)
    hipLaunchKernelGGL((k_chunk_rscan<DK, DV, TK, TV, true>), grid, dim3(64 * RsCfg<TK, TV>::NWV), 0, st,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldk, a.ldv, (bf16*)a.Rx, a.S_in, a.S_out, so, BH,
                       a.seqlen, a.heads, a.chunk, NC, tab);
  else
    hipLaunchKernelGGL((k_chunk_rscan<DK, DV, TK, TV, false>), grid, dim3(64 * RsCfg<TK, TV>::NWV), 0, st,
                       (const bf16*)a.K, (const bf16*)a.V, a.ldk, a.ldv, (bf16*)a.Rx, a.S_in, a.S_out, so, BH,
                       a.seqlen, a.heads, a.chunk, NC, tab);
}

// Tile: 256 x 128 (d_k x d_v) where that still gives about 200 workgroups,
// else 128 x 128.
template <int DK, int DV>
static void launch_rs_d(const ChunkArgs& a, int NC, const HeadTab& tab, const HeadScale& so, hipStream_t st) {
  const int BH = a.batch * a.heads;
  if constexpr (DK == 256) {
    if (BH * (DV / 128) >= 192) return launch_rs_t<DK, DV, 256, 128>(a, NC, tab, so, st);
  }
  launch_rs_t<DK, DV, 128, 128>(a, NC, tab, so, st);
}

hipError_t launch_chunk_rscan(const ChunkArgs& a, const HeadTab& tab, const HeadScale& so, hipStream_t st) {
  const int NC = (a.seqlen + a.chunk - 1) / a.chunk;
  if (!chunk_rscan_ok(a.elt, a.d_k, a.d_v, a.chunk, a.batch * a.heads)) return hipErrorInvalidValue;
#define MSR_RS(DK_, DV_) \
  if (a.d_k == DK_ && a.d_v == DV_) { launch_rs_d<DK_, DV_>(a, NC, tab, so, st); return hipGetLastError(); }
  MSR_RS(128, 128) MSR_RS(256, 256) MSR_RS(256, 512)
#undef MSR_RS
  return hipErrorInvalidValue;
}

}  // namespace msr
