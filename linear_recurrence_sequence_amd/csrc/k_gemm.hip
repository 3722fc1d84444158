// Projection GEMMs of the gated MSR layer on the gfx950 matrix cores.
//
// [RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、速度快、
// 性能強（2）", section "門控多尺度 Retention", Eq. (8): the layer projects X with
// W_Q, W_K, W_V, W_G and the gated, normalised heads with W_O.
//
// C[M, N] = A[M, K] * B[K, N], both row-major (the weights exactly as the
// layer stores them, [in, out]).  B may be split into up to four column
// segments with their own base pointer and row stride (W_Q | W_K | W_V |
// W_G in one launch).  The matrix-core B operand wants the reduction index
// contiguous: B tiles are copied into LDS as they are ([k][n]) and read
// with the transposing LDS read (see load_frag_rm).  Leading segments can get the
// rotation epilogue: output column pairs (2j, 2j+1) of each head are rotated
// by the (cos, sin) of their row's position (row % seqlen) before the single
// rounding to the output type.
//
// The epilogue optionally applies gelu or a sigmoid, adds a per-segment
// bias and a residual matrix (the RetNet block's feed-forward network and
// skip connections, the RG-LRU gates).
//
// Two kernels:
//   k_gemm_dc: bf16 with more than 128 rows whose weight segments start on
//     256-column boundaries (every projection of the layer, block and
//     RG-LRU at the benchmark shapes): 256x256 tiles, 8 waves, operand slabs
//     streamed into LDS by direct copies through a 4-slot ring.
//   k_gemm: everything else -- f32 (128x128 tiles, 32-deep slabs), bf16
//     with at most 128 rows (128x64 tiles, split-K, the decode step) and
//     bf16 with other segment boundaries (256x256 tiles, 4 waves of 128x128,
//     64-deep slabs double-buffered through registers).
#include "msr_launch.h"

namespace msr {

// Epilogue option sets (a compile-time parameter, so that a launch carries
// only the code of the options it uses; kEpiAny checks every option at run
// time and serves any combination).
enum : int {
  kEpiRope = 1, kEpiGelu = 2, kEpiSigmoid = 4, kEpiBias = 8, kEpiResid = 16, kEpiPart = 32, kEpiAny = 63
};

// Epilogue through LDS: each wave stages 32 of its rows at a time in
// float32, then every lane takes 8 consecutive columns of one row -- a
// rotation pair lives in one lane -- applies the rotation if the columns
// belong to a rotated segment, then bias, activation and residual, rounds
// once and writes 16 contiguous bytes.  stg0: at least
// WM WN 32 (BN / WN + 4) floats of LDS that no wave reads or writes any
// more (the caller's barrier); each wave then uses its own part of it.
template <class T, int BM, int BN, int WM, int WN, int EPI, int TM = BM / WM / 32, int TN = BN / WN / 32>
__device__ __forceinline__ void gemm_epilogue(f32x16 (&acc)[TM][TN], float* stg0, const GemmB& bp, T* __restrict__ C,
                                              int64_t ldc, int M, int N, int m0, int n0, int wave, int lane) {
  const int lr = lane & 31, hh = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  auto seg_of = [&](int n) { return (n >= bp.start[1]) + (n >= bp.start[2]) + (n >= bp.start[3]); };
  auto sel = [&](int sg, auto a0, auto a1, auto a2, auto a3) {
    return sg == 0 ? a0 : (sg == 1 ? a1 : (sg == 2 ? a2 : a3));
  };
  constexpr int WCOLS = BN / WN;                 // columns per wave
  constexpr int SLD = WCOLS + 4;                 // staged row stride (floats)
  float* stg = stg0 + wave * 32 * SLD;
  const int cw0 = n0 + wn * WCOLS;               // first column of this wave
  constexpr int ITER = 32 * (WCOLS / 8) / 64;    // 8-column groups per lane per 32 rows
  static_assert(32 * (WCOLS / 8) % 64 == 0, "whole iterations");
  // rows and columns past the end are clamped for the loads (table, bias,
  // residual) and only the stores are predicated: the iterations stay
  // branch-free, so their loads can all be in flight together
  auto where = [&](int i, int it, int& row, int& col, bool& ok) {
    const int g = lane + 64 * it, rr = g / (WCOLS / 8), c8 = g % (WCOLS / 8);
    const int row0 = m0 + wm * (BM / WM) + 32 * i + rr, col0 = cw0 + 8 * c8;
    ok = row0 < M && col0 < N;
    row = min(row0, M - 1);
    col = min(col0, N - 8);
  };
  // (cos, sin) of the 4 column pairs of an 8-column group at its row's
  // position.  A lane's 8 columns are the same in every iteration, so its
  // segment, rotation flag and pair offset are found once; the wave's rows
  // are consecutive, so row 32 i + rr of the wave sits at pos0 + 32 i + rr,
  // wrapped once at seqlen when seqlen covers the wave's rows (no integer
  // division per row: each costs a dozen instructions and a quarter-rate
  // reciprocal).
  static_assert(64 % (WCOLS / 8) == 0, "a lane's column group is the same in every iteration");
  bool rot = false;
  int cpair = 0, pos0 = 0;
  if constexpr ((EPI & kEpiRope) != 0) {
    int row, col;
    bool ok;
    where(0, 0, row, col, ok);
    const int sg = seg_of(col);
    rot = sg < bp.rope_segs && !bp.part;
    cpair = ((col - sel(sg, bp.start[0], bp.start[1], bp.start[2], bp.start[3])) % bp.rope_d) >> 1;
    pos0 = (m0 + wm * (BM / WM)) % bp.seqlen;
  }
  auto rope_cs = [&](int i, int it) {
    const int rr = (lane + 64 * it) / (WCOLS / 8);
    int p;
    if (bp.seqlen >= BM / WM) {
      p = pos0 + 32 * i + rr;
      p = p >= bp.seqlen ? p - bp.seqlen : p;
    } else {
      p = min(m0 + wm * (BM / WM) + 32 * i + rr, M - 1) % bp.seqlen;
    }
    return reinterpret_cast<const float4*>(bp.rope_tab + (size_t)p * (bp.rope_d / 2) + cpair);
  };
  constexpr bool PRE = (EPI & kEpiRope) && ITER <= 4;   // table values loaded before the staging
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float4 csv[PRE ? ITER : 1][2];
    if constexpr (PRE) {
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        if (rot) {
          const float4* cs = rope_cs(i, it);
          csv[it][0] = cs[0];
          csv[it][1] = cs[1];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stg[(8 * (r >> 2) + 4 * hh + (r & 3)) * SLD + 32 * j + lr] = acc[i][j][r];
    // the staging rows are this wave's own and a wave's LDS operations are
    // performed in order: no workgroup barrier, only a compiler fence
    asm volatile("" ::: "memory");
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int g = lane + 64 * it, rr = g / (WCOLS / 8), c8 = g % (WCOLS / 8);
      int row, col;
      bool ok;
      where(i, it, row, col, ok);
      const float* src = stg + rr * SLD + 8 * c8;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = src[e];
      const int sg = seg_of(col);
      if ((EPI & kEpiRope) && rot) {
        float4 c0, c1;
        if constexpr (PRE) {
          c0 = csv[PRE ? it : 0][0];
          c1 = csv[PRE ? it : 0][1];
        } else {
          const float4* cs = rope_cs(i, it);
          c0 = cs[0];
          c1 = cs[1];
        }
        const float t[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float x = v[2 * p], y = v[2 * p + 1];
          v[2 * p] = x * t[2 * p] - y * t[2 * p + 1];
          v[2 * p + 1] = x * t[2 * p + 1] + y * t[2 * p];
        }
      }
      if (const float* bias = (EPI & kEpiBias) ? sel(sg, bp.bias[0], bp.bias[1], bp.bias[2], bp.bias[3]) : nullptr) {
        const float* bs = bias + (col - sel(sg, bp.start[0], bp.start[1], bp.start[2], bp.start[3]));
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += bs[e];
      }
      if ((EPI & kEpiGelu) && bp.act == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.5f * v[e] * (1.0f + erff(v[e] * 0.70710678118654752f));
      } else if ((EPI & kEpiSigmoid) && bp.act == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e)   // sigmoid from the hardware exp2 and reciprocal (about 2 ulp)
          v[e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v[e] * -1.4426950408889634f));
      }
      if ((EPI & kEpiResid) && bp.resid) {
        Row8<T> rr8;
        load_row8(rr8, reinterpret_cast<const T*>(bp.resid) + (size_t)row * bp.ldr + col, true);
        float rv[8];
        unpack_row8(rv, rr8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += rv[e];
      }
      if ((EPI & kEpiPart) && bp.part) {           // split-K partial: float32, no rotation
        Row8<float> o;
        pack_row8(o, v);
        if (ok) store_row8(bp.part + (size_t)blockIdx.z * M * ldc + (size_t)row * ldc + col, o);
        continue;
      }
      Row8<T> o;
      pack_row8(o, v);
      if (ok) store_row8_nt(C + (size_t)row * ldc + col, o);
    }
    asm volatile("" ::: "memory");
  }
}

template <class T, int BM, int BN, int BK, int WM, int WN, bool UNI, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm(const T* __restrict__ A, int64_t lda, GemmB bp,
                                                       T* __restrict__ C, int64_t ldc, int M, int N, int K) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDA = BK + 16 / (int)sizeof(T);         // A tile [BM][LDA], k contiguous
  constexpr int LDB = BN + rm_pad<T>();                 // B tile [BK][LDB], n contiguous
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;   // 32x32 tiles per wave
  constexpr int AUNITS = BM * BK / 8, AU = (AUNITS + NT - 1) / NT;
  constexpr int BUNITS = BK * BN / 8, BU = (BUNITS + NT - 1) / NT;
  constexpr int STAGE = BM * LDA + BK * LDB;
  __shared__ __attribute__((aligned(16))) T smem[2][STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  // Tile order: blocks are dispatched round-robin over the 8 XCDs (each with
  // its own L2).  Give every XCD a contiguous range of tiles in grouped order
  // (8 tile-rows at a time, N fastest), so the tiles in flight on one XCD
  // share A row panels and B column panels in that XCD's L2.
  // XCD x (= bid % 8) takes q + (x < r) consecutive tiles starting at
  // x q + min(x, r), q = total / 8, r = total % 8: a permutation of 0..total-1.
  const int Mt = gridDim.y, Nt = gridDim.x, total = Mt * Nt;
  const int bid = blockIdx.y * Nt + blockIdx.x;
  const int xcd = bid % 8, q8 = total / 8, r8 = total % 8;
  const int t = xcd * q8 + min(xcd, r8) + bid / 8;
  constexpr int GM = 8;
  const int grp = t / (GM * Nt), first = grp * GM, gm = min(GM, Mt - first);
  const int w = t % (GM * Nt);
  const int m0 = (first + w % gm) * BM, n0 = (w / gm) * BN;
  auto seg_of = [&](int n) { return (n >= bp.start[1]) + (n >= bp.start[2]) + (n >= bp.start[3]); };

  // Global loads: uniform base (scalar registers) + loop-invariant 32-bit
  // per-thread offset + uniform K offset.  Rows of A past M and columns of B
  // past N are clamped to valid addresses instead of masked: they only feed
  // output rows / columns that are never stored.
  Row8<T> ra[AU], rb[BU];
  const int kz = blockIdx.z * K;                 // split-K: this workgroup's first K row
  const T* Ab = A + (size_t)m0 * lda + kz;
  uint32_t aoff[AU];
#pragma unroll
  for (int u = 0; u < AU; ++u) {
    const int idx = min(tid + NT * u, AUNITS - 1);
    const int row = min(idx / (BK / 8), M - 1 - m0), c8 = idx % (BK / 8);
    aoff[u] = (uint32_t)(row * lda + 8 * c8);
  }
  // B: the whole tile inside one weight segment (the usual case) -> one base.
  // UNI: the launcher checked that no tile straddles two segments.
  const int seg0 = seg_of(n0);
  const T* s0 = reinterpret_cast<const T*>(bp.ptr[0]);
  const T* s1 = reinterpret_cast<const T*>(bp.ptr[1]);
  const T* s2 = reinterpret_cast<const T*>(bp.ptr[2]);
  const T* s3 = reinterpret_cast<const T*>(bp.ptr[3]);
  auto sel = [&](int sg, auto a0, auto a1, auto a2, auto a3) {
    return sg == 0 ? a0 : (sg == 1 ? a1 : (sg == 2 ? a2 : a3));
  };
  const T* Bb = sel(seg0, s0, s1, s2, s3) + (n0 - sel(seg0, bp.start[0], bp.start[1], bp.start[2], bp.start[3])) +
                (size_t)kz * sel(seg0, bp.ld[0], bp.ld[1], bp.ld[2], bp.ld[3]);
  const int64_t ldb0 = sel(seg0, bp.ld[0], bp.ld[1], bp.ld[2], bp.ld[3]);
  uint32_t boff[BU];
  int bcol[BU];
#pragma unroll
  for (int u = 0; u < BU; ++u) {
    const int idx = min(tid + NT * u, BUNITS - 1);
    const int row = idx / (BN / 8), c8 = idx % (BN / 8);
    bcol[u] = min(n0 + 8 * c8, N - 8);           // N is a multiple of 8
    boff[u] = (uint32_t)(row * ldb0 + (bcol[u] - n0));
  }
  auto gload = [&](int k0) {
    const T* Ak = Ab + k0;
#pragma unroll
    for (int u = 0; u < AU; ++u) load_row8(ra[u], Ak + aoff[u], true);
    if constexpr (UNI) {
      const T* Bk = Bb + (size_t)k0 * ldb0;
#pragma unroll
      for (int u = 0; u < BU; ++u) load_row8(rb[u], Bk + boff[u], true);
    } else {
#pragma unroll
      for (int u = 0; u < BU; ++u) {
        const int idx = min(tid + NT * u, BUNITS - 1);
        const int row = idx / (BN / 8);
        const int sg = seg_of(bcol[u]);
        const T* src = sel(sg, s0, s1, s2, s3) + (bcol[u] - sel(sg, bp.start[0], bp.start[1], bp.start[2], bp.start[3]));
        load_row8(rb[u], src + (size_t)(kz + k0 + row) * sel(sg, bp.ld[0], bp.ld[1], bp.ld[2], bp.ld[3]), true);
      }
    }
  };
  auto sstore = [&](int buf) {
    T* sA = smem[buf];
    T* sB = sA + BM * LDA;
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int idx = tid + NT * u;
      if (AUNITS % NT != 0 && idx >= AUNITS) break;
      const int row = idx / (BK / 8), c8 = idx % (BK / 8);
      store_row8(sA + row * LDA + 8 * c8, ra[u]);
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int idx = tid + NT * u;
      if (BUNITS % NT != 0 && idx >= BUNITS) break;
      const int row = idx / (BN / 8), c8 = idx % (BN / 8);
      store_row8(sB + row * LDB + 8 * c8, rb[u]);
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
  auto lfr = [&](const T* sA, int s, Frag<T>* af, Frag<T>* bfr) {
    const T* sB = sA + BM * LDA;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = load_frag(sA + (wm * (BM / WM) + 32 * i + lr) * LDA + 16 * s + 8 * hh);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = load_frag_rm<KMAP_CONTIG>(sB + 16 * s * LDB + wn * (BN / WN) + 32 * j, LDB);
  };
  auto mm = [&](const Frag<T>* af, const Frag<T>* bfr) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) mma16(acc[i][j], af[i], bfr[j]);
  };
  if constexpr (sizeof(T) == 2 && BK == 64 && TM == 4 && TN == 4 && AU == 8 && BU == 8) {
    // Software pipeline with an explicit instruction interleave.  With one
    // wave per SIMD nothing else hides LDS or global latency, and left alone
    // the compiler waits on every fragment read right before its matrix-core
    // instructions.  Fragments are double-buffered in registers (set s & 1
    // holds k16 step s); each step issues the next step's 12 LDS reads (4 A +
    // 8 transposing B) between its 16 MFMAs, step 0 also the next slab's 16
    // global loads, step 3 the 16 LDS writes of that slab into the other
    // buffer.  sched_barrier fences keep each step's group in place.
    constexpr int NRD = TM + 2 * TN;                  // LDS fragment reads per k16 step (4 A + 8 transposing B)
    Frag<T> af[2][TM], bfr[2][TN];
    for (int kt = 0; kt < KT; ++kt) {
      const T* sA = smem[kt & 1];
      lfr(sA, 0, af[0], bfr[0]);
      __builtin_amdgcn_sched_barrier(0);
      gload(min(kt + 1, KT - 1) * BK);        // last slab: a harmless reload
      lfr(sA, 1, af[1], bfr[1]);
      mm(af[0], bfr[0]);
#pragma unroll
      for (int i = 0; i < NRD; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      }
#pragma unroll
      for (int i = NRD; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 1; s < 3; ++s) {
        lfr(sA, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
        mm(af[s & 1], bfr[s & 1]);
#pragma unroll
        for (int i = 0; i < NRD; ++i) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 16 - NRD, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      mm(af[1], bfr[1]);
      sstore((kt + 1) & 1);                    // last slab: the idle buffer
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gload((kt + 1) * BK);
      const T* sA = smem[kt & 1];
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        Frag<T> af[TM], bfr[TN];
        lfr(sA, s, af, bfr);
        mm(af, bfr);
      }
      if (kt + 1 < KT) sstore((kt + 1) & 1);
      __syncthreads();
    }
  }

  // epilogue through LDS (free after the main loop)
  gemm_epilogue<T, BM, BN, WM, WN, EPI>(acc, reinterpret_cast<float*>(&smem[0][0]), bp, C, ldc, M, N, m0, n0, wave,
                                        lane);
}

// ---------------------------------------------------------------------------
// k_gemm_dc: bf16 C = A B (B row-major, in up to four column segments whose
// boundaries fall on 256-column tile edges), 256 x 256 output tiles, 8
// waves of 128 x 64 (two per SIMD, so that one wave's matrix-core work
// covers the other's waits; 4 waves of 128 x 128 measured slower).  Both operand tiles
// stream into LDS by direct 16-byte copies (no staging registers, no LDS
// write instructions) through a ring of NS slots of 32-deep K slabs, NS - 2
// slabs in flight ahead of the one being read.
//   A slab: the 256 rows of A, 4 16-byte chunks (32 k) per row, row r's
//   chunk c in slot c ^ ((r / 4) % 4) of the row -- the 16 lanes that one
//   LDS read pass serves (rows r0 .. r0 + 15, one chunk) fall on 16
//   different 16-byte bank groups; and the 32 k-rows of B, 512 bytes each,
//   64-byte group g of k-row r in group g ^ (r % 4) -- the four k-rows that
//   one pass of the transposing read serves fall on four different 64-byte
//   bank groups.  A copy still fills 64 consecutive slots.
// Per slab, two k16 steps per wave; the fragments of the next step are read
// during the current one, and the wait + barrier for the next slab sits
// between the two steps, so the first fragments of a slab are read before
// its first MFMA is due.
// ---------------------------------------------------------------------------
// PRIO > 0: each k16 step's fragment reads and matrix-core instructions run
// at that wave priority, the waits and barriers between them at 0.
template <int EPI, int NS, int NW, int PRIO>
__global__ __launch_bounds__(64 * NW) void k_gemm_dc(const bf16* __restrict__ A, int64_t lda, GemmB bp,
                                                     bf16* __restrict__ C, int64_t ldc, int M, int N, int K) {
  constexpr int BM = 256, BN = 256, BK = 32, WM = 2, WN = NW / 2, TM = 4, TN = 4 / (NW / 4);
  constexpr int SLOTS = (BM + BN) * (BK / 8);        // 16-byte slots per slab
  constexpr int CPW = SLOTS / 64 / NW;               // copies per wave per slab
  static_assert(NW == 8 && NS >= 3, "slab layout");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NS * SLOTS * 8];
  static_assert(NS * SLOTS * 8 * 2 >= NW * 32 * (BN / WN + 4) * 4, "epilogue staging fits in the ring");

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int KT = K / BK;
  // tile order: as k_gemm (contiguous tile ranges per XCD), 4 tile-rows at
  // a time (4, 2, 1, 8 and 16 measured on the projection shapes: 4 fastest)
  const int Mt = gridDim.y, Nt = gridDim.x, total = Mt * Nt;
  const int bid = blockIdx.y * Nt + blockIdx.x;
  const int xcd = bid % 8, q8 = total / 8, r8 = total % 8;
  const int t8 = xcd * q8 + min(xcd, r8) + bid / 8;
  constexpr int GM = 4;
  const int grp = t8 / (GM * Nt), first = grp * GM, gm = min(GM, Mt - first);
  const int w8 = t8 % (GM * Nt);
  const int m0 = (first + w8 % gm) * BM, n0 = (w8 / gm) * BN;

  // Copies: this wave fills slots [64 (CPW wave + t), +64) of a slab; the
  // first half of the waves the A rows, the second half the B k-rows (of
  // the weight segment that holds the tile).  Rows past M and columns past
  // N are clamped: they feed outputs that are never stored.
  const int kz = blockIdx.z * K;                     // split-K: first K row of this workgroup
  const bool isA = wave < NW / 2;                    // wave-uniform
  const int sg0 = (n0 >= bp.start[1]) + (n0 >= bp.start[2]) + (n0 >= bp.start[3]);
  const bf16* bseg = reinterpret_cast<const bf16*>(sg0 == 0 ? bp.ptr[0] : sg0 == 1 ? bp.ptr[1] : sg0 == 2 ? bp.ptr[2]
                                                                                                          : bp.ptr[3]);
  const int64_t ldb = sg0 == 0 ? bp.ld[0] : sg0 == 1 ? bp.ld[1] : sg0 == 2 ? bp.ld[2] : bp.ld[3];
  const int nb0 = n0 - (sg0 == 0 ? bp.start[0] : sg0 == 1 ? bp.start[1] : sg0 == 2 ? bp.start[2] : bp.start[3]);
  const bf16* src = isA ? A + (size_t)m0 * lda + kz : bseg + nb0 + (size_t)kz * ldb;
  const int64_t kstep = isA ? BK : BK * ldb;         // elements from one slab to the next
  uint32_t off[CPW];
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int u = ((wave % (NW / 2)) * CPW + t) * 64 + lane;  // slot within this operand's 1024
    if (isA) {
      const int row = u >> 2, c = (u & 3) ^ ((row >> 2) & 3);
      off[t] = (uint32_t)((min(row, M - 1 - m0) * lda + 8 * c) * 2);
    } else {
      const int kr = u >> 5, pc = u & 31;
      const int lc = 4 * ((pc >> 2) ^ (kr & 3)) + (pc & 3);           // logical 16-byte chunk of the row
      off[t] = (uint32_t)((kr * ldb + (min(n0 + 8 * lc, N - 8) - n0)) * 2);
    }
  }
  const uint32_t lbase = lds_addr(smem) + (uint32_t)(wave * CPW * 64 * 16);
  // copy t of slab kt into its ring slot; slabs past the end copy the last
  // slab again (into a slot no slab still needs), so that every step issues
  // the same copies and the waits are fixed
  auto issue = [&](int kt, int t) {
    copy16_to_lds(src + min(kt, KT - 1) * kstep, off[t], lbase + (uint32_t)((kt % NS) * SLOTS * 16 + t * 1024));
  };

  // Fragments: lane lr reads row lr of a 32-row block, chunk 2 s + hh of
  // k16 step s, i.e. slot (2 s + hh) ^ ((lr / 4) % 4) (block rows are
  // multiples of 16, so the swizzle depends on the lane only).
  const int sw = (lr >> 2) & 3;
  const int fo0 = lr * 32 + 8 * ((0 + hh) ^ sw), fo1 = lr * 32 + 8 * ((2 + hh) ^ sw);   // elements
  // B: the transposing read of lane (hh, c, j, q) (lane = 32 hh + 16 c +
  // 4 j + q) takes k-row 16 s + 8 hh + 4 p + j, columns 16 c + 4 q of the
  // fragment's 32-column group
  const int tc = (lane >> 4) & 1, tj = (lane >> 2) & 3, tq = lane & 3;
  auto rd = [&](const bf16* slab, int s, Frag<bf16>* af, Frag<bf16>* bfr) {
    const int fo = s ? fo1 : fo0;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = load_frag(slab + (wm * 128 + 32 * i) * 32 + fo);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int grp = (wn * (BN / WN) + 32 * j) >> 5;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const bf16* a = slab + BM * 32 + (16 * s + 8 * hh + 4 * p + tj) * BN + 32 * (grp ^ tj) + 16 * tc + 4 * tq;
        const bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)a);
#pragma unroll
        for (int e = 0; e < 4; ++e) bfr[j].v[4 * p + e] = r[e];
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  // prologue: slabs 0 .. NS - 2 in flight, wait for slab 0
#pragma unroll
  for (int a = 0; a < NS - 1; ++a)
#pragma unroll
    for (int t = 0; t < CPW; ++t) issue(a, t);
  copies_wait_barrier<CPW * (NS - 2)>();
  Frag<bf16> af[2][TM], bfr[2][TN];
  rd(smem, 0, af[0], bfr[0]);
  for (int kt = 0; kt < KT; ++kt) {
    const bf16* slab = smem + (kt % NS) * SLOTS * 8;
    // step 0: read step 1's fragments, MFMAs of step 0
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(PRIO);
    rd(slab, 1, af[1], bfr[1]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) mma16(acc[i][j], af[0][i], bfr[0][j]);
    constexpr int NRD = TM + 2 * TN;                  // LDS reads per k16 step (A, then two per B fragment)
    static_assert(NRD <= TM * TN, "one read per MFMA at most");
#pragma unroll
    for (int i = 0; i < NRD; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, TM * TN - NRD, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    // slab kt + 1 landed (this wave's copies, then everyone's), every wave
    // is past slab kt - 1: its slot takes slab kt + NS - 1
    copies_wait_barrier<CPW * (NS - 3)>();
    // step 1: the next slab's step-0 fragments (after the last slab: a
    // harmless read of a slot nobody writes) and the refill copies between
    // the MFMAs of step 1
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(PRIO);
    rd(smem + ((kt + 1) % NS) * SLOTS * 8, 0, af[0], bfr[0]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        mma16(acc[i][j], af[1][i], bfr[1][j]);
        constexpr int EVERY = TM * TN / CPW;         // one copy per EVERY MFMAs
        if ((i * TN + j) % EVERY == EVERY - 1) issue(kt + NS - 1, (i * TN + j) / EVERY);
      }
    }
#pragma unroll
    for (int i = 0; i < NRD; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, TM * TN - NRD, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  }
  copies_wait_barrier<0>();                          // the trailing copies landed, every wave is done with the ring
  gemm_epilogue<bf16, BM, BN, WM, WN, EPI>(acc, reinterpret_cast<float*>(smem), bp, C, ldc, M, N, m0, n0, wave, lane);
}

// ---------------------------------------------------------------------------
// k_gemm_sk: bf16 C = A B for at most 128 rows of A (one token per sequence
// in decode), where the product is a stream of the weights B: 128 x 64
// output tiles, 64-deep K slabs of both operands copied straight to LDS
// (direct 16-byte copies) through a ring of 5 slots, 4 slabs (32 KiB of
// the weight stream) in flight per CU.  8 waves (two per SIMD), wave w:
// rows 32 (w % 4), columns 32 (w / 4).  Plain bf16 output or float32
// split-K partials (blockIdx.z = split), no other epilogue.
//   A slab: 128 rows x 8 chunks (8 k each), chunk c of row r in slot
//   c ^ ((r / 2) % 8): the 16 rows that one LDS pass of a fragment read
//   serves fall on 16 different 16-byte bank groups.
//   B slab: 64 k-rows x 8 chunks (8 columns each), chunk c of k-row r in
//   slot c ^ 4 ((r / 2) % 2): the four k-rows that one pass of the
//   transposing read serves fall on four different 64-byte bank groups.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

struct SkCfg {
  static constexpr int BM = 128, BN = 64, BK = 64, NW = 8;
  static constexpr int NS = 5;                       // ring slots (120 KiB)
  static constexpr int TJ = BN / 64;                 // 32 x 32 tiles per wave
  static constexpr int CPR = BN / 8;                 // chunks per B k-row
  static constexpr int ASL = BM * BK / 8, BSL = BK * BN / 8;   // 16-byte slots of the A and B slabs
  static constexpr int STG = (ASL + BSL) * 16;       // bytes per ring slot
  static constexpr int CPW = (ASL + BSL) / 64 / NW;  // copies per wave per slab
  static constexpr int ACP = ASL / 64 / NW;          // of which A
  static_assert(CPW * 64 * NW == ASL + BSL && ACP * 64 * NW == ASL, "whole copies per wave");
  static_assert(NS * STG <= 160 * 1024, "ring fits in LDS");
  static __device__ __forceinline__ int bsw(int r) { return 4 * ((r >> 1) & 1); }
};

template <bool PART>
__global__ __launch_bounds__(512) void k_gemm_sk(const bf16* __restrict__ A, int64_t lda, GemmB bp,
                                                 bf16* __restrict__ C, int64_t ldc, int M, int N, int K) {
  using SC = SkCfg;
  constexpr int BN = SC::BN, BK = SC::BK, NS = SC::NS, AHEAD = NS - 1, NW = SC::NW, TJ = SC::TJ, CPW = SC::CPW, ACP = SC::ACP;
  constexpr int ASL = SC::ASL, STG = SC::STG, CPR = SC::CPR;
  __shared__ __attribute__((aligned(1024))) char smem[NS * STG];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * BN;
  const int kz = blockIdx.z * K;                     // this split's first K row
  const int KT = K / BK;
  // the tile lies inside one weight segment (checked by the launcher)
  const int sg = (n0 >= bp.start[1]) + (n0 >= bp.start[2]) + (n0 >= bp.start[3]);
  auto sel = [&](auto a0, auto a1, auto a2, auto a3) { return sg == 0 ? a0 : (sg == 1 ? a1 : (sg == 2 ? a2 : a3)); };
  const bf16* Bs = reinterpret_cast<const bf16*>(sel(bp.ptr[0], bp.ptr[1], bp.ptr[2], bp.ptr[3]));
  const int64_t ldb = sel(bp.ld[0], bp.ld[1], bp.ld[2], bp.ld[3]);
  const bf16* Bt = Bs + (n0 - sel(bp.start[0], bp.start[1], bp.start[2], bp.start[3])) + (size_t)kz * ldb;
  const bf16* At = A + kz;

  // Per-lane source offsets (elements) of this wave's copies; copy t fills
  // slots 64 (NW t + wave) + lane of the slab (A for t < ACP, then B).
  uint32_t off[CPW];
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int u = 64 * (NW * t + wave) + lane;
    if (t < ACP) {
      const int r = u / 8, c = (u % 8) ^ ((r >> 1) & 7);
      off[t] = (uint32_t)(min(r, M - 1) * lda + 8 * c);
    } else {
      const int v = u - ASL, r = v / CPR, c = (v % CPR) ^ SC::bsw(r);
      off[t] = (uint32_t)(r * ldb + 8 * c);
    }
  }
  lds_char* const lds = (lds_char*)smem;
  // copies of slab j into its slot (slabs past the last re-copy the last
  // one, into a slot no wave reads again, so that every slab issues CPW
  // copies and the waits are fixed)
  auto issue = [&](int j) {
    const int jj = min(j, KT - 1);
    const uint32_t dst = (uint32_t)(uintptr_t)(lds + (j % NS) * STG) + wave * 1024;
    const bf16* a = At + (size_t)jj * BK;
    const bf16* b = Bt + (size_t)jj * BK * ldb;
#pragma unroll
    for (int t = 0; t < CPW; ++t)
      copy16_to_lds(t < ACP ? a : b, 2 * off[t], __builtin_amdgcn_readfirstlane(dst + t * NW * 1024));
  };
#pragma unroll
  for (int j = 0; j < AHEAD; ++j) issue(j);

  // fragment offsets within a slot: A row 32 (w % 4) + lr, chunk 2 s + hh;
  // B (transposing read, as load_frag_rm): k-row 16 s + 8 hh' + 4 p + jj,
  // columns (BN / 2) (w / 4) + 32 tj + 16 c + 4 q
  const int ar = 32 * (wave & 3) + lr;
  const uint32_t abase = (uint32_t)(ar * 128);
  const int af = (ar >> 1) & 7;
  const int g = lane >> 4, i16 = lane & 15, bh = g >> 1, bc = g & 1, jj = i16 >> 2, q = i16 & 3;
  f32x16 acc[TJ];
#pragma unroll
  for (int tj = 0; tj < TJ; ++tj) acc[tj] = (f32x16){};
  for (int j = 0; j < KT; ++j) {
    copies_wait_barrier<(AHEAD - 1) * CPW>();
    issue(j + AHEAD);
    const lds_char* sa = lds + (j % NS) * STG;
    const lds_char* sb = sa + ASL * 16;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      Frag<bf16> a;
      a.v = *(const lds_bf16x8_t*)(sa + abase + 16 * ((2 * s + hh) ^ af));
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        Frag<bf16> b;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int kr = 16 * s + 8 * bh + 4 * p + jj;
          const int col = (BN / 2) * (wave >> 2) + 32 * tj + 16 * bc + 4 * q;
          const int ch = (col >> 3) ^ SC::bsw(kr);
          const bf16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)(sb + kr * (BN * 2) + 16 * ch + 2 * (col & 7)));
#pragma unroll
          for (int e = 0; e < 4; ++e) b.v[4 * p + e] = r4[e];
        }
        mma16(acc[tj], a, b);
      }
    }
  }
  copies_wait_barrier<0>();                          // the trailing copies landed
  // epilogue: lane holds column lr of each 32 x 32 tile, rows 8 (r / 4) + 4 hh + r % 4
#pragma unroll
  for (int tj = 0; tj < TJ; ++tj) {
    const int n = n0 + (BN / 2) * (wave >> 2) + 32 * tj + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * (wave & 3) + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m < M) {
        if constexpr (PART) bp.part[(size_t)blockIdx.z * M * ldc + (size_t)m * ldc + n] = acc[tj][r];
        else C[(size_t)m * ldc + n] = (bf16)acc[tj][r];
      }
    }
  }
}

// Sum of the split-K partials, rounded once: 8 consecutive columns per thread.
template <class T>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int splits,
                                                       T* __restrict__ C, int64_t ldc, int M, int N) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / (N / 8), col = (g % (N / 8)) * 8;
  if (row >= M) return;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) {
    const float* p = part + ((int64_t)z * M + row) * N + col;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] += a[e]; v[4 + e] += b[e]; }
  }
  Row8<T> o;
  pack_row8(o, v);
  store_row8(C + row * ldc + col, o);
}

// bf16 products of at most 128 rows (one token per sequence in decode) use
// 128 x 64 tiles: the weight stream is split over many more workgroups, and
// no matrix-core work is spent on empty rows.
static bool skinny(Elt elt, int M) { return elt == kBF16 && M <= 128; }



int gemm_splits(Elt elt, int M, int N, int K) {
  if (skinny(elt, M) && N % 64 == 0) {
    // k_gemm_sk: one workgroup per CU, at most 8 slices
    const int tiles = N / 64;
    int s = 1;
    while (s < 8 && tiles * s < 256 && K % (64 * 2 * s) == 0) s *= 2;
    return s;
  }
  if (skinny(elt, M)) {
    // at least two workgroups per CU, at most 4 slices (more only adds partials traffic)
    const int tiles = (N + 63) / 64;
    int s = 1;
    while (s < 4 && tiles * s < 512 && K % (64 * 2 * s) == 0) s *= 2;
    return s;
  }
  // enough workgroups to cover the CUs, at most 8 slices, each a multiple of 64 rows of K
  const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int s = 1;
  while (s < 8 && tiles * s < 256 && K % (64 * 2 * s) == 0) s *= 2;
  return s;
}

// Segment boundaries all on multiples of the tile width: the uniform B path.
static bool uniform_segments(const GemmB& b, int N, int BN) {
  for (int sgi = 1; sgi < 4; ++sgi)
    if (b.start[sgi] < N && b.start[sgi] % BN) return false;
  return true;
}

// The epilogue option set of a launch.
static int epilogue_set(const GemmB& b) {
  int m = 0;
  if (b.rope_segs > 0) m |= kEpiRope;
  if (b.act == 1) m |= kEpiGelu;
  if (b.act == 2) m |= kEpiSigmoid;
  if (b.bias[0] || b.bias[1] || b.bias[2] || b.bias[3]) m |= kEpiBias;
  if (b.resid) m |= kEpiResid;
  if (b.part) m |= kEpiPart;
  return m;
}

// One tile configuration: picks the uniform-B variant and the instantiation
// for the epilogue option set (the sets the library launches have their
// own; any other combination runs the all-options instantiation).
template <class T, int BM, int BN, int BK, int WM, int WN>
static void launch_tiles(dim3 grid, const T* A, int64_t lda, const GemmB& b, T* C, int64_t ldc, int M, int N, int K,
                         hipStream_t st) {
  const bool uni = uniform_segments(b, N, BN);
  const dim3 block(64 * WM * WN);
#define MSR_GEMM_EPI(E)                                                                                             \
  if (uni)                                                                                                         \
    hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, true, E>), grid, block, 0, st, A, lda, b, C, ldc, M, N, K); \
  else                                                                                                             \
    hipLaunchKernelGGL((k_gemm<T, BM, BN, BK, WM, WN, false, E>), grid, block, 0, st, A, lda, b, C, ldc, M, N, K); \
  return;
  switch (epilogue_set(b)) {
    case 0: MSR_GEMM_EPI(0)
    case kEpiRope: MSR_GEMM_EPI(kEpiRope)
    case kEpiResid: MSR_GEMM_EPI(kEpiResid)
    case kEpiGelu: MSR_GEMM_EPI(kEpiGelu)
    case kEpiBias | kEpiSigmoid: MSR_GEMM_EPI(kEpiBias | kEpiSigmoid)
    case kEpiPart: MSR_GEMM_EPI(kEpiPart)
    default: MSR_GEMM_EPI(kEpiAny)
  }
#undef MSR_GEMM_EPI
}

// The direct-copy bf16 product on 256 x 256 tiles, instantiated for the
// epilogue option set as launch_tiles does.  8 waves and four ring slots:
// the fastest of 4 / 8 waves x 3 / 4 / 5 slots on the layer's projection
// shapes.  Products of at most 8192 columns raise the waves' issue priority
// while they issue matrix-core work (M 32768, N 4096, K 8192: 4.5 % faster;
// M 16384, N 8192, K 2048: 10 %; at N 24576, K 4096 it was 0.6 % slower).
static void launch_dc(dim3 grid, const bf16* A, int64_t lda, const GemmB& b, bf16* C, int64_t ldc, int M, int N, int K,
                      hipStream_t st) {
  constexpr int NS = 4, NW = 8;
  const bool prio = N <= 8192;
#define MSR_GEMM_BT(E)                                                                                         \
  if (prio)                                                                                                    \
    hipLaunchKernelGGL((k_gemm_dc<E, NS, NW, 1>), grid, dim3(64 * NW), 0, st, A, lda, b, C, ldc, M, N, K);    \
  else                                                                                                         \
    hipLaunchKernelGGL((k_gemm_dc<E, NS, NW, 0>), grid, dim3(64 * NW), 0, st, A, lda, b, C, ldc, M, N, K);    \
  return;
  switch (epilogue_set(b)) {
    case 0: MSR_GEMM_BT(0)
    case kEpiRope: MSR_GEMM_BT(kEpiRope)
    case kEpiResid: MSR_GEMM_BT(kEpiResid)
    case kEpiGelu: MSR_GEMM_BT(kEpiGelu)
    case kEpiBias | kEpiSigmoid: MSR_GEMM_BT(kEpiBias | kEpiSigmoid)
    case kEpiPart: MSR_GEMM_BT(kEpiPart)
    default: MSR_GEMM_BT(kEpiAny)
  }
#undef MSR_GEMM_BT
}

// bf16 and f32 products on their usual tiles, or on the skinny tiles.
static void launch_any(Elt elt, const void* A, int64_t lda, const GemmB& b, void* C, int64_t ldc, int M, int N,
                       int K, int splits, hipStream_t st) {
  const int epi = epilogue_set(b);
  if (skinny(elt, M) && N % 64 == 0 && K % 64 == 0 && (epi == 0 || epi == kEpiPart) && uniform_segments(b, N, 64)) {
    const dim3 grid(N / 64, 1, splits);
    if (epi == kEpiPart)
      hipLaunchKernelGGL((k_gemm_sk<true>), grid, dim3(512), 0, st, (const bf16*)A, lda, b, (bf16*)C, ldc, M, N, K);
    else
      hipLaunchKernelGGL((k_gemm_sk<false>), grid, dim3(512), 0, st, (const bf16*)A, lda, b, (bf16*)C, ldc, M, N, K);
  } else if (skinny(elt, M)) {
    launch_tiles<bf16, 128, 64, 64, 2, 2>(dim3((N + 63) / 64, 1, splits), (const bf16*)A, lda, b, (bf16*)C, ldc, M,
                                          N, K, st);
  } else if (elt == kBF16 && uniform_segments(b, N, 256)) {
    launch_dc(dim3((N + 255) / 256, (M + 255) / 256, splits), (const bf16*)A, lda, b, (bf16*)C, ldc, M, N, K, st);
  } else if (elt == kBF16) {
    launch_tiles<bf16, 256, 256, 64, 2, 2>(dim3((N + 255) / 256, (M + 255) / 256, splits), (const bf16*)A, lda, b,
                                           (bf16*)C, ldc, M, N, K, st);
  } else {
    launch_tiles<float, 128, 128, 32, 2, 2>(dim3((N + 127) / 128, (M + 127) / 128, splits), (const float*)A, lda, b,
                                            (float*)C, ldc, M, N, K, st);
  }
}

hipError_t launch_gemm_splitk(Elt elt, const void* A, int64_t lda, const GemmB& b, void* C, int64_t ldc, int M,
                              int N, int K, int splits, float* part, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (b.act || b.resid || b.bias[0] || b.bias[1] || b.bias[2] || b.bias[3]) return hipErrorInvalidValue;
  GemmB bs = b;
  bs.part = part;
  bs.rope_segs = 0;
  hipError_t err;
  {
    TraceScope ts("k_gemm", st);
    launch_any(elt, A, lda, bs, nullptr, (int64_t)N, M, N, K / splits, splits, st);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  TraceScope ts("k_splitk_reduce", st);
  const int64_t groups = (int64_t)M * (N / 8);
  const dim3 grid((unsigned)((groups + 255) / 256));
  if (elt == kBF16)
    hipLaunchKernelGGL((k_splitk_reduce<bf16>), grid, dim3(256), 0, st, part, splits, (bf16*)C, ldc, M, N);
  else
    hipLaunchKernelGGL((k_splitk_reduce<float>), grid, dim3(256), 0, st, part, splits, (float*)C, ldc, M, N);
  return hipGetLastError();
}

hipError_t launch_gemm(Elt elt, const void* A, int64_t lda, const GemmB& b, void* C, int64_t ldc, int M, int N,
                       int K, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  TraceScope ts("k_gemm", st);
  launch_any(elt, A, lda, b, C, ldc, M, N, K, 1, st);
  return hipGetLastError();
}

}  // namespace msr
