// Output kernel of chunkwise and parallel retention for d_k = 256, bf16,
// with 16 query rows per wave on the 16x16x32 matrix-core instruction.
//
// Method ([RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、
// 速度快、性能強（2）", section "3) Retention 分塊循環表征", Eq. (7)): for the
// rows t of chunk i (L rows in the chunk, keys s of the same chunk),
//   O_[i] = ((Q_[i] K_[i]^T) * scale (.) D) V_[i] + scale * (Q_[i] R_{i-1}) (.) xi,
//   D[t, s] = gamma^(t - s) (t >= s, else 0), xi_t = gamma^(t + 1);
// the parallel form (section "1) Retention 的並行表征", Eq. (5)) is one chunk
// spanning the sequence with no state.  Optionally followed by the per-head
// GroupNorm and the swish gate of section "門控多尺度 Retention", Eq. (8).
// The reversed variant (REV, for the backward's anti-causal passes) runs the
// same recurrence on the time-reversed sequence: row t of Q, K, V is read
// from row N - 1 - t and output row t written to row N - 1 - t.
//
// Work split: tiles of (batch, head, chunk, 128 query rows), run by a
// persistent grid of one workgroup of 8 waves (two per SIMD) per CU; each
// wave owns 16 query rows and the whole d_v width of their outputs, so the
// score tile never leaves the wave and the accumulators (d_v = 512: 128
// registers) leave room for a second wave per SIMD.  A workgroup walks its
// tiles with one continuous stream of stages -- the tile's Q rows (two
// 64-row stages), the d_k slabs of R_{i-1}^T, then blocks of 32 keys with K
// and V together -- through a ring of LDS slots filled by direct
// global->LDS copies, NS - 1 stages in flight, so the next tile's first
// stages land while the current tile finishes.  Tiles are stored unpadded
// and swizzled in 16-byte units (the copies pick each lane's source so that
// the data lands swizzled), which keeps every fragment read conflict-free:
//   Q, K [rows][32 chunks]     chunk c of row r at c ^ (r & 15)
//   V   [32 keys][d_v/8]       chunk c of row r at c ^ (2 (r & 7))
//   R^T [d_v][SK/8]            chunk c of row r at c ^ f(r), f(r) = (r >> 2) & 3
//                              (SK = 32) or (r >> 1) & 7 (SK = 64)
// The tiles of one (batch, head, chunk) run at the same time on one XCD
// (workgroup ids 8 apart), so K and V are fetched from HBM once per chunk
// and re-read from that XCD's L2.
//
// 16x16x32 fragments (lane l, i = l % 16, g = l / 16): A = row i, elements
// k = 8 g .. 8 g + 7; B = column i, the same k; the accumulator tile holds
// column i, rows 4 g .. 4 g + 3.  The score tile is computed transposed, S^T
// = K Q^T (keys in rows, so Q is the B operand kept in registers), in two
// 16-key halves; lane l then holds query i, keys 4 g + r and 16 + 4 g + r,
// and uses them directly as the A operand of P V with that key order; the V
// fragment is read in the same order with the transposing LDS read.
#include <atomic>
#include "msr_launch.h"

namespace msr {

namespace {

__device__ __forceinline__ void mma_16x32(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A wave-uniform value the compiler cannot prove uniform, moved to scalar
// registers (the direct copy takes its base and LDS address there).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Sum over the 16 lanes of each DPP row, returned to all of them.
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x141>(x);   // row_half_mirror
  x = dpp_add<0x140>(x);   // row_mirror
  return x;
}

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

template <int DV>
struct O16Cfg {
  static constexpr int DK = 256, NT = 512, NW = 8, RT = 128, KB = 32;
  static constexpr int CPK = DK / 8;                  // 16-byte chunks per K row
  static constexpr int CPV = DV / 8;                  // per V row
  static constexpr int SK = DV > 256 ? 32 : 64;       // d_k columns per R^T slab
  static constexpr int CPR = SK / 8;                  // chunks per R^T slab row
  static constexpr int KCH = KB * CPK;                // K chunks per key stage
  static constexpr int VCH = KB * CPV;                // V chunks per key stage
  static constexpr int RCH = DV * CPR;                // chunks per R^T slab
  static constexpr int NCP = (KCH + VCH) / 64;        // 1 KiB copies per stage
  static constexpr int LPW = NCP / NW;                // per wave
  static constexpr int STG = NCP * 1024;              // bytes per ring slot
  static constexpr int NS = DV > 256 ? 3 : 4;         // ring slots
  static constexpr int AHEAD = NS - 1;                // stages in flight
  static constexpr int NJ = DV / 16;                  // 16-column output tiles
  static constexpr int NR = DK / SK;                  // R^T slabs
  // fragment reads in flight ahead of the matrix-core step that uses them
  // (one 16x16x32 step is 16 cycles, an LDS read under load several times
  // that)
  static constexpr int PF = DV > 256 ? 3 : 6;
  static constexpr int SLH = DV / 2 + 16;             // epilogue staging row (floats, half of d_v): the 4 lane
                                                      // groups' rows, 16 banks apart, hit disjoint banks
  static_assert(NCP % NW == 0 && RCH % (64 * NW) == 0 && RCH / 64 <= NCP, "whole copies per wave");
  static_assert(NS * STG <= 160 * 1024, "ring fits in LDS");
  static_assert(NW * 4 * SLH * 4 <= STG, "epilogue staging (4 half rows per wave) fits in one slot");
  static_assert(64 * CPK / 64 <= NCP, "a Q stage (64 rows) fits the stage's copies");
  static_assert(KCH % (64 * NW) == 0 && CPK % NW == 0, "each part of a stage fills whole rounds of copies");
};

}  // namespace

template <int DV, bool STATE, bool GN, bool ROPE, bool REV>
__global__ __launch_bounds__(512) void k_chunk_o16(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, int64_t ldq, int64_t ldk,
    int64_t ldv, const bf16* __restrict__ Rx, const bf16* __restrict__ G, int64_t ldg,
    bf16* __restrict__ O, int64_t ldo, int BH, int N, int H, int chunk, int NC, int TPC, int P, float scale,
    float eps, HeadTab tab, const float2* __restrict__ rtab) {
  using C = O16Cfg<DV>;
  constexpr int DK = C::DK, KB = C::KB, NS = C::NS, AHEAD = C::AHEAD, NJ = C::NJ, LPW = C::LPW, RT = C::RT;
  __shared__ __attribute__((aligned(1024))) char smem[NS * C::STG];

  const int tid = threadIdx.x, lane = tid & 63, i16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroup (xg, j) of the P on XCD xg takes, at its iteration k, unit
  // (k (P / TPC) + j / TPC) * 8 + xg: a unit's TPC row tiles run at the same
  // time on one XCD, so that each K, V and R_{i-1} stage they share comes
  // from HBM once and from that XCD's L2 for the others -- if they read it
  // at about the same time.  Row tiles differ in length (the causal key
  // range), so the tiles are paired: at even k workgroup j takes row tile
  // l = (j + k / 2) % TPC and walks it forward (Q, R_{i-1}, key blocks in
  // order), at odd k row tile TPC - 1 - l of the next unit, walked backward
  // (Q, key blocks from the diagonal down, R_{i-1} last).  Every workgroup
  // then does the same work per pair of iterations: the forward tiles of a
  // unit start together and the backward ones end together, and either way
  // they reach each shared stage at the same time (measured at the block
  // workload: fetched bytes 2.38 -> 1.34 GB per launch, exactly the
  // compulsory ones).  With the GroupNorm + gate epilogue the tiles keep
  // the earlier order -- row tile TPC - 1 - (j + k) % TPC, always walked
  // forward -- which measured 5 % faster there (the paired tiles' gate
  // loads and stores come in step), and so do the variants that rotate Q
  // (the second Q R_{i-1} pass would not fit their registers).
  constexpr bool PAIR = !GN && !ROPE;
  const int U = NC * BH;
  const int xg = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int UG = (U + 7) / 8, upi = P / TPC;
  const int iters = (UG + upi - 1) / upi;
  struct Tile { int ok, ci, bh, c0, r0, nR, nKV, bwd; };
  auto tile_at = [&](int k) {
    Tile t{};
    const int ug = k * upi + j / TPC;
    const int unit = ug * 8 + xg;
    int li;
    if constexpr (PAIR) {
      const int le = (j % TPC + (k >> 1)) % TPC;
      t.bwd = k & 1;
      li = t.bwd ? TPC - 1 - le : le;
    } else {
      t.bwd = 0;
      li = TPC - 1 - (j % TPC + k) % TPC;
    }
    t.ok = 0;
    if (ug >= UG || unit >= U) return t;
    t.ci = unit / BH; t.bh = unit % BH;
    t.c0 = t.ci * chunk; t.r0 = t.c0 + li * RT;
    // a row tile past the sequence end (last chunk cut short) is still
    // run, with every row inactive: its copies are clamped to the last
    // token, nothing is stored, and the tile list then only ends at its tail
    t.ok = 1;
    // every tile of the state variant runs Q R_{i-1}, the first chunk's
    // too: the scan stores that chunk's incoming state (zero without an
    // initial state), and one code path keeps the accumulators out of a
    // merge of two register sets
    t.nR = STATE ? C::NR : 0;
    t.nKV = (min(t.r0 + RT, N) - t.c0 + KB - 1) / KB;
    return t;
  };
  // two Q stages, then R slabs and key blocks (forward) or key blocks from
  // the last one down and R slabs (backward)
  auto nst_of = [&](const Tile& t) { return 2 + t.nR + t.nKV; };

  const int ldk32 = (int)ldk, ldv32 = (int)ldv, ldq32 = (int)ldq;
  // LDS addresses are 32-bit (so that constant parts fold into the
  // instructions' offsets)
  lds_char* const lds = (lds_char*)smem;
  // ring slots by byte offset, stepped with a compare instead of a modulo
  // by NS (a multiply-high sequence per use for NS = 3)
  auto next_off = [&](uint32_t o) { return o + C::STG == (uint32_t)(NS * C::STG) ? 0u : o + C::STG; };
  auto prev_off = [&](uint32_t o) { return o == 0u ? (uint32_t)((NS - 1) * C::STG) : o - C::STG; };

  // ---- the copy stream: every stage of every tile of this workgroup ----
  // Per-lane byte offsets (from the stage's first row) of copy t of this
  // wave, which fills 16-byte slots 64 (NW t + wave) + lane of the stage
  // (copies strided over the waves: which part of the stage -- K or V, data
  // or pad -- a copy fills then depends on t alone, so each copy's formula
  // is fixed at compile time); rows past the sequence end are clamped to its
  // last row (lim): such keys are in the future of every stored query
  // (weight 0), such query rows are never stored.  Unsigned arithmetic: the
  // divisions are shifts.
  // Slot u = 512 t + w64 (w64 = 64 wave + lane) of a stage splits into a
  // part that depends on t alone and one that depends on the lane alone:
  //   K, Q rows (32 chunks each): row 16 t + w64 / 32, chunk (w64 % 32) ^ (row & 15)
  //   V rows (CPV chunks):        row (t - KR) 512 / CPV + w64 / CPV,
  //                               chunk (w64 % CPV) ^ (2 (row & 7))
  //   R^T rows (CPR chunks):      row 512 t / CPR + w64 / CPR, chunk p ^ f(row)
  // (512 / CPV is a multiple of 8 and 512 / CPR of 32, so the swizzles only
  // see the lane part).  The lane parts, kept in five registers:
  struct LaneOff { uint32_t rk, ck, rv, cv, ro; };
  LaneOff lo0;
  {
    const uint32_t w64 = (uint32_t)(wave * 64 + lane);
    lo0.rk = w64 / C::CPK;
    lo0.ck = 16u * ((w64 % C::CPK) ^ (lo0.rk & 15u));
    lo0.rv = w64 / C::CPV;
    lo0.cv = 16u * ((w64 % C::CPV) ^ (2u * (lo0.rv & 7u)));
    const uint32_t r = w64 / C::CPR, p = w64 % C::CPR;
    const uint32_t c = DV > 256 ? (p ^ ((r >> 2) & 3u)) : (p ^ ((r >> 1) & 7u));
    lo0.ro = (r * DK + 8u * c) * 2u;
  }
  constexpr int KR = C::KCH / 64 / C::NW;            // rounds of copies holding K
  // row r of a stage (clamped to lim) lies r rows after the stage's base
  // row, or, reversed, lim - r rows after it (the base is then the stage's
  // last row in time order, the lowest in memory)
  auto srow = [&](uint32_t r, uint32_t ul) { return REV ? ul - min(r, ul) : min(r, ul); };
  // row (< 64) times the row stride in bytes on the full-rate 24-bit
  // multiplier: the strides are below 2^20 bytes (a token row of the widest
  // buffer, heads (2 d_k + 2 d_v) elements, stays below 2^19)
  auto kv_off = [&](const LaneOff& lo, int t, int lim) -> uint32_t {
    const uint32_t ul = (uint32_t)lim;
    if (t < KR) return __umul24(srow(lo.rk + 16u * t, ul), (uint32_t)(2 * ldk32)) + lo.ck;
    return __umul24(srow(lo.rv + (uint32_t)((t - KR) * (512 / C::CPV)), ul), (uint32_t)(2 * ldv32)) + lo.cv;
  };
  // Q stages: 64 rows x 32 chunks, K's swizzle; R stages: rows of the R^T
  // slab.  Copies past the data (d_v = 512) re-read its first 16 bytes into
  // the unused tail of the slot, so that every stage issues LPW copies.
  auto q_off = [&](const LaneOff& lo, int t, int lim) -> uint32_t {
    if (t < 64 * C::CPK / 64 / C::NW) return __umul24(srow(lo.rk + 16u * t, (uint32_t)lim), (uint32_t)(2 * ldq32)) + lo.ck;
    return 0u;
  };
  auto r_off = [&](const LaneOff& lo, int t) -> uint32_t {
    if (t < C::RCH / 64 / C::NW) return lo.ro + (uint32_t)(t * (512 / C::CPR) * DK * 2);
    return 0u;
  };
  // The prefetch position (tile iteration pk, its stage pl) runs AHEAD
  // stages ahead of the consumed one; past the last stage of the last tile
  // it re-copies that stage into a free slot, so that every stage issues
  // the same copies and the waits are fixed.
  struct Cp { const bf16* src[2]; uint32_t dst; uint32_t off[LPW]; };
  int pk = 0, pl = 0;                                // prefetch tile iteration, stage in it
  uint32_t pgo = 0;                                  // its ring slot (byte offset)
  Tile pt = tile_at(0);
  const bool any = pt.ok;
  // Bases of the prefetch position's tile, set once when it enters the
  // tile (not per stage: the (batch, head) split is a scalar division and
  // the row products 64-bit): Q, K, V at row 0 of its sequence and head,
  // and its R_{i-1}^T.
  const bf16 *pqb, *pkb, *pvb, *prb;
  auto enter = [&](const Tile& t) {
    const int b = t.bh / H, h = t.bh % H;
    const size_t tokb = (size_t)b * N;
    pqb = Q + tokb * ldq + (size_t)h * DK;
    pkb = K + tokb * ldk + (size_t)h * DK;
    pvb = V + tokb * ldv + (size_t)h * DV;
    prb = STATE ? Rx + ((size_t)t.bh * NC + t.ci) * DV * DK : nullptr;
  };
  enter(pt);
  auto prep_next = [&](Cp& c) {
    c.dst = (uint32_t)(uintptr_t)(lds + pgo) + wave * 1024;
    pgo = next_off(pgo);
    // the lane parts made opaque here: otherwise the compiler keeps every
    // stage kind's per-copy offsets live across the whole tile loop
    LaneOff lo = lo0;
    asm volatile("" : "+v"(lo.rk), "+v"(lo.ck), "+v"(lo.rv), "+v"(lo.cv), "+v"(lo.ro));
    if (pl < 2) {                                    // Q rows r0 + 64 pl ..
      const int base = min(pt.r0 + 64 * pl, N - 1);
      const int lim = min(63, N - 1 - base);
      c.src[0] = c.src[1] = pqb + (uint64_t)(uint32_t)(REV ? N - 1 - base - lim : base) * (uint32_t)ldq32;
#pragma unroll
      for (int t = 0; t < LPW; ++t) c.off[t] = q_off(lo, t, lim);
    } else if (pt.bwd ? pl >= 2 + pt.nKV : pl < 2 + pt.nR) {   // R_{i-1}^T slab
      c.src[0] = c.src[1] = prb + (pt.bwd ? pl - 2 - pt.nKV : pl - 2) * C::SK;
#pragma unroll
      for (int t = 0; t < LPW; ++t) c.off[t] = r_off(lo, t);
    } else {                                         // keys kb .. kb + 31
      const int kb = pt.c0 + (pt.bwd ? pt.nKV - 1 - (pl - 2) : pl - 2 - pt.nR) * KB;
      const int lim = min(KB - 1, N - 1 - kb);
      const int row = REV ? N - 1 - kb - lim : kb;
      c.src[0] = pkb + (uint64_t)(uint32_t)row * (uint32_t)ldk32;
      c.src[1] = pvb + (uint64_t)(uint32_t)row * (uint32_t)ldv32;
#pragma unroll
      for (int t = 0; t < LPW; ++t) c.off[t] = kv_off(lo, t, lim);
    }
    // advance the position, unless this was the very last stage
    if (pl + 1 < nst_of(pt)) {
      ++pl;
    } else if (pk + 1 < iters) {
      const Tile t2 = tile_at(pk + 1);
      if (t2.ok) { ++pk; pt = t2; pl = 0; enter(pt); }
    }
  };
  auto cp = [&](const Cp& c, int t) {
    copy16_to_lds(uniform_ptr(t < C::KCH / 64 / C::NW ? c.src[0] : c.src[1]), c.off[t],
                  __builtin_amdgcn_readfirstlane(c.dst + t * C::NW * 1024));
  };
  if (!any) return;
  Cp cn;
#pragma unroll
  for (int a = 0; a < AHEAD; ++a) {
    prep_next(cn);
#pragma unroll
    for (int t = 0; t < LPW; ++t) cp(cn, t);
  }
  uint32_t gso = 0;                                  // ring slot (byte offset) of the stage being consumed
  // wait for the consumed stage's copies, then prepare those of the stage
  // AHEAD after it into the slot of the stage before it, which every wave
  // is past (issued during the consumed stage)
  auto advance = [&]() {
    copies_wait_barrier<(AHEAD - 1) * LPW>();
    prep_next(cn);
  };

  const uint32_t kbase = (uint32_t)(i16 * (C::CPK * 16));
  const int jj = i16 >> 2, m = i16 & 3, wv = (4 * g + jj) & 7;
  const uint32_t vbase = (uint32_t)(C::KCH * 16 + (4 * g + jj) * (C::CPV * 16) + 16 * (m >> 1) + 8 * (m & 1));
  const int fr = DV > 256 ? ((i16 >> 2) & 3) : ((i16 >> 1) & 7);

  for (int k = 0; k < iters; ++k) {
    const Tile t = tile_at(k);
    if (!t.ok) break;                                // uniform; the tile list ends
    const int h = t.bh % H, b = t.bh / H;
    const size_t tokb = (size_t)b * N;
    const int q0 = t.r0 + 16 * wave;
    const bool active = q0 < N;                      // wave-uniform
    const float lg2 = tab.lg2[h];

    // ---- Q: rows of this wave from the Q stage that holds them (element e
    // of fragment s is column 32 s + 8 g + e of row q0 + i16) ----
    bf16x8 qf[DK / 32];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs, gso = next_off(gso)) {
      advance();
#pragma unroll
      for (int tt = 0; tt < LPW; ++tt) cp(cn, tt);
      if ((wave >> 2) == qs) {
        uint32_t kb_l = kbase + (uint32_t)((wave & 3) * 16 * (C::CPK * 16));
        asm volatile("" : "+v"(kb_l));
        const lds_char* sq = lds + gso;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
          qf[s] = *(const lds_bf16x8*)(sq + kb_l + 16 * ((4 * (s & 3) + g) ^ i16) + (s >> 2) * 256);
      }
    }
    if constexpr (ROPE) {
      // rotation by the position of the row ([RN-zh] section "Retention", Eq. (3)-(4))
      const int qr = min(q0 + i16, N - 1);
      const float2* tp = rtab + (size_t)qr * (DK / 2) + 4 * g;
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)qf[s][e];
        rotate8(x, tp + 16 * s);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = (bf16)x[e];
      }
    }

    f32x4 acc[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) acc[jt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // ---- Q R_{i-1}: acc[jt] += Q[:, slab] R^T[16 jt .., slab]^T; the lane
    // reads R^T row 16 jt + i16, chunk 4 s2 + g swizzled by f(row), which
    // does not depend on jt ----
    auto r_phase = [&]() {
      static_for<C::NR>([&](auto slc) {
        constexpr int sl = decltype(slc)::value;
        advance();
        uint32_t rl[C::SK / 32];
#pragma unroll
        for (int s2 = 0; s2 < C::SK / 32; ++s2) rl[s2] = (uint32_t)(i16 * (C::CPR * 16) + 16 * ((4 * s2 + g) ^ fr));
        asm volatile("" : "+v"(rl[0]));
        if constexpr (C::SK / 32 > 1) asm volatile("" : "+v"(rl[C::SK / 32 - 1]));
        const lds_char* sR = lds + gso;
        constexpr int T = NJ * (C::SK / 32);
        auto rd = [&](int tt) {
          const int jt = tt / (C::SK / 32), s2 = tt % (C::SK / 32);
          return *(const lds_bf16x8*)(sR + rl[s2] + jt * (16 * C::CPR * 16));
        };
        constexpr int PF = C::PF;
        bf16x8 rf[PF + 1];
#pragma unroll
        for (int tt = 0; tt < PF; ++tt) rf[tt] = rd(tt);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          if (tt + PF < T) rf[(tt + PF) % (PF + 1)] = rd(tt + PF);
          mma_16x32(acc[tt / (C::SK / 32)], qf[sl * (C::SK / 32) + tt % (C::SK / 32)], rf[tt % (PF + 1)]);
          if (tt < LPW) cp(cn, tt);                  // next stages' copies between the MFMAs
        }
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          if (tt + PF < T) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        gso = next_off(gso);
      });
    };
    if constexpr (STATE) {
      if (!t.bwd) {
        r_phase();
        // rows scaled by scale * xi_t = scale * gamma^(t + 1), t = row in the chunk
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = scale * gpow(q0 - t.c0 + 4 * g + r + 1, lg2);
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) acc[jt][r] *= x;
        }
      }
    }

    // ---- key blocks ----
    // Decay gamma^n from the hardware exp2 of n log2(gamma), log2(0) = -inf
    // replaced by a large finite value so that n = 0 gives exactly 1 (0^0 =
    // 1 on the diagonal) and n > 0 underflows to 0.  Off the diagonal block
    // (every key before every row of the wave) gamma^(q - k) = u * w[e] with
    // u = gamma^(q0 - kb - 31) for the wave and w[e] = gamma^(31 + i16 - 16
    // (e / 4) - 4 g - e % 4) per lane, both exponents >= 0.
    const float lg2f = fmaxf(lg2, -1.0e30f);
    auto pw = [&](int n) { return __builtin_amdgcn_exp2f((float)n * lg2f); };
    int ex0 = 31 + i16 - 4 * g;                      // opaque: not hoisted out of the tile loop
    asm volatile("" : "+v"(ex0));
    float wk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) wk[e] = scale * pw(ex0 - 16 * (e >> 2) - (e & 3));
    for (int kv = 0; kv < t.nKV; ++kv, gso = next_off(gso)) {
      advance();
      const lds_char* sb = lds + gso;
      const int kb = t.c0 + (t.bwd ? t.nKV - 1 - kv : kv) * KB;
      // per-lane bases made opaque each stage: otherwise every (lane part +
      // constant) sum of the unrolled reads is hoisted out of the loop into
      // its own register instead of folding the constant into the offset
      uint32_t kb_l = kbase, vb_l = vbase, wv_l = (uint32_t)wv;
      asm volatile("" : "+v"(kb_l), "+v"(vb_l), "+v"(wv_l));
      // Every wave runs every key block: P is exactly 0 for keys in its
      // future (and its results are not stored when it has no rows), so
      // there is one code path for the accumulators -- a skip branch would
      // make them a loop-carried merge that the compiler copies.
      f32x4 st[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
      // S^T: 16 steps (k-step s = tt / 2, key half ks = tt % 2)
      {
        constexpr int T = 2 * (DK / 32);
        auto rd = [&](int tt) {
          const int s = tt >> 1, ks = tt & 1;
          return *(const lds_bf16x8*)(sb + kb_l + 16 * ((4 * (s & 3) + g) ^ i16) + (s >> 2) * 256 +
                                      ks * (16 * C::CPK * 16));
        };
        constexpr int PF = C::PF;
        bf16x8 kf[PF + 1];
#pragma unroll
        for (int tt = 0; tt < PF; ++tt) kf[tt] = rd(tt);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          if (tt + PF < T) kf[(tt + PF) % (PF + 1)] = rd(tt + PF);
          mma_16x32(st[tt & 1], kf[tt % (PF + 1)], qf[tt >> 1]);
          if (tt < LPW) cp(cn, tt);
        }
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          if (tt + PF < T) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // P = S * scale * gamma^(q - k) for k <= q, else 0 (query q0 + i16,
      // key kb + 16 (e / 4) + 4 g + e % 4)
      bf16x8 pa;
      if (kb + 31 < q0) {                            // wave-uniform
        const float u = pw(q0 - kb - 31);
#pragma unroll
        for (int e = 0; e < 8; ++e) pa[e] = (bf16)(st[e >> 2][e & 3] * (u * wk[e]));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = q0 - kb + i16 - 16 * (e >> 2) - 4 * g - (e & 3);
          pa[e] = (bf16)(n >= 0 ? st[e >> 2][e & 3] * (scale * pw(max(n, 0))) : 0.0f);
        }
      }
      // P V: one step per 16-column tile; the V fragment (tile jt, key half
      // hr): lane 16 g + 4 jj + m addresses row 16 hr + 4 g + jj, columns
      // 16 jt + 4 m .. + 3: chunk 2 jt + m / 2 swizzled by 2 w, w = (4 g +
      // jj) & 7, to 16 (jt >> 3) + 2 ((jt & 7) ^ w) + m / 2
      {
        auto rd = [&](int jt) {
          const lds_char* vb = sb + vb_l + 32 * ((jt & 7) ^ wv_l) + (jt >> 3) * 256;
          bf16x8 vf;
#pragma unroll
          for (int hr = 0; hr < 2; ++hr) {
            const bf16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + hr * (16 * C::CPV * 16)));
#pragma unroll
            for (int e = 0; e < 4; ++e) vf[4 * hr + e] = r4[e];
          }
          return vf;
        };
        constexpr int PF = C::PF;
        bf16x8 vq[PF + 1];
#pragma unroll
        for (int tt = 0; tt < PF; ++tt) vq[tt] = rd(tt);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          if (jt + PF < NJ) vq[(jt + PF) % (PF + 1)] = rd(jt + PF);
          mma_16x32(acc[jt], pa, vq[jt % (PF + 1)]);
        }
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
          if (jt + PF < NJ) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if constexpr (STATE) {
      if (t.bwd) {
        // Q R_{i-1} last: the Q rows (query q0 + i16 of every fragment) scaled
        // by scale * xi_t first, rounded to bf16
        const float x = scale * gpow(q0 - t.c0 + i16 + 1, lg2);
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[s][e] = (bf16)((float)qf[s][e] * x);
        r_phase();
      }
    }

    // ---- epilogue: lane holds column 16 jt + i16 of rows q0 + 4 g + r.
    // Pass p stages the rows q0 + 4 g + p / 2 (all four lane groups) over
    // the column half p % 2 in this wave's part of the last stage's slot,
    // so that each lane then takes whole 8-column chunks: 16-byte gate loads
    // and output stores.  The slot is free once every wave is past that
    // stage (the barrier; the copies in flight, which it does not wait for,
    // fill the other slots) and until the next stage's barrier.  Waves with
    // no rows skip the rest. ----
    copies_wait_barrier<AHEAD * LPW>();
    if (active) {
      float mu[4], rs[4];
      if constexpr (GN) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) sum += acc[jt][r];
          mu[r] = row16_sum(sum) * (1.0f / DV);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) {
            const float d = acc[jt][r] - mu[r];
            sum += d * d;
          }
          rs[r] = rsqrtf(row16_sum(sum) * (1.0f / DV) + eps);
          mu[r] *= -rs[r];                           // y = x rs - mu rs, one fused multiply-add
        }
      }
      lds_float* stg = (lds_float*)(lds + prev_off(gso)) + wave * 4 * C::SLH;
      constexpr int NCH = DV / 16;                   // 8-column chunks per half row
      constexpr int CH = 4 * NCH / 64;               // per lane per pass
      auto gate = [&](int pass, Row8<bf16>* gv) {
        const int r = pass >> 1, hv = pass & 1;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int id = lane + 64 * c, sr = id / NCH, c8 = id % NCH;
          const int q = min(q0 + 4 * sr + r, N - 1);
          load_row8(gv[c], G + (tokb + q) * ldg + (size_t)h * DV + hv * (DV / 2) + 8 * c8, true);
        }
      };
      Row8<bf16> gv[2][CH];
      if constexpr (GN) gate(0, gv[0]);
#pragma unroll
      for (int pass = 0; pass < 8; ++pass) {
        const int r = pass >> 1, hv = pass & 1;
        if constexpr (GN) {
          if (pass + 1 < 8) gate(pass + 1, gv[(pass + 1) & 1]);
        }
#pragma unroll
        for (int jh = 0; jh < NJ / 2; ++jh) {
          const int jt = hv * (NJ / 2) + jh;
          const float y = GN ? fmaf(acc[jt][r], rs[r], mu[r]) : acc[jt][r];
          stg[g * C::SLH + 16 * jh + i16] = y;
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int id = lane + 64 * c, sr = id / NCH, c8 = id % NCH;
          const int q = q0 + 4 * sr + r;
          const f32x4 y0 = *(const lds_f32x4*)(stg + sr * C::SLH + 8 * c8);
          const f32x4 y1 = *(const lds_f32x4*)(stg + sr * C::SLH + 8 * c8 + 4);
          float z[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
          if constexpr (GN) {
            float gg[8];
            unpack_row8(gg, gv[pass & 1][c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] *= swish_fast(gg[e]);
          }
          Row8<bf16> o;
          pack_row8(o, z);
          if (q < N) store_row8(O + (tokb + (REV ? N - 1 - q : q)) * ldo + (size_t)h * DV + hv * (DV / 2) + 8 * c8, o);
        }
        asm volatile("" ::: "memory");
      }
    }
  }
  copies_wait_barrier<0>();                          // no copy may land after the workgroup ends
}

// ---------------------------------------------------------------------------
bool chunk_out_o16(Elt elt, int d_k, int d_v, int chunk) {
  return elt == kBF16 && d_k == 256 && (d_v == 256 || d_v == 512) && chunk % 128 == 0;
}

// Workgroups per XCD: one per CU (one workgroup fills a CU's LDS), rounded
// down to a multiple of the row tiles per chunk; at most what the work needs.
static int o16_per_xcd(int U, int TPC) {
  static std::atomic<int> cu_count[64];             // per device, 0 = not read yet
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    cus = cu_count[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
      cu_count[dev].store(cus, std::memory_order_relaxed);
    }
  }
  const int need = ((U + 7) / 8) * TPC;
  int P = (cus / 8) / TPC * TPC;
  if (P < TPC) P = TPC;
  return P < need ? P : need;
}

template <int DV, bool STATE, bool GN, bool ROPE, bool REV = false>
static void launch_o16_t(const ChunkArgs& a, int chunk, int NC, int TPC, int has_sin, const HeadTab& tab,
                         hipStream_t st) {
  const int BH = a.batch * a.heads;
  const int U = NC * BH;
  const int P = o16_per_xcd(U, TPC);
  dim3 grid(8 * P);
  hipLaunchKernelGGL((k_chunk_o16<DV, STATE, GN, ROPE, REV>), grid, dim3(512), 0, st, (const bf16*)a.Q,
                     (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx,
                     (const bf16*)a.G, a.ldg, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC, P, a.scale,
                     a.eps, tab, a.q_rope_tab);
}

template <int DV, bool STATE>
static void launch_o16_d(const ChunkArgs& a, int chunk, int NC, int TPC, int has_sin, const HeadTab& tab,
                         hipStream_t st) {
  // the reversed passes (the backward's) carry neither the fused epilogue
  // nor the rotation
  if (a.rev_in) {
    launch_o16_t<DV, STATE, false, false, true>(a, chunk, NC, TPC, has_sin, tab, st);
    return;
  }
  if (a.fuse_gn_gate) {
    if (a.q_rope_tab) launch_o16_t<DV, STATE, true, true>(a, chunk, NC, TPC, has_sin, tab, st);
    else launch_o16_t<DV, STATE, true, false>(a, chunk, NC, TPC, has_sin, tab, st);
  } else {
    if (a.q_rope_tab) launch_o16_t<DV, STATE, false, true>(a, chunk, NC, TPC, has_sin, tab, st);
    else launch_o16_t<DV, STATE, false, false>(a, chunk, NC, TPC, has_sin, tab, st);
  }
}

hipError_t launch_out_o16(const ChunkArgs& a, bool state, int chunk, int NC, int TPC, int has_sin,
                          const HeadTab& tab, hipStream_t st) {
  if (a.d_v == 512) {
    if (state) launch_o16_d<512, true>(a, chunk, NC, TPC, has_sin, tab, st);
    else launch_o16_d<512, false>(a, chunk, NC, TPC, has_sin, tab, st);
  } else {
    if (state) launch_o16_d<256, true>(a, chunk, NC, TPC, has_sin, tab, st);
    else launch_o16_d<256, false>(a, chunk, NC, TPC, has_sin, tab, st);
  }
  return hipGetLastError();
}

}  // namespace msr
