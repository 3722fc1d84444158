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
//
// Work split: one workgroup of 8 waves (two per SIMD) per (batch, head,
// chunk, tile of 128 query rows); each wave owns 16 query rows and the whole
// d_v width of their outputs, so the score tile never leaves the wave and
// the accumulators (d_v = 512: 128 registers) leave room for a second wave
// per SIMD.  Stages -- d_k slabs of R_{i-1}^T, then blocks of 32 keys with
// K and V together -- stream through a ring of LDS slots filled by direct
// global->LDS copies, NS - 1 stages in flight.  Tiles are stored unpadded
// and swizzled in 16-byte units (the copies pick each lane's source so that
// the data lands swizzled), which keeps every fragment read conflict-free:
//   K   [32 keys][32 chunks]   chunk c of row r at c ^ (r & 15)
//   V   [32 keys][d_v/8]       chunk c of row r at c ^ (2 (r & 7))
//   R^T [d_v][SK/8]            chunk c of row r at c ^ f(r), f(r) = (r >> 2) & 3
//                              (SK = 32) or (r >> 1) & 7 (SK = 64)
// The tiles of one (batch, head, chunk) are dispatched to one XCD (block
// ids 8 apart), heaviest first, so K and V are fetched from HBM once per
// chunk and re-read from that XCD's L2.
//
// 16x16x32 fragments (lane l, i = l % 16, g = l / 16): A = row i, elements
// k = 8 g .. 8 g + 7; B = column i, the same k; the accumulator tile holds
// column i, rows 4 g .. 4 g + 3.  The score tile is computed transposed, S^T
// = K Q^T (keys in rows, so Q is the B operand kept in registers), in two
// 16-key halves; lane l then holds query i, keys 4 g + r and 16 + 4 g + r,
// and uses them directly as the A operand of P V with that key order; the V
// fragment is read in the same order with the transposing LDS read.
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
  static constexpr int PF = DV > 256 ? 4 : 6;
  static constexpr int SLD = DV + 8;                  // epilogue staging row (floats): 4 lane groups
                                                      // writing rows 2 apart hit disjoint banks
  static_assert(NCP % NW == 0 && RCH % (64 * NW) == 0 && RCH / 64 <= NCP, "whole copies per wave");
  static_assert(NS * STG <= 160 * 1024, "ring fits in LDS");
  static_assert(NW * 8 * SLD * 4 <= NS * STG, "epilogue staging fits in the ring");
};

}  // namespace

template <int DV, bool STATE, bool GN, bool ROPE>
__global__ __launch_bounds__(512) void k_chunk_o16(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, int64_t ldq, int64_t ldk,
    int64_t ldv, const bf16* __restrict__ Rx, int has_sin, const bf16* __restrict__ G, int64_t ldg,
    bf16* __restrict__ O, int64_t ldo, int BH, int N, int H, int chunk, int NC, int TPC, float scale, float eps,
    HeadTab tab, const float2* __restrict__ rtab) {
  using C = O16Cfg<DV>;
  constexpr int DK = C::DK, KB = C::KB, NS = C::NS, AHEAD = C::AHEAD, NJ = C::NJ, LPW = C::LPW;
  __shared__ __attribute__((aligned(1024))) char smem[NS * C::STG];

  const int tid = threadIdx.x, lane = tid & 63, i16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // block id -> (chunk unit, row tile): units 8 apart in block id share an
  // XCD; a unit's tiles are consecutive groups of 8, heaviest first
  const int U = NC * BH;
  const int xg = blockIdx.x & 7, yg = blockIdx.x >> 3;
  const int li = TPC - 1 - yg % TPC;
  const int unit = (yg / TPC) * 8 + xg;
  if (unit >= U) return;
  const int ci = unit / BH, bh = unit % BH;
  const int h = bh % H, b = bh / H;
  const int c0 = ci * chunk;
  const int r0 = c0 + li * C::RT;
  if (r0 >= N) return;
  const int q0 = r0 + 16 * wave;
  const bool active = q0 < N;                        // wave-uniform
  const float lg2 = tab.lg2[h];
  const size_t tokb = (size_t)b * N;

  // ---- stage list: nR slabs of R_{i-1}^T, then nKV blocks of 32 keys ----
  const bool inter = STATE && (ci > 0 || has_sin);
  const int nR = inter ? C::NR : 0;
  const int kend = min(r0 + C::RT, N);
  const int nKV = (kend - c0 + KB - 1) / KB;
  const int nst = nR + nKV;
  const bf16* Rt = STATE ? Rx + ((size_t)bh * NC + ci) * DV * DK : nullptr;
  const bf16* Kh = K + (size_t)h * DK + tokb * ldk;
  const bf16* Vh = V + (size_t)h * DV + tokb * ldv;
  const int ldk32 = (int)ldk, ldv32 = (int)ldv;
  // LDS addresses are 32-bit (so that constant parts fold into the
  // instructions' offsets)
  lds_char* const lds = (lds_char*)smem;
  auto slot = [&](int s) { return lds + (s % NS) * C::STG; };

  // Byte offsets (from the block's first row) of this lane's copies: copy t
  // of this wave fills 16-byte slots 64 (wave LPW + t) + lane of the stage.
  // Rows past the sequence end are clamped to its last row (lim): such keys
  // are in the future of every stored query, so their weights are 0.
  // (unsigned arithmetic throughout: the divisions are shifts, and no
  // per-lane condition becomes a branch)
  auto kv_off = [&](int t, int lim) -> uint32_t {
    const uint32_t u = (uint32_t)((wave * LPW + t) * 64 + lane);
    const uint32_t ul = (uint32_t)lim;
    const uint32_t rk = u / C::CPK, ck = (u % C::CPK) ^ (rk & 15u);
    const uint32_t v = u - C::KCH, rv = v / C::CPV, cv = (v % C::CPV) ^ (2u * (rv & 7u));
    const uint32_t ok = (min(rk, ul) * (uint32_t)ldk32 + 8u * ck) * 2u;
    const uint32_t ov = (min(rv, ul) * (uint32_t)ldv32 + 8u * cv) * 2u;
    return u < (uint32_t)C::KCH ? ok : ov;           // both formed: a select, not a branch
  };
  // R stages: rows of the R^T slab; copies past the slab (d_v = 512) re-read
  // its first 16 bytes into the unused tail of the slot, so that every stage
  // issues LPW copies
  auto r_off = [&](int t) -> uint32_t {
    const uint32_t u = (uint32_t)((wave * LPW + t) * 64 + lane);
    const uint32_t r = u / C::CPR, p = u % C::CPR;
    const uint32_t c = DV > 256 ? (p ^ ((r >> 2) & 3u)) : (p ^ ((r >> 1) & 7u));
    return ((r * DK + 8u * c) * 2u) & (0u - (uint32_t)(u < (uint32_t)C::RCH));
  };
  // one stage's copies: wave-uniform sources, LDS destination and kind; the
  // per-lane offsets are formed as each copy is issued (a few integer
  // operations), which keeps them out of the registers the accumulators need.
  // Stages past the last one copy the last again into a free slot, so that
  // every stage issues the same copies and the waits are fixed.
  struct Cp { const bf16* src[2]; uint32_t dst; int lim; bool rs; };
  auto prep = [&](int s, Cp& c) {
    const int idx = min(s, nst - 1);
    c.dst = (uint32_t)(uintptr_t)slot(s) + wave * LPW * 1024;
    c.rs = idx < nR;
    if (c.rs) {
      c.src[0] = c.src[1] = Rt + idx * C::SK;
      c.lim = KB - 1;
    } else {
      const int kb = c0 + (idx - nR) * KB;
      c.lim = min(KB - 1, N - 1 - kb);
      c.src[0] = Kh + (size_t)kb * ldk;
      c.src[1] = Vh + (size_t)kb * ldv;
    }
  };
  auto cp = [&](const Cp& c, int t) {
    const int ii = wave * LPW + t;                   // wave-uniform
    // both offsets formed and blended without a branch (a branch here would
    // cut the matrix-core sequences it sits in into separate blocks)
    const uint32_t msk = 0u - (uint32_t)c.rs;
    const uint32_t off = (r_off(t) & msk) | (kv_off(t, c.lim) & ~msk);
    copy16_to_lds(uniform_ptr(ii < C::KCH / 64 ? c.src[0] : c.src[1]), off,
                  __builtin_amdgcn_readfirstlane(c.dst + t * 1024));
  };
  {
    Cp c;
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) {
      prep(a, c);
#pragma unroll
      for (int t = 0; t < LPW; ++t) cp(c, t);
    }
  }

  // Query rows as fragments: element e of fragment s is column 32 s + 8 g + e
  // of row q0 + i16 (rows past the end clamped, never stored); rotated here
  // when a (cos, sin) table is given: the pair (2j, 2j+1) at position n turns
  // by n theta_j ([RN-zh] section "Retention", Eq. (3)-(4)).
  bf16x8 qf[DK / 32];
  {
    const int qr = min(q0 + i16, N - 1);
    const bf16* p = Q + (tokb + qr) * ldq + (size_t)h * DK + 8 * g;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(p + 32 * s);
    if constexpr (ROPE) {
      const float2* tp = rtab + (size_t)qr * (DK / 2) + 4 * g;
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        const f32x4 cs0 = *reinterpret_cast<const f32x4*>(tp + 16 * s);
        const f32x4 cs1 = *reinterpret_cast<const f32x4*>(tp + 16 * s + 2);
        const float cs[8] = {cs0[0], cs0[1], cs0[2], cs0[3], cs1[0], cs1[1], cs1[2], cs1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = (float)qf[s][2 * j], x1 = (float)qf[s][2 * j + 1];
          const float c = cs[2 * j], sn = cs[2 * j + 1];
          qf[s][2 * j] = (bf16)(x0 * c - x1 * sn);
          qf[s][2 * j + 1] = (bf16)(x0 * sn + x1 * c);
        }
      }
    }
  }
  // retire the Q loads here (with the copies issued before them): a wait for
  // them left inside the loop would drain the copies in flight
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) asm volatile("" ::"v"(qf[s]));

  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  Cp cn;
  auto advance = [&](int idx) {
    copies_wait_barrier<(AHEAD - 1) * LPW>();
    prep(idx + AHEAD, cn);
  };

  // ---- Q R_{i-1}: acc[jt] += Q[:, slab] R^T[16 jt .., slab]^T ----
  // lane reads R^T row 16 jt + i16, chunk 4 s2 + g (swizzled by f(row),
  // which does not depend on jt)
  const int fr = DV > 256 ? ((i16 >> 2) & 3) : ((i16 >> 1) & 7);
  if (inter) {
    static_for<C::NR>([&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      advance(sl);
      // (per-lane parts made opaque, as in the key loop below)
      uint32_t rl[C::SK / 32];
#pragma unroll
      for (int s2 = 0; s2 < C::SK / 32; ++s2) rl[s2] = (uint32_t)(i16 * (C::CPR * 16) + 16 * ((4 * s2 + g) ^ fr));
      asm volatile("" : "+v"(rl[0]));
      if constexpr (C::SK / 32 > 1) asm volatile("" : "+v"(rl[C::SK / 32 - 1]));
      const lds_char* sR = slot(sl);
      constexpr int T = NJ * (C::SK / 32);         // steps: tile jt = t / (SK/32), k-step t % (SK/32)
      auto rd = [&](int t) {
        const int jt = t / (C::SK / 32), s2 = t % (C::SK / 32);
        return *(const lds_bf16x8*)(sR + rl[s2] + jt * (16 * C::CPR * 16));
      };
      constexpr int PF = C::PF;
      bf16x8 rf[PF + 1];
#pragma unroll
      for (int t = 0; t < PF; ++t) rf[t] = rd(t);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (t + PF < T) rf[(t + PF) % (PF + 1)] = rd(t + PF);
        mma_16x32(acc[t / (C::SK / 32)], qf[sl * (C::SK / 32) + t % (C::SK / 32)], rf[t % (PF + 1)]);
        if (t < LPW) cp(cn, t);                      // next stages' copies between the MFMAs
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (t + PF < T) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // rows scaled by scale * xi_t = scale * gamma^(t + 1), t = row in the chunk
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = scale * gpow(q0 - c0 + 4 * g + r + 1, lg2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j][r] *= x;
    }
  }

  // ---- key blocks ----
  // Decay gamma^n from the hardware exp2 of n log2(gamma), log2(0) = -inf
  // replaced by a large finite value so that n = 0 gives exactly 1 (0^0 = 1
  // on the diagonal) and n > 0 underflows to 0.  Off the diagonal block
  // (every key before every row of the wave) gamma^(q - k) = u * w[e] with
  // u = gamma^(q0 - kb - 31) for the wave and w[e] = gamma^(31 + i16 - 16
  // (e / 4) - 4 g - e % 4) per lane, both exponents >= 0.
  const float lg2f = fmaxf(lg2, -1.0e30f);
  auto pw = [&](int n) { return __builtin_amdgcn_exp2f((float)n * lg2f); };
  float wk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wk[e] = scale * pw(31 + i16 - 16 * (e >> 2) - 4 * g - (e & 3));
  // K fragment (key half ks, step s): row 16 ks + i16, chunk 4 s + g,
  // swizzled to (4 s + g) ^ i16 -- for s >= 4 that is 16 + ((4 (s - 4) + g) ^ i16)
  const uint32_t kbase = (uint32_t)(i16 * (C::CPK * 16));
  // V fragment (tile jt, key half hr): lane 16 g + 4 jj + m addresses row
  // 16 hr + 4 g + jj, columns 16 jt + 4 m .. + 3: chunk 2 jt + m / 2, swizzled
  // by 2 w, w = (4 g + jj) & 7, to 16 (jt >> 3) + 2 ((jt & 7) ^ w) + m / 2
  const int jj = i16 >> 2, m = i16 & 3, wv = (4 * g + jj) & 7;
  const uint32_t vbase = (uint32_t)(C::KCH * 16 + (4 * g + jj) * (C::CPV * 16) + 16 * (m >> 1) + 8 * (m & 1));

  int idx = nR;
  for (; idx < nst; ++idx) {
    advance(idx);
    const lds_char* sb = slot(idx);
    // per-lane bases made opaque each stage: otherwise every (lane part +
    // constant) sum of the unrolled reads is hoisted out of the loop into its
    // own register instead of folding the constant into the read's offset
    uint32_t kb_l = kbase, vb_l = vbase, wv_l = (uint32_t)wv;
    asm volatile("" : "+v"(kb_l), "+v"(vb_l), "+v"(wv_l));
    const int kb = c0 + (idx - nR) * KB;
    // Every wave runs every key block: P is exactly 0 for keys in its future
    // (and its results are not stored when it has no rows), so there is one
    // code path for the accumulators -- a skip branch would make them a
    // loop-carried merge that the compiler copies (twice the registers).
    {
      f32x4 st[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
      // S^T: 16 steps (k-step s = t / 2, key half ks = t % 2), fragments read
      // two steps ahead
      {
        constexpr int T = 2 * (DK / 32);
        auto rd = [&](int t) {
          const int s = t >> 1, ks = t & 1;
          return *(const lds_bf16x8*)(sb + kb_l + 16 * ((4 * (s & 3) + g) ^ i16) + (s >> 2) * 256 +
                                      ks * (16 * C::CPK * 16));
        };
        constexpr int PF = C::PF;
        bf16x8 kf[PF + 1];
#pragma unroll
        for (int t = 0; t < PF; ++t) kf[t] = rd(t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if (t + PF < T) kf[(t + PF) % (PF + 1)] = rd(t + PF);
          mma_16x32(st[t & 1], kf[t % (PF + 1)], qf[t >> 1]);
          if (t < LPW) cp(cn, t);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if (t + PF < T) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // P = S * scale * gamma^(q - k) for k <= q, else 0 (query q0 + i16, key
      // kb + 16 (e / 4) + 4 g + e % 4)
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
      // P V: one step per 16-column tile, V fragments two steps ahead
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
        for (int t = 0; t < PF; ++t) vq[t] = rd(t);
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
  }
  copies_wait_barrier<0>();                          // no copy may land after the workgroup ends

  // ---- epilogue: lane holds column 16 jt + i16 of rows q0 + 4 g + r ----
  if (!active) return;
  float mu[4], rs[4];
  if constexpr (GN) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) sum += acc[j][r];
      mu[r] = row16_sum(sum) * (1.0f / DV);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float d = acc[j][r] - mu[r];
        sum += d * d;
      }
      rs[r] = rsqrtf(row16_sum(sum) * (1.0f / DV) + eps);
    }
  }
  // Rows go through this wave's part of the (now idle) ring, 8 at a time
  // (registers r = 2 rh, 2 rh + 1 of each lane group), so that each lane then
  // takes whole 8-column chunks: 16-byte gate loads and output stores.
  lds_float* stg = (lds_float*)lds + wave * 8 * C::SLD;
  constexpr int CH = 8 * (DV / 8) / 64;              // 8-column chunks per lane per pass
#pragma unroll
  for (int rh = 0; rh < 2; ++rh) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = 2 * rh + rr;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float y = GN ? (acc[j][r] - mu[r]) * rs[r] : acc[j][r];
        stg[(2 * g + rr) * C::SLD + 16 * j + i16] = y;
      }
    }
    asm volatile("" ::: "memory");
    Row8<bf16> gv[CH];
    if constexpr (GN) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int id = lane + 64 * k, sr = id / (DV / 8), c8 = id % (DV / 8);
        const int q = min(q0 + 4 * (sr >> 1) + 2 * rh + (sr & 1), N - 1);
        load_row8(gv[k], G + (tokb + q) * ldg + (size_t)h * DV + 8 * c8, true);
      }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int id = lane + 64 * k, sr = id / (DV / 8), c8 = id % (DV / 8);
      const int q = q0 + 4 * (sr >> 1) + 2 * rh + (sr & 1);
      const f32x4 y0 = *(const lds_f32x4*)(stg + sr * C::SLD + 8 * c8);
      const f32x4 y1 = *(const lds_f32x4*)(stg + sr * C::SLD + 8 * c8 + 4);
      float z[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      if constexpr (GN) {
        float gg[8];
        unpack_row8(gg, gv[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] *= swish_fast(gg[e]);
      }
      Row8<bf16> o;
      pack_row8(o, z);
      if (q < N) store_row8(O + (tokb + q) * ldo + (size_t)h * DV + 8 * c8, o);
    }
    asm volatile("" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
bool chunk_out_o16(Elt elt, int d_k, int d_v, int chunk) {
  return elt == kBF16 && d_k == 256 && (d_v == 256 || d_v == 512) && chunk % 128 == 0;
}

template <int DV, bool STATE, bool GN, bool ROPE>
static void launch_o16_t(const ChunkArgs& a, int chunk, int NC, int TPC, int has_sin, const HeadTab& tab,
                         hipStream_t st) {
  const int BH = a.batch * a.heads;
  const int U = NC * BH;
  dim3 grid(((U + 7) / 8) * 8 * TPC);
  hipLaunchKernelGGL((k_chunk_o16<DV, STATE, GN, ROPE>), grid, dim3(512), 0, st, (const bf16*)a.Q,
                     (const bf16*)a.K, (const bf16*)a.V, a.ldq, a.ldk, a.ldv, (const bf16*)a.Rx, has_sin,
                     (const bf16*)a.G, a.ldg, (bf16*)a.O, a.ldo, BH, a.seqlen, a.heads, chunk, NC, TPC, a.scale,
                     a.eps, tab, a.q_rope_tab);
}

template <int DV, bool STATE>
static void launch_o16_d(const ChunkArgs& a, int chunk, int NC, int TPC, int has_sin, const HeadTab& tab,
                         hipStream_t st) {
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
