// Device-side building blocks shared by the libmsr kernels (gfx950 / CDNA4).
//
// Matrix-core convention used throughout: one "k16 step" multiplies a 32x16
// A fragment by a 16x32 B fragment into a 32x32 float32 accumulator tile.
//   * bf16: one v_mfma_f32_32x32x16_bf16.
//   * f32 : eight v_mfma_f32_32x32x2_f32 (k = 2 per instruction).
// Per lane (lane = 0..63, lr = lane % 32, hh = lane / 32) a fragment holds 8
// elements: A fragment = row lr, B fragment = column lr, and element t (0..7)
// of lane half hh is reduction index kmap(hh, t).  The hardware pairs A and B
// by (hh, t), so any kmap works as long as A and B use the same one.  The
// accumulator tile C[i][j] lives in lane j + 32*((i/4)%2), register
// (i%4) + 4*(i/8), i.e. lane owns column lr and rows 8*(r/4) + 4*hh + r%4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>
#include <utility>

namespace msr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxHeads = 128;

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1: a loop whose index
// is a compile-time constant in the body.
template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier (LLVM AMDGPU
// scheduling-group masks).
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200 };

// Per-head decay constants, computed on the host in double precision and
// passed by value: log2(gamma_h) (-inf when gamma_h == 0), gamma_h^chunk,
// gamma_h^L of the last (possibly short) chunk, and gamma_h itself.
struct HeadTab {
  float lg2[kMaxHeads];
  float gchunk[kMaxHeads];
  float glast[kMaxHeads];
  float gam[kMaxHeads];
};

// gamma^n for an integer n >= 0 from log2(gamma); gamma^0 == 1 also when
// gamma == 0 (lg2 == -inf).
__device__ __forceinline__ float gpow(int n, float lg2) {
  float e = exp2f((float)n * lg2);
  return n == 0 ? 1.0f : e;
}

template <class T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ void mma16(f32x16& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[t], b.v[t], c, 0, 0, 0);
}

// 8 contiguous elements (16-byte aligned for bf16, 32-byte span for f32).
__device__ __forceinline__ Frag<bf16> load_frag(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> load_frag(const float* p) {
  Frag<float> f;
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
// Two groups of 4 contiguous elements (elements 0-3 from p0, 4-7 from p1).
__device__ __forceinline__ Frag<bf16> load_frag2(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  Frag<bf16> f;
  f.v = (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
__device__ __forceinline__ Frag<float> load_frag2(const float* p0, const float* p1) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p0);
  f32x4 b = *reinterpret_cast<const f32x4*>(p1);
  Frag<float> f;
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
template <class T> __device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = (T)0.0f;
  return f;
}
template <class T> __device__ __forceinline__ Frag<T> frag_from(const float* x) {
  Frag<T> f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = (T)x[t];
  return f;
}

// ---------------------------------------------------------------------------
// 16-byte global <-> register moves of 8 elements ("row8").
// ---------------------------------------------------------------------------
template <class T> struct Row8;
template <> struct Row8<bf16> { uint4 u; };                 // 8 x bf16
template <> struct Row8<float> { uint4 lo, hi; };           // 8 x f32

__device__ __forceinline__ void load_row8(Row8<bf16>& r, const bf16* p, bool ok) {
  r.u = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void load_row8(Row8<float>& r, const float* p, bool ok) {
  if (ok) {
    r.lo = *reinterpret_cast<const uint4*>(p);
    r.hi = *reinterpret_cast<const uint4*>(p + 4);
  } else {
    r.lo = r.hi = make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void store_row8(bf16* p, const Row8<bf16>& r) {
  *reinterpret_cast<uint4*>(p) = r.u;
}
__device__ __forceinline__ void store_row8(float* p, const Row8<float>& r) {
  *reinterpret_cast<uint4*>(p) = r.lo;
  *reinterpret_cast<uint4*>(p + 4) = r.hi;
}
// One element as loaded, not yet converted: a bf16 stays zero-extended in its
// own 32-bit register until used (converting -- or packing two per register
// -- right after the load would make the load complete at once).
template <class T> struct RawElt;
template <> struct RawElt<bf16> {
  using type = uint32_t;
  static __device__ __forceinline__ uint32_t load(const bf16* p) { return *reinterpret_cast<const uint16_t*>(p); }
  static __device__ __forceinline__ float value(uint32_t r) { return __uint_as_float(r << 16); }
};
template <> struct RawElt<float> {
  using type = float;
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float value(float r) { return r; }
};

// swish(x) = x sigmoid(x) from the hardware exp2 and reciprocal (about 2 ulp).
__device__ __forceinline__ float swish_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// Non-temporal variants for the GEMM's output tiles (the stores of a whole
// tile leave at once; marked streaming they stall the next tile's loads
// less -- measured faster for the projection GEMM and for the kernels that
// read its output; slower where the next kernel re-reads a smaller output).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t as_u32x4(uint4 u) { return u32x4_t{u.x, u.y, u.z, u.w}; }
__device__ __forceinline__ void store_row8_nt(bf16* p, const Row8<bf16>& r) {
  __builtin_nontemporal_store(as_u32x4(r.u), reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_row8_nt(float* p, const Row8<float>& r) {
  __builtin_nontemporal_store(as_u32x4(r.lo), reinterpret_cast<u32x4_t*>(p));
  __builtin_nontemporal_store(as_u32x4(r.hi), reinterpret_cast<u32x4_t*>(p + 4));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two floats rounded (to nearest even) to a bf16 pair in one 32-bit word:
// written as a vector conversion, one v_cvt_pk_bf16_f32.
typedef float f32x2_pk __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_pk __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_pk){lo, hi}, bf16x2_pk));
}

__device__ __forceinline__ void pack_row8(Row8<bf16>& r, const float* v) {
  r.u = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
}
__device__ __forceinline__ void pack_row8(Row8<float>& r, const float* v) {
  r.lo = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  r.hi = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7]));
}

__device__ __forceinline__ void unpack_row8(float* v, const Row8<bf16>& r) {
  const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
}
__device__ __forceinline__ void unpack_row8(float* v, const Row8<float>& r) {
  const uint32_t w[8] = {r.lo.x, r.lo.y, r.lo.z, r.lo.w, r.hi.x, r.hi.y, r.hi.z, r.hi.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
}

// Rotate the 4 interleaved pairs (x[2p], x[2p+1]) of an 8-element row (or
// fragment) by the angles whose (cos, sin) are cs[0..3] (32-byte aligned):
// ([RN-zh] section "Retention", Eq. (3)-(4)): (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).
__device__ __forceinline__ void rotate8(float* x, const float2* __restrict__ cs) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(cs), b = *reinterpret_cast<const f32x4*>(cs + 2);
  const float c[4] = {a[0], a[2], b[0], b[2]}, sn[4] = {a[1], a[3], b[1], b[3]};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = x[2 * q], x1 = x[2 * q + 1];
    x[2 * q] = x0 * c[q] - x1 * sn[q];
    x[2 * q + 1] = x0 * sn[q] + x1 * c[q];
  }
}
template <class T>
__device__ __forceinline__ void rotate_row8(Row8<T>& r, const float2* __restrict__ cs) {
  float x[8];
  unpack_row8(x, r);
  rotate8(x, cs);
  pack_row8(r, x);
}
template <class T>
__device__ __forceinline__ void rotate_frag(Frag<T>& f, const float2* __restrict__ cs) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)f.v[e];
  rotate8(x, cs);
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (T)x[e];
}

// Multiply the 8 elements of a row by s (rounding back to the storage type).
__device__ __forceinline__ void scale_row8(Row8<bf16>& r, float s) {
  uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16(bf16_lo(w[i]) * s, bf16_hi(w[i]) * s);
  r.u = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void scale_row8(Row8<float>& r, float s) {
  r.lo = make_uint4(__float_as_uint(__uint_as_float(r.lo.x) * s), __float_as_uint(__uint_as_float(r.lo.y) * s),
                    __float_as_uint(__uint_as_float(r.lo.z) * s), __float_as_uint(__uint_as_float(r.lo.w) * s));
  r.hi = make_uint4(__float_as_uint(__uint_as_float(r.hi.x) * s), __float_as_uint(__uint_as_float(r.hi.y) * s),
                    __float_as_uint(__uint_as_float(r.hi.z) * s), __float_as_uint(__uint_as_float(r.hi.w) * s));
}

// ---------------------------------------------------------------------------
// Fragments of a matrix stored row-major [k][n] (n contiguous) in LDS, i.e.
// with the reduction index strided.  This lane receives column lr of the
// 32-column tile starting at `tile` and, as element t = 4p + j, row
// koff(p, hh) + j, where koff = 8 hh + 4 p (KMAP_CONTIG: the same order as a
// k-contiguous fragment) or 8 p + 4 hh (KMAP_ACC: the key order of a 32x32
// accumulator tile reused as an A operand, see k_chunk_out).
//
// bf16 uses the gfx950 transposing LDS read ds_read_b64_tr_b16: within each
// group of 16 lanes, lane i receives as element j the (i % 4)-th 16-bit value
// of the 8 bytes addressed by lane 4 j + i / 4.  So lane 4 j + q of group g
// (hh = g / 2, column half c = g % 2) addresses row koff + j, columns
// 16 c + 4 q .. + 3; two reads (p = 0, 1) give the 8 elements.  With a row
// stride of 16 or 48 banks (mod 64) the 32 lanes serviced together touch 64
// distinct banks.  f32 has no such instruction: 8 scalar reads.
// ---------------------------------------------------------------------------
enum { KMAP_CONTIG = 0, KMAP_ACC = 1 };

template <int KM>
__device__ __forceinline__ Frag<bf16> load_frag_rm(const bf16* tile, int ld) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  const int hh = g >> 1, c = g & 1, j = i >> 2, q = i & 3;
  Frag<bf16> f;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int koff = KM == KMAP_CONTIG ? 8 * hh + 4 * p : 8 * p + 4 * hh;
    const bf16* a = tile + (koff + j) * ld + 16 * c + 4 * q;
    const bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)a);
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[4 * p + e] = r[e];
  }
  return f;
}

template <int KM>
__device__ __forceinline__ Frag<float> load_frag_rm(const float* tile, int ld) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, hh = lane >> 5;
  Frag<float> f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int p = t >> 2, j = t & 3;
    const int koff = KM == KMAP_CONTIG ? 8 * hh + 4 * p : 8 * p + 4 * hh;
    f.v[t] = tile[(koff + j) * ld + lr];
  }
  return f;
}

// Row padding (elements) of a row-major tile read with load_frag_rm: bf16
// rows of a multiple of 128 bytes get 64 bytes more, making the stride 16 or
// 48 banks mod 64.
template <class T> constexpr int rm_pad() { return sizeof(T) == 2 ? 32 : 4; }

// ---------------------------------------------------------------------------
// Direct global -> LDS copies (gfx950 global_load_lds_dwordx4).  Each lane
// copies 16 bytes from gbase + its own byte offset to LDS address
// lds + 16 * lane, so one instruction fills 1 KiB of LDS and no register
// holds the data while it is in flight.  gbase and lds must be wave-uniform.
// The copy is issued from inline asm: the compiler's own wait insertion
// does not model these LDS writes precisely and would otherwise wait for
// every copy in flight before each LDS read.  In exchange the caller waits
// for its copies itself (copies_wait_barrier) and, because vector-memory
// loads complete in issue order, counts every vector load it issued after
// the copies it waits for.  The copy asm carries no memory clobber, so the
// compiler may move LDS reads across it: callers never copy into an LDS
// region that is being read, and the ordering that matters -- copies into
// a region only after every wave has left it, reads only after the copies
// landed -- goes through copies_wait_barrier, which is a compiler memory
// barrier.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

__device__ __forceinline__ void copy16_to_lds(const void* gbase, uint32_t byte_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(byte_off), "s"(gbase), "s"(lds) : "m0");
}

// Wait until at most N vector-memory loads of this wave are outstanding and
// all its LDS operations are done, then the workgroup barrier.
template <int N>
__device__ __forceinline__ void copies_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Butterfly sum over the 32 lanes of one half-wave (xor masks < 32 stay
// inside the half).
// Sum over the 32 lanes of each half of the wave, returned to all of them,
// with lane moves (DPP) instead of LDS round trips: quad exchanges, then the
// half-row and row mirrors give every lane its 16-lane row sum; a row
// broadcast adds row 0 into row 1 and row 2 into row 3, whose last lanes
// (31 and 63) then hold the two half sums.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float half_wave_sum(float x) {
  x = dpp_add<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x141>(x);   // row_half_mirror
  x = dpp_add<0x140>(x);   // row_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));   // row_bcast:15, rows 1 and 3
  // (readlane is integer-typed: move the bits, not a converted value)
  const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  return (__lane_id() & 32) ? s1 : s0;
}

}  // namespace msr
