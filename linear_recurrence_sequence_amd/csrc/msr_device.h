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

namespace msr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxHeads = 128;

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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16 a = (bf16)lo, b = (bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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

// Transposing store: rows r[0..3] are 4 consecutive source rows (k, k+1,
// k+2, k+3) of 8 consecutive columns c..c+7.  Writes dst[(c+e)*ld + k + 0..3]
// for e = 0..7, i.e. the tile lands column-major (the reduction index k
// contiguous) as the matrix-core fragments want it.
__device__ __forceinline__ void store_transposed4x8(bf16* dst, int ld, const Row8<bf16>* r) {
  const uint32_t w0[4] = {r[0].u.x, r[0].u.y, r[0].u.z, r[0].u.w};
  const uint32_t w1[4] = {r[1].u.x, r[1].u.y, r[1].u.z, r[1].u.w};
  const uint32_t w2[4] = {r[2].u.x, r[2].u.y, r[2].u.z, r[2].u.w};
  const uint32_t w3[4] = {r[3].u.x, r[3].u.y, r[3].u.z, r[3].u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint2 even, odd;
    even.x = (w0[i] & 0xffffu) | (w1[i] << 16);
    even.y = (w2[i] & 0xffffu) | (w3[i] << 16);
    odd.x = (w0[i] >> 16) | (w1[i] & 0xffff0000u);
    odd.y = (w2[i] >> 16) | (w3[i] & 0xffff0000u);
    *reinterpret_cast<uint2*>(dst + (2 * i) * ld) = even;
    *reinterpret_cast<uint2*>(dst + (2 * i + 1) * ld) = odd;
  }
}
__device__ __forceinline__ void store_transposed4x8(float* dst, int ld, const Row8<float>* r) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(&r[0]);
  const uint32_t* b = reinterpret_cast<const uint32_t*>(&r[1]);
  const uint32_t* c = reinterpret_cast<const uint32_t*>(&r[2]);
  const uint32_t* d = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint4*>(dst + e * ld) = make_uint4(a[e], b[e], c[e], d[e]);
}

// Butterfly sum over the 32 lanes of one half-wave (xor masks < 32 stay
// inside the half).
__device__ __forceinline__ float half_wave_sum(float x) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace msr
