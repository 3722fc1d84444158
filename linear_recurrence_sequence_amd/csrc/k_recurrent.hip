// Recurrent decode step and rotation kernels for gfx950.
//
// Decode ([RN-zh] = page "Transformer取代者登場！微軟、清華剛推出RetNet：成本低、
// 速度快、性能強（2）", section "2) Retention 的循環表征", Eq. (6)): for every
// (batch, head)
//   S <- gamma S + k^T v ;   o = scale * q S
// with q, k rotated at the absolute position (section "Retention", Eq. (3)-(4),
// xPos).  The step reads and writes the d_k x d_v float32 state once, so it is
// bound by HBM bandwidth: workgroups stream the state row by row, each lane
// owning 4 contiguous d_v columns (16-byte non-temporal accesses), with 8
// rows in flight per lane.
#include "msr_launch.h"

namespace msr {

// (cos, sin) of p * theta_j, theta_j = base^(-2j/d).  The angle is reduced in
// double precision (p can be ~1e4 radians, where float32 would lose ~1e-3 of
// absolute accuracy) and evaluated as sincospi of the reduced half-turns.
// theta_j / pi of pair j
__device__ __forceinline__ double rope_w(int j, int d, float base) {
  return exp2(-2.0 * (double)j / (double)d * log2((double)base)) * 0.31830988618379067154;
}
// cos and sin of p theta_j, given w = theta_j / pi
__device__ __forceinline__ void rope_cs_w(int64_t p, double w, float* c, float* s) {
  double t = (double)p * w;
  t -= 2.0 * rint(0.5 * t);
  sincospif((float)t, s, c);
}
__device__ __forceinline__ void rope_cs(int64_t p, int j, int d, float base, float* c, float* s) {
  rope_cs_w(p, rope_w(j, d, base), c, s);
}

template <class T> __device__ __forceinline__ float ld1(const T* p) { return (float)*p; }

template <class T, class OT, int DK, int DV, int CS>
__global__ __launch_bounds__(256) void k_recurrent_step(const T* __restrict__ q, int64_t ldq, const T* __restrict__ k,
                                                        int64_t ldk, const T* __restrict__ v, int64_t ldv,
                                                        float* __restrict__ S, OT* __restrict__ o, int64_t ldo,
                                                        int H, float scale, int64_t pos, float rope_base,
                                                        HeadTab tab) {
  // CS workgroups per (batch, head), each owning DV / CS columns: the sum
  // over d_k rows of a column stays inside one workgroup, and the finer grid
  // avoids a mostly idle last round of workgroups.  The state is touched
  // exactly once per step, so its loads and stores are non-temporal.
  constexpr int CPT = 4;               // d_v columns per lane
  constexpr int SW = DV / CS;          // columns per workgroup
  constexpr int TPR = SW / CPT;        // lanes per state row
  constexpr int RG = 256 / TPR;        // rows processed in parallel
  __shared__ float sq[DK], sk[DK];
  __shared__ f32x4 red[RG][TPR];
  const int bh = blockIdx.x / CS, cs = blockIdx.x % CS, h = bh % H, b = bh / H, tid = threadIdx.x;
  const T* qb = q + (size_t)b * ldq + (size_t)h * DK;
  const T* kb = k + (size_t)b * ldk + (size_t)h * DK;
  for (int j = tid; j < DK / 2; j += 256) {
    float q0 = ld1(qb + 2 * j), q1 = ld1(qb + 2 * j + 1), k0 = ld1(kb + 2 * j), k1 = ld1(kb + 2 * j + 1);
    if (rope_base > 0.f) {
      float c, s;
      rope_cs(pos, j, DK, rope_base, &c, &s);
      const float a0 = q0 * c - q1 * s, a1 = q0 * s + q1 * c;
      const float b0 = k0 * c - k1 * s, b1 = k0 * s + k1 * c;
      q0 = a0; q1 = a1; k0 = b0; k1 = b1;
    }
    sq[2 * j] = q0; sq[2 * j + 1] = q1;
    sk[2 * j] = k0; sk[2 * j + 1] = k1;
  }
  __syncthreads();

  const int rg = tid / TPR, c = cs * SW + (tid % TPR) * CPT;
  const T* vb = v + (size_t)b * ldv + (size_t)h * DV + c;
  const f32x4 vv = {ld1(vb), ld1(vb + 1), ld1(vb + 2), ld1(vb + 3)};
  const float g = tab.gam[h];
  float* Sb = S + (size_t)bh * DK * DV + c;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int i = rg; i < DK; i += RG) {
    f32x4* p = reinterpret_cast<f32x4*>(Sb + (size_t)i * DV);
    f32x4 s = __builtin_nontemporal_load(p);
    const float ki = sk[i], qi = sq[i];
    s = g * s + ki * vv;
    __builtin_nontemporal_store(s, p);
    acc += qi * s;
  }
  red[rg][tid % TPR] = acc;
  __syncthreads();
  if (rg == 0) {
    f32x4 t = red[0][tid];
#pragma unroll
    for (int r = 1; r < RG; ++r) t += red[r][tid];
    OT* ob = o + (size_t)b * ldo + (size_t)h * DV + c;
    ob[0] = (OT)(scale * t[0]);
    ob[1] = (OT)(scale * t[1]);
    ob[2] = (OT)(scale * t[2]);
    ob[3] = (OT)(scale * t[3]);
  }
}

template <class T, int DK, int DV>
static hipError_t run_step(int batch, int heads, const StepIO& io, float* S, float scale, int64_t pos, float base,
                           const HeadTab& tab, hipStream_t st) {
  constexpr int CS = DV >= 256 ? 2 : 1;
  TraceScope ts("k_recurrent_step", st);
  const dim3 grid(batch * heads * CS);
  if (io.o_f32)
    hipLaunchKernelGGL((k_recurrent_step<T, float, DK, DV, CS>), grid, dim3(256), 0, st, (const T*)io.q, io.ldq,
                       (const T*)io.k, io.ldk, (const T*)io.v, io.ldv, S, (float*)io.o, io.ldo, heads, scale, pos,
                       base, tab);
  else
    hipLaunchKernelGGL((k_recurrent_step<T, T, DK, DV, CS>), grid, dim3(256), 0, st, (const T*)io.q, io.ldq,
                       (const T*)io.k, io.ldk, (const T*)io.v, io.ldv, S, (T*)io.o, io.ldo, heads, scale, pos,
                       base, tab);
  return hipGetLastError();
}

hipError_t launch_recurrent_step(Elt elt, int d_k, int d_v, int batch, int heads, const StepIO& io, float* S,
                                 float scale, int64_t pos, float base, const HeadTab& tab, hipStream_t st) {
#define MSR_STEP(T)                                                                                        \
  if (d_k == 64 && d_v == 64) return run_step<T, 64, 64>(batch, heads, io, S, scale, pos, base, tab, st);     \
  if (d_k == 128 && d_v == 128) return run_step<T, 128, 128>(batch, heads, io, S, scale, pos, base, tab, st); \
  if (d_k == 256 && d_v == 256) return run_step<T, 256, 256>(batch, heads, io, S, scale, pos, base, tab, st); \
  if (d_k == 256 && d_v == 512) return run_step<T, 256, 512>(batch, heads, io, S, scale, pos, base, tab, st);
  if (elt == kBF16) {
    MSR_STEP(bf16)
  } else {
    MSR_STEP(float)
  }
#undef MSR_STEP
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// GroupNorm + swish gate of a decode step ([RN-zh] "門控多尺度 Retention",
// Eq. (8)): per (batch element, head), statistics over the head's d_v
// outputs (biased variance), z = swish(g) (.) (o - mean) / sqrt(var + eps).
// One wave per (batch element, head); lane l holds columns l, l + 64, ...
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <class T, int DV>
__global__ __launch_bounds__(256) void k_gn_gate(const float* __restrict__ o, int64_t ldo, const T* __restrict__ g,
                                                 int64_t ldg, T* __restrict__ z, int64_t ldz, int rows, int H,
                                                 float eps) {
  constexpr int PER = DV / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;                         // wave-uniform; no barrier below
  const int b = row / H, h = row % H;
  const float* ob = o + (size_t)b * ldo + (size_t)h * DV + lane;
  const T* gb = g + (size_t)b * ldg + (size_t)h * DV + lane;
  T* zb = z + (size_t)b * ldz + (size_t)h * DV + lane;
  float x[PER];
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) sum += (x[e] = ob[64 * e]);
  const float mu = wave_sum(sum) * (1.0f / DV);
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) sq += (x[e] - mu) * (x[e] - mu);
  const float rs = rsqrtf(wave_sum(sq) * (1.0f / DV) + eps);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float gv = (float)gb[64 * e];
    zb[64 * e] = (T)(gv / (1.0f + __expf(-gv)) * (x[e] - mu) * rs);
  }
}

hipError_t launch_gn_gate(Elt elt, int d_v, int batch, int heads, const float* o, int64_t ldo, const void* g,
                          int64_t ldg, void* z, int64_t ldz, float eps, hipStream_t st) {
  const int rows = batch * heads;
  const dim3 grid((rows + 3) / 4);
  TraceScope ts("k_gn_gate", st);
#define MSR_GN(T, D)                                                                                    \
  if (d_v == D) {                                                                                       \
    hipLaunchKernelGGL((k_gn_gate<T, D>), grid, dim3(256), 0, st, o, ldo, (const T*)g, ldg, (T*)z, ldz, rows, \
                       heads, eps);                                                                     \
    return hipGetLastError();                                                                           \
  }
  if (elt == kBF16) {
    MSR_GN(bf16, 64) MSR_GN(bf16, 128) MSR_GN(bf16, 256) MSR_GN(bf16, 512)
  } else {
    MSR_GN(float, 64) MSR_GN(float, 128) MSR_GN(float, 256) MSR_GN(float, 512)
  }
#undef MSR_GN
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Rotation: a (cos, sin) table per call, then an elementwise pass.
// ---------------------------------------------------------------------------
// One lane per (pair j, RPL consecutive positions): theta_j / pi (float64
// exp2 and log2) once per lane; lanes of a wave take consecutive pairs, so
// every store of a position is one contiguous row segment.
constexpr int RPL = 4;
__global__ void k_rope_table(float2* tab, int npos, int d, int64_t pos0, float base) {
  const int half = d / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nblk = (npos + RPL - 1) / RPL;
  if (i >= nblk * half) return;
  const int j = (int)(i % half), n0 = (int)(i / half) * RPL;
  const double w = rope_w(j, d, base);
  for (int u = 0; u < RPL && n0 + u < npos; ++u) {
    float c, s;
    rope_cs_w(pos0 + n0 + u, w, &c, &s);
    tab[(int64_t)(n0 + u) * half + j] = make_float2(c, s);
  }
}

hipError_t launch_rope_table(float2* tab, int npos, int d, int64_t pos0, float base, hipStream_t st) {
  const int64_t n = (int64_t)((npos + RPL - 1) / RPL) * (d / 2);
  if (n == 0) return hipSuccess;
  TraceScope ts("k_rope_table", st);
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab, npos, d, pos0, base);
  return hipGetLastError();
}

// One lane rotates 4 pairs (8 contiguous elements) of one (token, head).
template <class T>
__global__ void k_rope_apply(const T* src, int64_t lds, T* dst, int64_t ldd, int rows, int seqlen, int heads, int d,
                             const float2* __restrict__ tab, float sgn) {
  const int groups = d / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)heads * groups;
  if (i >= (int64_t)rows * per_row) return;
  const int row = (int)(i / per_row);
  const int rem = (int)(i % per_row);
  const int h = rem / groups, g = rem % groups;
  const int n = row % seqlen;
  const T* s = src + (size_t)row * lds + (size_t)h * d + 8 * g;
  T* o = dst + (size_t)row * ldd + (size_t)h * d + 8 * g;
  const float2* cs = tab + (size_t)n * (d / 2) + 4 * g;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)s[e];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float2 t = cs[p];
    const float sn = sgn * t.y;
    const float a = x[2 * p], b = x[2 * p + 1];
    x[2 * p] = a * t.x - b * sn;
    x[2 * p + 1] = a * sn + b * t.x;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (T)x[e];
}

hipError_t launch_rope_apply(Elt elt, const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int seqlen,
                             int heads, int d, const float2* tab, hipStream_t st, bool inverse) {
  const int64_t n = (int64_t)rows * heads * (d / 8);
  const float sgn = inverse ? -1.f : 1.f;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  TraceScope ts("k_rope_apply", st);
  if (elt == kBF16)
    hipLaunchKernelGGL(k_rope_apply<bf16>, grid, dim3(256), 0, st, (const bf16*)src, lds, (bf16*)dst, ldd, rows,
                       seqlen, heads, d, tab, sgn);
  else
    hipLaunchKernelGGL(k_rope_apply<float>, grid, dim3(256), 0, st, (const float*)src, lds, (float*)dst, ldd, rows,
                       seqlen, heads, d, tab, sgn);
  return hipGetLastError();
}

}  // namespace msr
