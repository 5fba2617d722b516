// Device-side helpers shared by the scan and update kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 is carried as its raw 16-bit pattern.  Widening to fp32 puts the 16
// bits in the top half of the word (exact).
__device__ __forceinline__ float io_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
__device__ __forceinline__ float io_to_f32(float v) { return v; }

// Narrowing with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ void io_store(uint16_t* p, float v) { *p = __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ void io_store(float* p, float v) { *p = v; }

// 2^v on the hardware transcendental unit (no range reduction or denormal
// fix-up; results below the normal range flush towards zero).
__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Turn-taking between the waves that share a SIMD.  The issue arbiter favours
// the older of two waves; with equal work per wave (the Mamba-1.4B layer's
// scan and backward launch exactly two per SIMD) the older wave of the scan
// finished in ~1370 us and the younger in ~1625 us, which then ran alone for
// the last 15%.  Waves of odd and even slots (HW_ID bits 3:0, read through
// hwreg(HW_REG_HW_ID, 0, 32)) instead take the higher priority in turns, one
// block each: both then finish within ~5% of each other (scan 1.64 -> 1.56
// ms, backward from checkpoints 7.30 -> 6.91 ms; results unchanged).
__device__ __forceinline__ int wave_slot_parity() { return (int)(__builtin_amdgcn_s_getreg(4 | (31 << 11)) & 1u); }
__device__ __forceinline__ void take_turn(int block, int parity) {
  if ((block + parity) & 1) {
    __builtin_amdgcn_s_setprio(1);
  } else {
    __builtin_amdgcn_s_setprio(0);
  }
}
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }
__device__ __forceinline__ float hw_log2(float v) { return __builtin_amdgcn_logf(v); }

// softplus(raw + bias) = log(1 + e^v), v = raw + bias, to about 2 ulp of the
// value at the exact sum.  softplus(v) ~ e^v for v < 0 has relative
// condition number |v|, so the rounding of raw + bias alone would cost ~|v|/2
// ulp; the sum is therefore kept as vh + vl (Knuth's two-sum, exact).  Then
// softplus(v) = max(v, 0) + log1p(t) with t = e^-|v| in (0, 1]:
//  * t = 2^(a log2 e), a = -|v|: the exponent is split into yh + yl (the
//    rounding of yh, log2(e)'s low part and vl's share), so t = th + tl with
//    th = 2^yh from the hardware unit and tl = th * yl * ln2 (first order);
//  * log1p(t) = 2 atanh(s) with s = t / (2 + t) <= 1/3 (the atanh series
//    of log((1 + s) / (1 - s))): s0 = th / d with d = 2 + th rounded, then one
//    residual step on (th + tl) - s0 (d + dl + tl), dl = d's rounding error
//    (exact), gives s to ~0.5 ulp; the series tail 2s (s^2/3 + ... + s^14/15)
//    is below 4% of the result, so its own rounding hardly shows.
// For |v| beyond 1e30 the low part is dropped and below -200 the exponent is
// clamped (+inf stays +inf, -inf gives 0); NaN propagates.  Results below
// fp32's normal range flush towards zero.
constexpr float kLog2eLo = 1.925963e-8f;  // log2(e) - (float)log2(e)
__device__ __forceinline__ float softplus(float raw, float bias) {
  const float vh = raw + bias;
  const float bb = vh - raw;
  const float vl = __builtin_fabsf(vh) < 1e30f ? (raw - (vh - bb)) + (bias - bb) : 0.0f;
  const bool pos = vh > 0.0f;
  float a = pos ? -vh : vh;
  a = a < -200.0f ? -200.0f : a;  // e^-200 is 0 in fp32; keeps -inf out of the exponent (NaN passes)
  const float al = pos ? -vl : vl;
  const float yh = a * kLog2e;
  const float yl = __builtin_fmaf(a, kLog2e, -yh) + __builtin_fmaf(al, kLog2e, a * kLog2eLo);
  const float th = hw_exp2(yh);
  const float tl = th * (yl * kLn2);
  const float d = 2.0f + th;
  const float dl = th - (d - 2.0f);
  const float r = hw_rcp(d);
  const float s0 = th * r;
  float e = __builtin_fmaf(-s0, d, th);
  e = __builtin_fmaf(-s0, dl + tl, e + tl);
  const float s = __builtin_fmaf(e, r, s0);
  const float z = s * s;
  float q = 1.0f / 15.0f;
  q = __builtin_fmaf(q, z, 1.0f / 13.0f);
  q = __builtin_fmaf(q, z, 1.0f / 11.0f);
  q = __builtin_fmaf(q, z, 1.0f / 9.0f);
  q = __builtin_fmaf(q, z, 1.0f / 7.0f);
  q = __builtin_fmaf(q, z, 1.0f / 5.0f);
  q = __builtin_fmaf(q, z, 1.0f / 3.0f);
  const float s2 = s + s;
  const float lp = __builtin_fmaf(s2, z * q, s2);
  return pos ? vh + (lp + vl) : lp;
}

// v * sigmoid(v) = v / (1 + exp(-v)).  For v -> -inf the exponential
// overflows to +inf and the result is -0; NaN propagates.
__device__ __forceinline__ float silu(float v) { return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// Coefficient of B*x in the exact zero-order hold, (exp(delta a) - 1) / a,
// from y = delta * a * log2(e), abar = 2^y and inv_a = 1/a:
//   |y| < 1/2: delta * phi, phi = (e^v - 1)/v = sum_k v^k/(k+1)! with v = y ln 2,
//              to 6th order (truncation < 2e-8 relative); this also covers a = 0;
//   otherwise: (abar - 1) * inv_a, where |abar - 1| > 0.29, so abar's error
//              (under 0.8 ulp) grows at most ~2.4x.
// Relative error about 3 ulp or less over the whole range.
constexpr float kZoh1 = 0.34657359f;     // ln2 / 2!
constexpr float kZoh2 = 0.080075503f;    // ln2^2 / 3!
constexpr float kZoh3 = 0.013876027f;    // ln2^3 / 4!
constexpr float kZoh4 = 0.0019236258f;   // ln2^4 / 5!
constexpr float kZoh5 = 2.2222597e-4f;   // ln2^5 / 6!
constexpr float kZoh6 = 2.2005043e-5f;   // ln2^6 / 7!
__device__ __forceinline__ float zoh_coef(float y, float abar, float delta, float inv_a) {
  float p = __builtin_fmaf(y, kZoh6, kZoh5);
  p = __builtin_fmaf(p, y, kZoh4);
  p = __builtin_fmaf(p, y, kZoh3);
  p = __builtin_fmaf(p, y, kZoh2);
  p = __builtin_fmaf(p, y, kZoh1);
  const float phi = __builtin_fmaf(p, y, 1.0f);
  const float small = delta * phi;
  const float big = __builtin_fmaf(abar, inv_a, -inv_a);
  return __builtin_fabsf(y) < 0.5f ? small : big;
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X
// (workgroup i runs on XCD i % 8).  Remap so that each XCD receives one
// contiguous range of logical workgroup ids: tiles that share B and C rows
// then share one XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  constexpr int kXcd = 8;
  const int q = n / kXcd, r = n % kXcd;
  const int xcd = i % kXcd, idx = i / kXcd;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Read-only view of global memory in the constant address space.  B and C
// are never written while a kernel runs, and loads through this address space
// with a wave-uniform address always compile to scalar loads (through a
// generic pointer the compiler must first prove that no store in the kernel
// can clobber them, and inside the sweep loop that proof fails).
typedef const uint32_t __attribute__((address_space(4)))* const_u32_ptr;
typedef const float __attribute__((address_space(4)))* const_f32_ptr;

// B/C row fragment for one wave: NS consecutive states of one (b, t), held in
// SGPRs and fed to the VALU as scalar operands.
template <typename T, int NS>
struct StateRow;

template <int NS>
struct StateRow<uint16_t, NS> {
  static_assert(NS % 2 == 0, "bf16 rows are loaded as dwords");
  uint32_t w[NS / 2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const_u32_ptr q = (const_u32_ptr)(const void*)p;
#pragma unroll
    for (int k = 0; k < NS / 2; ++k) w[k] = q[k];
  }
  // Marks the row as consumed here (an empty asm reading an SGPR), which
  // makes the compiler wait for its scalar load at this point.  The memory
  // clobber keeps later row loads from being hoisted above it.
  __device__ __forceinline__ void touch() const { asm volatile("" ::"s"(w[0]) : "memory"); }
  __device__ __forceinline__ float get(int n) const {
    const uint32_t v = w[n >> 1];
    return __builtin_bit_cast(float, (n & 1) ? (v & 0xffff0000u) : (v << 16));
  }
};

template <int NS>
struct StateRow<float, NS> {
  float w[NS];
  __device__ __forceinline__ void load(const float* p) {
    const_f32_ptr q = (const_f32_ptr)(const void*)p;
#pragma unroll
    for (int k = 0; k < NS; ++k) w[k] = q[k];
  }
  __device__ __forceinline__ void touch() const {
    asm volatile("" ::"s"(__builtin_bit_cast(uint32_t, w[0])) : "memory");
  }
  __device__ __forceinline__ float get(int n) const { return w[n]; }
};

// A wave-uniform pointer re-read through readfirstlane: the compiler then
// treats it as an opaque SGPR value.  Row pointers that move by a fixed
// amount per block are passed through this so that loop strength reduction
// does not turn "SGPR base + 32-bit lane offset" into one 64-bit per-lane
// pointer per tensor and step (which would hold ~100 VGPRs).
// The result is typed as a global-memory pointer, so loads and stores
// through it stay global (SGPR base + VGPR offset) instead of flat.
typedef char __attribute__((address_space(1))) gchar;
__device__ __forceinline__ gchar* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gchar*>(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T gldr(const gchar* base, uint32_t off) {
  return *reinterpret_cast<const T __attribute__((address_space(1)))*>(base + off);
}
template <typename T>
__device__ __forceinline__ void gstr(gchar* base, uint32_t off, T v) {
  *reinterpret_cast<T __attribute__((address_space(1)))*>(base + off) = v;
}

}  // namespace ssm
