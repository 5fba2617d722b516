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
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }
__device__ __forceinline__ float hw_log2(float v) { return __builtin_amdgcn_logf(v); }

// softplus(v) = log(1 + e^v).
//  * e^v = 2^(v log2 e): the rounding of the product v * log2(e) (|v| up to
//    ~10 here) would cost ~5e-7 relative in e^v, so the product is split into
//    hi + lo (one FMA, plus log2(e)'s own low part) and e^v is corrected to
//    first order in lo.
//  * With u = 1 + e^v rounded, log(u) loses the low bits of a small e^v; the
//    factor e^v / (u - 1) restores them (Kahan's log1p rearrangement).
// For v > 20 the result is v to fp32 precision (and e^v may overflow).
constexpr float kLog2eLo = 1.925963e-8f;  // log2(e) - (float)log2(e)
__device__ __forceinline__ float softplus(float v) {
  const float yh = v * kLog2e;
  const float yl = __builtin_fmaf(v, kLog2e, -yh) + v * kLog2eLo;
  float e = hw_exp2(yh);
  e = __builtin_fmaf(e, yl * kLn2, e);
  const float u = 1.0f + e;
  const float um1 = u - 1.0f;
  const float r = um1 == 0.0f ? e : hw_log2(u) * kLn2 * (e * hw_rcp(um1));
  return v > 20.0f ? v : r;
}

// v * sigmoid(v) = v / (1 + exp(-v)).  For v -> -inf the exponential
// overflows to +inf and the result is -0; NaN propagates.
__device__ __forceinline__ float silu(float v) { return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// Coefficient of B*x in the exact zero-order hold, (exp(delta a) - 1) / a,
// from y = delta * a * log2(e), abar = 2^y and inv_a = 1/a:
//   |y| < 1/4: delta * phi, phi = (e^v - 1)/v = sum_k v^k/(k+1)! with v = y ln 2,
//              to 4th order (truncation < 3e-7 relative); this also covers a = 0;
//   otherwise: (abar - 1) * inv_a, where abar's rounding is small against
//              abar - 1 (|abar - 1| > 0.16).
// Relative error below ~5e-7 over the whole range.
constexpr float kZoh1 = 0.3465736f;    // ln2 / 2!
constexpr float kZoh2 = 0.0800755f;    // ln2^2 / 3!
constexpr float kZoh3 = 0.013876027f;  // ln2^3 / 4!
constexpr float kZoh4 = 0.0019236258f; // ln2^4 / 5!
__device__ __forceinline__ float zoh_coef(float y, float abar, float delta, float inv_a) {
  const float phi =
      __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(__builtin_fmaf(y, kZoh4, kZoh3), y, kZoh2), y, kZoh1), y, 1.0f);
  const float small = delta * phi;
  const float big = __builtin_fmaf(abar, inv_a, -inv_a);
  return __builtin_fabsf(y) < 0.25f ? small : big;
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
