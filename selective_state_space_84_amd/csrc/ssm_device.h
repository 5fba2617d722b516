// Device-side helpers shared by the scan and update kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

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

// v * sigmoid(v) = v / (1 + exp(-v)).  For v -> -inf the exponential
// overflows to +inf and the result is -0; NaN propagates.
__device__ __forceinline__ float silu(float v) { return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

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

}  // namespace ssm
