// Register-only probe of the gfx950 VALU issue rates behind the VALU-slot
// roof that bench.py reports: a stream of independent wave64 v_fmac_f32, a
// stream of v_exp_f32, and the scan's per-state mix (decay product, exp,
// readout FMA, input product, state FMA), each launched with a chosen number
// of waves per SIMD
// (1024 one-wave workgroups per wave per SIMD: 256 CUs x 4 SIMDs).  No memory
// is touched but one store per lane of the final values, at
// out[block * 64 + lane] (the caller sizes out to blocks * 64 floats).
#include <hip/hip_runtime.h>
#include <stdint.h>

#define F8(op) op op op op op op op op
template <int V>
__global__ void __launch_bounds__(64) k_rate(float* __restrict__ out, int iters) {
  // (V == 2 reads a2..a5 as the decay rates and the input terms.)
  float a0 = threadIdx.x * 1e-3f, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3, a4 = a0 + 4, a5 = a0 + 5, a6 = a0 + 6,
        a7 = a0 + 7;
  const float m = 0.999f, c = 1e-3f;
  for (int it = 0; it < iters; ++it) {
    if constexpr (V == 0) {
      // 64 FMAs in 8 independent chains.
      asm volatile(F8("v_fmac_f32 %0, %8, %9\n v_fmac_f32 %1, %8, %9\n v_fmac_f32 %2, %8, %9\n v_fmac_f32 %3, %8, %9\n"
                      "v_fmac_f32 %4, %8, %9\n v_fmac_f32 %5, %8, %9\n v_fmac_f32 %6, %8, %9\n v_fmac_f32 %7, %8, %9\n")
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                   : "v"(m), "v"(c));
    } else if constexpr (V == 2) {
      // 16 state updates (8 states, two steps) in the scan's order:
      // t = d*a_n; t = exp2(t); acc += c*h_(n-1); u = b*w; h_n = t*h_n + u.
      float t, u;
      asm volatile(
          F8("v_mul_f32 %[t], %[d], %[a0]\n v_exp_f32 %[t], %[t]\n v_fmac_f32 %[acc], %[c], %[h7]\n"
             "v_mul_f32 %[u], %[b], %[w]\n v_fma_f32 %[h0], %[t], %[h0], %[u]\n"
             "v_mul_f32 %[t], %[d], %[a1]\n v_exp_f32 %[t], %[t]\n v_fmac_f32 %[acc], %[c], %[h0]\n"
             "v_mul_f32 %[u], %[b], %[w]\n v_fma_f32 %[h1], %[t], %[h1], %[u]\n")
          : [h0] "+v"(a0), [h1] "+v"(a1), [h7] "+v"(a7), [acc] "+v"(a6), [t] "=&v"(t), [u] "=&v"(u)
          : [d] "v"(m), [a0] "v"(a2), [a1] "v"(a3), [c] "v"(c), [b] "v"(a4), [w] "v"(a5));
    } else {
      // 64 exponentials in 8 independent chains.
      asm volatile(F8("v_exp_f32 %0, %0\n v_exp_f32 %1, %1\n v_exp_f32 %2, %2\n v_exp_f32 %3, %3\n"
                      "v_exp_f32 %4, %4\n v_exp_f32 %5, %5\n v_exp_f32 %6, %6\n v_exp_f32 %7, %7\n")
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
    }
  }
  out[(int64_t)blockIdx.x * 64 + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

// kind 0: FMA stream, 1: exp stream, 2: the scan's state mix.  Returns 0,
// or -1 for a bad argument.
extern "C" int valu_rate_probe(int kind, float* out, int blocks, int iters, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipStream_t st = (hipStream_t)stream;
  if (kind == 0) {
    hipLaunchKernelGGL(k_rate<0>, dim3(blocks), dim3(64), 0, st, out, iters);
  } else if (kind == 1) {
    hipLaunchKernelGGL(k_rate<1>, dim3(blocks), dim3(64), 0, st, out, iters);
  } else if (kind == 2) {
    hipLaunchKernelGGL(k_rate<2>, dim3(blocks), dim3(64), 0, st, out, iters);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
