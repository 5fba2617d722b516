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
__global__ void __launch_bounds__(64) k_rate(float* __restrict__ out, int iters, float su) {
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
    } else if constexpr (V == 3) {
      // 64 FMAs in 8 independent chains, one operand a wave-uniform SGPR value.
      asm volatile(F8("v_fmac_f32 %0, %8, %9\n v_fmac_f32 %1, %8, %9\n v_fmac_f32 %2, %8, %9\n v_fmac_f32 %3, %8, %9\n"
                      "v_fmac_f32 %4, %8, %9\n v_fmac_f32 %5, %8, %9\n v_fmac_f32 %6, %8, %9\n v_fmac_f32 %7, %8, %9\n")
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                   : "s"(su), "v"(c));
    } else if constexpr (V == 4 || V == 5) {
      // The structured scan's state mix (decay product, input product with
      // B, state FMA, readout FMA with C; B and C wave-uniform in SGPRs), 16
      // states per iteration.  V == 4 first unpacks each bf16 B and C value on
      // the scalar unit as the compiled loop does (s_pack_*: the same cost as
      // its shift and mask, and SCC is left alone); V == 5 has them as fp32.
      float t, u;
      if constexpr (V == 4) {
        asm volatile(
            F8("v_mul_f32 %[t], %[q], %[r]\n s_pack_ll_b32_b16 s4, 0, %[b]\n v_mul_f32 %[u], s4, %[w]\n"
               "v_fmac_f32 %[u], %[t], %[h0]\n s_pack_ll_b32_b16 s5, 0, %[c]\n v_fmac_f32 %[acc], s5, %[u]\n"
               "v_mul_f32 %[t], %[q], %[r]\n s_pack_hh_b32_b16 s4, 0, %[b]\n v_mul_f32 %[h0], s4, %[w]\n"
               "v_fmac_f32 %[h0], %[t], %[h1]\n s_pack_hh_b32_b16 s5, 0, %[c]\n v_fmac_f32 %[acc], s5, %[h0]\n")
            : [h0] "+v"(a0), [h1] "+v"(a1), [acc] "+v"(a6), [t] "=&v"(t), [u] "=&v"(u)
            : [q] "v"(m), [r] "v"(a2), [c] "s"(su), [b] "s"(su), [w] "v"(a5)
            : "s4", "s5");
      } else {
        asm volatile(
            F8("v_mul_f32 %[t], %[q], %[r]\n v_mul_f32 %[u], %[b], %[w]\n"
               "v_fmac_f32 %[u], %[t], %[h0]\n v_fmac_f32 %[acc], %[c], %[u]\n"
               "v_mul_f32 %[t], %[q], %[r]\n v_mul_f32 %[h0], %[b], %[w]\n"
               "v_fmac_f32 %[h0], %[t], %[h1]\n v_fmac_f32 %[acc], %[c], %[h0]\n")
            : [h0] "+v"(a0), [h1] "+v"(a1), [acc] "+v"(a6), [t] "=&v"(t), [u] "=&v"(u)
            : [q] "v"(m), [r] "v"(a2), [c] "s"(su), [b] "s"(su), [w] "v"(a5));
      }
    } else {
      // 64 exponentials in 8 independent chains.
      asm volatile(F8("v_exp_f32 %0, %0\n v_exp_f32 %1, %1\n v_exp_f32 %2, %2\n v_exp_f32 %3, %3\n"
                      "v_exp_f32 %4, %4\n v_exp_f32 %5, %5\n v_exp_f32 %6, %6\n v_exp_f32 %7, %7\n")
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
    }
  }
  out[(int64_t)blockIdx.x * 64 + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

// Two waves per SIMD with different work: 8-wave workgroups, one per CU
// (256), so waves w and w + 4 share SIMD w.  Waves 0-3 run iters_e
// iterations of 64 independent exponentials, waves 4-7 iters_f iterations of
// 64 independent FMAs; either count may be 0.  Stores one value per thread at
// out[block * 512 + thread].
__global__ void __launch_bounds__(512) k_split(float* __restrict__ out, int iters_e, int iters_f) {
  float a0 = threadIdx.x * 1e-3f, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3, a4 = a0 + 4, a5 = a0 + 5, a6 = a0 + 6,
        a7 = a0 + 7;
  const float m = 0.999f, c = 1e-3f;
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4) {
    for (int it = 0; it < iters_e; ++it)
      asm volatile(F8("v_exp_f32 %0, %0\n v_exp_f32 %1, %1\n v_exp_f32 %2, %2\n v_exp_f32 %3, %3\n"
                      "v_exp_f32 %4, %4\n v_exp_f32 %5, %5\n v_exp_f32 %6, %6\n v_exp_f32 %7, %7\n")
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
  } else {
    for (int it = 0; it < iters_f; ++it)
      asm volatile(F8("v_fmac_f32 %0, %8, %9\n v_fmac_f32 %1, %8, %9\n v_fmac_f32 %2, %8, %9\n v_fmac_f32 %3, %8, %9\n"
                      "v_fmac_f32 %4, %8, %9\n v_fmac_f32 %5, %8, %9\n v_fmac_f32 %6, %8, %9\n v_fmac_f32 %7, %8, %9\n")
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                   : "v"(m), "v"(c));
  }
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

// 256 workgroups of k_split; out holds 256 * 512 floats.  Returns 0, or -1
// for a bad argument.
extern "C" int valu_split_probe(float* out, int iters_e, int iters_f, void* stream) {
  if (out == nullptr || iters_e < 0 || iters_f < 0) return -1;
  hipLaunchKernelGGL(k_split, dim3(256), dim3(512), 0, (hipStream_t)stream, out, iters_e, iters_f);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// kind 0: FMA stream, 1: exp stream, 2: the scan's state mix, 3: FMA stream
// with an SGPR operand, 4 / 5: the structured state mix with bf16 B and C
// unpacked on the scalar unit / given as fp32.  Returns 0, or -1 for a bad
// argument.
extern "C" int valu_rate_probe(int kind, float* out, int blocks, int iters, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipStream_t st = (hipStream_t)stream;
  const float su = 0.5f;
  if (kind == 0) {
    hipLaunchKernelGGL(k_rate<0>, dim3(blocks), dim3(64), 0, st, out, iters, su);
  } else if (kind == 1) {
    hipLaunchKernelGGL(k_rate<1>, dim3(blocks), dim3(64), 0, st, out, iters, su);
  } else if (kind == 2) {
    hipLaunchKernelGGL(k_rate<2>, dim3(blocks), dim3(64), 0, st, out, iters, su);
  } else if (kind == 3) {
    hipLaunchKernelGGL(k_rate<3>, dim3(blocks), dim3(64), 0, st, out, iters, su);
  } else if (kind == 4) {
    hipLaunchKernelGGL(k_rate<4>, dim3(blocks), dim3(64), 0, st, out, iters, su);
  } else if (kind == 5) {
    hipLaunchKernelGGL(k_rate<5>, dim3(blocks), dim3(64), 0, st, out, iters, su);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
