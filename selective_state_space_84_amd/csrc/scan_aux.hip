// Small helper kernels of the scan: chunk carries and the empty-sequence
// state hand-over, plus the dispatch over compile-time modes.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// Entry state of every chunk: H[0] = h0, H[c+1] = P[c] * H[c] + S[c], with
// the decay product P[c] = exp(A[d][n] T[c]) formed here from the chunk's step
// sum T[c][b][d] exactly as the sweep forms a decay (A * log2(e), times the
// step, then exp2), so the result does not depend on where it is computed.
// One lane per (b, d, n) state; lanes are contiguous in memory, so every
// access is coalesced (the d_state lanes of a row share one step sum).  The
// chunk loop is the associative combine applied in order (the pairs are few,
// so a tree would only add work).
__global__ void __launch_bounds__(256) k_chunk_carry(const float* __restrict__ h0, const float* __restrict__ A,
                                                     const int linear_a, const float* __restrict__ sumT,
                                                     const float* __restrict__ sumS, float* __restrict__ h_entry,
                                                     int64_t rows, int32_t d_state, int64_t d_inner,
                                                     int64_t n_chunks) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t states = rows * d_state;
  if (s >= states) return;
  const int64_t row = s / d_state;  // b * d_inner + d
  const int n = (int)(s - row * d_state);
  const int64_t d = row % d_inner;
  const float a = linear_a ? (float)(n + 1) * A[d * d_state] : A[d * d_state + n];
  const float al2 = a * kLog2e;
  float hc = h0 != nullptr ? h0[s] : 0.f;
  h_entry[s] = hc;
  // The pairs of four chunks are loaded before they are combined (the loads
  // do not depend on the state), so they are in flight together.
  int64_t c = 0;
  for (; c + 4 < n_chunks; c += 4) {
    float T[4], S[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      T[j] = sumT[(c + j) * rows + row];
      S[j] = sumS[(c + j) * states + s];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hc = __builtin_fmaf(hw_exp2(al2 * T[j]), hc, S[j]);
      h_entry[(c + j + 1) * states + s] = hc;
    }
  }
  for (; c + 1 < n_chunks; ++c) {
    hc = __builtin_fmaf(hw_exp2(al2 * sumT[c * rows + row]), hc, sumS[c * states + s]);
    h_entry[(c + 1) * states + s] = hc;
  }
}

// h_last for an empty sequence: the state is handed over unchanged.
__global__ void __launch_bounds__(256) k_state_fill(float* __restrict__ dst, const float* __restrict__ src,
                                                    int64_t states) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s < states) dst[s] = src != nullptr ? src[s] : 0.f;
}

}  // namespace

hipError_t launch_chunk_carry(const float* h0, const float* A, bool linear_a, const float* sumT, const float* sumS,
                              float* h_entry, int64_t rows, int64_t d_state, int64_t d_inner, int64_t n_chunks,
                              hipStream_t stream) {
  const int64_t states = rows * d_state;
  return launch(k_chunk_carry, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, stream, h0, A, linear_a ? 1 : 0,
                sumT, sumS, h_entry, rows, (int32_t)d_state, d_inner, n_chunks);
}

hipError_t launch_state_fill(float* dst, const float* src, int64_t states, hipStream_t stream) {
  return launch(k_state_fill, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, stream, dst, src, states);
}

hipError_t launch_scan(const ScanLaunch& p) {
  switch (p.flags & 7u) {
    case 0: return launch_scan_mode<0>(p);
    case 1: return launch_scan_mode<1>(p);
    case 2: return launch_scan_mode<2>(p);
    case 3: return launch_scan_mode<3>(p);
    case 4: return launch_scan_mode<4>(p);
    case 5: return launch_scan_mode<5>(p);
    case 6: return launch_scan_mode<6>(p);
    default: return launch_scan_mode<7>(p);
  }
}

}  // namespace ssm
