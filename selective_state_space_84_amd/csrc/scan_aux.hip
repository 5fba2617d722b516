// Small helper kernels of the scan: chunk carries and the empty-sequence
// state hand-over, plus the dispatch over compile-time modes.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// Entry state of every chunk: H[0] = h0, H[c+1] = P[c] * H[c] + S[c].
// One lane per (b, d, n) state; lanes are contiguous in memory, so every
// access is coalesced.  The chunk loop is the associative combine applied in
// order (the pairs are few, so a tree would only add work).
__global__ void __launch_bounds__(256) k_chunk_carry(const float* __restrict__ h0, const float* __restrict__ sumP,
                                                     const float* __restrict__ sumS, float* __restrict__ h_entry,
                                                     int64_t states, int64_t n_chunks) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= states) return;
  float hc = h0 != nullptr ? h0[s] : 0.f;
  h_entry[s] = hc;
  // The pairs of four chunks are loaded before they are combined (the loads
  // do not depend on the state), so they are in flight together.
  int64_t c = 0;
  for (; c + 4 < n_chunks; c += 4) {
    float P[4], S[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      P[j] = sumP[(c + j) * states + s];
      S[j] = sumS[(c + j) * states + s];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hc = __builtin_fmaf(P[j], hc, S[j]);
      h_entry[(c + j + 1) * states + s] = hc;
    }
  }
  for (; c + 1 < n_chunks; ++c) {
    hc = __builtin_fmaf(sumP[c * states + s], hc, sumS[c * states + s]);
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

hipError_t launch_chunk_carry(const float* h0, const float* sumP, const float* sumS, float* h_entry, int64_t states,
                              int64_t n_chunks, hipStream_t stream) {
  return launch(k_chunk_carry, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, stream, h0, sumP, sumS, h_entry,
                states, n_chunks);
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
