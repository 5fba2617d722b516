// Internal interface between the C ABI layer (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Timesteps per block of the scan sweep (prefetch and readout granularity).
constexpr int kTimeBlock = 8;
// Largest number of waves that may share one 64-channel tile.
constexpr int kMaxSplit = 8;

// One launch of the scan.  Pointers are device pointers; element type of the
// io tensors is fp32 or bf16 (raw 16-bit) according to bf16.
struct ScanLaunch {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* h0;     // nullable
  void* y;
  float* h_last;       // nullable
  float* workspace;    // nullable when n_chunks == 1
  int64_t batch, seqlen, d_inner;
  int32_t d_state;
  int32_t n_split;     // waves per 64-channel tile (1, 2, 4, 8)
  int64_t chunk_len;   // timesteps per chunk
  int64_t n_chunks;    // ceil(seqlen / chunk_len)
  bool bf16;
  hipStream_t stream;
};

struct UpdateLaunch {
  float* h;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;  // nullable
  const void* z;   // nullable
  void* y;
  int64_t batch, d_inner;
  int32_t d_state;
  bool bf16;
  hipStream_t stream;
};

// Workspace layout used when n_chunks > 1, in floats, with S = batch*d_inner*d_state:
//   [0, (n_chunks-1)*S)             chunk decay products  P[c][b][d][n]
//   [(n_chunks-1)*S, 2(n_chunks-1)*S) chunk end states from zero  S[c][b][d][n]
//   [2(n_chunks-1)*S, ...+n_chunks*S) chunk entry states  H[c][b][d][n]
inline int64_t scan_workspace_floats(int64_t n_chunks, int64_t states) {
  return n_chunks > 1 ? (3 * n_chunks - 2) * states : 0;
}

hipError_t launch_scan(const ScanLaunch& p);
hipError_t launch_state_fill(float* dst, const float* src, int64_t states, hipStream_t stream);
hipError_t launch_update(const UpdateLaunch& p);

}  // namespace ssm
