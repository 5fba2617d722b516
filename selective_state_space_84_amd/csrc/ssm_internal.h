// Internal interface between the C ABI layer (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

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
  float* ckpt;         // nullable: states at 8-step block starts for the backward pass
  const float* dt_bias;  // [d_inner], used with SSM_FLAG_DELTA_SOFTPLUS
  uint32_t flags;        // SSM_FLAG_* (bit 0 softplus step, bit 1 exact ZOH)
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
  const float* dt_bias;  // [d_inner], used with SSM_FLAG_DELTA_SOFTPLUS
  uint32_t flags;
  int64_t batch, d_inner;
  int32_t d_state;
  bool bf16;
  hipStream_t stream;
};

// One causal conv1d launch (or decode step: x = x_t, y = y_t, state_out = the
// in-place state, seqlen unused).
struct ConvLaunch {
  const void* x;
  const float* w;         // [d_inner][d_conv]
  const float* bias;      // nullable
  const float* state_in;  // nullable
  void* y;
  float* state_out;       // nullable (sweep); the state (decode step)
  int64_t batch, seqlen, d_inner;
  int32_t d_conv;
  bool silu;
  bool bf16;
  hipStream_t stream;
};

// Workspace layout used when n_chunks > 1, in floats, with R = batch*d_inner
// rows and S = R*d_state states (each section 256-byte aligned):
//   [0, up((n_chunks-1)*R))      chunk step sums  T[c][b][d] (sum of the chunk's steps)
//   next (n_chunks-1)*S           chunk end states from zero  S[c][b][d][n]
//   next n_chunks*S               chunk entry states  H[c][b][d][n]
// A chunk's decay products exp(A[d][n] * T[c][b][d]) are formed where they
// are used, so one float per row replaces d_state of them.
inline int64_t scan_stepsum_floats(int64_t n_chunks, int64_t rows) {
  return n_chunks > 1 ? ((n_chunks - 1) * rows + 63) / 64 * 64 : 0;
}

// Gradient of the scan (one launch sequence).  io tensors (x, delta, z, dy,
// dx, ddelta, dz) are fp32 or bf16 according to bf16; the rest are fp32.
struct BwdLaunch {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* h0;       // nullable
  const float* dt_bias;  // used with SSM_FLAG_DELTA_SOFTPLUS
  const void* dy;
  const float* dh_last;  // nullable
  const float* ckpt;     // nullable: block-start states written by the forward sweep
  void* dx;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;         // nullable (required when D is given)
  void* dz;          // nullable (required when z is given)
  float* dh0;        // nullable
  float* d_dt_bias;  // used with SSM_FLAG_DELTA_SOFTPLUS
  uint32_t flags;
  int64_t batch, seqlen, d_inner;
  int32_t d_state;
  bool bf16;
  hipStream_t stream;
};

// Steps per checkpoint block of the backward pass.  The forward sweep writes
// the checkpoints ([batch][ceil(seqlen/8)][d_state][d_inner], the state
// before every block) with its own block length, and ssm_scan_ckpt_bytes
// sizes them the same way: the two must stay equal.
constexpr int kBwdBlock = kTimeBlock;
static_assert(kBwdBlock == kTimeBlock, "forward checkpoints and backward blocks share one block length");

// Sequence chunks of the backward pass: (chunk_len, n_chunks), chunk_len a
// multiple of kBwdBlock.  Chunks are used only when channels alone leave the
// chip idle; they add a forward summary (standalone calls) and a reverse
// adjoint summary.
struct BwdPlan {
  int64_t chunk_len;
  int64_t n_chunks;
};
BwdPlan bwd_plan(int64_t batch, int64_t seqlen, int64_t d_inner);

// Sections of the backward workspace (floats, each 256-byte aligned), with
// S = batch * d_inner * d_state states and c = n_chunks.  When the caller
// passes the forward call's checkpoints (ckpt_given), the sections that only
// serve to compute them (ckpt, fT, fS, fH) are left out.
//   ckpt    [batch][ceil(seqlen/8)][d_state][d_inner]  states at block starts
//   part_bc [tiles][batch][seqlen][2*d_state]          per-tile dB | dC sums
//   part_a  [c][batch][d_inner][d_state]               per-(chunk, row) dA
//   part_d, part_t [c][batch][d_inner]                 per-(chunk, row) dD, d_dt_bias
//   when c > 1: forward chunk step sums fT [c-1][batch][d_inner], zero-start
//   end states fS [c-1][S] and entry states fH
//   [c][S]; adjoint chunk summaries lP, lS [c-1][S] and incoming adjoints
//   lIn [c][S];
//   when d_state > 16: part_el [3][batch][seqlen][d_inner], the state groups'
//   per-element sums.
struct BwdWorkspace {
  float* ckpt;
  float* part_bc;
  float* part_a;
  float* part_d;
  float* part_t;
  float* fT;
  float* fS;
  float* fH;
  float* lP;
  float* lS;
  float* lIn;
  float* part_el;  // more than 16 states: per-element sums of the state groups, [3][batch][seqlen][d_inner]
};
BwdWorkspace bwd_workspace_layout(float* base, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                  const BwdPlan& plan, bool ckpt_given, int64_t* total_floats);
hipError_t launch_scan_bwd(const BwdLaunch& p, const BwdWorkspace& ws, const BwdPlan& pl);

// Scan with a scalar decay per head (Mamba-2 / SSD form).  bf16 io (x, dt,
// B, C, z, y), fp32 A, D, dt_bias, h0, h_last; headdim 64.
struct SsdLaunch {
  const void* x;      // [batch][seqlen][nheads][64]
  const void* dt;     // [batch][seqlen][nheads]
  const float* A;     // [nheads]
  const void* B;      // [batch][seqlen][ngroups][d_state]
  const void* C;
  const float* D;     // nullable
  const void* z;      // nullable
  const float* h0;    // nullable, [batch][nheads][64][d_state]
  void* y;
  float* h_last;      // nullable
  const float* dt_bias;  // used with SSM_FLAG_DELTA_SOFTPLUS
  uint32_t flags;
  int64_t batch, seqlen, nheads, ngroups;
  int32_t d_state;
  hipStream_t stream;
};
hipError_t launch_ssd(const SsdLaunch& p);

hipError_t launch_scan(const ScanLaunch& p);
template <int MODE>
hipError_t launch_scan_mode(const ScanLaunch& p);  // one translation unit per MODE
// Entry states of every chunk from the step sums T and zero-start end states
// S of the chunks before it; A is read as the sweep reads it (structured when
// linear_a).
hipError_t launch_chunk_carry(const float* h0, const float* A, bool linear_a, const float* sumT, const float* sumS,
                              float* h_entry, int64_t rows, int64_t d_state, int64_t d_inner, int64_t n_chunks,
                              hipStream_t stream);
hipError_t launch_state_fill(float* dst, const float* src, int64_t states, hipStream_t stream);
hipError_t launch_update(const UpdateLaunch& p);
hipError_t launch_conv1d(const ConvLaunch& p);
hipError_t launch_conv1d_update(const ConvLaunch& p);
int64_t conv_grid_blocks(int64_t batch, int64_t seqlen, int64_t d_inner);

// Launches kern with hipLaunchKernel, which reports this launch's own error
// (the sticky last-error state is left alone).  Arguments are converted to
// the kernel's parameter types first.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                         Args&&... args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&](auto&... v) {
    int k = 0;
    ((ptrs[k++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, shmem, s);
}

}  // namespace ssm
