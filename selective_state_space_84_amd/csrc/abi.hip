// C ABI of the selective-scan library: argument checks, launch planning and
// dispatch to the gfx950 kernels.  Every check runs on the host before any
// HIP call, so a rejected call has no side effects.
#include "ssm_scan.h"
#include "ssm_internal.h"

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <mutex>

namespace ssm {
int64_t update_grid_blocks(int64_t batch, int64_t d_inner, int32_t d_state);
}

namespace {

// Below this many waves an MI355X is underfilled (256 CUs x 4 SIMDs; one wave
// issues a VALU instruction only every ~4 cycles, so a SIMD needs two to fill
// its 2-cycle VALU).  At or above it, cutting the sequence into chunks costs
// more (the summary pass) than it gains (measured on the Mamba-1.4B layer:
// 2048 waves unchunked 1.64 ms, 2 chunks 2.11 ms, 4 chunks 2.22 ms; 2 waves
// per tile 1.85 ms).
constexpr int64_t kTargetWaves = 2048;
// Once a sequence is cut, aim for this many waves: measured on MI355X, more
// resident waves pay for the summary pass on the chunks (Mamba-2.8B long
// layer, 320 waves from channels: 8 chunks 4.31 ms, 26 chunks 3.73 ms, 32 or
// 64 chunks 3.26 ms; Mamba-130M layer: 8 chunks 0.21 ms, 32 chunks 0.17 ms).
constexpr int64_t kChunkTargetWaves = 16384;
// Shortest chunk the automatic plan will cut a sequence into.
constexpr int64_t kMinAutoChunk = 64;
// Workspace alignment the library asks for.
constexpr uintptr_t kWorkspaceAlign = 256;
constexpr uint32_t kKnownFlags = SSM_FLAG_DELTA_SOFTPLUS | SSM_FLAG_EXACT_ZOH | SSM_FLAG_A_LINEAR_N;

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  int64_t t;
  if (__builtin_mul_overflow(a, b, &t)) return false;
  if (__builtin_mul_overflow(t, c, out)) return false;
  return true;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Byte ranges [p, p+n) and [q, q+m) overlap (empty ranges never overlap).
bool overlap(const void* p, int64_t n, const void* q, int64_t m) {
  if (p == nullptr || q == nullptr || n <= 0 || m <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

struct Plan {
  int32_t n_split;
  int64_t chunk_len;
  int64_t n_chunks;
};

int make_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, const ssm_scan_opts_t* o, Plan* pl) {
  const int gmin = d_state > 16 ? (int)(d_state / 16) : 1;
  const int gmax = (int)(d_state / 2) < ssm::kMaxSplit ? (int)(d_state / 2) : ssm::kMaxSplit;
  if (gmin > gmax) return SSM_ERR_UNSUPPORTED;
  const int64_t tiles = (d_inner + 63) / 64;
  const int64_t base = batch * tiles;
  int g;
  if (o != nullptr && o->n_split != 0) {
    g = o->n_split;
    if (!is_pow2(g) || g < gmin || g > gmax) return SSM_ERR_UNSUPPORTED;
  } else {
    // Each extra wave per tile repeats the per-step fixed work (widening,
    // delta*x, loop and scalar traffic) and adds an LDS exchange: measured
    // on MI355X, 4 waves per tile cost ~1.4x the VALU work of 1, and 2 waves
    // with chunks lose to 1 wave with more chunks.  So parallelism comes from
    // sequence chunks; the states are split over a second wave only when the
    // sequence is too short to cut.
    g = gmin;
    if (seqlen < 2 * kMinAutoChunk) {
      const int gpref = gmax < 2 ? gmax : (gmin > 2 ? gmin : 2);
      while (g < gpref && base * g < kTargetWaves) g *= 2;
    }
  }
  int64_t chunk_len;
  if (o != nullptr && o->chunk_len < 0) return SSM_ERR_UNSUPPORTED;
  if (o != nullptr && o->chunk_len > 0) {
    chunk_len = o->chunk_len;
  } else {
    int64_t nch = 1;
    const int64_t waves = base * g;
    if (waves > 0 && waves < kTargetWaves && seqlen >= 2 * kMinAutoChunk) {
      nch = (kChunkTargetWaves + waves - 1) / waves;
      if (nch > seqlen / kMinAutoChunk) nch = seqlen / kMinAutoChunk;
    }
    chunk_len = (seqlen + nch - 1) / nch;
    chunk_len = (chunk_len + ssm::kTimeBlock - 1) / ssm::kTimeBlock * ssm::kTimeBlock;
  }
  if (chunk_len <= 0) chunk_len = 1;
  if (chunk_len > seqlen && seqlen > 0) chunk_len = seqlen;
  pl->n_split = g;
  pl->chunk_len = chunk_len;
  pl->n_chunks = seqlen > 0 ? (seqlen + chunk_len - 1) / chunk_len : 1;
  return SSM_OK;
}

bool scan_d_state_ok(int64_t n) { return n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64 || n == 128; }
bool update_d_state_ok(int64_t n) { return n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64; }

// The sweep counts time inside a chunk in int32 and addresses a block of
// kTimeBlock rows with 32-bit per-lane byte offsets; these bounds keep both
// exact (seqlen < 2^31 - 256, kTimeBlock * d_inner * 4 bytes < 2^32).
constexpr int64_t kMaxSeqlen = INT32_MAX - 256;
constexpr int64_t kMaxDInner = (int64_t)1 << 26;

int check_dims(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0) return SSM_ERR_BAD_DIM;
  if (seqlen > kMaxSeqlen || d_inner > kMaxDInner) return SSM_ERR_BAD_DIM;
  return SSM_OK;
}

int workspace_bytes_for(int64_t batch, int64_t d_inner, int64_t d_state, const Plan& pl, size_t* out) {
  int64_t states;
  if (!mul3(batch, d_inner, d_state, &states)) return SSM_ERR_BAD_DIM;
  const int64_t nch = pl.n_chunks;
  int64_t floats = 0;
  if (nch > 1) {
    // Step sums (one per row and chunk, rounded up to 64) and 2n - 1 state sets.
    int64_t sets, sums;
    if (__builtin_mul_overflow(2 * nch - 1, states, &sets) || __builtin_mul_overflow(nch - 1, batch * d_inner, &sums) ||
        __builtin_add_overflow(sets, sums + 63, &floats))
      return SSM_ERR_BAD_DIM;
    floats = sets + ssm::scan_stepsum_floats(nch, batch * d_inner);
  }
  int64_t bytes;
  if (__builtin_mul_overflow(floats, (int64_t)sizeof(float), &bytes)) return SSM_ERR_BAD_DIM;
  *out = (size_t)bytes;
  return SSM_OK;
}

// Device scratch of ssm_scan_fwd_noalloc: the chunk carries (step sums,
// zero-start end states, entry states) of a split sequence live here instead
// of in a caller workspace.  Each device holds its own copy from the first
// call on it until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken once per device
// with hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.  Calls that overlap on one device share it and race.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// The current device's scratch address (SSM_OK), or SSM_ERR_HIP.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return SSM_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return SSM_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return SSM_OK;
}

// With no caller workspace, the automatic plan keeps as many sequence chunks
// as the scratch holds: n chunks need up64((n - 1) * R) + (2n - 1) * S floats
// (R = batch * d_inner rows, S = R * d_state states).  Fewer than two fitting
// chunks means one unsplit sweep.
void cap_plan_to_scratch(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, Plan* pl) {
  const int64_t rows = batch * d_inner, states = rows * d_state;
  if (pl->n_chunks <= 1 || states <= 0) return;
  const int64_t cap = (int64_t)(kScratchBytes / sizeof(float));
  auto fits = [&](int64_t n) { return ssm::scan_stepsum_floats(n, rows) + (2 * n - 1) * states <= cap; };
  int64_t n_max = (cap - 64 + rows + states) / (rows + 2 * states);
  while (n_max > 1 && !fits(n_max)) --n_max;
  if (pl->n_chunks <= n_max) return;
  if (n_max < 2) {
    pl->chunk_len = seqlen;
    pl->n_chunks = 1;
    return;
  }
  int64_t cl = (seqlen + n_max - 1) / n_max;
  cl = (cl + ssm::kTimeBlock - 1) / ssm::kTimeBlock * ssm::kTimeBlock;
  if (cl > seqlen) cl = seqlen;
  pl->chunk_len = cl;
  pl->n_chunks = (seqlen + cl - 1) / cl;
}

int scan_impl(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
              const void* z, const float* h0, void* y, float* h_last, int64_t batch, int64_t seqlen,
              int64_t d_inner, int64_t d_state, int32_t io_dtype, const ssm_scan_opts_t* opts, void* workspace,
              size_t workspace_bytes, void* stream, bool use_scratch = false) {
  int rc = check_dims(batch, seqlen, d_inner, d_state);
  if (rc != SSM_OK) return rc;
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
  if (!scan_d_state_ok(d_state)) return SSM_ERR_UNSUPPORTED;
  const uint32_t flags = opts != nullptr ? opts->flags : 0u;
  const float* dt_bias = (flags & SSM_FLAG_DELTA_SOFTPLUS) ? opts->dt_bias : nullptr;
  float* ckpt = opts != nullptr ? opts->ckpt_out : nullptr;
  if (flags & ~kKnownFlags) return SSM_ERR_UNSUPPORTED;
  if (ckpt != nullptr && opts->chunk_len > 0 && opts->chunk_len % ssm::kTimeBlock != 0) return SSM_ERR_UNSUPPORTED;
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;

  int64_t n_io, n_bc, n_h, n_a;
  if (!mul3(batch, seqlen, d_inner, &n_io) || !mul3(batch, seqlen, d_state, &n_bc) ||
      !mul3(batch, d_inner, d_state, &n_h) || !mul3(1, d_inner, d_state, &n_a))
    return SSM_ERR_BAD_DIM;
  int64_t b_io, b_bc, b_h, b_a;
  if (__builtin_mul_overflow(n_io, es, &b_io) || __builtin_mul_overflow(n_bc, es, &b_bc) ||
      __builtin_mul_overflow(n_h, (int64_t)4, &b_h) || __builtin_mul_overflow(n_a, (int64_t)4, &b_a))
    return SSM_ERR_BAD_DIM;
  const int64_t b_d = d_inner * 4;

  // Required pointers (a tensor with no elements may be NULL).
  if (n_io > 0 && (x == nullptr || delta == nullptr || y == nullptr)) return SSM_ERR_NULL_ARG;
  if (n_bc > 0 && n_io > 0 && (B == nullptr || C == nullptr)) return SSM_ERR_NULL_ARG;
  if (n_a > 0 && n_io > 0 && A == nullptr) return SSM_ERR_NULL_ARG;
  if ((flags & SSM_FLAG_DELTA_SOFTPLUS) && d_inner > 0 && dt_bias == nullptr) return SSM_ERR_NULL_ARG;

  // Alignment.
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(z, es) || !aligned(y, es)) return SSM_ERR_MISALIGNED;
  if (!aligned(B, 4) || !aligned(C, 4) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) || !aligned(h_last, 4) ||
      !aligned(dt_bias, 4))
    return SSM_ERR_MISALIGNED;

  if (!aligned(ckpt, 4)) return SSM_ERR_MISALIGNED;
  int64_t b_ck = 0;
  if (ckpt != nullptr) {
    int64_t n_ck;
    if (!mul3(batch, (seqlen + ssm::kTimeBlock - 1) / ssm::kTimeBlock, d_state, &n_ck) ||
        __builtin_mul_overflow(n_ck, d_inner * 4, &b_ck))
      return SSM_ERR_BAD_DIM;
  }

  // Aliasing: y overlaps nothing; h_last overlaps nothing except h0 exactly;
  // the checkpoints overlap nothing.
  {
    const void* all[] = {x, delta, z, B, C, A, D, h0, y, h_last, dt_bias};
    const int64_t allb[] = {b_io, b_io, z ? b_io : 0, b_bc, b_bc, b_a, D ? b_d : 0, h0 ? b_h : 0, b_io,
                            h_last ? b_h : 0, dt_bias ? b_d : 0};
    for (int k = 0; k < 11; ++k)
      if (overlap(ckpt, b_ck, all[k], allb[k])) return SSM_ERR_ALIAS;
  }
  const void* ins[] = {x, delta, z, B, C, A, D, h0};
  const int64_t inb[] = {b_io, b_io, z ? b_io : 0, b_bc, b_bc, b_a, D ? b_d : 0, h0 ? b_h : 0};
  for (int k = 0; k < 8; ++k)
    if (overlap(y, b_io, ins[k], inb[k])) return SSM_ERR_ALIAS;
  if (overlap(y, b_io, h_last, h_last ? b_h : 0)) return SSM_ERR_ALIAS;
  if (overlap(y, b_io, dt_bias, dt_bias ? b_d : 0) || overlap(h_last, h_last ? b_h : 0, dt_bias, dt_bias ? b_d : 0))
    return SSM_ERR_ALIAS;
  if (h_last != nullptr) {
    for (int k = 0; k < 7; ++k)
      if (overlap(h_last, b_h, ins[k], inb[k])) return SSM_ERR_ALIAS;
    if (h0 != nullptr && h0 != h_last && overlap(h_last, b_h, h0, b_h)) return SSM_ERR_ALIAS;
  }

  Plan pl;
  rc = make_plan(batch, seqlen, d_inner, d_state, opts, &pl);
  if (rc != SSM_OK) return rc;
  const bool auto_chunks = opts == nullptr || opts->chunk_len == 0;
  if (use_scratch && auto_chunks) cap_plan_to_scratch(batch, seqlen, d_inner, d_state, &pl);
  size_t need;
  rc = workspace_bytes_for(batch, d_inner, d_state, pl, &need);
  if (rc != SSM_OK) return rc;
  const int64_t tiles = (d_inner + 63) / 64;
  int64_t grid;
  if (!mul3(batch, pl.n_chunks, tiles, &grid) || grid > INT32_MAX) return SSM_ERR_BAD_DIM;
  if (use_scratch) {
    // An explicit chunk length whose carries do not fit the scratch.
    if (need > kScratchBytes) return SSM_ERR_WORKSPACE;
  } else if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return SSM_ERR_WORKSPACE;
    if (!aligned(workspace, kWorkspaceAlign)) return SSM_ERR_MISALIGNED;
    const void* all[] = {x, delta, z, B, C, A, D, h0, y, h_last, dt_bias};
    const int64_t allb[] = {b_io, b_io, z ? b_io : 0, b_bc, b_bc, b_a, D ? b_d : 0, h0 ? b_h : 0, b_io,
                            h_last ? b_h : 0, dt_bias ? b_d : 0};
    for (int k = 0; k < 11; ++k)
      if (overlap(workspace, (int64_t)need, all[k], allb[k])) return SSM_ERR_ALIAS;
    if (overlap(workspace, (int64_t)need, ckpt, b_ck)) return SSM_ERR_ALIAS;
  }
  int64_t state_blocks = (n_h + 255) / 256;
  if (state_blocks > INT32_MAX) return SSM_ERR_BAD_DIM;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0 || d_inner == 0) return SSM_OK;
  if (seqlen == 0) {
    if (h_last == nullptr || h_last == h0) return SSM_OK;
    return ssm::launch_state_fill(h_last, h0, n_h, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  if (use_scratch) {
    workspace = nullptr;
    if (need > 0) {
      rc = device_scratch(&workspace);
      if (rc != SSM_OK) return rc;
    }
  }
  ssm::ScanLaunch p{x, delta, A, B, C, D, z, h0, y, h_last, static_cast<float*>(workspace), ckpt, dt_bias, flags, batch,
                    seqlen, d_inner, (int32_t)d_state, pl.n_split, pl.chunk_len, pl.n_chunks,
                    io_dtype == SSM_DTYPE_BF16, s};
  return ssm::launch_scan(p) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int update_impl(float* h, const void* x_t, const void* delta_t, const float* A, const void* B_t, const void* C_t,
                const float* D, const void* z_t, void* y_t, int64_t batch, int64_t d_inner, int64_t d_state,
                int32_t io_dtype, uint32_t flags, const float* dt_bias, void* stream) {
  if (batch < 0 || d_inner < 0 || d_state <= 0) return SSM_ERR_BAD_DIM;
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
  if (!update_d_state_ok(d_state)) return SSM_ERR_UNSUPPORTED;
  if (flags & ~kKnownFlags) return SSM_ERR_UNSUPPORTED;
  if (!(flags & SSM_FLAG_DELTA_SOFTPLUS)) dt_bias = nullptr;
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  int64_t n_io, n_h, n_bc;
  if (!mul3(batch, d_inner, 1, &n_io) || !mul3(batch, d_inner, d_state, &n_h) || !mul3(batch, d_state, 1, &n_bc))
    return SSM_ERR_BAD_DIM;
  int64_t b_io, b_h, b_bc, b_a;
  if (__builtin_mul_overflow(n_io, es, &b_io) || __builtin_mul_overflow(n_h, (int64_t)4, &b_h) ||
      __builtin_mul_overflow(n_bc, es, &b_bc) || __builtin_mul_overflow(d_inner * d_state, (int64_t)4, &b_a))
    return SSM_ERR_BAD_DIM;
  if (n_io > 0 && (h == nullptr || x_t == nullptr || delta_t == nullptr || y_t == nullptr || A == nullptr ||
                   B_t == nullptr || C_t == nullptr))
    return SSM_ERR_NULL_ARG;
  if ((flags & SSM_FLAG_DELTA_SOFTPLUS) && n_io > 0 && dt_bias == nullptr) return SSM_ERR_NULL_ARG;
  if (!aligned(dt_bias, 4)) return SSM_ERR_MISALIGNED;
  const uintptr_t ha = d_state >= 4 ? 16 : 8;
  if (!aligned(h, ha) || !aligned(A, ha)) return SSM_ERR_MISALIGNED;
  if (!aligned(x_t, es) || !aligned(delta_t, es) || !aligned(z_t, es) || !aligned(y_t, es)) return SSM_ERR_MISALIGNED;
  if (!aligned(B_t, io_dtype == SSM_DTYPE_BF16 ? 4 : ha) || !aligned(C_t, io_dtype == SSM_DTYPE_BF16 ? 4 : ha) ||
      !aligned(D, 4))
    return SSM_ERR_MISALIGNED;
  const void* ins[] = {x_t, delta_t, z_t, B_t, C_t, A, D};
  const int64_t inb[] = {b_io, b_io, z_t ? b_io : 0, b_bc, b_bc, b_a, D ? d_inner * 4 : 0};
  for (int k = 0; k < 7; ++k) {
    if (overlap(y_t, b_io, ins[k], inb[k])) return SSM_ERR_ALIAS;
    if (overlap(h, b_h, ins[k], inb[k])) return SSM_ERR_ALIAS;
  }
  if (overlap(h, b_h, y_t, b_io)) return SSM_ERR_ALIAS;
  if (overlap(y_t, b_io, dt_bias, dt_bias ? d_inner * 4 : 0) || overlap(h, b_h, dt_bias, dt_bias ? d_inner * 4 : 0))
    return SSM_ERR_ALIAS;
  if (ssm::update_grid_blocks(batch, d_inner, (int32_t)d_state) > INT32_MAX) return SSM_ERR_BAD_DIM;
  if (n_io == 0) return SSM_OK;
  ssm::UpdateLaunch p{h, x_t, delta_t, A, B_t, C_t, D, z_t, y_t, dt_bias, flags, batch, d_inner, (int32_t)d_state,
                      io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream)};
  return ssm::launch_update(p) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

bool bwd_d_state_ok(int64_t n) { return n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64 || n == 128; }

// Floats of backward workspace, or -1 when a size overflows.
int64_t bwd_workspace_floats(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, bool ckpt_given) {
  const int64_t tiles = (d_inner + 63) / 64;
  const int64_t nblk = (seqlen + ssm::kBwdBlock - 1) / ssm::kBwdBlock;
  int64_t a, b, c;
  // Largest sections: checkpoints and per-tile partials; the rest are smaller.
  if (!mul3(batch, nblk, d_state, &a) || __builtin_mul_overflow(a, d_inner, &a)) return -1;
  if (!mul3(tiles, batch, seqlen, &b) || __builtin_mul_overflow(b, 2 * d_state, &b)) return -1;
  if (!mul3(batch, d_inner, d_state, &c)) return -1;
  int64_t el;  // per-element sums of the state groups (d_state > 16): 3 floats per element
  if (!mul3(batch, seqlen, d_inner, &el)) return -1;
  if (a > INT64_MAX / 8 || b > INT64_MAX / 8 || c > INT64_MAX / 8 || el > INT64_MAX / 16) return -1;
  int64_t total;
  ssm::bwd_workspace_layout(nullptr, batch, seqlen, d_inner, d_state, ssm::bwd_plan(batch, seqlen, d_inner), ckpt_given,
                            &total);
  return total;
}

int bwd_impl(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
             const void* z, const float* h0, const float* dt_bias, const void* dy, const float* dh_last,
             const float* ckpt, void* dx,
             void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* dh0, float* d_dt_bias,
             int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int32_t io_dtype, uint32_t flags,
             void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(batch, seqlen, d_inner, d_state);
  if (rc != SSM_OK) return rc;
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
  if (!bwd_d_state_ok(d_state)) return SSM_ERR_UNSUPPORTED;
  if (flags & ~kKnownFlags) return SSM_ERR_UNSUPPORTED;
  const bool sp = (flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;
  if (!sp) {
    dt_bias = nullptr;
    d_dt_bias = nullptr;
  }
  if (D == nullptr) dD = nullptr;
  if (z == nullptr) dz = nullptr;
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  int64_t n_io, n_bc, n_h;
  if (!mul3(batch, seqlen, d_inner, &n_io) || !mul3(batch, seqlen, d_state, &n_bc) ||
      !mul3(batch, d_inner, d_state, &n_h))
    return SSM_ERR_BAD_DIM;
  int64_t b_io, b_bc, b_bc32, b_h;
  if (__builtin_mul_overflow(n_io, es, &b_io) || __builtin_mul_overflow(n_bc, es, &b_bc) ||
      __builtin_mul_overflow(n_bc, (int64_t)4, &b_bc32) || __builtin_mul_overflow(n_h, (int64_t)4, &b_h))
    return SSM_ERR_BAD_DIM;
  const int64_t b_a = d_inner * d_state * 4, b_d = d_inner * 4;

  // Required pointers.
  if (n_io > 0 && (x == nullptr || delta == nullptr || dy == nullptr || dx == nullptr || ddelta == nullptr))
    return SSM_ERR_NULL_ARG;
  if (n_io > 0 && (B == nullptr || C == nullptr || dB == nullptr || dC == nullptr)) return SSM_ERR_NULL_ARG;
  if (b_a > 0 && (A == nullptr || dA == nullptr)) return SSM_ERR_NULL_ARG;
  if (D != nullptr && d_inner > 0 && dD == nullptr) return SSM_ERR_NULL_ARG;
  if (z != nullptr && n_io > 0 && dz == nullptr) return SSM_ERR_NULL_ARG;
  if (sp && d_inner > 0 && (dt_bias == nullptr || d_dt_bias == nullptr)) return SSM_ERR_NULL_ARG;

  // Alignment.
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(z, es) || !aligned(dy, es) || !aligned(dx, es) ||
      !aligned(ddelta, es) || !aligned(dz, es))
    return SSM_ERR_MISALIGNED;
  const void* f4[] = {A, B, C, D, h0, dt_bias, dh_last, ckpt, dA, dB, dC, dD, dh0, d_dt_bias};
  for (const void* q : f4)
    if (!aligned(q, 4)) return SSM_ERR_MISALIGNED;

  // Aliasing: no output overlaps an input, another output or the workspace.
  int64_t b_ck = 0;
  if (ckpt != nullptr) {
    int64_t n_ck;
    if (!mul3(batch, (seqlen + ssm::kBwdBlock - 1) / ssm::kBwdBlock, d_state, &n_ck) ||
        __builtin_mul_overflow(n_ck, d_inner * 4, &b_ck))
      return SSM_ERR_BAD_DIM;
  }
  const void* ins[] = {x, delta, A, B, C, D, z, h0, dt_bias, dy, dh_last, ckpt};
  const int64_t inb[] = {b_io, b_io, b_a, b_bc, b_bc, D ? b_d : 0, z ? b_io : 0, h0 ? b_h : 0,
                         dt_bias ? b_d : 0, b_io, dh_last ? b_h : 0, b_ck};
  const void* outs[] = {dx, ddelta, dA, dB, dC, dD, dz, dh0, d_dt_bias};
  const int64_t outb[] = {b_io, b_io, b_a, b_bc32, b_bc32, dD ? b_d : 0, dz ? b_io : 0, dh0 ? b_h : 0,
                          d_dt_bias ? b_d : 0};
  for (int o = 0; o < 9; ++o) {
    for (int k = 0; k < 12; ++k)
      if (overlap(outs[o], outb[o], ins[k], inb[k])) return SSM_ERR_ALIAS;
    for (int k = o + 1; k < 9; ++k)
      if (overlap(outs[o], outb[o], outs[k], outb[k])) return SSM_ERR_ALIAS;
  }

  const int64_t floats = bwd_workspace_floats(batch, seqlen, d_inner, d_state, ckpt != nullptr);
  if (floats < 0) return SSM_ERR_BAD_DIM;
  const int64_t need = floats * 4;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < (size_t)need) return SSM_ERR_WORKSPACE;
    if (!aligned(workspace, kWorkspaceAlign)) return SSM_ERR_MISALIGNED;
    for (int k = 0; k < 12; ++k)
      if (overlap(workspace, need, ins[k], inb[k])) return SSM_ERR_ALIAS;
    for (int k = 0; k < 9; ++k)
      if (overlap(workspace, need, outs[k], outb[k])) return SSM_ERR_ALIAS;
  }
  const int64_t tiles = (d_inner + 63) / 64;
  const ssm::BwdPlan bplan = ssm::bwd_plan(batch, seqlen, d_inner);
  if (batch * tiles * bplan.n_chunks > INT32_MAX || (n_bc * 2 + 255) / 256 > INT32_MAX ||
      (d_inner * d_state + 255) / 256 > INT32_MAX || (n_h + 255) / 256 > INT32_MAX)
    return SSM_ERR_BAD_DIM;

  if (d_inner == 0) return SSM_OK;
  float* ws = static_cast<float*>(workspace);
  const ssm::BwdPlan plan = ssm::bwd_plan(batch, seqlen, d_inner);
  const ssm::BwdWorkspace lay =
      ssm::bwd_workspace_layout(ws, batch, seqlen, d_inner, d_state, plan, ckpt != nullptr, nullptr);
  ssm::BwdLaunch p{x, delta, A, B, C, D, z, h0, dt_bias, dy, dh_last, ckpt, dx, ddelta, dA, dB, dC, dD, dz, dh0,
                   d_dt_bias, flags, batch, seqlen, d_inner, (int32_t)d_state, io_dtype == SSM_DTYPE_BF16,
                   static_cast<hipStream_t>(stream)};
  return ssm::launch_scan_bwd(p, lay, plan) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssd_impl(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
             const void* z, const float* h0, void* y, float* h_last, int64_t batch, int64_t seqlen, int64_t nheads,
             int64_t headdim, int64_t ngroups, int64_t d_state, int32_t io_dtype, uint32_t flags,
             const float* dt_bias, void* stream) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || ngroups <= 0 || d_state <= 0) return SSM_ERR_BAD_DIM;
  // The kernel addresses a 32-step chunk with 24-bit row multiplies: 32768
  // heads of 64 channels (or groups of 128 states) keep a step below 2^24 bytes.
  if (seqlen > kMaxSeqlen || nheads > (1 << 15)) return SSM_ERR_BAD_DIM;
  if (io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
  if (headdim != 64 || (d_state != 64 && d_state != 128) || nheads % ngroups != 0) return SSM_ERR_UNSUPPORTED;
  if (flags & ~(uint32_t)SSM_FLAG_DELTA_SOFTPLUS) return SSM_ERR_UNSUPPORTED;
  if (!(flags & SSM_FLAG_DELTA_SOFTPLUS)) dt_bias = nullptr;
  int64_t n_io, n_dt, n_bc, n_h;
  if (!mul3(batch, seqlen, nheads * headdim, &n_io) || !mul3(batch, seqlen, nheads, &n_dt) ||
      !mul3(batch, seqlen, ngroups * d_state, &n_bc) || !mul3(batch, nheads * headdim, d_state, &n_h))
    return SSM_ERR_BAD_DIM;
  if (n_io > INT64_MAX / 4 || n_bc > INT64_MAX / 4 || n_h > INT64_MAX / 8) return SSM_ERR_BAD_DIM;
  const int64_t b_io = n_io * 2, b_dt = n_dt * 2, b_bc = n_bc * 2, b_h = n_h * 4, b_p = nheads * 4;
  if (n_io > 0 && (x == nullptr || dt == nullptr || y == nullptr || B == nullptr || C == nullptr || A == nullptr))
    return SSM_ERR_NULL_ARG;
  if ((flags & SSM_FLAG_DELTA_SOFTPLUS) && nheads > 0 && dt_bias == nullptr) return SSM_ERR_NULL_ARG;
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(B, 16) || !aligned(C, 16) ||
      !aligned(dt, 2) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) || !aligned(h_last, 4) ||
      !aligned(dt_bias, 4))
    return SSM_ERR_MISALIGNED;
  const void* ins[] = {x, dt, A, B, C, D, z, h0, dt_bias};
  const int64_t inb[] = {b_io, b_dt, b_p, b_bc, b_bc, D ? b_p : 0, z ? b_io : 0, h0 ? b_h : 0, dt_bias ? b_p : 0};
  for (int k = 0; k < 9; ++k)
    if (overlap(y, b_io, ins[k], inb[k])) return SSM_ERR_ALIAS;
  if (h_last != nullptr) {
    for (int k = 0; k < 7; ++k)
      if (overlap(h_last, b_h, ins[k], inb[k])) return SSM_ERR_ALIAS;
    if (overlap(h_last, b_h, y, b_io) || overlap(h_last, b_h, dt_bias, dt_bias ? b_p : 0)) return SSM_ERR_ALIAS;
    if (h0 != nullptr && h0 != h_last && overlap(h_last, b_h, h0, b_h)) return SSM_ERR_ALIAS;
  }
  if (batch * nheads > INT32_MAX) return SSM_ERR_BAD_DIM;
  if (batch == 0 || nheads == 0) return SSM_OK;
  ssm::SsdLaunch p{x, dt, A, B, C, D, z, h0, y, h_last, dt_bias, flags, batch, seqlen, nheads, ngroups,
                   (int32_t)d_state, static_cast<hipStream_t>(stream)};
  return ssm::launch_ssd(p) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int conv_impl(const void* x, const float* w, const float* bias, const float* state_in, void* y, float* state_out,
              int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_conv, int32_t io_dtype, int32_t apply_silu,
              void* stream, bool update) {
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_conv <= 0) return SSM_ERR_BAD_DIM;
  if (seqlen > kMaxSeqlen || d_inner > kMaxDInner) return SSM_ERR_BAD_DIM;
  if (io_dtype != SSM_DTYPE_F32 && io_dtype != SSM_DTYPE_BF16) return SSM_ERR_UNSUPPORTED;
  if (d_conv < 2 || d_conv > 4) return SSM_ERR_UNSUPPORTED;
  if (apply_silu != 0 && apply_silu != 1) return SSM_ERR_UNSUPPORTED;
  const int64_t es = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  int64_t n_io, n_st;
  if (!mul3(batch, update ? 1 : seqlen, d_inner, &n_io) || !mul3(batch, d_inner, d_conv - 1, &n_st))
    return SSM_ERR_BAD_DIM;
  int64_t b_io, b_st;
  if (__builtin_mul_overflow(n_io, es, &b_io) || __builtin_mul_overflow(n_st, (int64_t)4, &b_st))
    return SSM_ERR_BAD_DIM;
  const int64_t b_w = d_inner * d_conv * 4, b_b = d_inner * 4;
  if (n_io > 0 && (x == nullptr || y == nullptr || w == nullptr)) return SSM_ERR_NULL_ARG;
  if (update && n_st > 0 && state_out == nullptr) return SSM_ERR_NULL_ARG;
  if (!aligned(x, es) || !aligned(y, es) || !aligned(w, 4) || !aligned(bias, 4) || !aligned(state_in, 4) ||
      !aligned(state_out, 4))
    return SSM_ERR_MISALIGNED;
  const void* ins[] = {x, w, bias, state_in};
  const int64_t inb[] = {b_io, b_w, bias ? b_b : 0, state_in ? b_st : 0};
  for (int k = 0; k < 4; ++k)
    if (overlap(y, b_io, ins[k], inb[k])) return SSM_ERR_ALIAS;
  if (state_out != nullptr) {
    for (int k = 0; k < 3; ++k)
      if (overlap(state_out, b_st, ins[k], inb[k])) return SSM_ERR_ALIAS;
    if (overlap(state_out, b_st, y, b_io)) return SSM_ERR_ALIAS;
    if (state_in != nullptr && state_in != state_out && overlap(state_out, b_st, state_in, b_st)) return SSM_ERR_ALIAS;
  }
  const int64_t blocks = update ? (batch * d_inner + 255) / 256 : ssm::conv_grid_blocks(batch, seqlen, d_inner);
  if (blocks > INT32_MAX || (batch * d_inner + 255) / 256 > INT32_MAX) return SSM_ERR_BAD_DIM;
  if (batch == 0 || d_inner == 0) return SSM_OK;
  ssm::ConvLaunch p{x, w, bias, state_in, y, state_out, batch, seqlen, d_inner, (int32_t)d_conv, apply_silu == 1,
                    io_dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream)};
  if (update) return ssm::launch_conv1d_update(p) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  if (seqlen == 0 && state_out == nullptr) return SSM_OK;
  return ssm::launch_conv1d(p) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_conv1d_fwd(const void* x, const float* w, const float* bias, const float* state_in, void* y,
                   float* state_out, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_conv,
                   int32_t io_dtype, int32_t apply_silu, void* stream) {
  return conv_impl(x, w, bias, state_in, y, state_out, batch, seqlen, d_inner, d_conv, io_dtype, apply_silu, stream,
                   false);
}

int ssm_conv1d_update(float* state, const void* x_t, const float* w, const float* bias, void* y_t, int64_t batch,
                      int64_t d_inner, int64_t d_conv, int32_t io_dtype, int32_t apply_silu, void* stream) {
  return conv_impl(x_t, w, bias, nullptr, y_t, state, batch, 1, d_inner, d_conv, io_dtype, apply_silu, stream, true);
}


size_t ssm_scan_bwd_workspace_size_ex(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                      int32_t ckpt_given) {
  if (check_dims(batch, seqlen, d_inner, d_state) != SSM_OK || !bwd_d_state_ok(d_state)) return (size_t)-1;
  if (ckpt_given != 0 && ckpt_given != 1) return (size_t)-1;
  const int64_t floats = bwd_workspace_floats(batch, seqlen, d_inner, d_state, ckpt_given == 1);
  if (floats < 0) return (size_t)-1;
  return (size_t)floats * 4;
}

size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  return ssm_scan_bwd_workspace_size_ex(batch, seqlen, d_inner, d_state, 0);
}

size_t ssm_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  if (check_dims(batch, seqlen, d_inner, d_state) != SSM_OK) return (size_t)-1;
  int64_t n, bytes;
  if (!mul3(batch, (seqlen + ssm::kTimeBlock - 1) / ssm::kTimeBlock, d_state, &n) ||
      __builtin_mul_overflow(n, d_inner * 4, &bytes))
    return (size_t)-1;
  return (size_t)bytes;
}

int ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* h0, const float* dt_bias, const void* dy, const float* dh_last,
                 const float* ckpt, void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                 float* dh0, float* d_dt_bias, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                 int32_t io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(x, delta, A, B, C, D, z, h0, dt_bias, dy, dh_last, ckpt, dx, ddelta, dA, dB, dC, dD, dz, dh0, d_dt_bias,
                  batch, seqlen, d_inner, d_state, io_dtype, flags, workspace, workspace_bytes, stream);
}

int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                const void* z, const float* h0, void* y, float* h_last, int64_t batch, int64_t seqlen,
                int64_t nheads, int64_t headdim, int64_t ngroups, int64_t d_state, int32_t io_dtype, uint32_t flags,
                const float* dt_bias, void* stream) {
  return ssd_impl(x, dt, A, B, C, D, z, h0, y, h_last, batch, seqlen, nheads, headdim, ngroups, d_state, io_dtype,
                  flags, dt_bias, stream);
}

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_strerror(int status) {
  switch (status) {
    case SSM_OK: return "success";
    case SSM_ERR_NULL_ARG: return "a required pointer is NULL";
    case SSM_ERR_BAD_DIM: return "invalid size (negative, overflowing, or beyond launch limits)";
    case SSM_ERR_UNSUPPORTED: return "unsupported d_state, dtype, flag or option";
    case SSM_ERR_MISALIGNED: return "pointer not aligned as required";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "HIP runtime error while launching";
    case SSM_ERR_ALIAS: return "an output overlaps an input it must not overlap";
    default: return "unknown status";
  }
}

size_t ssm_scan_fwd_ex_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                      const ssm_scan_opts_t* opts) {
  if (check_dims(batch, seqlen, d_inner, d_state) != SSM_OK || !scan_d_state_ok(d_state)) return (size_t)-1;
  Plan pl;
  if (make_plan(batch, seqlen, d_inner, d_state, opts, &pl) != SSM_OK) return (size_t)-1;
  size_t need;
  if (workspace_bytes_for(batch, d_inner, d_state, pl, &need) != SSM_OK) return (size_t)-1;
  return need;
}

size_t ssm_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  return ssm_scan_fwd_ex_workspace_size(batch, seqlen, d_inner, d_state, nullptr);
}

int ssm_scan_fwd_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, const ssm_scan_opts_t* opts,
                      int32_t* n_split_out, int64_t* chunk_len_out, int64_t* n_chunks_out) {
  int rc = check_dims(batch, seqlen, d_inner, d_state);
  if (rc != SSM_OK) return rc;
  if (!scan_d_state_ok(d_state)) return SSM_ERR_UNSUPPORTED;
  Plan pl;
  rc = make_plan(batch, seqlen, d_inner, d_state, opts, &pl);
  if (rc != SSM_OK) return rc;
  if (n_split_out) *n_split_out = pl.n_split;
  if (chunk_len_out) *chunk_len_out = pl.chunk_len;
  if (n_chunks_out) *n_chunks_out = pl.n_chunks;
  return SSM_OK;
}

int ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* h0, void* y, float* h_last, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int64_t d_state, int32_t io_dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return scan_impl(x, delta, A, B, C, D, z, h0, y, h_last, batch, seqlen, d_inner, d_state, io_dtype, nullptr,
                   workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                    const void* z, const float* h0, void* y, float* h_last, int64_t batch, int64_t seqlen,
                    int64_t d_inner, int64_t d_state, int32_t io_dtype, const ssm_scan_opts_t* opts,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return scan_impl(x, delta, A, B, C, D, z, h0, y, h_last, batch, seqlen, d_inner, d_state, io_dtype, opts,
                   workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* h0, void* y, float* h_last, int64_t batch,
                         int64_t seqlen, int64_t d_inner, int64_t d_state, int32_t io_dtype,
                         const ssm_scan_opts_t* opts, void* stream) {
  return scan_impl(x, delta, A, B, C, D, z, h0, y, h_last, batch, seqlen, d_inner, d_state, io_dtype, opts, nullptr, 0,
                   stream, true);
}

size_t ssm_scan_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int ssm_state_update(float* h, const void* x_t, const void* delta_t, const float* A, const void* B_t,
                     const void* C_t, const float* D, const void* z_t, void* y_t, int64_t batch, int64_t d_inner,
                     int64_t d_state, int32_t io_dtype, void* stream) {
  return update_impl(h, x_t, delta_t, A, B_t, C_t, D, z_t, y_t, batch, d_inner, d_state, io_dtype, 0, nullptr,
                     stream);
}

int ssm_state_update_ex(float* h, const void* x_t, const void* delta_t, const float* A, const void* B_t,
                        const void* C_t, const float* D, const void* z_t, void* y_t, int64_t batch, int64_t d_inner,
                        int64_t d_state, int32_t io_dtype, uint32_t flags, const float* dt_bias, void* stream) {
  return update_impl(h, x_t, delta_t, A, B_t, C_t, D, z_t, y_t, batch, d_inner, d_state, io_dtype, flags, dt_bias,
                     stream);
}

}  // extern "C"
