// Backward pass (gradient) of the selective scan on gfx950 (MI355X).
//
// For the loss L = sum(dy * y) + sum(dh_last * h_last), with lam_t[n] =
// dL/dh_t[n] (the adjoint of the state), the chain rule on
//   h_t = abar_t h_{t-1} + dt_t B_t x_t,   abar_t = exp(dt_t A)
//   y_t = (sum_n C_t h_t + D x_t) * silu(z_t)
// runs backwards in time:
//   g_t    = dy_t silu(z_t)                         (gradient of the pre-gate output)
//   lam_t  = abar_{t+1} lam_{t+1} + g_t C_t          (starting from dh_last)
//   dx_t   = g_t D + dt_t sum_n lam_t B_t
//   ddt_t  = sum_n lam_t (A abar_t h_{t-1} + B_t x_t)
//   dA    += lam_t dt_t abar_t h_{t-1}     dB_t += lam_t dt_t x_t   (summed over channels)
//   dC_t  += g_t h_t (summed over channels)   dD += g_t x_t   dz_t = dy_t ypre_t silu'(z_t)
//   dh0    = abar_0 lam_0
// With a softplus step, ddt is carried through softplus' derivative (the
// logistic sigmoid) to the raw input and summed per channel into d_dt_bias.
// Training back-propagates through the scan along time, keeping a few states
// and recomputing the intermediate ones ("SSMs for long-document QA"
// (pwwt.cn/news/5168881), sections 3.2-3.3; "Deriving and implementing Mamba
// from scratch" (dpshk.com/news/3333417), section 5.3: the fused scan keeps
// only what the backward pass needs).
//
// Mapping onto CDNA4 (lane = channel, as in the forward sweep):
//   1. Checkpoints: the state at the start of every block of kBB = 8 steps,
//      ckpt[b][k][n][d] (each state row one coalesced line per wave), from
//      the forward scan's checkpoint output or, in a standalone call, from
//      the forward sweep's state-only mode (k_scan_sweep, summary mode).
//   2. k_bwd_sweep: one wave per (batch row, 64-channel tile) walks the blocks
//      from last to first.  A block is recomputed forward from its checkpoint,
//      keeping abar * h_{t-1} for its steps in VGPRs (the recurrence's inputs
//      are not invertible in a stable way, so states are never run backwards),
//      then walked backwards with lam in VGPRs.  B_t and C_t are wave-uniform
//      and come through scalar loads; the per-lane rows and the checkpoint
//      go through buffer resources (lane offset in a VGPR, row offset in an
//      SGPR), so no 64-bit address is formed on the VALU.  dB_t and dC_t are
//      sums over the 64 channels of the wave: each lane writes its per-state
//      terms to LDS as rows of a [state-step][lane] table and lane r then adds
//      up row r with 16-byte reads (a transpose-and-add: per state and step,
//      one LDS write and a sixteenth of a row read, instead of a 6-level
//      cross-lane tree).
//      The per-tile sums go to a partial buffer.  dA, dD and the dt-bias
//      gradient accumulate per lane over time and are written per batch row.
//   3. k_bwd_reduce_bc / k_bwd_reduce_params: sum the partials over tiles (dB,
//      dC) and over batch rows (dA, dD, d_dt_bias) in a fixed order, so the
//      result does not depend on scheduling.
#include "scan_sweep.h"  // the forward summary sweep gives chunk entry states
#include "ssm_device.h"
#include "ssm_internal.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kBB = kBwdBlock;  // steps per checkpoint block
constexpr int kRedStride = 68;  // LDS row stride in floats (64 lanes + 4 pad: row reads stay conflict-free)

struct BwdDims {
  int64_t batch, seqlen, d_inner;
  int32_t tiles, nblk;
  int32_t n_chunks, chunk_blocks;  // sequence chunks, blocks per chunk
};

// Blocks [kb, ke) of chunk c.
__device__ __forceinline__ void chunk_blocks(const BwdDims& dm, int c, int& kb, int& ke) {
  kb = c * dm.chunk_blocks;
  ke = min(dm.nblk, kb + dm.chunk_blocks);
}

__device__ __forceinline__ float sigmoid(float v) { return hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// d/da of the exact-ZOH coefficient (exp(delta a) - 1)/a, with y = delta *
// a * log2(e), abar = 2^y, v = y ln 2 and coef from zoh_coef:
//   |v| >= 1: (delta abar - coef) / a, whose two terms differ by at least a
//             third of the larger one, so coef's error grows at most ~3x;
//   |v| < 1:  delta^2 phi'(v), phi'(v) = sum_{k>=0} (k+1) v^k / (k+2)!, to
//             10 terms (truncation < 1e-7 relative); this also covers a = 0.
__device__ __forceinline__ float zoh_coef_da(float y, float abar, float delta, float coef, float inv_a) {
  constexpr float c[10] = {1.f / 2,    2.f / 6,     3.f / 24,     4.f / 120,     5.f / 720,
                           6.f / 5040, 7.f / 40320, 8.f / 362880, 9.f / 3628800, 10.f / 39916800};
  const float v = y * kLn2;
  float p = c[9];
#pragma unroll
  for (int k = 8; k >= 0; --k) p = __builtin_fmaf(p, v, c[k]);
  const float small = delta * delta * p;
  const float big = __builtin_fmaf(delta, abar, -coef) * inv_a;
  return __builtin_fabsf(v) < 1.0f ? small : big;
}

// Raw io rows of one stage: bf16 values two to a dword (widened when read;
// the compiler folds the packing away when the values are used right after
// the load), fp32 as is.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
template <typename T, int NV>
struct RawRows;
template <int NV>
struct RawRows<uint16_t, NV> {
  u16x2 v[(NV + 1) / 2];
  __device__ __forceinline__ void set(int i, uint16_t x) { v[i >> 1][i & 1] = x; }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = __builtin_bit_cast(uint32_t, v[i >> 1]);
    return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <int NV>
struct RawRows<float, NV> {
  float v[NV];
  __device__ __forceinline__ void set(int i, float x) { v[i] = x; }
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};

// fp32 to the io type: bf16 with round-to-nearest-even, or unchanged.
template <typename T>
__device__ __forceinline__ T to_io(float v);
template <>
__device__ __forceinline__ uint16_t to_io<uint16_t>(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
template <>
__device__ __forceinline__ float to_io<float>(float v) {
  return v;
}

// Adjoint summary of chunk c >= 1: processing its steps backwards maps the
// incoming adjoint lam to P * lam + S (P = exp(A * sum delta) per state, S
// the result from lam = 0), the same affine form as the forward carry.  P is
// accumulated as the product of the very decays the sweep multiplies lam by:
// for slowly decaying channels (small delta) this matches the unsplit sweep
// far more closely than exp of the rounded sum.
// NF is the full state count of the tensors (A rows, B/C rows, lP/lS): a
// launch with N < NF covers states n_off .. n_off + N - 1 of them.
template <typename T, int N, int MODE, int NF = N>
__global__ void __launch_bounds__(64)
    k_bwd_lam_summary(const T* __restrict__ delta, const float* __restrict__ A, const T* __restrict__ C,
                      const T* __restrict__ z, const T* __restrict__ dy, const float* __restrict__ dt_bias,
                      float* __restrict__ lP, float* __restrict__ lS, const BwdDims dm, const int n_off) {
  const int lane = threadIdx.x;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = bid % dm.tiles;
  bid /= dm.tiles;
  const int chunk = 1 + bid % (dm.n_chunks - 1);
  const int64_t b = bid / (dm.n_chunks - 1);
  const int64_t DI = dm.d_inner, L = dm.seqlen;
  const int64_t d = (int64_t)tile * 64 + lane;
  const bool dvalid = d < DI;
  const int64_t dc = dvalid ? d : DI - 1;
  const int64_t cbase = (int64_t)tile * 64;
  const int lc = (int)(dc - cbase);
  const bool has_z = z != nullptr;
  int kb, ke;
  chunk_blocks(dm, chunk, kb, ke);
  const int64_t t_lo = (int64_t)kb * kBB, t_hi = min(L, (int64_t)ke * kBB);

  float Al2[N], lam[N], P[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    Al2[n] = A[dc * NF + n_off + n] * kLog2e;
    lam[n] = 0.f;
    P[n] = 1.f;
  }
  const float dtb = (MODE & 1) ? dt_bias[dc] : 0.f;
  const uint32_t row_bytes = (uint32_t)(DI * (int64_t)sizeof(T));
  const uint32_t lo = (uint32_t)lc * (uint32_t)sizeof(T);
  const uint32_t blk_span = (uint32_t)kBB * row_bytes;
  auto rs = [&](const void* base, int64_t t) {
    return block_rsrc(reinterpret_cast<const char*>(base) + ((b * L + t) * DI + cbase) * (int64_t)sizeof(T), blk_span);
  };
  const T* Cb = C + b * L * NF + n_off;
  // Blocks run from the chunk's end backwards.  The raw delta / dy / z rows
  // of the next (earlier) block load while the current one computes, and
  // each step's C row is requested one step ahead through SGPRs.
  T dn[kBB], yn[kBB], zn[kBB];
  auto fetch = [&](int64_t t1) {
    const int64_t t0 = max(t_lo, t1 - kBB);
    const int nt = (int)(t1 - t0);
    const __amdgpu_buffer_rsrc_t rd = rs(delta, t0), ry = rs(dy, t0), rz = rs(has_z ? z : delta, t0);
#pragma unroll
    for (int i = 0; i < kBB; ++i) {
      const uint32_t so = (uint32_t)min(i, nt - 1) * row_bytes;  // past the end: repeat the last row
      dn[i] = buf_ld<T>(rd, lo, so);
      yn[i] = buf_ld<T>(ry, lo, so);
      zn[i] = buf_ld<T>(rz, lo, so);
    }
  };
  StateRow<T, N> cq;
  if (t_hi > t_lo) {
    fetch(t_hi);
    cq.load(Cb + (t_hi - 1) * NF);
  }
  for (int64_t t1 = t_hi; t1 > t_lo; t1 -= kBB) {
    const int64_t t0 = max(t_lo, t1 - kBB);
    const int nt = (int)(t1 - t0);
    T dr[kBB], yr[kBB], zr[kBB];
#pragma unroll
    for (int i = 0; i < kBB; ++i) {
      dr[i] = dn[i];
      yr[i] = yn[i];
      zr[i] = zn[i];
    }
    if (t0 > t_lo) fetch(t0);
    float dt[kBB], g[kBB];
#pragma unroll
    for (int i = 0; i < kBB; ++i) {
      float v = io_to_f32(dr[i]);
      if (MODE & 1) v = softplus(v, dtb);
      dt[i] = v;
      const float dyv = dvalid ? io_to_f32(yr[i]) : 0.f;
      const float zv = io_to_f32(zr[i]);
      g[i] = has_z ? dyv * zv * sigmoid(zv) : dyv;
    }
#pragma unroll
    for (int i = kBB - 1; i >= 0; --i) {
      if (i < nt) {
        cq.touch();
        __builtin_amdgcn_sched_barrier(0);
        const StateRow<T, N> cr = cq;
        const int64_t t = t0 + i;
        cq.load(Cb + (t > t_lo ? t - 1 : t) * NF);  // at the chunk start: repeat the row
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < N; ++n) {
          const float a = hw_exp2(dt[i] * Al2[n]);
          lam[n] = __builtin_fmaf(g[i], cr.get(n), lam[n]) * a;
          P[n] *= a;
        }
      }
    }
  }
  if (t_hi > t_lo) cq.touch();  // let the last row request land
  if (dvalid) {
    const int64_t o = (((int64_t)(chunk - 1) * dm.batch + b) * DI + d) * NF + n_off;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      lP[o + n] = P[n];
      lS[o + n] = lam[n];
    }
  }
}

// Incoming adjoint of every chunk, last first: lIn[c-1] = lP[c-1] * lIn[c] +
// lS[c-1], lIn[n_chunks-1] = dh_last (or 0).  One lane per state.
__global__ void __launch_bounds__(256) k_bwd_lam_carry(const float* __restrict__ dh_last,
                                                       const float* __restrict__ lP, const float* __restrict__ lS,
                                                       float* __restrict__ lIn, int64_t states, int64_t n_chunks) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= states) return;
  float v = dh_last != nullptr ? dh_last[s] : 0.f;
  lIn[(n_chunks - 1) * states + s] = v;
  // Four chunks' pairs are loaded before they are combined (see k_chunk_carry).
  int64_t c = n_chunks - 1;
  for (; c >= 4; c -= 4) {
    float P[4], S[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      P[j] = lP[(c - 1 - j) * states + s];
      S[j] = lS[(c - 1 - j) * states + s];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v = __builtin_fmaf(P[j], v, S[j]);
      lIn[(c - 1 - j) * states + s] = v;
    }
  }
  for (; c >= 1; --c) {
    v = __builtin_fmaf(lP[(c - 1) * states + s], v, lS[(c - 1) * states + s]);
    lIn[(c - 1) * states + s] = v;
  }
}

// Steps of abar * h_{t-1} a lane keeps in VGPRs at once.  With 16 states a
// block is handled as two halves, the second one first: each half is
// reached by a forward pass from the block's checkpoint that keeps w only
// for that half (so the second half's pass also steps through the first
// half: one extra decay + FMA per state for half of the steps), then walked
// back.  This holds 64 values instead of 128, which lets two waves share a
// SIMD.
template <int N>
constexpr int bwd_sub() {
  return N * kBB <= 64 ? kBB : 64 / N;
}

// Compiled for two waves per SIMD (256 VGPRs).  The exact-ZOH variant at 16
// states spills ~130 B per lane at that size and is still faster than at one
// wave per SIMD without spills.
//
// State groups (NF > N): with more states than fit one lane's registers the
// sweep runs once per group of N states, n_off .. n_off + N - 1 of the NF in
// the tensors.  The per-state results (lam, dA, dB, dC, dh0) are the group's
// own; the per-element ones are sums over every state, so each group adds its
// part, in fp32, to part_el = [3][batch][seqlen][d_inner]: the readout
// sum_n C h (for dz), sum_n lam dt B (for dx) and the delta gradient before
// the softplus factor.  The first group writes, the others add (the groups
// run one after another on the stream); k_bwd_finalize then adds the skip and
// gate terms and writes dx, ddelta, dz, and the dD and dt-bias partials.
template <typename T, int N, int MODE, int NF = N>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_bwd_sweep(const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
                const T* __restrict__ B, const T* __restrict__ C, const float* __restrict__ D,
                const T* __restrict__ z, const T* __restrict__ dy, const float* __restrict__ dh_last,
                const float* __restrict__ dt_bias, const float* __restrict__ ckpt, T* __restrict__ dx,
                T* __restrict__ ddelta, T* __restrict__ dz, float* __restrict__ dh0, float* __restrict__ part_bc,
                float* __restrict__ part_a, float* __restrict__ part_d, float* __restrict__ part_t,
                const float* __restrict__ lam_in, const BwdDims dm, const int n_off,
                float* __restrict__ part_el) {
  constexpr bool kPart = NF > N;
  constexpr int SUB = bwd_sub<N>();                   // steps of w held at once
  constexpr int NSUB = kBB / SUB;                     // sub-blocks per block
  constexpr int GS = (64 / N) < SUB ? (64 / N) : SUB;  // steps per LDS reduction group
  constexpr int ROWS = GS * N;
  static_assert(kBB % SUB == 0 && SUB % GS == 0 && ROWS <= 64, "bad block split");
  __shared__ __align__(16) float red[ROWS * kRedStride];

  const int lane = threadIdx.x;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = bid % dm.tiles;
  bid /= dm.tiles;
  const int chunk = bid % dm.n_chunks;
  const int64_t b = bid / dm.n_chunks;
  const int64_t DI = dm.d_inner, L = dm.seqlen;
  const int64_t d = (int64_t)tile * 64 + lane;
  const bool dvalid = d < DI;
  const int64_t dc = dvalid ? d : DI - 1;
  const bool has_z = z != nullptr;
  int kb, ke;
  chunk_blocks(dm, chunk, kb, ke);

  // Lanes past d_inner run on a copy of the last channel with g = 0 and
  // lam = 0, so every term they add to the channel sums is zero.  The
  // incoming adjoint is dh_last for one chunk, else the chunk's carry.
  const float* li = lam_in != nullptr ? lam_in + (((int64_t)chunk * dm.batch + b) * DI + d) * NF + n_off
                                      : (dh_last != nullptr ? dh_last + (b * DI + d) * NF + n_off : nullptr);
  float Al2[N], lam[N], gA[N];
  float ia[(MODE & kExactZoh) ? N : 1];  // 1/a for the exact-ZOH coefficient
#pragma unroll
  for (int n = 0; n < N; ++n) {
    Al2[n] = A[dc * NF + n_off + n] * kLog2e;
    if (MODE & kExactZoh) ia[n] = 1.0f / A[dc * NF + n_off + n];
    lam[n] = (dvalid && li != nullptr) ? li[n] : 0.f;
    gA[n] = 0.f;
  }
  const float Dv = D != nullptr ? D[dc] : 0.f;
  const float dtb = (MODE & 1) ? dt_bias[dc] : 0.f;
  float accD = 0.f, accT = 0.f;
  const int wslot = wave_slot_parity();  // for take_turn (ssm_device.h)

  // Addressing (as in the forward sweep): the io tensors share one layout,
  // so a block of kBB rows is one buffer resource per tensor (SGPRs), the
  // lane's byte offset in one VGPR and the row's offset in an SGPR.
  const int64_t cbase = (int64_t)tile * 64;
  const int lc = (int)(dc - cbase);
  const uint32_t row_bytes = (uint32_t)(DI * (int64_t)sizeof(T));
  const uint32_t lane_b = (uint32_t)lc * (uint32_t)sizeof(T);
  auto rowp = [&](const void* base, int64_t t) {
    return block_rsrc(reinterpret_cast<const char*>(base) + ((b * L + t) * DI + cbase) * (int64_t)sizeof(T),
                      0xffffffffu);
  };
  auto st = [&](__amdgpu_buffer_rsrc_t r, uint32_t so, float v) { buf_st(to_io<T>(v), r, lane_b, so); };
  const T* Bb = B + b * L * NF + n_off;
  const T* Cb = C + b * L * NF + n_off;
  float* pbc = part_bc + ((int64_t)tile * dm.batch + b) * L * (2 * NF) + n_off;
  // fp32 per-element sums of a state group (plane 0 readout, 1 dx, 2 ddelta).
  const int64_t plane = dm.batch * L * DI;
  auto add_part = [&](int pl, int64_t t, float v) {
    float* q = part_el + pl * plane + (b * L + t) * DI + d;
    *q = n_off == 0 ? v : *q + v;
  };

  // B/C rows run one step ahead through SGPRs: each step waits for its own
  // rows (issued one step earlier), then requests the rows of the step that
  // follows it in processing order.
  StateRow<T, N> bq, cq;
  auto issue = [&](int64_t t) {
    bq.load(Bb + t * NF);
    cq.load(Cb + t * NF);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto take = [&](StateRow<T, N>& bc, StateRow<T, N>& cc) {
    bq.touch();
    cq.touch();
    __builtin_amdgcn_sched_barrier(0);
    bc = bq;
    cc = cq;
  };

  // Sum of the ROWS x 64 table over lanes; row r = (step s, state n) of the
  // group starting at step g0 lands in the partial buffer at step
  // t0 + g0 + s, column which + n (which = 0 for dB, N for dC).  Four
  // 16-byte reads are in flight at a time.
  auto reduce = [&](int64_t t0, int g0, int nt, int which) {
    __syncthreads();
    if (lane < ROWS) {
      const float4* row = reinterpret_cast<const float4*>(red + lane * kRedStride);
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int q0 = 0; q0 < 16; q0 += 4) {
        float4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = row[q0 + q];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s0 += v[q].x;
          s1 += v[q].y;
          s2 += v[q].z;
          s3 += v[q].w;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const int st_ = lane / N, n = lane % N;
      if (g0 + st_ < nt) pbc[(t0 + g0 + st_) * (2 * NF) + which + n] = (s0 + s1) + (s2 + s3);
    }
    __syncthreads();
  };

  // Each stage requests its rows when it starts: a block its x and delta
  // rows, a pass its dy and z rows and its checkpoint.  Requesting them one
  // stage earlier, into registers free at that point, kept more values live
  // and measured slower at two waves per SIMD.  Loads are unconditional (z
  // falls back to x; tail lanes read a valid channel) and past a ragged end
  // they repeat the last row, so no load waits behind a branch.
  RawRows<T, kBB> px, pd;
  RawRows<T, SUB> pdy, pz;
  float ph[N];
  const uint32_t coff = (uint32_t)lc * 4u;
  const uint32_t crow = (uint32_t)DI * 4u;
  auto steps_of = [&](int k) { return (int)min((int64_t)kBB, L - (int64_t)k * kBB); };
  auto request_block = [&](int k) {
    const int nt = steps_of(k);
    const __amdgpu_buffer_rsrc_t xb = rowp(x, (int64_t)k * kBB);
    const __amdgpu_buffer_rsrc_t db = rowp(delta, (int64_t)k * kBB);
#pragma unroll
    for (int i = 0; i < kBB; ++i) {
      const uint32_t o = (uint32_t)min(i, nt - 1) * row_bytes;
      px.set(i, buf_ld<T>(xb, lane_b, o));
      pd.set(i, buf_ld<T>(db, lane_b, o));
    }
  };
  auto request_pass = [&](int k, int j) {
    const int nt = steps_of(k);
    const __amdgpu_buffer_rsrc_t yb = rowp(dy, (int64_t)k * kBB);
    const __amdgpu_buffer_rsrc_t zb = rowp(has_z ? (const void*)z : (const void*)x, (int64_t)k * kBB);
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const uint32_t o = (uint32_t)min(j * SUB + i, nt - 1) * row_bytes;
      pdy.set(i, buf_ld<T>(yb, lane_b, o));
      pz.set(i, buf_ld<T>(zb, lane_b, o));
    }
    // The checkpoint's state rows are DI floats apart: one buffer resource
    // for the block, the lane's column in a VGPR and the row offset in an
    // SGPR that is advanced per state (the empty asm keeps the compiler from
    // precomputing all N row offsets, which would hold 2N SGPRs).
    const __amdgpu_buffer_rsrc_t cpr =
        block_rsrc(ckpt + ((b * dm.nblk + k) * NF + n_off) * DI + cbase, 0xffffffffu);
    uint32_t so = 0;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      ph[n] = buf_ld<float>(cpr, coff, so);
      so += crow;
      asm volatile("" : "+s"(so));
    }
  };

  auto block = [&](int k) {
    take_turn(k, wslot);
    const int64_t t0 = (int64_t)k * kBB;
    const int nt = steps_of(k);
    const int nsub = (nt + SUB - 1) / SUB;  // sub-blocks holding steps
    request_block(k);
    float xv[kBB], dt[kBB], sg[(MODE & 1) ? kBB : 1];
#pragma unroll
    for (int i = 0; i < kBB; ++i) {
      xv[i] = px.get(i);
      const float raw = pd.get(i);
      if (MODE & 1) {
        const float v = raw + dtb;
        dt[i] = softplus(raw, dtb);
        sg[i] = sigmoid(v);
      } else {
        dt[i] = raw;
      }
    }

#pragma unroll
    for (int j = NSUB - 1; j >= 0; --j) {
      if (j >= nsub) continue;
      const int lo = j * SUB, hi = min(nt, lo + SUB);  // this pass covers steps [lo, hi)
      request_pass(k, j);
      // dy and the gate terms of this sub-block.
      float g[SUB], dsz[SUB];
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const float dyv = dvalid ? pdy.get(i) : 0.f;
        const float zv = pz.get(i);
        const float s = sigmoid(zv);
        g[i] = has_z ? dyv * zv * s : dyv;
        dsz[i] = dyv * s * __builtin_fmaf(zv, 1.f - s, 1.f);
      }

      // Forward from the checkpoint to the end of this sub-block.  Steps
      // before it only advance h; its own steps keep w = abar * h_{i-1},
      // read out the pre-gate output (for dz) and write the rows g * h_i
      // (for dC).  Each pass reads the steps through its own opaque copy, so
      // the compiler cannot merge the decays of different passes (keeping
      // them alive between passes would cost more VGPRs than recomputing).
      float w[SUB][N];
      float dtp[kBB];
      const __amdgpu_buffer_rsrc_t zo = rowp(has_z ? (const void*)dz : (const void*)dx, t0);  // used only with z
#pragma unroll
      for (int i = 0; i < kBB; ++i) {
        dtp[i] = dt[i];
        if (i < lo + SUB) asm volatile("" : "+v"(dtp[i]));
      }
      {
        float h[N];
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = ph[n];
#pragma unroll
        for (int i = 0; i < lo; ++i) {
          StateRow<T, N> br, cr;
          take(br, cr);
          issue(t0 + i + 1);
          const float dtx = dtp[i] * xv[i];
#pragma unroll
          for (int n = 0; n < N; ++n) {
            if (MODE & kExactZoh) {
              const float yv = dtp[i] * Al2[n];
              const float ab = hw_exp2(yv);
              h[n] = __builtin_fmaf(zoh_coef(yv, ab, dtp[i], ia[n]), xv[i] * br.get(n), ab * h[n]);
            } else {
              h[n] = __builtin_fmaf(dtx, br.get(n), hw_exp2(dtp[i] * Al2[n]) * h[n]);
            }
          }
        }
#pragma unroll
        for (int g0 = 0; g0 < SUB; g0 += GS) {
          if (lo + g0 >= hi) break;
#pragma unroll
          for (int s = 0; s < GS; ++s) {
            const int ii = g0 + s, i = lo + ii;
            if (i < hi) {
              StateRow<T, N> br, cr;
              take(br, cr);
              issue(i + 1 < hi ? t0 + i + 1 : t0 + hi - 1);
              const float dtx = dtp[i] * xv[i];
              float acc = kPart ? 0.f : Dv * xv[i];
#pragma unroll
              for (int n = 0; n < N; ++n) {
                if (MODE & kExactZoh) {
                  const float yv = dtp[i] * Al2[n];
                  const float ab = hw_exp2(yv);
                  const float wv = ab * h[n];
                  w[ii][n] = wv;
                  h[n] = __builtin_fmaf(zoh_coef(yv, ab, dtp[i], ia[n]), xv[i] * br.get(n), wv);
                } else {
                  const float wv = hw_exp2(dtp[i] * Al2[n]) * h[n];
                  w[ii][n] = wv;
                  h[n] = __builtin_fmaf(dtx, br.get(n), wv);
                }
                acc = __builtin_fmaf(cr.get(n), h[n], acc);
                red[(s * N + n) * kRedStride + lane] = g[ii] * h[n];
              }
              if constexpr (kPart) {
                if (has_z && dvalid) add_part(0, t0 + i, acc);
              } else {
                if (has_z && dvalid) st(zo, (uint32_t)i * row_bytes, acc * dsz[ii]);
              }
            }
          }
          reduce(t0, lo + g0, nt, NF);
        }
      }

      // Backward through this sub-block.
      const __amdgpu_buffer_rsrc_t xo = rowp(dx, t0);
      const __amdgpu_buffer_rsrc_t po = rowp(ddelta, t0);
#pragma unroll
      for (int g0 = SUB - GS; g0 >= 0; g0 -= GS) {
        if (lo + g0 >= hi) continue;
#pragma unroll
        for (int s = GS - 1; s >= 0; --s) {
          const int ii = g0 + s, i = lo + ii;
          if (i < hi) {
            StateRow<T, N> br, cr;
            take(br, cr);
            issue(i > lo ? t0 + i - 1 : (j > 0 ? t0 : (k > kb ? t0 - kBB : t0)));
            // The decays are recomputed here rather than kept from the
            // forward pass (that would hold another SUB * N values in
            // VGPRs); the empty asm keeps the compiler from merging the two
            // computations.
            float dti = dt[i];
            asm volatile("" : "+v"(dti));
            const float dtx = dti * xv[i];
            // sb = sum_n lam B (the input term's adjoint per unit coefficient);
            // with the exact ZOH the coefficient differs per state, so sb
            // carries it (sum_n lam coef B) and sa = sum_n lam abar B is its
            // derivative in delta.
            float dd = 0.f, sb = 0.f, sa = 0.f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
              lam[n] = __builtin_fmaf(g[ii], cr.get(n), lam[n]);
              const float tw = lam[n] * w[ii][n];
              dd = __builtin_fmaf(tw, Al2[n], dd);
              gA[n] = __builtin_fmaf(dti, tw, gA[n]);
              if (MODE & kExactZoh) {
                const float yv = dti * Al2[n];
                const float ab = hw_exp2(yv);
                const float coef = zoh_coef(yv, ab, dti, ia[n]);
                const float lb = lam[n] * br.get(n);
                sb = __builtin_fmaf(lb, coef, sb);
                sa = __builtin_fmaf(lb, ab, sa);
                gA[n] = __builtin_fmaf(lb * xv[i], zoh_coef_da(yv, ab, dti, coef, ia[n]), gA[n]);
                red[(s * N + n) * kRedStride + lane] = lam[n] * coef * xv[i];
                lam[n] *= ab;
              } else {
                sb = __builtin_fmaf(lam[n], br.get(n), sb);
                red[(s * N + n) * kRedStride + lane] = lam[n] * dtx;
                lam[n] *= hw_exp2(dti * Al2[n]);
              }
            }
            if constexpr (kPart) {
              if (dvalid) {
                add_part(1, t0 + i, (MODE & kExactZoh) ? sb : dti * sb);
                add_part(2, t0 + i, __builtin_fmaf(dd, kLn2, xv[i] * ((MODE & kExactZoh) ? sa : sb)));
              }
            } else {
              const float dxv =
                  (MODE & kExactZoh) ? __builtin_fmaf(g[ii], Dv, sb) : __builtin_fmaf(g[ii], Dv, dti * sb);
              float ddt = __builtin_fmaf(dd, kLn2, xv[i] * ((MODE & kExactZoh) ? sa : sb));
              if (MODE & 1) ddt *= sg[i];
              accT += ddt;
              accD = __builtin_fmaf(g[ii], xv[i], accD);
              if (dvalid) {
                st(xo, (uint32_t)i * row_bytes, dxv);
                st(po, (uint32_t)i * row_bytes, ddt);
              }
            }
          }
        }
        reduce(t0, lo + g0, nt, 0);
      }
    }
  };

  if (ke > kb) {
    issue((int64_t)(ke - 1) * kBB);
    for (int k = ke - 1; k >= kb; --k) block(k);
    // Let the last row request land before the wave ends.
    bq.touch();
    cq.touch();
  }

  if (dvalid) {
    if (dh0 != nullptr && chunk == 0) {
#pragma unroll
      for (int n = 0; n < N; ++n) dh0[(b * DI + d) * NF + n_off + n] = lam[n];
    }
    const int64_t row = (int64_t)chunk * dm.batch + b;
#pragma unroll
    for (int n = 0; n < N; ++n) part_a[(row * DI + d) * NF + n_off + n] = gA[n];
    if (!kPart) {
      part_d[row * DI + d] = accD;
      part_t[row * DI + d] = accT;
    }
  }
}

// sum over k = 0..count-1 of p[k * stride], in a fixed order: eight partial
// sums (k mod 8) added pairwise at the end, so that eight loads are in flight
// per thread (one running sum waits for every load in turn: with few
// elements per launch, such as the Mamba-130M layer's 24576 dA entries over
// 256 rows, that latency chain was the whole cost).
__device__ __forceinline__ float strided_sum(const float* __restrict__ p, int64_t count, int64_t stride) {
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = 0.f;
  int64_t k = 0;
  for (; k + 8 <= count; k += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] += p[(k + j) * stride];
  }
#pragma unroll
  for (int j = 0; j < 7; ++j)
    if (k + j < count) s[j] += p[(k + j) * stride];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// dB[r][n] = sum over tiles of part[tile][r][n], dC[r][n] likewise from
// column N + n; r runs over (b, t).
__global__ void __launch_bounds__(256) k_bwd_reduce_bc(const float* __restrict__ part, float* __restrict__ dB,
                                                       float* __restrict__ dC, int64_t rows, int32_t N,
                                                       int32_t tiles) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = rows * 2 * N;
  if (i >= total) return;
  const float s = strided_sum(part + i, tiles, total);
  const int64_t r = i / (2 * N);
  const int c = (int)(i - r * 2 * N);
  if (c < N) {
    dB[r * N + c] = s;
  } else {
    dC[r * N + c - N] = s;
  }
}

// dA[d][n], dD[d], d_dt_bias[d]: sums over batch rows.
__global__ void __launch_bounds__(256) k_bwd_reduce_params(const float* __restrict__ part_a,
                                                           const float* __restrict__ part_d,
                                                           const float* __restrict__ part_t, float* __restrict__ dA,
                                                           float* __restrict__ dD, float* __restrict__ d_dt_bias,
                                                           int64_t batch, int64_t d_inner, int32_t N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t na = d_inner * N;
  if (i < na) dA[i] = strided_sum(part_a + i, batch, na);
  if (i < d_inner) {
    if (dD != nullptr) dD[i] = strided_sum(part_d + i, batch, d_inner);
    if (d_dt_bias != nullptr) d_dt_bias[i] = strided_sum(part_t + i, batch, d_inner);
  }
}

template <typename T, int N, int MODE>
hipError_t launch_bwd_t(const BwdLaunch& p, const BwdWorkspace& ws, const BwdPlan& pl) {
  const int64_t tiles = (p.d_inner + 63) / 64;
  const int nch = (int)pl.n_chunks;
  const BwdDims dm{p.batch, p.seqlen, p.d_inner, (int32_t)tiles, (int32_t)((p.seqlen + kBB - 1) / kBB), nch,
                   (int32_t)(pl.chunk_len / kBB)};
  const T* x = static_cast<const T*>(p.x);
  const T* dl = static_cast<const T*>(p.delta);
  const T* Bm = static_cast<const T*>(p.B);
  const T* Cm = static_cast<const T*>(p.C);
  const T* zz = static_cast<const T*>(p.z);
  const T* dyy = static_cast<const T*>(p.dy);
  const int64_t states = p.batch * p.d_inner * N;
  hipError_t e;
  const unsigned waves = (unsigned)(p.batch * tiles);
  if (waves > 0) {
    const float* ck = p.ckpt;
    if (ck == nullptr && dm.nblk > 0) {
      const float* h_entry = nullptr;
      if (nch > 1) {
        // Entry state of every chunk: the forward scan's chunk summaries
        // (k_scan_sweep in summary mode) and their carry.
        SweepDims sd{p.batch, p.seqlen, p.d_inner, pl.chunk_len, (int32_t)tiles, nch - 1, nch, 0, nullptr};
        e = launch(k_scan_sweep<T, N, N, true, MODE>, dim3((unsigned)(p.batch * (nch - 1) * tiles)), dim3(64), 0,
                   p.stream, x, dl, p.A, Bm, Cm, (const float*)nullptr, zz, (const float*)nullptr, (T*)nullptr,
                   (float*)nullptr, ws.fT, ws.fS, p.dt_bias, sd);
        if (e != hipSuccess) return e;
        e = launch_chunk_carry(p.h0, p.A, (MODE & kLinearA) != 0, ws.fT, ws.fS, ws.fH, p.batch * p.d_inner, N,
                               p.d_inner, nch, p.stream);
        if (e != hipSuccess) return e;
        h_entry = ws.fH;
      }
      // The checkpoints: the forward sweep's state-only (summary) mode, run
      // from each chunk's entry state, writes the state before every block.
      SweepDims cd{p.batch, p.seqlen, p.d_inner, pl.chunk_len, (int32_t)tiles, nch, nch, h_entry != nullptr ? 1 : 0,
                   ws.ckpt};
      e = launch(k_scan_sweep<T, N, N, true, MODE>, dim3(waves * nch), dim3(64), 0, p.stream, x, dl, p.A, Bm, Cm,
                 (const float*)nullptr, zz, h_entry != nullptr ? h_entry : p.h0, (T*)nullptr, (float*)nullptr,
                 (float*)nullptr, (float*)nullptr, p.dt_bias, cd);
      if (e != hipSuccess) return e;
      ck = ws.ckpt;
    }
    const float* lam_in = nullptr;
    if (nch > 1) {
      e = launch(k_bwd_lam_summary<T, N, MODE>, dim3((unsigned)(p.batch * (nch - 1) * tiles)), dim3(64), 0,
                 p.stream, dl, p.A, Cm, zz, dyy, p.dt_bias, ws.lP, ws.lS, dm, 0);
      if (e != hipSuccess) return e;
      e = launch(k_bwd_lam_carry, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, p.stream, p.dh_last, ws.lP,
                 ws.lS, ws.lIn, states, (int64_t)nch);
      if (e != hipSuccess) return e;
      lam_in = ws.lIn;
    }
    e = launch(k_bwd_sweep<T, N, MODE>, dim3(waves * nch), dim3(64), 0, p.stream, x, dl, p.A, Bm, Cm, p.D, zz, dyy,
               p.dh_last, p.dt_bias, ck, static_cast<T*>(p.dx), static_cast<T*>(p.ddelta), static_cast<T*>(p.dz),
               p.dh0, ws.part_bc, ws.part_a, ws.part_d, ws.part_t, lam_in, dm, 0, (float*)nullptr);
    if (e != hipSuccess) return e;
  }
  const int64_t rows = p.batch * p.seqlen;
  if (rows > 0) {
    const int64_t total = rows * 2 * N;
    e = launch(k_bwd_reduce_bc, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, p.stream, ws.part_bc, p.dB,
               p.dC, rows, (int32_t)N, (int32_t)tiles);
    if (e != hipSuccess) return e;
  }
  const int64_t na = p.d_inner * N;
  if (na > 0) {
    // Partials are [chunk][batch] rows: sum over both.
    e = launch(k_bwd_reduce_params, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, p.stream, ws.part_a,
               ws.part_d, ws.part_t, p.dA, p.dD, p.d_dt_bias, p.batch * nch, p.d_inner, (int32_t)N);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Per-element gradients of a state-group backward (NF > 16): the groups'
// fp32 sums in part_el plus the skip and gate terms, one thread per (b, d)
// walking the sequence (a wave reads and writes whole rows).  Also the
// per-row partials of dD (sum g x) and d_dt_bias (sum of the step gradient
// through softplus' derivative), in row c = 0 of the [chunk][batch] layout
// that k_bwd_reduce_params sums; rows of later chunks are zeroed.
template <typename T, int MODE>
__global__ void __launch_bounds__(256)
    k_bwd_finalize(const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ D,
                   const T* __restrict__ z, const T* __restrict__ dy, const float* __restrict__ dt_bias,
                   const float* __restrict__ part_el, T* __restrict__ dx, T* __restrict__ ddelta, T* __restrict__ dz,
                   float* __restrict__ part_d, float* __restrict__ part_t, int64_t batch, int64_t seqlen,
                   int64_t d_inner, int32_t n_chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= batch * d_inner) return;
  const int64_t b = i / d_inner, d = i - b * d_inner;
  const float Dv = D != nullptr ? D[d] : 0.f;
  const float dtb = (MODE & 1) ? dt_bias[d] : 0.f;
  const int64_t plane = batch * seqlen * d_inner;
  float accD = 0.f, accT = 0.f;
  for (int64_t t = 0; t < seqlen; ++t) {
    const int64_t o = (b * seqlen + t) * d_inner + d;
    const float xv = io_to_f32(x[o]);
    const float dyv = io_to_f32(dy[o]);
    float g = dyv;
    if (z != nullptr) {
      const float zv = io_to_f32(z[o]);
      const float sz = sigmoid(zv);
      g = dyv * zv * sz;
      const float ypre = __builtin_fmaf(Dv, xv, part_el[o]);
      dz[o] = to_io<T>(ypre * (dyv * sz * __builtin_fmaf(zv, 1.f - sz, 1.f)));
    }
    dx[o] = to_io<T>(__builtin_fmaf(g, Dv, part_el[plane + o]));
    float ddt = part_el[2 * plane + o];
    if (MODE & 1) ddt *= sigmoid(io_to_f32(delta[o]) + dtb);
    ddelta[o] = to_io<T>(ddt);
    accT += ddt;
    accD = __builtin_fmaf(g, xv, accD);
  }
  part_d[b * d_inner + d] = accD;
  part_t[b * d_inner + d] = accT;
  for (int c = 1; c < n_chunks; ++c) {
    part_d[((int64_t)c * batch + b) * d_inner + d] = 0.f;
    part_t[((int64_t)c * batch + b) * d_inner + d] = 0.f;
  }
}

// Backward for NF = 32, 64 or 128 states: the 16-state sweep once per group
// of 16 states (see k_bwd_sweep), then k_bwd_finalize.  Checkpoints come
// from the forward sweep's state-only mode with NF / 16 waves per tile.
template <typename T, int NF, int MODE>
hipError_t launch_bwd_groups(const BwdLaunch& p, const BwdWorkspace& ws, const BwdPlan& pl) {
  constexpr int NG = 16;
  constexpr int G = NF / NG;
  const int64_t tiles = (p.d_inner + 63) / 64;
  const int nch = (int)pl.n_chunks;
  const BwdDims dm{p.batch, p.seqlen, p.d_inner, (int32_t)tiles, (int32_t)((p.seqlen + kBB - 1) / kBB), nch,
                   (int32_t)(pl.chunk_len / kBB)};
  const T* x = static_cast<const T*>(p.x);
  const T* dl = static_cast<const T*>(p.delta);
  const T* Bm = static_cast<const T*>(p.B);
  const T* Cm = static_cast<const T*>(p.C);
  const T* zz = static_cast<const T*>(p.z);
  const T* dyy = static_cast<const T*>(p.dy);
  const int64_t states = p.batch * p.d_inner * NF;
  hipError_t e;
  const unsigned waves = (unsigned)(p.batch * tiles);
  if (waves > 0) {
    const float* ck = p.ckpt;
    if (ck == nullptr && dm.nblk > 0) {
      const float* h_entry = nullptr;
      if (nch > 1) {
        SweepDims sd{p.batch, p.seqlen, p.d_inner, pl.chunk_len, (int32_t)tiles, nch - 1, nch, 0, nullptr};
        e = launch(k_scan_sweep<T, NF, NG, true, MODE>, dim3((unsigned)(p.batch * (nch - 1) * tiles)), dim3(64 * G),
                   0, p.stream, x, dl, p.A, Bm, Cm, (const float*)nullptr, zz, (const float*)nullptr, (T*)nullptr,
                   (float*)nullptr, ws.fT, ws.fS, p.dt_bias, sd);
        if (e != hipSuccess) return e;
        e = launch_chunk_carry(p.h0, p.A, (MODE & kLinearA) != 0, ws.fT, ws.fS, ws.fH, p.batch * p.d_inner, NF,
                               p.d_inner, nch, p.stream);
        if (e != hipSuccess) return e;
        h_entry = ws.fH;
      }
      SweepDims cd{p.batch, p.seqlen, p.d_inner, pl.chunk_len, (int32_t)tiles, nch, nch, h_entry != nullptr ? 1 : 0,
                   ws.ckpt};
      e = launch(k_scan_sweep<T, NF, NG, true, MODE>, dim3(waves * nch), dim3(64 * G), 0, p.stream, x, dl, p.A, Bm,
                 Cm, (const float*)nullptr, zz, h_entry != nullptr ? h_entry : p.h0, (T*)nullptr, (float*)nullptr,
                 (float*)nullptr, (float*)nullptr, p.dt_bias, cd);
      if (e != hipSuccess) return e;
      ck = ws.ckpt;
    }
    const float* lam_in = nullptr;
    if (nch > 1) {
      for (int gi = 0; gi < G; ++gi) {
        e = launch(k_bwd_lam_summary<T, NG, MODE, NF>, dim3((unsigned)(p.batch * (nch - 1) * tiles)), dim3(64), 0,
                   p.stream, dl, p.A, Cm, zz, dyy, p.dt_bias, ws.lP, ws.lS, dm, NG * gi);
        if (e != hipSuccess) return e;
      }
      e = launch(k_bwd_lam_carry, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, p.stream, p.dh_last, ws.lP,
                 ws.lS, ws.lIn, states, (int64_t)nch);
      if (e != hipSuccess) return e;
      lam_in = ws.lIn;
    }
    for (int gi = 0; gi < G; ++gi) {
      e = launch(k_bwd_sweep<T, NG, MODE, NF>, dim3(waves * nch), dim3(64), 0, p.stream, x, dl, p.A, Bm, Cm, p.D, zz,
                 dyy, p.dh_last, p.dt_bias, ck, static_cast<T*>(p.dx), static_cast<T*>(p.ddelta),
                 static_cast<T*>(p.dz), p.dh0, ws.part_bc, ws.part_a, ws.part_d, ws.part_t, lam_in, dm, NG * gi,
                 ws.part_el);
      if (e != hipSuccess) return e;
    }
    const int64_t rows_bd = p.batch * p.d_inner;
    e = launch(k_bwd_finalize<T, MODE>, dim3((unsigned)((rows_bd + 255) / 256)), dim3(256), 0, p.stream, x, dl, p.D,
               zz, dyy, p.dt_bias, (const float*)ws.part_el, static_cast<T*>(p.dx), static_cast<T*>(p.ddelta),
               static_cast<T*>(p.dz), ws.part_d, ws.part_t, p.batch, p.seqlen, p.d_inner, (int32_t)nch);
    if (e != hipSuccess) return e;
  }
  const int64_t rows = p.batch * p.seqlen;
  if (rows > 0) {
    const int64_t total = rows * 2 * NF;
    e = launch(k_bwd_reduce_bc, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, p.stream, ws.part_bc, p.dB,
               p.dC, rows, (int32_t)NF, (int32_t)tiles);
    if (e != hipSuccess) return e;
  }
  const int64_t na = p.d_inner * NF;
  if (na > 0) {
    e = launch(k_bwd_reduce_params, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, p.stream, ws.part_a,
               ws.part_d, ws.part_t, p.dA, p.dD, p.d_dt_bias, p.batch * nch, p.d_inner, (int32_t)NF);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int MODE>
hipError_t launch_bwd_n(const BwdLaunch& p, const BwdWorkspace& ws, const BwdPlan& pl) {
  switch (p.d_state) {
    case 2: return launch_bwd_t<T, 2, MODE>(p, ws, pl);
    case 4: return launch_bwd_t<T, 4, MODE>(p, ws, pl);
    case 8: return launch_bwd_t<T, 8, MODE>(p, ws, pl);
    case 16: return launch_bwd_t<T, 16, MODE>(p, ws, pl);
    case 32: return launch_bwd_groups<T, 32, MODE>(p, ws, pl);
    case 64: return launch_bwd_groups<T, 64, MODE>(p, ws, pl);
    case 128: return launch_bwd_groups<T, 128, MODE>(p, ws, pl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Below kBwdFillWaves waves from channels (256 CUs x 4 SIMDs x 2) the
// sequence is cut into chunks, aiming at kBwdChunkTargetWaves waves with
// chunks of at least kBwdMinChunk steps.  Measured on MI355X: the
// Mamba-2.8B long layer takes 27.2 ms with ~2048 waves and 17.5 ms with
// ~16384 (32768: no further gain); the Mamba-1.4B layer (2048 waves) is
// faster unchunked (11.4 ms against 13.4 ms cut into chunks).
constexpr int64_t kBwdFillWaves = 2048;
constexpr int64_t kBwdChunkTargetWaves = 16384;
constexpr int64_t kBwdMinChunk = 64;

BwdPlan bwd_plan(int64_t batch, int64_t seqlen, int64_t d_inner) {
  const int64_t waves = batch * ((d_inner + 63) / 64);
  int64_t nch = 1;
  if (waves > 0 && waves < kBwdFillWaves && seqlen >= 2 * kBwdMinChunk) {
    nch = (kBwdChunkTargetWaves + waves - 1) / waves;
    if (nch > seqlen / kBwdMinChunk) nch = seqlen / kBwdMinChunk;
  }
  const int64_t nblk = (seqlen + kBB - 1) / kBB;
  int64_t cb = nblk > 0 ? (nblk + nch - 1) / nch : 1;  // blocks per chunk
  if (cb < 1) cb = 1;
  BwdPlan p;
  p.chunk_len = cb * kBB;
  p.n_chunks = nblk > 0 ? (nblk + cb - 1) / cb : 1;
  return p;
}

BwdWorkspace bwd_workspace_layout(float* base, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                  const BwdPlan& plan, bool ckpt_given, int64_t* total_floats) {
  auto up = [](int64_t v) { return (v + 63) / 64 * 64; };  // 256-byte sections
  const int64_t tiles = (d_inner + 63) / 64;
  const int64_t nblk = (seqlen + kBB - 1) / kBB;
  const int64_t nch = plan.n_chunks;
  const int64_t states = batch * d_inner * d_state;
  const int64_t n_ck = ckpt_given ? 0 : up(batch * nblk * d_state * d_inner);
  const int64_t n_bc = up(tiles * batch * seqlen * 2 * d_state);
  const int64_t n_a = up(nch * states);
  const int64_t n_d = up(nch * batch * d_inner);
  const int64_t n_sum = nch > 1 ? up((nch - 1) * states) : 0;
  const int64_t n_ent = nch > 1 ? up(nch * states) : 0;
  // Forward chunk summaries (step sums, end states) and entry states: only to
  // compute checkpoints.
  const int64_t n_ftsum = ckpt_given ? 0 : scan_stepsum_floats(nch, batch * d_inner);
  const int64_t n_fsum = ckpt_given ? 0 : n_sum;
  const int64_t n_fent = ckpt_given ? 0 : n_ent;
  // Per-element sums of the state groups (more than 16 states).
  const int64_t n_el = d_state > 16 ? up(3 * batch * seqlen * d_inner) : 0;
  BwdWorkspace ws{};
  if (base != nullptr) {
    ws.ckpt = ckpt_given ? nullptr : base;
    ws.part_bc = base + n_ck;
    ws.part_a = ws.part_bc + n_bc;
    ws.part_d = ws.part_a + n_a;
    ws.part_t = ws.part_d + n_d;
    float* f = ws.part_t + n_d;
    ws.fT = ckpt_given ? nullptr : f;
    ws.fS = ckpt_given ? nullptr : f + n_ftsum;
    ws.fH = ckpt_given ? nullptr : f + n_ftsum + n_fsum;
    ws.lP = f + n_ftsum + n_fsum + n_fent;
    ws.lS = ws.lP + n_sum;
    ws.lIn = ws.lS + n_sum;
    ws.part_el = n_el > 0 ? ws.lIn + n_ent : nullptr;
  }
  if (total_floats != nullptr)
    *total_floats = n_ck + n_bc + n_a + 2 * n_d + n_ftsum + n_fsum + n_fent + 2 * n_sum + n_ent + n_el;
  return ws;
}

hipError_t launch_scan_bwd(const BwdLaunch& p, const BwdWorkspace& ws, const BwdPlan& pl) {
  // MODE bits as in the forward sweep: kSoftplusDelta, kExactZoh.
  switch (p.flags & 3u) {
    case 0: return p.bf16 ? launch_bwd_n<uint16_t, 0>(p, ws, pl) : launch_bwd_n<float, 0>(p, ws, pl);
    case 1: return p.bf16 ? launch_bwd_n<uint16_t, 1>(p, ws, pl) : launch_bwd_n<float, 1>(p, ws, pl);
    case 2: return p.bf16 ? launch_bwd_n<uint16_t, 2>(p, ws, pl) : launch_bwd_n<float, 2>(p, ws, pl);
    default: return p.bf16 ? launch_bwd_n<uint16_t, 3>(p, ws, pl) : launch_bwd_n<float, 3>(p, ws, pl);
  }
}

}  // namespace ssm
