// Single-token recurrent state update (decode) for gfx950.
//
// For each batch row b and channel d, with the state h[b,d,:] resident in HBM:
//   h[n] <- exp(delta*A[d,n]) * h[n] + delta * B[b,n] * x
//   y     = (sum_n C[b,n] * h[n] + D[d] * x) * silu(z)
// One recurrent step of the diagonal selective SSM: "State space models vs
// Transformer: a practical guide" (datadaily.news), "How SSMs actually work";
// state shape (batch, d_inner, d_state) from "Mamba from principle to code"
// (lshu.cn/news/79586) section 6.5; the update itself is section 3.2 of
// "Deriving and implementing Mamba from scratch" (dpshk.com/news/3333417).
//
// The step moves 2 x 4 x d_state bytes of state per channel and a few bytes
// of io, against ~6 VALU slots per state: it is HBM-bound.  The layout is
// chosen for the memory system:
//   * LPC lanes share one channel, each owning 4 consecutive states, so one
//     wave's 16-byte state loads cover 1 KiB of contiguous memory (fully
//     coalesced, no partial cache lines per instruction).
//   * The readout is reduced across the LPC lanes with DPP / swizzle moves;
//     every lane of the group then holds y, and the first one stores it.
//   * x, delta, z are read once per lane group (the group's lanes hit the same
//     cache line); B and C rows are tiny and shared by the whole row.
#include "ssm_device.h"
#include "ssm_internal.h"


namespace ssm {
namespace {

constexpr int kUpdBlock = 256;

// Sum over aligned groups of LPC lanes (LPC a power of two <= 16).
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  if (LPC >= 2)  // quad_perm [1,0,3,2]: partner lane ^ 1
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  if (LPC >= 4)  // quad_perm [2,3,0,1]: partner lane ^ 2
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if (LPC >= 8)  // ds_swizzle bit mode: and 0x1F, xor 4
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x101F));
  if (LPC >= 16)  // xor 8
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x201F));
  return v;
}

// SPL consecutive fp32 states of one lane, moved as 16-byte (or 8-byte for
// SPL = 2) vector accesses.
template <int SPL>
struct LaneStates {
  static_assert(SPL == 2 || SPL % 4 == 0, "lane state width");
  static __device__ __forceinline__ void load(const float* p, float (&v)[SPL]) {
    if constexpr (SPL == 2) {
      const float2 q = *reinterpret_cast<const float2*>(p);
      v[0] = q.x;
      v[1] = q.y;
    } else {
#pragma unroll
      for (int k = 0; k < SPL / 4; ++k) {
        const float4 q = reinterpret_cast<const float4*>(p)[k];
        v[4 * k] = q.x;
        v[4 * k + 1] = q.y;
        v[4 * k + 2] = q.z;
        v[4 * k + 3] = q.w;
      }
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[SPL]) {
    if constexpr (SPL == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
      for (int k = 0; k < SPL / 4; ++k)
        reinterpret_cast<float4*>(p)[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    }
  }
};

// SPL values of a B or C row as fp32 (bf16 pairs are read as dwords).
template <int SPL>
__device__ __forceinline__ void load_row(const uint16_t* p, float (&v)[SPL]) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
  for (int k = 0; k < SPL / 2; ++k) {
    const uint32_t w = q[k];
    v[2 * k] = __builtin_bit_cast(float, w << 16);
    v[2 * k + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
  }
}
template <int SPL>
__device__ __forceinline__ void load_row(const float* p, float (&v)[SPL]) {
  float tmp[SPL];
  LaneStates<SPL>::load(p, tmp);
#pragma unroll
  for (int k = 0; k < SPL; ++k) v[k] = tmp[k];
}

// MODE bit 0: the step is softplus(delta + dt_bias[d]); bit 1: exact
// zero-order-hold input term (exp(delta a) - 1) / a * B (limit delta * B at
// a = 0), as in the scan sweep.
template <typename T, int SPL, int LPC, int MODE, int R>
__global__ void __launch_bounds__(kUpdBlock)
    k_state_update(float* __restrict__ h, const T* __restrict__ x, const T* __restrict__ delta,
                   const float* __restrict__ A, const T* __restrict__ B, const T* __restrict__ C,
                   const float* __restrict__ D, const T* __restrict__ z, T* __restrict__ y,
                   const float* __restrict__ dt_bias, int64_t batch, int64_t d_inner, int32_t blocks_per_row) {
  constexpr int N = SPL * LPC;
  constexpr int kChan = kUpdBlock / LPC;  // channels per workgroup
  // Each thread updates the same channel in R batch rows (b0 + r * stride),
  // so A, D and dt_bias are read once per R rows.
  const int64_t rows = (batch + R - 1) / R;
  const int64_t b0 = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x % blocks_per_row;
  const int sub = threadIdx.x % LPC;
  const int64_t d = (int64_t)blk * kChan + threadIdx.x / LPC;
  const bool valid = d < d_inner;
  const int64_t dc = valid ? d : d_inner - 1;
  const int s0 = sub * SPL;

  float al[SPL];
  LaneStates<SPL>::load(A + dc * N + s0, al);
  const float Dv = D != nullptr ? D[dc] : 0.f;
  const float dtb = (MODE & 1) ? dt_bias[dc] : 0.f;
  // All rows' loads are issued before any row is computed or stored (a row
  // past the batch reads row b0 and stores nothing), so a thread has every
  // load of its R rows in flight at once; the per-channel inputs go first,
  // since in a decode loop they are the cold data (the state, rewritten every
  // step, is more likely to be found in the on-package cache).
  // Measured at 256 x 5120 x 16 bf16 with fresh inputs each step: 36.9 us
  // per step with each row loaded after the previous row's store, 35.3 us
  // this way.
  float hv[R][SPL], Bv[R][SPL], Cv[R][SPL], xr[R], dr[R], zr[R];
  bool rv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t bq = b0 + r * rows;
    rv[r] = r == 0 || bq < batch;
    const int64_t b = rv[r] ? bq : b0;
    const int64_t io = b * d_inner + dc;
    xr[r] = io_to_f32(x[io]);
    dr[r] = io_to_f32(delta[io]);
    zr[r] = z != nullptr ? io_to_f32(z[io]) : 0.f;
    load_row<SPL>(B + b * N + s0, Bv[r]);
    load_row<SPL>(C + b * N + s0, Cv[r]);
    LaneStates<SPL>::load(h + (b * d_inner + dc) * N + s0, hv[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = b0 + r * rows;
    const float xv = xr[r];
    float dv = dr[r];
    if (MODE & 1) dv = softplus(dv, dtb);
    const float wx = dv * xv;
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < SPL; ++n) {
      const float yv = dv * (al[n] * kLog2e);
      const float ab = hw_exp2(yv);
      if (MODE & 2) {
        const float coef = zoh_coef(yv, ab, dv, 1.0f / al[n]);
        hv[r][n] = __builtin_fmaf(coef, xv * Bv[r][n], ab * hv[r][n]);
      } else {
        hv[r][n] = __builtin_fmaf(ab, hv[r][n], wx * Bv[r][n]);
      }
      acc = __builtin_fmaf(Cv[r][n], hv[r][n], acc);
    }
    acc = group_sum<LPC>(acc);
    if (valid && rv[r]) {
      LaneStates<SPL>::store(h + (b * d_inner + dc) * N + s0, hv[r]);
      if (sub == 0) {
        float v = __builtin_fmaf(Dv, xv, acc);
        if (z != nullptr) v *= silu(zr[r]);
        io_store(y + b * d_inner + dc, v);
      }
    }
  }
}

// Batch rows per thread: A, D and dt_bias loads are shared by this many rows
// (measured at 256 x 5120 x 16 bf16 with the loads issued first: 1 row
// 38.4 us, 2 rows 35.9, 4 rows 35.9).
constexpr int kUpdRows = 2;

template <typename T, int SPL, int LPC, int MODE>
hipError_t launch_update_m(const UpdateLaunch& p) {
  constexpr int kChan = kUpdBlock / LPC;
  const int64_t per_row = (p.d_inner + kChan - 1) / kChan;
  const int64_t rows = (p.batch + kUpdRows - 1) / kUpdRows;
  return launch(k_state_update<T, SPL, LPC, MODE, kUpdRows>, dim3((unsigned)(rows * per_row)), dim3(kUpdBlock), 0,
                p.stream, p.h, static_cast<const T*>(p.x), static_cast<const T*>(p.delta), p.A,
                static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.D, static_cast<const T*>(p.z),
                static_cast<T*>(p.y), p.dt_bias, p.batch, p.d_inner, (int32_t)per_row);
}

template <typename T, int SPL, int LPC>
hipError_t launch_update_t(const UpdateLaunch& p) {
  switch (p.flags & 3u) {
    case 0: return launch_update_m<T, SPL, LPC, 0>(p);
    case 1: return launch_update_m<T, SPL, LPC, 1>(p);
    case 2: return launch_update_m<T, SPL, LPC, 2>(p);
    default: return launch_update_m<T, SPL, LPC, 3>(p);
  }
}

template <typename T>
hipError_t launch_update_n(const UpdateLaunch& p) {
  switch (p.d_state) {
    case 2: return launch_update_t<T, 2, 1>(p);
    case 4: return launch_update_t<T, 4, 1>(p);
    case 8: return launch_update_t<T, 4, 2>(p);
    case 16: return launch_update_t<T, 4, 4>(p);
    case 32: return launch_update_t<T, 4, 8>(p);
    case 64: return launch_update_t<T, 4, 16>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t update_grid_blocks(int64_t batch, int64_t d_inner, int32_t d_state) {
  const int lpc = d_state <= 4 ? 1 : d_state / 4;
  const int64_t chan = kUpdBlock / lpc;
  return (batch + kUpdRows - 1) / kUpdRows * ((d_inner + chan - 1) / chan);
}

hipError_t launch_update(const UpdateLaunch& p) {
  return p.bf16 ? launch_update_n<uint16_t>(p) : launch_update_n<float>(p);
}

}  // namespace ssm
