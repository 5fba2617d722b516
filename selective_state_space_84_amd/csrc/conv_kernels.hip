// Causal depthwise conv1d over time (+ SiLU) and its decode step, gfx950.
//
//   out[b,t,d] = silu(bias[d] + sum_{k<K} w[d,k] * xe[b, t+k, d])
// where xe is x extended on the left by the K-1 carried inputs (state_in, or
// zeros).  This is the Mamba block's Conv1d(d_inner, d_inner, kernel d_conv,
// padding d_conv-1, groups d_inner) cut to the first seqlen outputs, then SiLU
// ("Deriving and implementing Mamba from scratch" (dpshk.com/news/3333417),
// section 5.2).  The carried state (last K-1 inputs) is the convolution half
// of the decode cache ("SSM series #12" (dpshk.com/news/5205047), section 1.3).
//
// The op is HBM-bound (one read and one write per element, ~6 VALU slots).
// Layout and mapping:
//   * x and y are [batch][seqlen][d_inner]: a wave owns 64 consecutive
//     channels, so every row access is one contiguous 128-byte (bf16) line.
//   * A thread covers kSeg consecutive steps of its channel: it issues the
//     K-1 halo loads and all kSeg loads up front (deep memory-level
//     parallelism), then slides the K-tap window in registers.
//   * The carried state is written by a second small kernel after the sweep,
//     so state_out may be the state_in buffer.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kSeg = 64;  // timesteps per thread (measured: 64 > 32 > 16)
constexpr int kConvBlock = 256;

template <typename T, int K, bool SILU>
__global__ void __launch_bounds__(kConvBlock)
    k_conv1d_fwd(const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
                 const float* __restrict__ state_in, T* __restrict__ y, int64_t seqlen, int64_t d_inner,
                 int32_t tiles, int32_t segs) {
  constexpr int S = K - 1;
  const int lane = threadIdx.x & 63;
  // blockIdx.x -> (b, seg, group of 4 tiles); one wave per tile.
  int bid = blockIdx.x;
  const int tgroups = (tiles + 3) / 4;
  const int tg = bid % tgroups;
  bid /= tgroups;
  const int seg = bid % segs;
  const int64_t b = bid / segs;
  const int tile = tg * 4 + (threadIdx.x >> 6);
  if (tile >= tiles) return;  // whole wave exits together
  const int64_t d = (int64_t)tile * 64 + lane;
  const bool valid = d < d_inner;
  const int64_t dc = valid ? d : d_inner - 1;
  const int64_t t0 = (int64_t)seg * kSeg;
  const int nt = (int)min((int64_t)kSeg, seqlen - t0);

  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = w[dc * K + k];
  const float bv = bias != nullptr ? bias[dc] : 0.f;

  const T* xc = x + (b * seqlen) * d_inner + dc;
  float win[S + kSeg];
  // Halo: the S inputs before t0 (from x, or the carried state, or zeros).
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int64_t t = t0 - S + j;
    float v;
    if (t >= 0) {
      v = io_to_f32(xc[t * d_inner]);
    } else if (state_in != nullptr) {
      v = state_in[(b * d_inner + dc) * S + (S + t)];
    } else {
      v = 0.f;
    }
    win[j] = v;
  }
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    const int64_t t = t0 + min(i, nt - 1);  // clamped rows are loaded but not stored
    win[S + i] = io_to_f32(xc[t * d_inner]);
  }
  T* yc = y + (b * seqlen + t0) * d_inner + dc;
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    if (i < nt) {
      float acc = bv;
#pragma unroll
      for (int k = 0; k < K; ++k) acc = __builtin_fmaf(wk[k], win[i + k], acc);
      if (SILU) acc = silu(acc);
      if (valid) io_store(yc + (int64_t)i * d_inner, acc);
    }
  }
}

// state_out[b,d,j] = xe[b, seqlen + j, d]: the last K-1 entries of the
// extended input.  Each thread reads everything it needs before writing, so
// state_out may be the state_in buffer.
template <typename T, int K>
__global__ void __launch_bounds__(kConvBlock)
    k_conv_state_out(const T* __restrict__ x, const float* state_in, float* state_out, int64_t batch,
                     int64_t seqlen, int64_t d_inner) {
  constexpr int S = K - 1;
  const int64_t i = (int64_t)blockIdx.x * kConvBlock + threadIdx.x;
  if (i >= batch * d_inner) return;
  const int64_t b = i / d_inner, d = i % d_inner;
  float v[S > 0 ? S : 1];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int64_t e = seqlen + j;  // index into xe = [state (S) | x (seqlen)]
    if (e >= S) {
      v[j] = io_to_f32(x[(b * seqlen + (e - S)) * d_inner + d]);
    } else {
      v[j] = state_in != nullptr ? state_in[i * S + e] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < S; ++j) state_out[i * S + j] = v[j];
}

// One decode step: window = [state, x_t]; y_t = silu(bias + w . window);
// state <- window[1:], in place.
template <typename T, int K, bool SILU>
__global__ void __launch_bounds__(kConvBlock)
    k_conv1d_update(float* __restrict__ state, const T* __restrict__ x, const float* __restrict__ w,
                    const float* __restrict__ bias, T* __restrict__ y, int64_t batch, int64_t d_inner) {
  constexpr int S = K - 1;
  const int64_t i = (int64_t)blockIdx.x * kConvBlock + threadIdx.x;
  if (i >= batch * d_inner) return;
  const int64_t d = i % d_inner;
  float win[K];
#pragma unroll
  for (int j = 0; j < S; ++j) win[j] = state[i * S + j];
  win[S] = io_to_f32(x[i]);
  float acc = bias != nullptr ? bias[d] : 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(w[d * K + k], win[k], acc);
  if (SILU) acc = silu(acc);
  io_store(y + i, acc);
#pragma unroll
  for (int j = 0; j < S; ++j) state[i * S + j] = win[j + 1];
}

template <typename T, int K, bool SILU>
hipError_t launch_conv_t(const ConvLaunch& p) {
  const int64_t tiles = (p.d_inner + 63) / 64;
  const int64_t segs = (p.seqlen + kSeg - 1) / kSeg;
  const int64_t tgroups = (tiles + 3) / 4;
  const T* x = static_cast<const T*>(p.x);
  hipError_t e = hipSuccess;
  if (p.seqlen > 0) {
    e = launch(k_conv1d_fwd<T, K, SILU>, dim3((unsigned)(p.batch * segs * tgroups)), dim3(kConvBlock), 0, p.stream,
               x, p.w, p.bias, p.state_in, static_cast<T*>(p.y), p.seqlen, p.d_inner, (int32_t)tiles,
               (int32_t)segs);
    if (e != hipSuccess) return e;
  }
  if (p.state_out != nullptr && K > 1) {
    const int64_t n = p.batch * p.d_inner;
    e = launch(k_conv_state_out<T, K>, dim3((unsigned)((n + kConvBlock - 1) / kConvBlock)), dim3(kConvBlock), 0,
               p.stream, x, p.state_in, p.state_out, p.batch, p.seqlen, p.d_inner);
  }
  return e;
}

template <typename T, int K, bool SILU>
hipError_t launch_conv_update_t(const ConvLaunch& p) {
  const int64_t n = p.batch * p.d_inner;
  return launch(k_conv1d_update<T, K, SILU>, dim3((unsigned)((n + kConvBlock - 1) / kConvBlock)), dim3(kConvBlock),
                0, p.stream, p.state_out, static_cast<const T*>(p.x), p.w, p.bias, static_cast<T*>(p.y), p.batch,
                p.d_inner);
}

template <typename T, bool SILU>
hipError_t dispatch_k(const ConvLaunch& p, bool update) {
  switch (p.d_conv) {
    case 2: return update ? launch_conv_update_t<T, 2, SILU>(p) : launch_conv_t<T, 2, SILU>(p);
    case 3: return update ? launch_conv_update_t<T, 3, SILU>(p) : launch_conv_t<T, 3, SILU>(p);
    case 4: return update ? launch_conv_update_t<T, 4, SILU>(p) : launch_conv_t<T, 4, SILU>(p);
    default: return hipErrorInvalidValue;
  }
}

hipError_t dispatch_conv(const ConvLaunch& p, bool update) {
  if (p.bf16) return p.silu ? dispatch_k<uint16_t, true>(p, update) : dispatch_k<uint16_t, false>(p, update);
  return p.silu ? dispatch_k<float, true>(p, update) : dispatch_k<float, false>(p, update);
}

}  // namespace

int64_t conv_grid_blocks(int64_t batch, int64_t seqlen, int64_t d_inner) {
  const int64_t tiles = (d_inner + 63) / 64;
  return batch * ((seqlen + kSeg - 1) / kSeg) * ((tiles + 3) / 4);
}

hipError_t launch_conv1d(const ConvLaunch& p) { return dispatch_conv(p, false); }
hipError_t launch_conv1d_update(const ConvLaunch& p) { return dispatch_conv(p, true); }

}  // namespace ssm
