// Selective-scan kernels for gfx950 (MI355X).
//
// What is computed (per batch row b, channel d, state n; A diagonal):
//   abar = exp(delta[b,t,d] * A[d,n])                     -- decay
//   h[n] = abar * h[n] + delta[b,t,d] * B[b,t,n] * x[b,t,d] -- state update
//   y    = (sum_n C[b,t,n] * h[n] + D[d] * x) * silu(z)     -- readout + gate
// "Deriving and implementing Mamba from scratch" (dpshk.com/news/3333417),
// sections 2.2, 3.2, 4.2, 5.1 and 5.2; decode shape and segment hand-over in
// "Mamba from principle to code" (lshu.cn/news/79586) section 6.5 and
// "SSMs for long-document QA" (pwwt.cn/news/5168881) section 3.1.
//
// Mapping onto CDNA4:
//   * lane = channel: a wave owns 64 consecutive channels of one batch row, so
//     x / delta / z / y are read and written as contiguous 128-byte (bf16) or
//     256-byte (fp32) rows per timestep.
//   * The fp32 state of each channel lives in VGPRs for the whole sweep; the
//     recurrence runs sequentially over t inside the lane.  This is the
//     cheapest form of the recurrence (one FMA per state per step); the work
//     is VALU-bound, so a time-parallel scan per element would cost several
//     times more arithmetic.
//   * B_t and C_t are shared by every channel of a row: their address is
//     wave-uniform, so they arrive through scalar loads into SGPRs (prefetched
//     one timestep ahead) and feed the VALU as scalar operands.  No LDS
//     traffic and no VGPRs are spent on them.
//   * n-split: up to 8 waves share one channel tile, each owning d_state/g
//     states.  Their partial readouts meet in LDS once per block of 8
//     timesteps; the gate and the store are spread over the waves.  This
//     multiplies parallelism for shapes with few channels at a cost of a few
//     VALU ops per element.
//   * Sequence chunks: when even that leaves the chip idle, the sequence is
//     cut into chunks.  A summary sweep gives each chunk's affine map
//     h -> P*h + S (P = prod of decays = exp(A * sum delta), S = end state
//     from zero), an associative combine (a1,b1)o(a2,b2) = (a1*a2, a2*b1+b2)
//     over chunks gives every chunk its entry state, and the main sweep then
//     runs each chunk from its true entry state.
//   * Workgroup ids are remapped so each XCD gets a contiguous range of
//     (batch row, chunk, tile), keeping a row's B/C lines in one L2.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <tuple>
#include <utility>

namespace ssm {
namespace {

constexpr int kTB = kTimeBlock;

struct SweepDims {
  int64_t batch, seqlen, d_inner, chunk_len;
  int32_t d_state, n_split, tiles, n_chunks_grid;  // chunks covered by this launch
  int32_t n_chunks;                                // chunks of the whole sequence
  int32_t h_init_chunked;                          // h_init is [n_chunks][B][d][N] (else [B][d][N])
};

// SUMMARY = true: chunk summary sweep (state from zero, no readout); writes
// P = exp(A * sum(delta)) and the end state S for chunk c into sumP / sumS.
// SUMMARY = false: full sweep with readout, gate and y store.
template <typename T, int NS, bool SUMMARY>
__global__ void __launch_bounds__(64 * kMaxSplit)
    k_scan_sweep(const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
                 const T* __restrict__ B, const T* __restrict__ C, const float* __restrict__ D,
                 const T* __restrict__ z, const float* __restrict__ h_init, T* __restrict__ y,
                 float* __restrict__ h_last, float* __restrict__ sumP, float* __restrict__ sumS,
                 const SweepDims dm) {
  extern __shared__ float red[];  // [2][g][kTB][64] partial readouts when g > 1
  const int lane = threadIdx.x & 63;
  // Wave index within the workgroup; readfirstlane tells the compiler it is
  // wave-uniform, so everything derived from it stays in SGPRs.
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = dm.n_split;

  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = bid % dm.tiles;
  bid /= dm.tiles;
  const int chunk = bid % dm.n_chunks_grid;
  const int64_t b = bid / dm.n_chunks_grid;

  const int64_t DI = dm.d_inner, L = dm.seqlen;
  const int N = dm.d_state;
  const int64_t d = (int64_t)tile * 64 + lane;
  const bool dvalid = d < DI;
  const int64_t dc = dvalid ? d : DI - 1;  // tail lanes read a valid channel, store nothing
  const int n0 = wv * NS;
  const int64_t t_beg = (int64_t)chunk * dm.chunk_len;
  const int64_t t_end = min(L, t_beg + dm.chunk_len);

  float Al2[NS], h[NS];
  {
    const float* Ap = A + dc * N + n0;
#pragma unroll
    for (int n = 0; n < NS; ++n) Al2[n] = Ap[n] * kLog2e;
  }
  if (!SUMMARY && h_init != nullptr) {
    const int64_t row = dm.h_init_chunked ? ((int64_t)chunk * dm.batch + b) * DI + dc : b * DI + dc;
    const float* hp = h_init + row * N + n0;
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = hp[n];
  } else {
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = 0.f;
  }
  const float Dv = (!SUMMARY && D != nullptr && wv == 0) ? D[dc] : 0.f;
  const bool has_z = !SUMMARY && z != nullptr;

  // Row pointers are wave-uniform (SGPR); each lane adds its channel offset.
  const int64_t row0 = b * L;
  const int64_t cbase = (int64_t)tile * 64;
  const int lc = (int)(dc - cbase);
  const T* xrow = x + row0 * DI + cbase;
  const T* drow = delta + row0 * DI + cbase;
  const T* zrow = has_z ? z + row0 * DI + cbase : xrow;
  const T* Bp = B + row0 * N + n0;
  const T* Cp = C + row0 * N + n0;

  StateRow<T, NS> bn, cn;
  bn.load(Bp + t_beg * N);
  if (!SUMMARY) cn.load(Cp + t_beg * N);

  T xn[kTB], dn[kTB], zn[kTB];
#pragma unroll
  for (int i = 0; i < kTB; ++i) zn[i] = T(0);
  auto fetch = [&](int64_t tb) {
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const int64_t off = min(tb + i, t_end - 1) * DI;
      xn[i] = xrow[off + lc];
      dn[i] = drow[off + lc];
      if (has_z && (i & (g - 1)) == wv) zn[i] = zrow[off + lc];
    }
  };
  fetch(t_beg);

  float dsum = 0.f;
  int buf = 0;
  for (int64_t t0 = t_beg; t0 < t_end; t0 += kTB) {
    const int nt = (int)min((int64_t)kTB, t_end - t0);
    T xr[kTB], dr[kTB], zr[kTB];
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      xr[i] = xn[i];
      dr[i] = dn[i];
      zr[i] = zn[i];
    }
    if (t0 + kTB < t_end) fetch(t0 + kTB);

    float part[kTB];
    auto step = [&](int i) {
      const int64_t t = t0 + i;
      // Scalar loads return out of order, so consuming this step's B/C row
      // needs every outstanding scalar load to land.  Touch the row first,
      // then request the next row, so that request has a whole step of VALU
      // work to arrive in.
      const StateRow<T, NS> bc = bn, cc = cn;
      bc.touch();
      if (!SUMMARY) cc.touch();
      __builtin_amdgcn_sched_barrier(0);
      const int64_t tn = min(t + 1, t_end - 1);
      bn.load(Bp + tn * N);
      if (!SUMMARY) cn.load(Cp + tn * N);
      __builtin_amdgcn_sched_barrier(0);
      const float xv = io_to_f32(xr[i]);
      const float dv = io_to_f32(dr[i]);
      const float wx = dv * xv;
      float acc = Dv * xv;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const float ab = hw_exp2(dv * Al2[n]);
        h[n] = __builtin_fmaf(ab, h[n], wx * bc.get(n));
        if (!SUMMARY) acc = __builtin_fmaf(cc.get(n), h[n], acc);
      }
      if (SUMMARY) dsum += dv;
      part[i] = acc;
    };
    if (nt == kTB) {
#pragma unroll
      for (int i = 0; i < kTB; ++i) step(i);
    } else {
#pragma unroll
      for (int i = 0; i < kTB; ++i)
        if (i < nt) step(i);
    }

    if (!SUMMARY) {
      T* yb = y + (row0 + t0) * DI + cbase;
      if (g == 1) {
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
          if (i < nt) {
            float v = part[i];
            if (has_z) v *= silu(io_to_f32(zr[i]));
            if (dvalid) io_store(yb + i * DI + lc, v);
          }
        }
      } else {
        float* mine = red + ((buf * g + wv) * kTB) * 64 + lane;
#pragma unroll
        for (int i = 0; i < kTB; ++i) mine[i * 64] = part[i];
        __syncthreads();
        const float* base = red + (buf * g * kTB) * 64 + lane;
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
          if ((i & (g - 1)) == wv && i < nt) {
            float v = 0.f;
            for (int j = 0; j < g; ++j) v += base[(j * kTB + i) * 64];
            if (has_z) v *= silu(io_to_f32(zr[i]));
            if (dvalid) io_store(yb + i * DI + lc, v);
          }
        }
        buf ^= 1;
      }
    }
  }

  if (SUMMARY) {
    if (dvalid) {
      const int64_t o = (((int64_t)chunk * dm.batch + b) * DI + d) * N + n0;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        sumP[o + n] = hw_exp2(Al2[n] * dsum);
        sumS[o + n] = h[n];
      }
    }
  } else if (h_last != nullptr && chunk == dm.n_chunks - 1 && dvalid) {
    float* hp = h_last + (b * DI + d) * N + n0;
#pragma unroll
    for (int n = 0; n < NS; ++n) hp[n] = h[n];
  }
}

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
  for (int64_t c = 0; c + 1 < n_chunks; ++c) {
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

template <typename... KArgs, typename... Args>
hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args&&... args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... v) {
    int k = 0;
    ((ptrs[k++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, shmem, s);
}

template <typename T, int NS>
hipError_t launch_scan_t(const ScanLaunch& p) {
  const int g = p.n_split;
  const int64_t tiles = (p.d_inner + 63) / 64;
  const int64_t states = p.batch * p.d_inner * p.d_state;
  const size_t shmem = g > 1 ? (size_t)2 * g * kTB * 64 * sizeof(float) : 0;
  SweepDims dm{p.batch, p.seqlen, p.d_inner, p.chunk_len, p.d_state, g, (int32_t)tiles, 1, (int32_t)p.n_chunks, 0};
  const T* x = static_cast<const T*>(p.x);
  const T* dl = static_cast<const T*>(p.delta);
  const T* Bm = static_cast<const T*>(p.B);
  const T* Cm = static_cast<const T*>(p.C);
  const T* zz = static_cast<const T*>(p.z);
  T* y = static_cast<T*>(p.y);
  hipError_t e;
  if (p.n_chunks > 1) {
    float* sumP = p.workspace;
    float* sumS = sumP + (p.n_chunks - 1) * states;
    float* hent = sumS + (p.n_chunks - 1) * states;
    SweepDims ds = dm;
    ds.n_chunks_grid = (int32_t)(p.n_chunks - 1);
    e = launch(k_scan_sweep<T, NS, true>, dim3((unsigned)(p.batch * (p.n_chunks - 1) * tiles)), dim3(64 * g), 0,
               p.stream, x, dl, p.A, Bm, Cm, p.D, zz, (const float*)nullptr, y, p.h_last, sumP, sumS, ds);
    if (e != hipSuccess) return e;
    e = launch(k_chunk_carry, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, p.stream, p.h0,
               (const float*)sumP, (const float*)sumS, hent, states, p.n_chunks);
    if (e != hipSuccess) return e;
    dm.n_chunks_grid = (int32_t)p.n_chunks;
    dm.h_init_chunked = 1;
    return launch(k_scan_sweep<T, NS, false>, dim3((unsigned)(p.batch * p.n_chunks * tiles)), dim3(64 * g), shmem,
                  p.stream, x, dl, p.A, Bm, Cm, p.D, zz, (const float*)hent, y, p.h_last, (float*)nullptr,
                  (float*)nullptr, dm);
  }
  return launch(k_scan_sweep<T, NS, false>, dim3((unsigned)(p.batch * tiles)), dim3(64 * g), shmem, p.stream, x, dl,
                p.A, Bm, Cm, p.D, zz, p.h0, y, p.h_last, (float*)nullptr, (float*)nullptr, dm);
}

template <typename T>
hipError_t launch_scan_ns(const ScanLaunch& p) {
  switch (p.d_state / p.n_split) {
    case 2: return launch_scan_t<T, 2>(p);
    case 4: return launch_scan_t<T, 4>(p);
    case 8: return launch_scan_t<T, 8>(p);
    case 16: return launch_scan_t<T, 16>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scan(const ScanLaunch& p) {
  return p.bf16 ? launch_scan_ns<uint16_t>(p) : launch_scan_ns<float>(p);
}

hipError_t launch_state_fill(float* dst, const float* src, int64_t states, hipStream_t stream) {
  return launch(k_state_fill, dim3((unsigned)((states + 255) / 256)), dim3(256), 0, stream, dst, src, states);
}

}  // namespace ssm
