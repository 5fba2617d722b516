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
#include <type_traits>
#include <utility>

namespace ssm {
namespace {

constexpr int kTB = kTimeBlock;
// Steps ahead of the current block whose B/C lines are warmed into L2.
constexpr int kFar = 3 * kTB;

// Steps per scalar-load group: keeps the two groups of B/C rows in flight
// within ~32 SGPRs (bf16 rows are NS/2 dwords each for B and for C), which
// is kP * NS * 6 ~ 96 VALU slots of cover per group whatever NS is.
template <typename T, int NS>
constexpr int row_group() {
  constexpr int budget = sizeof(T) == 2 ? 16 : 8;
  return budget / NS < kTB ? (budget / NS > 0 ? budget / NS : 1) : kTB;
}

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

  const int64_t DI = dm.d_inner;
  const int N = dm.d_state;
  const int64_t d = (int64_t)tile * 64 + lane;
  const bool dvalid = d < DI;
  const int64_t dc = dvalid ? d : DI - 1;  // tail lanes read a valid channel, store nothing
  const int n0 = wv * NS;
  // Time inside the chunk runs in int32 (the host keeps seqlen below 2^31 - 64).
  const int64_t t_beg = (int64_t)chunk * dm.chunk_len;
  const int nsteps = (int)(min(dm.seqlen, t_beg + dm.chunk_len) - t_beg);

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

  // Wave-uniform pointers (SGPRs) to the chunk's first (b, t) row; each lane
  // adds its channel offset lc, so loads use the SGPR-base addressing form and
  // all per-step address arithmetic stays on the scalar unit.
  const int64_t row0 = b * dm.seqlen + t_beg;
  const int64_t cbase = (int64_t)tile * 64;
  const int lc = (int)(dc - cbase);
  const T* xrow = x + row0 * DI + cbase;
  const T* drow = delta + row0 * DI + cbase;
  const T* zrow = has_z ? z + row0 * DI + cbase : xrow;
  T* yrow = SUMMARY ? nullptr : y + row0 * DI + cbase;
  const T* Bp = B + row0 * N + n0;
  const T* Cp = C + row0 * N + n0;

  // B/C rows travel in groups of kP steps through SGPRs: the rows of group
  // k+1 are requested as soon as group k's rows have landed, so each request
  // has kP steps of VALU work to arrive in.  (Scalar loads may return out of
  // order; the only safe wait is for all of them, once per group.)
  constexpr int kP = row_group<T, NS>();
  StateRow<T, NS> bq[kP], cq[kP];
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const int tt = min(j, nsteps - 1);
    bq[j].load(Bp + (int64_t)tt * N);
    if (!SUMMARY) cq[j].load(Cp + (int64_t)tt * N);
  }

  T xn[kTB], dn[kTB], zn[kTB];
#pragma unroll
  for (int i = 0; i < kTB; ++i) zn[i] = T(0);
  auto fetch = [&](int tb) {
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const int64_t off = (int64_t)min(tb + i, nsteps - 1) * DI;
      const T* xs = xrow + off;
      const T* ds = drow + off;
      xn[i] = xs[lc];
      dn[i] = ds[lc];
      if (has_z && (i & (g - 1)) == wv) {
        const T* zs = zrow + off;
        zn[i] = zs[lc];
      }
    }
  };
  fetch(0);

  // L2 warm-up: 16 lanes touch the B and C rows kFar steps ahead with vector
  // loads (no scalar-counter wait); the value is folded into a sink so the
  // loads are kept, and consumed a block later when they have long landed.
  uint32_t pf_sink = 0, pf_last = 0;

  float dsum = 0.f;
  int buf = 0;
  for (int tb = 0; tb < nsteps; tb += kTB) {
    const int nt = min(kTB, nsteps - tb);
    T xr[kTB], dr[kTB], zr[kTB];
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      xr[i] = xn[i];
      dr[i] = dn[i];
      zr[i] = zn[i];
    }
    if (tb + kTB < nsteps) fetch(tb + kTB);
    pf_sink ^= pf_last;
    if (lane < 16) {
      const int tt = min(tb + kFar + (lane & 7), nsteps - 1);
      const T* src = ((lane & 8) && !SUMMARY) ? Cp + (int64_t)tt * N : Bp + (int64_t)tt * N;
      pf_last = *reinterpret_cast<const uint32_t*>(src);
    }

    float part[kTB];
    auto step = [&](int i, const StateRow<T, NS>& bc, const StateRow<T, NS>& cc) {
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
    auto group = [&](int sb, auto full_t) {
      constexpr bool kFull = decltype(full_t)::value;
      bq[0].touch();
      if (!SUMMARY) cq[0].touch();
      __builtin_amdgcn_sched_barrier(0);
      StateRow<T, NS> bc[kP], cc[kP];
#pragma unroll
      for (int j = 0; j < kP; ++j) {
        bc[j] = bq[j];
        cc[j] = cq[j];
      }
#pragma unroll
      for (int j = 0; j < kP; ++j) {
        const int tt = min(tb + sb + kP + j, nsteps - 1);
        bq[j].load(Bp + (int64_t)tt * N);
        if (!SUMMARY) cq[j].load(Cp + (int64_t)tt * N);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kP; ++j)
        if (kFull || sb + j < nt) step(sb + j, bc[j], cc[j]);
    };
    if (nt == kTB) {
#pragma unroll
      for (int sb = 0; sb < kTB; sb += kP) group(sb, std::true_type{});
    } else {
#pragma unroll
      for (int sb = 0; sb < kTB; sb += kP)
        if (sb < nt) group(sb, std::false_type{});
    }

    if (!SUMMARY) {
      T* yb = yrow + (int64_t)tb * DI;
      if (g == 1) {
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
          if (i < nt) {
            float v = part[i];
            if (has_z) v *= silu(io_to_f32(zr[i]));
            T* ys = yb + (int64_t)i * DI;
            if (dvalid) io_store(ys + lc, v);
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
            T* ys = yb + (int64_t)i * DI;
            if (dvalid) io_store(ys + lc, v);
          }
        }
        buf ^= 1;
      }
    }
  }
  // Let the last scalar and warm-up loads land before the wave ends.
  bq[0].touch();
  if (!SUMMARY) cq[0].touch();
  asm volatile("" ::"v"(pf_sink ^ pf_last));

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
