// Scan with a scalar decay per head (Mamba-2 / SSD form) on gfx950, with
// the dense parts on the matrix cores.
//
// Per batch row b, head h (group g of heads sharing B and C), channel p of
// the head (headdim 64) and state n:
//   a_t = exp(dt_t A_h),  H_t = a_t H_{t-1} + dt_t B_t x_t^T,  y_t = C_t H_t + D_h x_t  (then * silu(z_t))
// With a scalar decay the scan is y = M x for a lower-triangular
// semiseparable M[k,i] = C_k B_i^T (prod_{j=i+1..k} a_j) dt_i ("Deriving and
// implementing Mamba from scratch" (dpshk.com/news/3333417), section 6.1),
// which splits into blocks like attention ("SSMs for long-document QA"
// (pwwt.cn/news/5168881), section 2.3).  For a chunk of Q = 32 steps, with
// l_t the running sum of dt A inside the chunk and H[n][p] the state:
//   Y^T = X^T W^T + (H^T C^T) diag(exp(l))    W[k,i] = C_k.B_i exp(l_k - l_i) dt_i (i <= k), + D_h (i = k)
//   H'  = exp(l_Q) H + B^T (w o X)            w_i = exp(l_Q - l_i) dt_i
// Folding D_h into the diagonal of W gives the skip term for free.  The four
// products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation, and the
// state stays in fp32 accumulators for the whole sequence.
//
// Precision: x, B, C are bf16 inputs and enter the products exactly.  The
// derived operands (W, the state fed to C H, and w o X) are sums of terms much
// larger than the outputs they produce (random B and C give scores of size
// sqrt(N)); rounding any one of them to bf16 once costs percent-level errors
// on small outputs.  Each is therefore split into hi = bf16(v) and lo =
// bf16(v - hi) and multiplied twice (about 16 significant bits), which leaves
// the bf16 rounding of y as the dominant error.
//
// Mapping: one workgroup (4 waves) per (batch row, head) walks the chunks in
// order; wave w owns channels [16w, 16w+16) of the head, for Y and for H.
// Per chunk, x, B and C are staged row-major in LDS with 16-byte writes (B
// and C double-buffered, so two barriers per chunk suffice); the next chunk's
// rows are loaded into registers while this one computes.
//   * The operands that run over time (X^T for Y, w o X and B^T for the state
//     update) need eight consecutive steps per lane: they come from the
//     row-major tiles through ds_read_b64_tr_b16, which transposes 16 x 4
//     blocks across each group of 16 lanes.
//   * Waves 0-2 each compute one of the three causal 16 x 16 score tiles
//     (S^T = B C^T), mask them and share W through LDS.
//   * The state's accumulator layout (lane = channel, four states per lane
//     per tile) is used directly as the A operand of H^T C^T: the contraction
//     over n takes the states in the order the accumulators hold them, and C
//     is staged with its columns permuted to match, so the state never
//     leaves registers.
//
// MFMA operand layout (checked on the device): for a 16x32 A, lane l holds
// A[l % 16][8 (l / 16) + j], j < 8; for a 32x16 B, B[8 (l / 16) + j][l % 16];
// the 16x16 result: D[4 (l / 16) + j][l % 16], j < 4.
// ds_read_b64_tr_b16 (checked on the device): in each group of 16 lanes, if
// lane s supplies the address of row r(s / 4), columns c0 + 4 (s % 4) .. +3,
// then lane s receives column c0 + s of rows r(0..3).
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kQ = 32;           // chunk length
constexpr int kHP = 64;          // channels per head
constexpr int kSX = kHP + 16;    // x tile row stride (bf16): 40 dwords, transposing reads conflict-free
constexpr int kSW = kQ + 8;      // score tile row stride: 20 dwords, 16-byte reads conflict-free

struct SsdDims {
  int64_t batch, seqlen;
  int32_t nheads, ngroups;
};

__device__ __forceinline__ f32x4 mma(const u16x8& a, const u16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ u16x4 lds_tr4(const uint16_t* p) {
  return __builtin_bit_cast(u16x4,
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(s16x4*)const_cast<uint16_t*>(p)));
}

__device__ __forceinline__ uint16_t to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ float from_bf16(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = to_bf16(v);
  lo = to_bf16(v - from_bf16(hi));
}

__device__ __forceinline__ u16x8 cat(const u16x4& a, const u16x4& b) {
  return u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Position of state column o (0..31 inside a 32-wide slice) in the permuted
// C tile: the order in which the state accumulators hold the states.
__device__ __forceinline__ int cperm(int o) { return o < 16 ? 2 * o : 2 * (o - 16) + 4; }

template <int N, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))  // all (row, head) groups resident
k_ssd_fwd(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
          const uint16_t* __restrict__ B, const uint16_t* __restrict__ C, const float* __restrict__ D,
          const uint16_t* __restrict__ z, const float* __restrict__ h0, uint16_t* __restrict__ y,
          float* __restrict__ h_last, const float* __restrict__ dt_bias, const SsdDims dm) {
  constexpr int NT = N / 16;            // state tiles of 16
  constexpr int NK = N / 32;            // contraction slices over the state
  constexpr int SB = N + 16;            // B tile row stride: transposing reads conflict-free
  constexpr int SC = N + 8;             // C tile row stride: 16-byte reads conflict-free
  constexpr int PB = kQ * N / 8 / 256;  // 16-byte pieces of B (and of C) per thread
  __shared__ __align__(16) uint16_t sX[kQ * kSX];
  __shared__ __align__(16) uint16_t sB[2][kQ * SB];
  __shared__ __align__(16) uint16_t sC[2][kQ * SC];
  __shared__ __align__(16) uint16_t sW[2][kQ * kSW];  // masked scores [k][i], hi and lo planes
  __shared__ __align__(16) float sv[4][4][kQ];         // per wave: l (log2 units), dt, w, exp(l)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bid % dm.nheads;
  const int64_t b = bid / dm.nheads;
  const int g = h / (dm.nheads / dm.ngroups);
  const int64_t L = dm.seqlen;
  const int64_t HP = (int64_t)dm.nheads * kHP;
  const float Al2 = A[h] * kLog2e;
  const float Dh = D != nullptr ? D[h] : 0.f;
  const float dtb = (MODE & 1) ? dt_bias[h] : 0.f;
  const bool has_z = z != nullptr;
  float* const lv = &sv[w][0][0];
  float* const dv = &sv[w][1][0];
  float* const wv = &sv[w][2][0];
  float* const ev = &sv[w][3][0];

  // State H[n][p] for p = 16w + r16: accH[nt][j] = H[16 nt + 4 q4 + j][p].
  f32x4 accH[NT];
  {
    const float* hp = h0 != nullptr ? h0 + (((b * dm.nheads) + h) * kHP + 16 * w + r16) * N + 4 * q4 : nullptr;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) accH[nt][j] = hp != nullptr ? hp[16 * nt + j] : 0.f;
  }

  // Staging registers, one chunk ahead.
  const int sx_t = tid >> 3, sx_c = (tid & 7) * 8;
  u16x8 rx, rb[PB], rc[PB];
  uint16_t rdt = 0;
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const int nt_ = (int)min((int64_t)kQ, L - t0);
    const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
    rx = sx_t < nt_ ? *reinterpret_cast<const u16x8*>(x + (b * L + t0 + sx_t) * HP + (int64_t)h * kHP + sx_c) : zero;
#pragma unroll
    for (int r = 0; r < PB; ++r) {
      const int piece = tid + 256 * r;
      const int t = piece / (N / 8), n8 = (piece % (N / 8)) * 8;
      const int64_t o = ((b * L + t0 + t) * dm.ngroups + g) * N + n8;
      rb[r] = t < nt_ ? *reinterpret_cast<const u16x8*>(B + o) : zero;
      rc[r] = t < nt_ ? *reinterpret_cast<const u16x8*>(C + o) : zero;
    }
    rdt = lane < nt_ ? dt[(b * L + t0 + lane) * dm.nheads + h] : (uint16_t)0;
  };
  auto stage = [&](int buf) {
    *reinterpret_cast<u16x8*>(&sX[sx_t * kSX + sx_c]) = rx;
#pragma unroll
    for (int r = 0; r < PB; ++r) {
      const int piece = tid + 256 * r;
      const int t = piece / (N / 8), n8 = (piece % (N / 8)) * 8;
      *reinterpret_cast<u16x8*>(&sB[buf][t * SB + n8]) = rb[r];
      const int s0 = n8 & ~31, o = n8 & 31;
      *reinterpret_cast<u16x4*>(&sC[buf][t * SC + s0 + cperm(o)]) = u16x4{rc[r][0], rc[r][1], rc[r][2], rc[r][3]};
      *reinterpret_cast<u16x4*>(&sC[buf][t * SC + s0 + cperm(o + 4)]) = u16x4{rc[r][4], rc[r][5], rc[r][6], rc[r][7]};
    }
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  if (nchunks > 0) fetch(0);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int buf = (int)(c & 1);
    const int64_t t0 = c * kQ;
    const int nt_ = (int)min((int64_t)kQ, L - t0);
    stage(buf);
    const uint16_t dcur = rdt;
    if (c + 1 < nchunks) fetch(c + 1);
    // Gate inputs of this chunk in the Y^T layout: row k = 16 kt + r16, channels 16w + 4q4 .. +3.
    uint2 zv[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int k = 16 * kt + r16;
      zv[kt] = make_uint2(0u, 0u);
      if (has_z && k < nt_)
        zv[kt] = *reinterpret_cast<const uint2*>(z + (b * L + t0 + k) * HP + (int64_t)h * kHP + 16 * w + 4 * q4);
    }
    __syncthreads();

    // 1. Steps and decay sums (every wave for itself; lane = step).  Steps
    //    past the end count as dt = 0: decay 1, no input.
    {
      float d = 0.f;
      if (lane < nt_) {
        d = from_bf16(dcur);
        if (MODE & 1) d = softplus(d + dtb);
      }
      float l = d * Al2;
#pragma unroll
      for (int off = 1; off < kQ; off <<= 1) {
        const float o = __shfl_up(l, off, 64);
        if ((lane & (kQ - 1)) >= off) l += o;
      }
      const float lq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), kQ - 1));
      if (lane < kQ) {
        lv[lane] = l;
        dv[lane] = d;
        wv[lane] = hw_exp2(lq - l) * d;
        ev[lane] = hw_exp2(l);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const float decay = hw_exp2(lv[kQ - 1]);

    // 2. Score tile (it, kt) = (0,0), (0,1), (1,1) for waves 0, 1, 2:
    //    S^T = B C^T over the permuted state order, masked into W.
    if (w < 3) {
      const int it = w >> 1, kt = (w + 1) >> 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const uint16_t* bp = &sB[buf][(16 * it + r16) * SB + 32 * kk + 4 * q4];
        const u16x8 a = cat(*reinterpret_cast<const u16x4*>(bp), *reinterpret_cast<const u16x4*>(bp + 16));
        const u16x8 cb = *reinterpret_cast<const u16x8*>(&sC[buf][(16 * kt + r16) * SC + 32 * kk + 8 * q4]);
        acc = mma(a, cb, acc);
      }
      const int k = 16 * kt + r16;
      const float lk = lv[k];
      const f32x4 li = *reinterpret_cast<const f32x4*>(&lv[16 * it + 4 * q4]);
      const f32x4 di = *reinterpret_cast<const f32x4*>(&dv[16 * it + 4 * q4]);
      u16x4 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * it + 4 * q4 + j;
        float v = i <= k ? acc[j] * hw_exp2(lk - li[j]) * di[j] : 0.f;
        if (i == k) v += Dh;
        uint16_t vh, vl;
        split_bf16(v, vh, vl);
        hi[j] = vh;
        lo[j] = vl;
      }
      *reinterpret_cast<u16x4*>(&sW[0][k * kSW + 16 * it + 4 * q4]) = hi;
      *reinterpret_cast<u16x4*>(&sW[1][k * kSW + 16 * it + 4 * q4]) = lo;
    }
    // 3. This wave's x columns over the chunk's steps: lane (r16, q4) gets
    //    x[8 q4 + j][16 w + r16], j < 8.
    const uint16_t* xp = &sX[(8 * q4 + (r16 >> 2)) * kSX + 16 * w + 4 * (r16 & 3)];
    const u16x8 xt = cat(lds_tr4(xp), lds_tr4(xp + 4 * kSX));
    __syncthreads();  // W complete

    // 4. Y^T = X^T W^T + (H^T C^T) diag(exp(l)); gate; store.
    u16x8 hhi[NK], hlo[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t vh, vl;
        split_bf16(accH[2 * kk + (j >> 2)][j & 3], vh, vl);
        hhi[kk][j] = vh;
        hlo[kk][j] = vl;
      }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int k = 16 * kt + r16;
      const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
      const bool upper = kt == 0 && q4 >= 2;  // steps i >= 16 > k
      u16x8 whi = *reinterpret_cast<const u16x8*>(&sW[0][k * kSW + 8 * q4]);
      u16x8 wlo = *reinterpret_cast<const u16x8*>(&sW[1][k * kSW + 8 * q4]);
      whi = upper ? zero : whi;
      wlo = upper ? zero : wlo;
      f32x4 accY = {0.f, 0.f, 0.f, 0.f};
      accY = mma(xt, whi, accY);
      accY = mma(xt, wlo, accY);
      f32x4 accO = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u16x8 cb = *reinterpret_cast<const u16x8*>(&sC[buf][k * SC + 32 * kk + 8 * q4]);
        accO = mma(hhi[kk], cb, accO);
        accO = mma(hlo[kk], cb, accO);
      }
      const float ek = ev[k];
      if (k < nt_) {
        u16x4 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = accY[j] + ek * accO[j];
          if (has_z) {
            const uint32_t zw = j < 2 ? zv[kt].x : zv[kt].y;
            v *= silu(from_bf16((uint16_t)((j & 1) ? zw >> 16 : zw & 0xffffu)));
          }
          out[j] = to_bf16(v);
        }
        *reinterpret_cast<u16x4*>(y + (b * L + t0 + k) * HP + (int64_t)h * kHP + 16 * w + 4 * q4) = out;
      }
    }

    // 5. State: H = exp(l_Q) H + B^T (w o X).
    u16x8 xwh, xwl;
    {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wv[8 * q4]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wv[8 * q4 + 4]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t vh, vl;
        split_bf16((j < 4 ? w0[j] : w1[j - 4]) * from_bf16(xt[j]), vh, vl);
        xwh[j] = vh;
        xwl[j] = vl;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint16_t* bp = &sB[buf][(8 * q4 + (r16 >> 2)) * SB + 16 * nt + 4 * (r16 & 3)];
      const u16x8 bt = cat(lds_tr4(bp), lds_tr4(bp + 4 * SB));
      f32x4 acc = accH[nt] * decay;
      acc = mma(bt, xwh, acc);
      acc = mma(bt, xwl, acc);
      accH[nt] = acc;
    }
  }

  if (h_last != nullptr) {
    float* hp = h_last + (((b * dm.nheads) + h) * kHP + 16 * w + r16) * N + 4 * q4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) hp[16 * nt + j] = accH[nt][j];
  }
}

template <int N>
hipError_t launch_ssd_n(const SsdLaunch& p) {
  const SsdDims dm{p.batch, p.seqlen, (int32_t)p.nheads, (int32_t)p.ngroups};
  const unsigned grid = (unsigned)(p.batch * p.nheads);
  auto go = [&](auto kern) {
    return launch(kern, dim3(grid), dim3(256), 0, p.stream, static_cast<const uint16_t*>(p.x),
                  static_cast<const uint16_t*>(p.dt), p.A, static_cast<const uint16_t*>(p.B),
                  static_cast<const uint16_t*>(p.C), p.D, static_cast<const uint16_t*>(p.z), p.h0,
                  static_cast<uint16_t*>(p.y), p.h_last, p.dt_bias, dm);
  };
  return (p.flags & 1u) ? go(k_ssd_fwd<N, 1>) : go(k_ssd_fwd<N, 0>);
}

}  // namespace

hipError_t launch_ssd(const SsdLaunch& p) {
  switch (p.d_state) {
    case 64: return launch_ssd_n<64>(p);
    case 128: return launch_ssd_n<128>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssm
