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
// (pwwt.cn/news/5168881), section 2.3).  For a chunk of Q = 64 steps, with
// l_t the running sum of dt A inside the chunk:
//   Y   = (C B^T o L) (dt x) + diag(exp(l)) C H_prev        L[k,i] = exp(l_k - l_i), i <= k
//   H'  = exp(l_Q) H_prev + sum_i exp(l_Q - l_i) dt_i B_i x_i^T
// The products C B^T (Q x Q, contraction over N), the masked scores times X
// (Q x 64), C H_prev (Q x 64) and the state update (64 x N, contraction over
// Q) are dense: they run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
// The state stays in fp32 MFMA accumulators for the whole sequence.
//
// Precision: x, B, C are bf16 inputs and enter the products exactly.  The
// derived operands (masked scores, the scaled B^T and the state copy) are
// sums of terms much larger than the outputs they produce (random B and C
// give scores of size sqrt(N)); rounding them to bf16 once costs up to ~10%
// of small outputs.  Each is therefore split into hi = bf16(v) and lo =
// bf16(v - hi) and multiplied twice (about 16 significant bits), which
// leaves the bf16 rounding of y as the dominant error.  The matrix cores are
// not the bound here (HBM is), so the extra products are cheap.
//
// Mapping: one workgroup (4 waves) per (batch row, head) walks the chunks in
// order.  Wave w owns output rows [16w, 16w+16) of a chunk and channel rows
// [16w, 16w+16) of the state.  Per chunk: the decay sums go to LDS; X is
// staged transposed and B transposed with each row scaled by exp(l_Q - l_i)
// dt_i; each wave reads its C rows and the scores' B rows straight from
// global memory as 16-byte MFMA operands.
//
// MFMA operand layout (checked on the device): for a 16x32 A, lane l holds
// A[l % 16][8 (l / 16) + j], j < 8; for a 32x16 B, B[8 (l / 16) + j][l % 16];
// the 16x16 result: D[4 (l / 16) + j][l % 16], j < 4.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kQ = 64;    // chunk length
constexpr int kHP = 64;   // channels per head
constexpr int kPad = 8;   // LDS row padding in bf16 (keeps 16-byte row reads conflict-free)

struct SsdDims {
  int64_t batch, seqlen;
  int32_t nheads, ngroups;
};

__device__ __forceinline__ f32x4 mma(const u16x8& a, const u16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ uint16_t to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ float from_bf16(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
// v = hi + lo to about 16 significant bits.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = to_bf16(v);
  lo = to_bf16(v - from_bf16(hi));
}

template <int N, int MODE>
__global__ void __launch_bounds__(256)
    k_ssd_fwd(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
              const uint16_t* __restrict__ B, const uint16_t* __restrict__ C, const float* __restrict__ D,
              const uint16_t* __restrict__ z, const float* __restrict__ h0, uint16_t* __restrict__ y,
              float* __restrict__ h_last, const float* __restrict__ dt_bias, const SsdDims dm) {
  constexpr int NT = N / 16;  // state tiles of 16
  constexpr int NK = N / 32;  // contraction steps over the state
  // Derived operands are kept as hi/lo bf16 pairs (plane 0 = hi, 1 = lo).
  __shared__ __align__(16) uint16_t sXt[kHP][kQ + kPad];      // x^T of the chunk
  __shared__ __align__(16) uint16_t sBtw[2][N][kQ + kPad];    // (exp(l_Q - l_i) dt_i B_i)^T
  __shared__ __align__(16) uint16_t sW[2][kQ][kQ + kPad];     // masked scores
  __shared__ __align__(16) uint16_t sHt[2][kHP][N + kPad];    // copy of the state, [p][n]
  __shared__ float sl[kQ], sdt[kQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;  // MFMA row / quarter
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bid % dm.nheads;
  const int64_t b = bid / dm.nheads;
  const int g = h / (dm.nheads / dm.ngroups);
  const int64_t L = dm.seqlen;
  const int64_t HP = (int64_t)dm.nheads * kHP;
  const float Ah = A[h];
  const float Dh = D != nullptr ? D[h] : 0.f;
  const float dtb = (MODE & 1) ? dt_bias[h] : 0.f;
  const bool has_z = z != nullptr;

  // State H^T[p][n], p in [16w, 16w+16): accH[nt][j] = H^T[16w + 4 q4 + j][16 nt + r16].
  f32x4 accH[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = 16 * w + 4 * q4 + j, n = 16 * nt + r16;
      accH[nt][j] = h0 != nullptr ? h0[(((b * dm.nheads) + h) * kHP + p) * N + n] : 0.f;
    }
  }
  auto write_state_copy = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        split_bf16(accH[nt][j], sHt[0][16 * w + 4 * q4 + j][16 * nt + r16], sHt[1][16 * w + 4 * q4 + j][16 * nt + r16]);
  };
  write_state_copy();

  const int64_t nchunks = (L + kQ - 1) / kQ;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * kQ;
    const int nt_ = (int)min((int64_t)kQ, L - t0);
    // 1. Steps and decay sums (wave 0; lane = step).  Steps past the end
    //    count as dt = 0: decay 1, no input.
    if (w == 0) {
      float d = 0.f;
      if (lane < nt_) {
        d = from_bf16(dt[(b * L + t0 + lane) * dm.nheads + h]);
        if (MODE & 1) d = softplus(d + dtb);
      }
      float l = d * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(l, off, 64);
        if (lane >= off) l += o;
      }
      sl[lane] = l;
      sdt[lane] = d;
    }
    __syncthreads();
    // 2. Stage x^T and the scaled B^T.
    const float lQ = sl[kQ - 1];
    {
      // x: 64 rows x 64 channels = 512 pieces of 8; two per thread.
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int piece = tid + 256 * r;
        const int t = piece >> 3, p0 = (piece & 7) * 8;
        u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < nt_) v = *reinterpret_cast<const u16x8*>(x + (b * L + t0 + t) * HP + (int64_t)h * kHP + p0);
#pragma unroll
        for (int j = 0; j < 8; ++j) sXt[p0 + j][t] = v[j];
      }
      // B: 64 rows x N states = 8N pieces of 8.
#pragma unroll
      for (int r = 0; r < N / 32; ++r) {
        const int piece = tid + 256 * r;
        const int t = piece / (N / 8), n0 = (piece % (N / 8)) * 8;
        u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        float wt = 0.f;
        if (t < nt_) {
          v = *reinterpret_cast<const u16x8*>(B + ((b * L + t0 + t) * dm.ngroups + g) * N + n0);
          wt = hw_exp2((lQ - sl[t]) * kLog2e) * sdt[t];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) split_bf16(wt * from_bf16(v[j]), sBtw[0][n0 + j][t], sBtw[1][n0 + j][t]);
      }
    }
    __syncthreads();

    // 3. This wave's C rows as MFMA A operands (k = 16w + r16; rows past the
    //    end are zero).
    const int krow = 16 * w + r16;
    const bool kvalid = krow < nt_;
    const uint16_t* crow = C + ((b * L + t0 + (kvalid ? krow : 0)) * dm.ngroups + g) * N + 8 * q4;
    u16x8 ac[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      ac[kk] = *reinterpret_cast<const u16x8*>(crow + 32 * kk);
      if (!kvalid) ac[kk] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    // 4. Scores C B^T for the causal tiles, masked by the decay and dt.
    float lk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lk[j] = sl[16 * w + 4 * q4 + j];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt <= w) {
        const int irow = 16 * jt + r16;
        const uint16_t* brow = B + ((b * L + t0 + min(irow, nt_ - 1)) * dm.ngroups + g) * N + 8 * q4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc = mma(ac[kk], *reinterpret_cast<const u16x8*>(brow + 32 * kk), acc);
        const int i = 16 * jt + r16;
        const float li = sl[i], di = sdt[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = 16 * w + 4 * q4 + j;
          const float v = i <= k ? acc[j] * hw_exp2((lk[j] - li) * kLog2e) * di : 0.f;
          split_bf16(v, sW[0][k][i], sW[1][k][i]);
        }
      } else if (jt == w + 1 && (w & 1) == 0) {
        // The W X product below runs over whole 32-wide slices of i: this
        // tile is inside the slice and must read as zero.
#pragma unroll
        for (int j = 0; j < 4; ++j) sW[0][16 * w + 4 * q4 + j][16 * jt + r16] = sW[1][16 * w + 4 * q4 + j][16 * jt + r16] = 0;
      }
    }
    // 5. Y = W X (own rows of sW only) + diag(exp(l_k)) C H_prev.
    f32x4 accY[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (32 * kk <= 16 * w + 15) {
          const u16x8 bx = *reinterpret_cast<const u16x8*>(&sXt[16 * pt + r16][32 * kk + 8 * q4]);
#pragma unroll
          for (int pl = 0; pl < 2; ++pl)
            acc = mma(*reinterpret_cast<const u16x8*>(&sW[pl][krow][32 * kk + 8 * q4]), bx, acc);
        }
      }
      f32x4 off = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
          off = mma(ac[kk], *reinterpret_cast<const u16x8*>(&sHt[pl][16 * pt + r16][32 * kk + 8 * q4]), off);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += hw_exp2(lk[j] * kLog2e) * off[j];
      accY[pt] = acc;
    }
    // 6. Skip term, gate, store.
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 16 * w + 4 * q4 + j, p = 16 * pt + r16;
        if (k < nt_) {
          const int64_t o = (b * L + t0 + k) * HP + (int64_t)h * kHP + p;
          float v = accY[pt][j] + Dh * from_bf16(sXt[p][k]);
          if (has_z) v *= silu(from_bf16(z[o]));
          y[o] = to_bf16(v);
        }
      }
    }
    __syncthreads();  // every wave is done with sHt, sXt and sW
    // 7. State: H = exp(l_Q) H + sum_i x_i (exp(l_Q - l_i) dt_i B_i)^T.
    const float decay = hw_exp2(lQ * kLog2e);
    const int prow = 16 * w + r16;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = accH[nt] * decay;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u16x8 ax = *reinterpret_cast<const u16x8*>(&sXt[prow][32 * kk + 8 * q4]);
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
          acc = mma(ax, *reinterpret_cast<const u16x8*>(&sBtw[pl][16 * nt + r16][32 * kk + 8 * q4]), acc);
      }
      accH[nt] = acc;
    }
    __syncthreads();  // every wave is done with sXt and sBtw before restaging
    write_state_copy();
  }

  if (h_last != nullptr) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = 16 * w + 4 * q4 + j, n = 16 * nt + r16;
        h_last[(((b * dm.nheads) + h) * kHP + p) * N + n] = accH[nt][j];
      }
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
