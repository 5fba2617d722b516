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
// state stays in fp32 accumulators for the whole sequence, kept scaled by a
// power of two so that the decay exp(l_Q) is folded into w and exp(l) and
// applied to the accumulators only when the scale is reset.
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
// The next chunk's rows are loaded into registers while this one computes
// and staged in LDS per chunk:
//   * x row-major; this wave's columns over time (the X^T operand, and w o X)
//     need eight consecutive steps per lane and come out through
//     ds_read_b64_tr_b16, which transposes 16 x 4 blocks across each group of
//     16 lanes.
//   * B twice: rows in the permuted state order (the score operand), and B^T
//     for the state update, written transposed (a 4 x 4 transpose in
//     registers, 4 state rows per padded LDS group) so that every wave reads
//     it with 16-byte loads.  B^T is written between the chunk's two
//     barriers, so both copies are single-buffered.
//   * C in the permuted state order, double-buffered (it is read on both
//     sides of the second barrier).
//   * Waves 0-2 each compute one of the three causal 16 x 16 score tiles
//     (S^T = B C^T), mask them and share W through LDS.
//   * The state's accumulator layout (lane = channel, four states per lane
//     per tile) is used directly as the A operand of H^T C^T: the contraction
//     over n takes the states in the order the accumulators hold them, and C
//     is staged with its columns permuted to match, so the state never
//     leaves registers.

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
constexpr int kSZ = kHP + 8;     // gate-in / output-out tile row stride: 36 dwords

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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t pack_bf16(float v0, float v1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v0, v1}, bf16x2));
}
__device__ __forceinline__ float lo_f32(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float hi_f32(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }
// v0, v1 = hi + lo to about 16 significant bits, as packed bf16 pairs
// (.x = hi, .y = lo).
__device__ __forceinline__ uint2 split2(float v0, float v1) {
  const uint32_t hi = pack_bf16(v0, v1);
  return make_uint2(hi, pack_bf16(v0 - lo_f32(hi), v1 - hi_f32(hi)));
}
__device__ __forceinline__ u16x8 as_u16x8(const u32x4& v) { return __builtin_bit_cast(u16x8, v); }
__device__ __forceinline__ u16x8 cat(const u16x4& a, const u16x4& b) {
  return u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Inclusive prefix sum over lanes 0..31 (lanes 32..63 hold a second,
// unused scan).  DPP row shifts add within each row of 16 lanes (lanes whose
// source falls outside the row read 0), then row 0's total (lane 15) is
// broadcast into row 1: all on the VALU, no LDS round trips.
__device__ __forceinline__ float scan32(float v) {
  int x = __builtin_bit_cast(int, v);
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true)));
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true)));
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true)));
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true)));
  // row_bcast:15 into rows 1 and 3 only (row mask 0b1010); other rows add 0.
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false)));
  return __builtin_bit_cast(float, x);
}

// Position of state column o (0..31 inside a 32-wide slice) in the permuted
// C tile: the order in which the state accumulators hold the states.
__device__ __forceinline__ int cperm(int o) { return o < 16 ? 2 * o : 2 * (o - 16) + 4; }

// MODE bit 0: dt is softplus(dt + dt_bias); bit 1: gate with silu(z).
template <int N, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))  // all (row, head) groups resident
k_ssd_fwd(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
          const uint16_t* __restrict__ B, const uint16_t* __restrict__ C, const float* __restrict__ D,
          const uint16_t* __restrict__ z, const float* __restrict__ h0, uint16_t* __restrict__ y,
          float* __restrict__ h_last, const float* __restrict__ dt_bias, const SsdDims dm) {
  constexpr int NT = N / 16;            // state tiles of 16
  constexpr int NK = N / 32;            // contraction slices over the state
  constexpr int SC = N + 8;             // B and C tile row stride: 16-byte reads conflict-free
  constexpr int PB = kQ * N / 8 / 256;  // 16-byte pieces of C per thread
  constexpr int GT = 4 * kQ + 8;        // transposed B: groups of 4 state rows of kQ steps, padded
  constexpr int NQ = N / 4;             // 4-state column groups of B
  constexpr int BT = NQ * (kQ / 4);     // threads that stage B (4 steps x 4 states each)
  constexpr bool kGate = (MODE & 2) != 0;
  __shared__ __align__(16) uint16_t sX[kQ * kSX];
  __shared__ __align__(16) uint16_t sBp[kQ * SC];      // B rows, states in the permuted order (scores)
  __shared__ __align__(16) uint16_t sBt[NQ * GT];      // B^T: (n, t) at (n / 4) GT + (n % 4) kQ + t
  __shared__ __align__(16) uint16_t sC[2][kQ * SC];
  __shared__ __align__(16) uint16_t sW[2][kQ * kSW];  // masked scores [k][i], hi and lo planes
  __shared__ __align__(16) float sv[2][4][kQ];         // l (log2 units), dt, w, exp(l); double-buffered
  __shared__ float sfac[2];                            // per chunk: state rescale factor (negative: none)
  __shared__ float slam;                               // log2 of the scale of the kept state, at the end
  __shared__ __align__(16) uint16_t sZY[kQ * kSZ];    // gate inputs in, outputs out, row-major

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = bid % dm.nheads;
  const int64_t b = bid / dm.nheads;
  const int g = h / (dm.nheads / dm.ngroups);
  const int64_t L = dm.seqlen;
  // Bytes per step of x, z, y and of B, C: below 2^24 for at most 32768
  // heads, so row offsets use 24-bit multiplies.
  const uint32_t rowb = (uint32_t)dm.nheads * kHP * 2;
  const uint32_t growb = (uint32_t)dm.ngroups * N * 2;
  const float Al2 = A[h] * kLog2e;
  const float Dh = D != nullptr ? D[h] : 0.f;
  const float dtb = (MODE & 1) ? dt_bias[h] : 0.f;

  // State H[n][p] for p = 16w + r16: accH[nt][j] = H[16 nt + 4 q4 + j][p].
  f32x4 accH[NT];
  {
    const float* hp = h0 != nullptr ? h0 + (((b * dm.nheads) + h) * kHP + 16 * w + r16) * N + 4 * q4 : nullptr;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) accH[nt][j] = hp != nullptr ? hp[16 * nt + j] : 0.f;
  }
  // Scores with k < 16 <= i are never written: zero them once.
  if (tid < 64) {
    const int k = tid >> 2, i = 16 + 4 * (tid & 3);
    *reinterpret_cast<u16x4*>(&sW[0][k * kSW + i]) = u16x4{0, 0, 0, 0};
    *reinterpret_cast<u16x4*>(&sW[1][k * kSW + i]) = u16x4{0, 0, 0, 0};
  }

  // Staging registers, one chunk ahead.  Rows past the end of the sequence
  // repeat the last row: they only ever meet zero weights (dt = 0 there)
  // or feed outputs that are not stored.
  const int sx_t = tid >> 3, sx_c = (tid & 7) * 8;
  const int bq = tid % NQ, tq = tid / NQ;  // B: states 4 bq .. +3 of steps 4 tq .. +3
  u16x8 rx, rc[PB];
  u32x2 rb[4];
  u16x8 rz = {};
  uint16_t rdt = 0;
  // The next chunk's rows are requested in two groups, B and C after the
  // first barrier and x, dt and the gate inputs after the second, so that
  // the four waves do not put all their loads into the memory pipeline at
  // once.
  auto fetch_xz = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const int last = (int)min((int64_t)kQ, L - t0) - 1;
    const gchar* xb = uniform_ptr(x + ((b * L + t0) * dm.nheads + h) * kHP);
    rx = gldr<u16x8>(xb, __umul24((uint32_t)min(sx_t, last), rowb) + sx_c * 2);
    if (kGate) {
      // Gate inputs in whole rows, like x: they pass through LDS into the Y^T layout.
      const gchar* zb = uniform_ptr(z + ((b * L + t0) * dm.nheads + h) * kHP);
      rz = gldr<u16x8>(zb, __umul24((uint32_t)min(sx_t, last), rowb) + sx_c * 2);
    }
  };
  // The steps of chunk c (lane = step), for wave 3, which turns them into
  // decay sums a chunk ahead of their use.
  auto fetch_dt = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const int last = (int)min((int64_t)kQ, L - t0) - 1;
    const gchar* db = uniform_ptr(dt + (b * L + t0) * dm.nheads + h);
    rdt = gldr<uint16_t>(db, __umul24((uint32_t)min(lane, last), (uint32_t)dm.nheads * 2));
  };
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const int last = (int)min((int64_t)kQ, L - t0) - 1;
    const gchar* bb = uniform_ptr(B + ((b * L + t0) * dm.ngroups + g) * N);
    const gchar* cb = uniform_ptr(C + ((b * L + t0) * dm.ngroups + g) * N);
#pragma unroll
    for (int r = 0; r < PB; ++r) {
      const int piece = tid + 256 * r;
      const int t = piece / (N / 8), n8 = (piece % (N / 8)) * 8;
      rc[r] = gldr<u16x8>(cb, __umul24((uint32_t)min(t, last), growb) + n8 * 2);
    }
    if (BT == 256 || w < BT / 64) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rb[r] = gldr<u32x2>(bb, __umul24((uint32_t)min(4 * tq + r, last), growb) + 8 * bq);
    }
  };
  // x, C and the row copy of B, before the chunk's first barrier.
  auto stage = [&](int buf) {
    *reinterpret_cast<u16x8*>(&sX[sx_t * kSX + sx_c]) = rx;
    if (BT == 256 || w < BT / 64) {
      const int s0 = (4 * bq) & ~31, o = (4 * bq) & 31;
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x2*>(&sBp[(4 * tq + r) * SC + s0 + cperm(o)]) = rb[r];
    }
#pragma unroll
    for (int r = 0; r < PB; ++r) {
      const int piece = tid + 256 * r;
      const int t = piece / (N / 8), n8 = (piece % (N / 8)) * 8;
      const int s0 = n8 & ~31, o = n8 & 31;
      *reinterpret_cast<u16x4*>(&sC[buf][t * SC + s0 + cperm(o)]) = u16x4{rc[r][0], rc[r][1], rc[r][2], rc[r][3]};
      *reinterpret_cast<u16x4*>(&sC[buf][t * SC + s0 + cperm(o + 4)]) = u16x4{rc[r][4], rc[r][5], rc[r][6], rc[r][7]};
    }
  };

  // B^T, after the chunk's first barrier (the previous chunk's state update
  // is then done with it) and before the second: a 4 x 4 transpose in
  // registers, one 8-byte write per state.
  auto stage_bt = [&]() {
    if (BT == 256 || w < BT / 64) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int d = c4 >> 1, sh = (c4 & 1) * 16;
        const uint32_t t01 = ((rb[0][d] >> sh) & 0xffffu) | (((rb[1][d] >> sh) & 0xffffu) << 16);
        const uint32_t t23 = ((rb[2][d] >> sh) & 0xffffu) | (((rb[3][d] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(&sBt[bq * GT + c4 * kQ + 4 * tq]) = u32x2{t01, t23};
      }
    }
  };

  // Steps and decay sums of chunk cc (lane = step) into sv[cc & 1], by wave 3
  // (the one without a score tile), a chunk ahead of their use.  Steps past
  // the end count as dt = 0: decay 1, no input.
  // The state is kept scaled, G = H 2^-lam with lam the log2 of the decay
  // since the last rescale, so that a chunk adds to it without multiplying it
  // by the chunk's decay first: G += B^T (w' o X) with w'_i = 2^(-lam - l_i)
  // dt_i (lam before the chunk), and C H enters the outputs as
  // 2^(l_k + lam) C G.  When the scale would pass 2^60 the chunk rescales G to
  // H instead (factor 2^(lam + l_Q), passed on in sfac) and takes the unscaled
  // weights 2^(l_Q - l_i) dt_i, so no weight and no kept state exceeds 2^60
  // times its unscaled size.
  float lam = 0.f;  // wave 3's running lam
  auto decay_sums = [&](int64_t cc) {
    const int ntc = (int)min((int64_t)kQ, L - cc * kQ);
    float d = 0.f;
    if (lane < ntc) {
      d = lo_f32(rdt);
      if (MODE & 1) d = softplus(d, dtb);
    }
    const float l = scan32(d * Al2);
    const float lq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), kQ - 1));
    const bool rescale = lam + lq < -60.f;
    const float sigma = rescale ? lq : -lam;
    if (lane < kQ) {
      float* const sd = &sv[cc & 1][0][0];
      sd[lane] = l;
      sd[kQ + lane] = d;
      sd[2 * kQ + lane] = hw_exp2(sigma - l) * d;
      sd[3 * kQ + lane] = hw_exp2(l + lam);
    }
    if (lane == 0) sfac[cc & 1] = rescale ? hw_exp2(lam + lq) : -1.f;
    lam = rescale ? 0.f : lam + lq;
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  if (nchunks > 0) {
    fetch(0);
    fetch_xz(0);
    if (w == 3) {
      fetch_dt(0);
      decay_sums(0);
      if (nchunks > 1) fetch_dt(1);
    }
  }
  // Up to three workgroups share a CU: their waves take turns at the higher
  // priority, one chunk each (take_turn, ssm_device.h), so that no workgroup
  // runs its last chunks alone (0.402 -> 0.388 ms on the Mamba-2 2.7B layer).
  const int wslot = wave_slot_parity();
  for (int64_t c = 0; c < nchunks; ++c) {
    take_turn((int)c, wslot);
    const int buf = (int)(c & 1);
    const int64_t t0 = c * kQ;
    stage(buf);
    __syncthreads();
    // The previous chunk's outputs leave in whole 128-byte rows, and this
    // chunk's gate inputs take their place: every thread reads, stores and
    // refills the same 16 bytes of the tile (only the last chunk can be
    // short, and it is stored after the loop).
    {
      uint16_t* slot = &sZY[sx_t * kSZ + sx_c];
      if (c > 0) {
        gchar* yp = uniform_ptr(y + ((b * L + t0 - kQ) * dm.nheads + h) * kHP);
        gstr<u16x8>(yp, __umul24((uint32_t)sx_t, rowb) + sx_c * 2, *reinterpret_cast<const u16x8*>(slot));
      }
      if (kGate) *reinterpret_cast<u16x8*>(slot) = rz;
    }
    stage_bt();
    if (c + 1 < nchunks) fetch(c + 1);
    // Wave 3 has no score tile: the next chunk's decay sums fill its wait for
    // the second barrier (their steps were requested a chunk ago).
    if (w == 3 && c + 1 < nchunks) {
      decay_sums(c + 1);
      if (c + 2 < nchunks) fetch_dt(c + 2);
    }

    // 1. This chunk's decay sums (written by wave 3 before the barrier).
    const float* const lv = &sv[buf][0][0];
    const float* const dv = lv + kQ;
    const float* const wv = lv + 2 * kQ;
    const float* const ev = lv + 3 * kQ;
    const float fac = sfac[buf];

    // 2. Score tile (it, kt) = (0,0), (0,1), (1,1) for waves 0, 1, 2:
    //    S^T = B C^T over the permuted state order, masked into W.
    if (w < 3) {
      const int it = w >> 1, kt = (w + 1) >> 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u16x8 a = *reinterpret_cast<const u16x8*>(&sBp[(16 * it + r16) * SC + 32 * kk + 8 * q4]);
        const u16x8 cb = *reinterpret_cast<const u16x8*>(&sC[buf][(16 * kt + r16) * SC + 32 * kk + 8 * q4]);
        acc = mma(a, cb, acc);
      }
      const int k = 16 * kt + r16;
      const float lk = lv[k];
      const f32x4 li = *reinterpret_cast<const f32x4*>(&lv[16 * it + 4 * q4]);
      const f32x4 di = *reinterpret_cast<const f32x4*>(&dv[16 * it + 4 * q4]);
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * it + 4 * q4 + j;
        v[j] = i <= k ? acc[j] * hw_exp2(lk - li[j]) * di[j] : 0.f;
        if (i == k) v[j] += Dh;
      }
      const uint2 s01 = split2(v[0], v[1]), s23 = split2(v[2], v[3]);
      *reinterpret_cast<uint2*>(&sW[0][k * kSW + 16 * it + 4 * q4]) = make_uint2(s01.x, s23.x);
      *reinterpret_cast<uint2*>(&sW[1][k * kSW + 16 * it + 4 * q4]) = make_uint2(s01.y, s23.y);
    }
    // 3. This wave's x columns over the chunk's steps: lane (r16, q4) gets
    //    x[8 q4 + j][16 w + r16], j < 8.
    const uint16_t* xp = &sX[(8 * q4 + (r16 >> 2)) * kSX + 16 * w + 4 * (r16 & 3)];
    const u16x8 xt = cat(lds_tr4(xp), lds_tr4(xp + 4 * kSX));
    __syncthreads();  // W complete
    if (c + 1 < nchunks) fetch_xz(c + 1);

    // 4. Y^T = X^T W^T + (H^T C^T) diag(exp(l)); gate; store.  Software
    //    pipelined over the 32-state slices: the C operands of slice kk + 1
    //    are requested before slice kk's state is split into hi and lo and
    //    multiplied, so the split's VALU work covers the LDS latency.
    f32x4 accY[2], accO[2];
    {
      u16x8 wq[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int k = 16 * kt + r16;
        wq[kt][0] = *reinterpret_cast<const u16x8*>(&sW[0][k * kSW + 8 * q4]);
        wq[kt][1] = *reinterpret_cast<const u16x8*>(&sW[1][k * kSW + 8 * q4]);
      }
      auto cfrag = [&](int kt, int kk) {
        return *reinterpret_cast<const u16x8*>(&sC[buf][(16 * kt + r16) * SC + 32 * kk + 8 * q4]);
      };
      u16x8 cn[2] = {cfrag(0, 0), cfrag(1, 0)};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        accY[kt] = mma(xt, wq[kt][0], f32x4{0.f, 0.f, 0.f, 0.f});
        accY[kt] = mma(xt, wq[kt][1], accY[kt]);
        accO[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u16x8 cb0 = cn[0], cb1 = cn[1];
        if (kk + 1 < NK) {
          cn[0] = cfrag(0, kk + 1);
          cn[1] = cfrag(1, kk + 1);
        }
        u32x4 vh, vl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4& a = accH[2 * kk + (q >> 1)];
          const uint2 sp = split2(a[2 * (q & 1)], a[2 * (q & 1) + 1]);
          vh[q] = sp.x;
          vl[q] = sp.y;
        }
        const u16x8 hh = as_u16x8(vh), hl = as_u16x8(vl);
        accO[0] = mma(hh, cb0, accO[0]);
        accO[1] = mma(hh, cb1, accO[1]);
        accO[0] = mma(hl, cb0, accO[0]);
        accO[1] = mma(hl, cb1, accO[1]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int k = 16 * kt + r16;
      const float ek = ev[k];
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = accY[kt][j] + ek * accO[kt][j];
      // This lane's 8 bytes of the tile: its gate inputs, then its outputs.
      u32x2* const yz = reinterpret_cast<u32x2*>(&sZY[k * kSZ + 16 * w + 4 * q4]);
      if (kGate) {
        const u32x2 zz = *yz;
        v[0] *= silu(lo_f32(zz.x));
        v[1] *= silu(hi_f32(zz.x));
        v[2] *= silu(lo_f32(zz.y));
        v[3] *= silu(hi_f32(zz.y));
      }
      *yz = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }

    // 5. State: G += B^T (w' o X), after the rescale when the chunk has one.
    u16x8 xwh, xwl;
    {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wv[8 * q4]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wv[8 * q4 + 4]);
      const u32x4 xd = __builtin_bit_cast(u32x4, xt);
      u32x4 vh, vl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float wa = q < 2 ? w0[2 * q] : w1[2 * q - 4], wb = q < 2 ? w0[2 * q + 1] : w1[2 * q - 3];
        const uint2 sp = split2(wa * lo_f32(xd[q]), wb * hi_f32(xd[q]));
        vh[q] = sp.x;
        vl[q] = sp.y;
      }
      xwh = as_u16x8(vh);
      xwl = as_u16x8(vl);
    }
    if (fac >= 0.f) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) accH[nt] *= fac;
    }
    {
      auto bfrag = [&](int nt) {
        const int n = 16 * nt + r16;
        return *reinterpret_cast<const u16x8*>(&sBt[(n >> 2) * GT + (n & 3) * kQ + 8 * q4]);
      };
      u16x8 bn = bfrag(0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u16x8 bt = bn;
        if (nt + 1 < NT) bn = bfrag(nt + 1);
        accH[nt] = mma(bt, xwh, accH[nt]);
        accH[nt] = mma(bt, xwl, accH[nt]);
      }
    }
  }

  if (w == 3 && lane == 0) slam = lam;
  // The last chunk's outputs (its first nt rows).
  __syncthreads();
  if (nchunks > 0) {
    const int64_t t0 = (nchunks - 1) * kQ;
    if (sx_t < L - t0) {
      gchar* yp = uniform_ptr(y + ((b * L + t0) * dm.nheads + h) * kHP);
      gstr<u16x8>(yp, __umul24((uint32_t)sx_t, rowb) + sx_c * 2, *reinterpret_cast<const u16x8*>(&sZY[sx_t * kSZ + sx_c]));
    }
  }

  if (h_last != nullptr) {
    float* hp = h_last + (((b * dm.nheads) + h) * kHP + 16 * w + r16) * N + 4 * q4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) hp[16 * nt + j] = accH[nt][j] * hw_exp2(slam);
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
  const bool sp = (p.flags & 1u) != 0, gate = p.z != nullptr;
  if (gate) return sp ? go(k_ssd_fwd<N, 3>) : go(k_ssd_fwd<N, 2>);
  return sp ? go(k_ssd_fwd<N, 1>) : go(k_ssd_fwd<N, 0>);
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
