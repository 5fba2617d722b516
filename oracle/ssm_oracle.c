/*
 * ssm_oracle.c -- fp64 CPU oracle for the Mamba-1 selective scan and the
 * single-token recurrent state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and it shares no
 * code, header or helper with that path.
 *
 * What it computes (plain definitions, written as sequential loops):
 *
 *   Diagonal (S4D) state space model with zero-order-hold decay and the
 *   first-order input term used by Mamba:
 *       abar[t,n] = exp(delta[t] * A[n])                      (decay)
 *       h[t,n]    = abar[t,n] * h[t-1,n] + delta[t]*B[t,n]*x[t]
 *       y[t]      = sum_n C[t,n]*h[t,n] + D*x[t]
 *       y[t]     *= z[t] * sigmoid(z[t])                      (SiLU gate)
 *   Sources:
 *     - "Deriving and implementing Mamba from scratch" (dpshk.com/news/3333417),
 *       section 2.2 (discrete recurrence h_k = Abar h_{k-1} + Bbar x_k,
 *       y_k = C h_k + D x_k), section 3.2 (diagonal A: Abar = diag(exp(delta a_i)),
 *       elementwise update h^(i) = exp(delta a_i) h^(i) + delta b_i x),
 *       section 4.2 (selective Abar_k = exp(delta_k A), Bbar_k = delta_k B(x_k)),
 *       section 5.1 (SelectiveSSM: B, C of width d_state shared by every channel,
 *       Bbar = delta*B, state starts at zero, y_t = <h, C_t> + D x_t),
 *       section 5.2 (MambaBlock: SSM output multiplied by SiLU(gate)).
 *     - "Mamba from principle to code" (lshu.cn/news/79586), section 3.1
 *       (B, C have shape (batch, seq_len, d_state); delta = softplus(...) > 0)
 *       and section 6.5 (state cache shape (batch, d_inner, d_state)).
 *     - "SSMs for long-document QA" (pwwt.cn/news/5168881), section 3.1
 *       (segment-wise processing: the final state of one segment is the
 *       initial state of the next) -- this is the h0 / h_last contract.
 *     - "State space models vs Transformer: a practical guide"
 *       (datadaily.news), "How SSMs actually work" (one recurrent step:
 *       h_new from h, then y_t from h_new) -- the single-token update.
 *
 *   Readings taken where the pages are silent or loose:
 *     - y[t] is read from the state AFTER it absorbed x[t] (h_{-1} = h0);
 *       h_last is the state after the final step.
 *     - D == NULL means D = 0; z == NULL means no gate; h0 == NULL means a
 *       zero initial state; h_last == NULL means it is not written.
 *     - B and C are indexed [b][t][n] and shared by every channel d.
 *
 *   The exact-ZOH input term (input_mode 1) uses the unapproximated
 *   Bbar = (delta A)^{-1} (exp(delta A) - 1) delta B from section 2.2 of the
 *   derivation page and section 2.2 of "Mamba from principle to code"; for a
 *   diagonal A this is (exp(delta a) - 1)/a * B per state.  For a == 0 it is
 *   the limit delta*B.
 *
 *   Delta preprocessing (delta_mode 1) applies the selection step of
 *   section 4.1 of the derivation page, delta = softplus(raw + bias[d]),
 *   with softplus(v) = log(1 + exp(v)).
 *
 * Arithmetic: IEEE double, libm exp/log1p, no fast-math.  No blocking,
 * reordering or fusion beyond the loops above.  Single-threaded.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)

/* softplus(v) = log(1 + exp(v)), written to avoid overflow for large v. */
static double oracle_softplus(double v) {
  if (v > 30.0) return v + log1p(exp(-v));
  return log1p(exp(v));
}

/*
 * One channel (b, d) of the scan over t = 0..seqlen-1.
 * Strides are in elements.  state[] holds h on entry (initial state) and on
 * exit (final state).
 */
static void oracle_scan_channel(const double* x, const double* delta, const double* A_row, const double* B,
                                const double* C, double Dval, const double* z, double* y, double* state,
                                int64_t seqlen, int64_t d_state, int64_t io_stride, int64_t bc_stride,
                                int input_mode, int delta_mode, double dt_bias) {
  for (int64_t t = 0; t < seqlen; ++t) {
    double xv = x[t * io_stride];
    double dt = delta[t * io_stride];
    if (delta_mode == 1) dt = oracle_softplus(dt + dt_bias);
    const double* Bt = B + t * bc_stride;
    const double* Ct = C + t * bc_stride;
    double acc = 0.0;
    for (int64_t n = 0; n < d_state; ++n) {
      double a = A_row[n];
      double abar = exp(dt * a);
      double bbar;
      if (input_mode == 1) {
        /* exact ZOH for a diagonal entry: (exp(dt a) - 1) / a * B */
        bbar = (a != 0.0) ? (expm1(dt * a) / a) * Bt[n] : dt * Bt[n];
      } else {
        bbar = dt * Bt[n];
      }
      state[n] = abar * state[n] + bbar * xv;
      acc += Ct[n] * state[n];
    }
    double yv = acc + Dval * xv;
    if (z != NULL) {
      double zv = z[t * io_stride];
      yv = yv * (zv / (1.0 + exp(-zv)));
    }
    y[t * io_stride] = yv;
  }
}

/*
 * Full-sequence selective scan.
 *   x, delta, z, y : [batch][seqlen][d_inner]
 *   A              : [d_inner][d_state]
 *   B, C           : [batch][seqlen][d_state]
 *   D, dt_bias     : [d_inner]           (nullable)
 *   h0, h_last     : [batch][d_inner][d_state]  (nullable)
 * input_mode: 0 = Bbar = delta*B (the simplified term), 1 = exact ZOH.
 * delta_mode: 0 = delta used as given, 1 = softplus(delta + dt_bias[d]).
 */
int ssm_oracle_scan_f64(const double* x, const double* delta, const double* A, const double* B, const double* C,
                        const double* D, const double* z, const double* h0, const double* dt_bias, double* y,
                        double* h_last, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                        int input_mode, int delta_mode) {
  if (!x || !delta || !A || !B || !C || !y) return ORACLE_BAD_ARG;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0) return ORACLE_BAD_ARG;
  if (input_mode != 0 && input_mode != 1) return ORACLE_BAD_ARG;
  if (delta_mode != 0 && delta_mode != 1) return ORACLE_BAD_ARG;
  if (delta_mode == 1 && !dt_bias) return ORACLE_BAD_ARG;
  double* state = (double*)malloc((size_t)d_state * sizeof(double));
  if (!state) return ORACLE_BAD_ARG;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < d_inner; ++d) {
      for (int64_t n = 0; n < d_state; ++n)
        state[n] = h0 ? h0[(b * d_inner + d) * d_state + n] : 0.0;
      int64_t off = b * seqlen * d_inner + d;
      oracle_scan_channel(x + off, delta + off, A + d * d_state, B + b * seqlen * d_state,
                          C + b * seqlen * d_state, D ? D[d] : 0.0, z ? z + off : NULL, y + off, state, seqlen,
                          d_state, d_inner, d_state, input_mode, delta_mode, dt_bias ? dt_bias[d] : 0.0);
      if (h_last)
        for (int64_t n = 0; n < d_state; ++n) h_last[(b * d_inner + d) * d_state + n] = state[n];
    }
  }
  free(state);
  return ORACLE_OK;
}

/*
 * Single-token recurrent update (decode), in place on h.
 *   h           : [batch][d_inner][d_state]   (in/out)
 *   x_t, delta_t, z_t, y_t : [batch][d_inner]
 *   B_t, C_t    : [batch][d_state]
 * This is the scan body for one step: a scan of length 1 that starts from h
 * and writes its final state back into h.
 */
int ssm_oracle_update_f64(double* h, const double* x_t, const double* delta_t, const double* A, const double* B_t,
                          const double* C_t, const double* D, const double* z_t, const double* dt_bias, double* y_t,
                          int64_t batch, int64_t d_inner, int64_t d_state, int input_mode, int delta_mode) {
  if (!h) return ORACLE_BAD_ARG;
  /* x_t is [batch][1][d_inner]; B_t is [batch][1][d_state]; h is both h0 and h_last. */
  return ssm_oracle_scan_f64(x_t, delta_t, A, B_t, C_t, D, z_t, h, dt_bias, y_t, h, batch, 1, d_inner, d_state,
                             input_mode, delta_mode);
}

/*
 * Causal depthwise convolution over time, one filter per channel, followed
 * by an optional SiLU.  "Deriving and implementing Mamba from scratch"
 * (dpshk.com/news/3333417), section 5.2: Conv1d(d_inner, d_inner,
 * kernel_size=d_conv, padding=d_conv-1, groups=d_inner, bias=True), output
 * cut to the first seqlen positions, then SiLU.  With that padding the
 * output at t sees inputs t-(K-1) .. t, weight k multiplying input
 * t-(K-1)+k:
 *     out[t] = bias + sum_{k=0}^{K-1} w[k] * xe[t + k]
 * where xe is the input extended on the left by K-1 values: the carried
 * conv state (state_in) if given, else zeros.  The carried state is the
 * last K-1 entries of xe after the sequence ("SSM series #12" page,
 * section 1.3: the decode cache holds a convolution state next to the SSM
 * state).
 *   x, y      : [batch][seqlen][d_inner]
 *   w         : [d_inner][d_conv]
 *   bias      : [d_inner] (nullable: 0)
 *   state_in  : [batch][d_inner][d_conv-1] (nullable: zeros)
 *   state_out : [batch][d_inner][d_conv-1] (nullable)
 */
int ssm_oracle_conv1d_f64(const double* x, const double* w, const double* bias, const double* state_in, double* y,
                          double* state_out, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_conv,
                          int apply_silu) {
  if (!x || !w || !y) return ORACLE_BAD_ARG;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_conv < 1) return ORACLE_BAD_ARG;
  const int64_t K = d_conv, S = d_conv - 1;
  double* xe = (double*)malloc((size_t)(seqlen + S + 1) * sizeof(double));
  if (!xe) return ORACLE_BAD_ARG;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < d_inner; ++d) {
      for (int64_t j = 0; j < S; ++j) xe[j] = state_in ? state_in[(b * d_inner + d) * S + j] : 0.0;
      for (int64_t t = 0; t < seqlen; ++t) xe[S + t] = x[(b * seqlen + t) * d_inner + d];
      for (int64_t t = 0; t < seqlen; ++t) {
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) acc += w[d * K + k] * xe[t + k];
        if (apply_silu) acc = acc / (1.0 + exp(-acc));
        y[(b * seqlen + t) * d_inner + d] = acc;
      }
      if (state_out)
        for (int64_t j = 0; j < S; ++j) state_out[(b * d_inner + d) * S + j] = xe[seqlen + j];
    }
  }
  free(xe);
  return ORACLE_OK;
}

/*
 * d/d(a) of the exact-ZOH input coefficient coef(dt, a) = (exp(dt a) - 1)/a
 * (the a -> 0 limit being dt).  With y = dt*a and phi1(y) = (e^y - 1)/y,
 * coef = dt*phi1(y), so d coef/d a = dt^2 * phi1'(y), where
 *     phi1'(y) = (y e^y - e^y + 1) / y^2 = sum_{k>=1} k y^(k-1) / (k+1)!.
 * The closed form cancels badly for small |y|; there the series is summed.
 */
static double oracle_dcoef_da(double dt, double a) {
  double y = dt * a;
  double d1;
  if (fabs(y) < 0.5) {
    double term = 0.5; /* k = 1: 1 * y^0 / 2! */
    double fact = 2.0; /* (k+1)! */
    double ypow = 1.0;
    d1 = 0.0;
    for (int k = 1; k <= 30; ++k) {
      fact = (k == 1) ? 2.0 : fact * (double)(k + 1);
      term = (double)k * ypow / fact;
      d1 += term;
      ypow *= y;
    }
  } else {
    d1 = (y * exp(y) - expm1(y)) / (y * y);
  }
  return dt * dt * d1;
}

/*
 * Reverse-mode gradient of the full-sequence scan above (same input_mode /
 * delta_mode meanings), for the scalar loss
 *     L = sum(dy * y) + sum(dh_last * h_last).
 * It is the chain rule applied to the recurrence, taken backwards in time:
 * training back-propagates along the time axis through the scan ("SSMs for
 * long-document QA" (pwwt.cn/news/5168881), sections 3.2-3.3, which keep a
 * few states and recompute the intermediate ones for the backward pass;
 * "Deriving and implementing Mamba from scratch" (dpshk.com/news/3333417),
 * section 5.3, whose fused scan keeps what the backward pass needs).  Here
 * every state of the channel is kept, which is the plain definition.
 * Per channel (b, d), with lam[n] = dL/dh_t[n]:
 *     lam <- dh_last;  for t = L-1 .. 0:
 *        ypre = sum_n C h_t + D x;  g = dy * silu(z)  (dy if no gate)
 *        dz   = dy * ypre * silu'(z);  dD += g x;  dx = g D
 *        lam += g C_t;  dC_t += g h_t
 *        h_t  = abar h_{t-1} + bbar x   with abar = exp(dt a), bbar = dt B
 *               (exact ZOH: bbar = coef(dt, a) B)
 *        ddt += lam (a abar h_{t-1} + d bbar/d dt * x)
 *        dA  += lam (dt abar h_{t-1} + d bbar/d a * x)
 *        dB_t += lam coef x;  dx += lam coef B
 *        lam  = abar lam
 *     dh0 = lam
 * With delta_mode 1 the returned ddelta is d/d(raw) = ddt * sigmoid(raw + bias)
 * and d_dt_bias[d] accumulates the same quantity.
 *
 * Outputs: dx, ddelta, dz (if z), shaped like x; dA [d_inner][d_state];
 * dB, dC [batch][seqlen][d_state]; dD [d_inner] (if D); dh0 [batch][d_inner]
 * [d_state] (nullable); d_dt_bias [d_inner] (required with delta_mode 1).
 * dA, dB, dC, dD and d_dt_bias are sums over every channel / row that uses
 * them; they are zeroed here first.
 */
int ssm_oracle_scan_bwd_f64(const double* x, const double* delta, const double* A, const double* B, const double* C,
                            const double* D, const double* z, const double* h0, const double* dt_bias,
                            const double* dy, const double* dh_last, double* dx, double* ddelta, double* dA,
                            double* dB, double* dC, double* dD, double* dz, double* dh0, double* d_dt_bias,
                            int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int input_mode,
                            int delta_mode) {
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return ORACLE_BAD_ARG;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0) return ORACLE_BAD_ARG;
  if (input_mode != 0 && input_mode != 1) return ORACLE_BAD_ARG;
  if (delta_mode != 0 && delta_mode != 1) return ORACLE_BAD_ARG;
  if (delta_mode == 1 && (!dt_bias || !d_dt_bias)) return ORACLE_BAD_ARG;
  if ((D && !dD) || (z && !dz)) return ORACLE_BAD_ARG;
  const int64_t N = d_state;
  for (int64_t i = 0; i < d_inner * N; ++i) dA[i] = 0.0;
  for (int64_t i = 0; i < batch * seqlen * N; ++i) dB[i] = dC[i] = 0.0;
  for (int64_t i = 0; i < d_inner; ++i) {
    if (dD) dD[i] = 0.0;
    if (d_dt_bias) d_dt_bias[i] = 0.0;
  }
  /* hs[(t+1)*N + n] = h_t[n], with hs[0..N) = h_{-1} = h0. */
  double* hs = (double*)malloc((size_t)(seqlen + 1) * (size_t)N * sizeof(double));
  double* lam = (double*)malloc((size_t)N * sizeof(double));
  if (!hs || !lam) {
    free(hs);
    free(lam);
    return ORACLE_BAD_ARG;
  }
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < d_inner; ++d) {
      const double* Arow = A + d * N;
      const double bias = dt_bias ? dt_bias[d] : 0.0;
      const double Dv = D ? D[d] : 0.0;
      /* Forward, keeping every state. */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * d_inner + d) * N + n] : 0.0;
      for (int64_t t = 0; t < seqlen; ++t) {
        const int64_t io = (b * seqlen + t) * d_inner + d;
        double dt = delta[io];
        if (delta_mode == 1) dt = oracle_softplus(dt + bias);
        const double xv = x[io];
        const double* Bt = B + (b * seqlen + t) * N;
        for (int64_t n = 0; n < N; ++n) {
          double a = Arow[n];
          double coef = (input_mode == 1) ? ((a != 0.0) ? expm1(dt * a) / a : dt) : dt;
          hs[(t + 1) * N + n] = exp(dt * a) * hs[t * N + n] + coef * Bt[n] * xv;
        }
      }
      /* Backward. */
      for (int64_t n = 0; n < N; ++n) lam[n] = dh_last ? dh_last[(b * d_inner + d) * N + n] : 0.0;
      for (int64_t t = seqlen - 1; t >= 0; --t) {
        const int64_t io = (b * seqlen + t) * d_inner + d;
        const double raw = delta[io];
        const double dt = (delta_mode == 1) ? oracle_softplus(raw + bias) : raw;
        const double xv = x[io];
        const double* Bt = B + (b * seqlen + t) * N;
        const double* Ct = C + (b * seqlen + t) * N;
        const double* ht = hs + (t + 1) * N;
        const double* hp = hs + t * N;
        double ypre = Dv * xv;
        for (int64_t n = 0; n < N; ++n) ypre += Ct[n] * ht[n];
        double g = dy[io];
        if (z) {
          const double zv = z[io];
          const double sg = 1.0 / (1.0 + exp(-zv));
          g = dy[io] * zv * sg;
          dz[io] = dy[io] * ypre * sg * (1.0 + zv * (1.0 - sg));
        }
        if (dD) dD[d] += g * xv;
        double dxv = g * Dv;
        double ddt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double a = Arow[n];
          const double abar = exp(dt * a);
          double coef, dcoef_ddt, dcoef_da;
          if (input_mode == 1) {
            coef = (a != 0.0) ? expm1(dt * a) / a : dt;
            dcoef_ddt = abar;
            dcoef_da = oracle_dcoef_da(dt, a);
          } else {
            coef = dt;
            dcoef_ddt = 1.0;
            dcoef_da = 0.0;
          }
          lam[n] += g * Ct[n];
          dC[(b * seqlen + t) * N + n] += g * ht[n];
          ddt += lam[n] * (a * abar * hp[n] + dcoef_ddt * Bt[n] * xv);
          dA[d * N + n] += lam[n] * (dt * abar * hp[n] + dcoef_da * Bt[n] * xv);
          dB[(b * seqlen + t) * N + n] += lam[n] * coef * xv;
          dxv += lam[n] * coef * Bt[n];
          lam[n] *= abar;
        }
        dx[io] = dxv;
        if (delta_mode == 1) {
          const double sg = 1.0 / (1.0 + exp(-(raw + bias)));
          ddelta[io] = ddt * sg;
          d_dt_bias[d] += ddt * sg;
        } else {
          ddelta[io] = ddt;
        }
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * d_inner + d) * N + n] = lam[n];
    }
  }
  free(hs);
  free(lam);
  return ORACLE_OK;
}

/*
 * Mamba-2 style scan with a scalar decay per head (the SSD form).
 * "Deriving and implementing Mamba from scratch" (dpshk.com/news/3333417),
 * section 6.1: when A is a scalar per step the scan is y = M x with the
 * lower-triangular M[k,i] = c_k (prod_{j=i+1..k} a_j) b_i, whose rank is
 * bounded by the state size; section 6.2: A is a scalar, and groups of heads
 * share B and C (like grouped-query attention).  "SSMs for long-document QA"
 * (pwwt.cn/news/5168881), section 2.3: multi-head SSM, the state split over
 * heads.  Per batch row b, head h (group g = h / (nheads / ngroups)),
 * channel p of the head and state n:
 *     a        = exp(dt[b,t,h] * A[h])
 *     H[p,n]   = a * H[p,n] + dt[b,t,h] * B[b,t,g,n] * x[b,t,h,p]
 *     y[b,t,h,p] = (sum_n C[b,t,g,n] * H[p,n] + D[h] * x[b,t,h,p]) * silu(z[b,t,h,p])
 * (the input term dt*B follows the Mamba convention Bbar = delta*B).
 *   x, z, y : [batch][seqlen][nheads][headdim]
 *   dt      : [batch][seqlen][nheads] (delta_mode 1: softplus(dt + dt_bias[h]))
 *   A, D, dt_bias : [nheads]   (D, z nullable)
 *   B, C    : [batch][seqlen][ngroups][d_state]
 *   h0, h_last : [batch][nheads][headdim][d_state] (nullable)
 */
int ssm_oracle_ssd_f64(const double* x, const double* dt, const double* A, const double* B, const double* C,
                       const double* D, const double* z, const double* h0, const double* dt_bias, double* y,
                       double* h_last, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t ngroups, int64_t d_state, int delta_mode) {
  if (!x || !dt || !A || !B || !C || !y) return ORACLE_BAD_ARG;
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || ngroups <= 0 || d_state <= 0) return ORACLE_BAD_ARG;
  if (nheads % ngroups != 0) return ORACLE_BAD_ARG;
  if (delta_mode != 0 && delta_mode != 1) return ORACLE_BAD_ARG;
  if (delta_mode == 1 && !dt_bias) return ORACLE_BAD_ARG;
  const int64_t N = d_state, P = headdim, HP = nheads * headdim;
  double* state = (double*)malloc((size_t)N * sizeof(double));
  if (!state) return ORACLE_BAD_ARG;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < nheads; ++h) {
      const int64_t g = h / (nheads / ngroups);
      for (int64_t p = 0; p < P; ++p) {
        for (int64_t n = 0; n < N; ++n) state[n] = h0 ? h0[((b * nheads + h) * P + p) * N + n] : 0.0;
        for (int64_t t = 0; t < seqlen; ++t) {
          double d = dt[(b * seqlen + t) * nheads + h];
          if (delta_mode == 1) d = oracle_softplus(d + dt_bias[h]);
          const double a = exp(d * A[h]);
          const int64_t io = (b * seqlen + t) * HP + h * P + p;
          const double xv = x[io];
          const double* Bt = B + ((b * seqlen + t) * ngroups + g) * N;
          const double* Ct = C + ((b * seqlen + t) * ngroups + g) * N;
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            state[n] = a * state[n] + d * Bt[n] * xv;
            acc += Ct[n] * state[n];
          }
          double yv = acc + (D ? D[h] : 0.0) * xv;
          if (z) {
            const double zv = z[io];
            yv = yv * (zv / (1.0 + exp(-zv)));
          }
          y[io] = yv;
        }
        if (h_last)
          for (int64_t n = 0; n < N; ++n) h_last[((b * nheads + h) * P + p) * N + n] = state[n];
      }
    }
  }
  free(state);
  return ORACLE_OK;
}

int ssm_oracle_version(void) { return 4; }
