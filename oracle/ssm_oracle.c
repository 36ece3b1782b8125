/*
 * ssm_oracle.c -- plain fp64 CPU oracle for the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU kernels are
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP library, and it is never a fallback for it.
 *
 * Sources (the pages this follows; page titles as printed on them):
 *  [xw]  "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 *        (ai.xwebgame.com/papers/mamba), section on what an SSM is: the pair
 *        h_t = A h_{t-1} + B x_t, y_t = C h_t + D x_t.
 *  [fs]  fsdata.site article "mamba-state-space-model", section 3.2: the
 *        selective step -- dt = softplus(.), A_bar = exp(dt*A),
 *        B_bar = dt*B, h_new = A_bar*h + B_bar*x, y = C.h_new + D*x.
 *  [fg]  "Mamba: 基于选择状态空间的线性时间序列模型" (freeguideonline.com),
 *        section 2.2 (ZOH discretisation), section 4.2 step 2 (softplus with
 *        a bias inside), section 4.3 (channels are independent SSMs),
 *        section 5.1 (the scan reproduces the sequential recurrence).
 *  [xw-code] same page as [xw], "run it with PyTorch" section: the block
 *        gates the SSM output by SiLU of the second projection branch.
 *
 * What is computed (per batch b, channel d, state n; all in double):
 *   x      = delta[b,d,t] + bias[d]
 *   dt     = softplus(x) = max(x,0) + log1p(exp(-|x|))
 *   Abar   = exp(dt * A[d,n])
 *   Bbar   = dt * B[b,n,t]                       (default)
 *          = (exp(dt*A) - 1) / A * B[b,n,t]      (ZOH flag; dt*B when A == 0; evaluated as
 *                                                expm1(dt*A) / A, which keeps its digits as dt*A -> 0)
 *   h[n]   = Abar * h[n] + Bbar * u[b,d,t]
 *   y      = sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]   (h after the update)
 *   out    = y * z / (1 + exp(-z))               (when z is given)
 *   final_state[b,d,n] = h after the last processed step.
 * With the REVERSE flag, t runs from L-1 down to 0 (a backward-in-time SSM).
 * The initial state is zero unless h0 is given.
 *
 * Layouts (row-major, contiguous):
 *   u, delta, z, out : [Bsz, Dm, L]     B, C : [Bsz, N, L]
 *   A : [Dm, N]   D, bias : [Dm]   h0, final_state : [Bsz, Dm, N]
 *
 * The backward pass (oracle_scan_bwd_f64) is not described on the pages; it is
 * the chain rule applied to the forward definition above, written as the
 * reverse-time adjoint recurrence (see the comment on that function).
 *
 * The step that produces u (oracle_conv1d_f64) follows the block of [xw-code]:
 * a depthwise 1-D convolution of width K over time with K-1 zeros of padding
 * on the left, its output cut to the first L steps (so step t only sees steps
 * t-K+1 .. t), a per-channel bias, then SiLU.  Like the page's nn.Conv1d it
 * is a cross-correlation: weight tap k multiplies the input K-1-k steps back.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ZOH 1
#define ORACLE_REVERSE 2

static double softplus_f64(double x) {
  /* stable form of log(1 + exp(x)) */
  return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

static double silu_f64(double z) { return z / (1.0 + exp(-z)); }

/* Zero-order hold (freeguideonline tutorial, section 2.2): B_bar = e B with
   e = (exp(dt A) - 1) / A, taken as expm1(dt A) / A so that it keeps its digits as dt A -> 0.
   Its derivative in A, de/dA = (dt exp(dt A) - e) / A, cancels there; for |dt A| < 1e-2 it is
   taken from its Taylor series dt^2 sum_k (k + 1) (dt A)^k / (k + 2)!, whose terms past k = 6
   are below the fp64 rounding level (at A = 0 the series is the limit dt^2 / 2). */
static double zoh_e_dA_f64(double dt, double an, double a, double e) {
  const double x = dt * an;
  if (fabs(x) < 1e-2) {
    double s = 0.0, f = 2.0, p = 1.0; /* f = (k + 2)!, p = x^k */
    for (int k = 0; k <= 6; ++k) {
      s += (k + 1) * p / f;
      p *= x;
      f *= (k + 3);
    }
    return dt * dt * s;
  }
  return (dt * a - e) / an;
}

int oracle_abi_version(void) { return 5; }

/* Threads an OpenMP region of the oracle uses by default (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for one call: nthreads if positive, else the OpenMP default.  Passed to each parallel
 * region, so a call never changes the count later calls use. */
static int team_size(int nthreads) { return nthreads > 0 ? nthreads : oracle_max_threads(); }

/* Returns 0 on success, -1 on bad arguments. nthreads <= 0 uses the OpenMP default. */
int oracle_scan_f64(int64_t Bsz, int64_t Dm, int64_t N, int64_t L,
                    const double* u, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dv,
                    const double* z, const double* bias, const double* h0,
                    double* out, double* final_state, int flags, int nthreads) {
  if (Bsz < 0 || Dm < 0 || N <= 0 || L < 0) return -1;
  if (!u || !delta || !A || !Bm || !Cm || !out) return -1;
  const int64_t rows = Bsz * Dm;
  const int nt = team_size(nthreads);
  (void)nt;  /* unused without OpenMP */
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t b = r / Dm, d = r % Dm;
    double* h = (double*)malloc((size_t)N * sizeof(double));
    if (!h) { bad = 1; continue; }
    for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[r * N + n] : 0.0;
    const double* ur = u + r * L;
    const double* dr = delta + r * L;
    const double* zr = z ? z + r * L : NULL;
    double* yr = out + r * L;
    const double* Ab = Bm + b * N * L;
    const double* Cb = Cm + b * N * L;
    for (int64_t s = 0; s < L; ++s) {
      const int64_t t = (flags & ORACLE_REVERSE) ? (L - 1 - s) : s;
      const double dt = softplus_f64(dr[t] + (bias ? bias[d] : 0.0));
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double a_dn = A[d * N + n];
        const double abar = exp(dt * a_dn);
        double bbar;
        if ((flags & ORACLE_ZOH) && a_dn != 0.0)
          bbar = expm1(dt * a_dn) / a_dn * Ab[n * L + t];
        else
          bbar = dt * Ab[n * L + t];
        h[n] = abar * h[n] + bbar * ur[t];
        acc += Cb[n * L + t] * h[n];
      }
      double y = acc + (Dv ? Dv[d] : 0.0) * ur[t];
      if (zr) y *= silu_f64(zr[t]);
      yr[t] = y;
    }
    if (final_state)
      for (int64_t n = 0; n < N; ++n) final_state[r * N + n] = h[n];
    free(h);
  }
  return bad ? -1 : 0;
}

/* One generation step: the scan body with L = 1, state read and written in place.
 * u, delta, z, out : [Bsz, Dm]; B, C : [Bsz, N]; state : [Bsz, Dm, N]. */
int oracle_step_f64(int64_t Bsz, int64_t Dm, int64_t N, double* state,
                    const double* u, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dv,
                    const double* z, const double* bias, double* out, int flags,
                    int nthreads) {
  if (Bsz < 0 || Dm < 0 || N <= 0 || !state || !u || !delta || !A || !Bm || !Cm || !out)
    return -1;
  const int64_t rows = Bsz * Dm;
  const int nt = team_size(nthreads);
  (void)nt;  /* unused without OpenMP */
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t b = r / Dm, d = r % Dm;
    const double dt = softplus_f64(delta[r] + (bias ? bias[d] : 0.0));
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a_dn = A[d * N + n];
      const double abar = exp(dt * a_dn);
      double bbar;
      if ((flags & ORACLE_ZOH) && a_dn != 0.0)
        bbar = expm1(dt * a_dn) / a_dn * Bm[b * N + n];
      else
        bbar = dt * Bm[b * N + n];
      double* h = state + r * N + n;
      *h = abar * *h + bbar * u[r];
      acc += Cm[b * N + n] * *h;
    }
    double y = acc + (Dv ? Dv[d] : 0.0) * u[r];
    if (z) y *= silu_f64(z[r]);
    out[r] = y;
  }
  return 0;
}

/* Causal depthwise convolution + bias + SiLU (the block's step 2 in [xw-code]).
 *   x, u            : [Bsz, Dm, L]
 *   w               : [Dm, K]    tap k weighs input step t - (K-1) + k
 *   bias            : [Dm] or NULL (zero)
 *   state_in        : [Bsz, Dm, K-1] or NULL (zeros): the K-1 inputs before x,
 *                     oldest first, so a sequence can be processed in pieces
 *   state_out       : [Bsz, Dm, K-1] or NULL: the last K-1 inputs of the
 *                     sequence state_in followed by x, oldest first
 *   u[t] = silu(bias + sum_k w[k] * xe[t + k]), xe = state_in followed by x. */
int oracle_conv1d_f64(int64_t Bsz, int64_t Dm, int64_t L, int64_t K,
                      const double* x, const double* w, const double* bias,
                      const double* state_in, double* u, double* state_out,
                      int nthreads) {
  if (Bsz < 0 || Dm < 0 || L < 0 || K < 1 || !x || !w || !u) return -1;
  const int64_t rows = Bsz * Dm, H = K - 1;
  const int nt = team_size(nthreads);
  (void)nt;  /* unused without OpenMP */
  int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t d = r % Dm;
    double* xe = (double*)malloc((size_t)(H + L + 1) * sizeof(double));
    if (!xe) { bad = 1; continue; }
    for (int64_t j = 0; j < H; ++j) xe[j] = state_in ? state_in[r * H + j] : 0.0;
    for (int64_t t = 0; t < L; ++t) xe[H + t] = x[r * L + t];
    for (int64_t t = 0; t < L; ++t) {
      double v = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < K; ++k) v += w[d * K + k] * xe[t + k];
      u[r * L + t] = silu_f64(v);
    }
    if (state_out)
      for (int64_t j = 0; j < H; ++j) state_out[r * H + j] = xe[L + j];
    free(xe);
  }
  return bad ? -1 : 0;
}

/* Gradients of the scan (either discretisation, either direction) for a given output
 * gradient dout [Bsz,Dm,L] and optional final-state gradient dfs [Bsz,Dm,N].  Derived
 * with the chain rule from the forward definition.  Write B_bar = e * B, so e = dt by
 * default and e = (Abar - 1) / A under ZOH (dt when A == 0); then de/ddt = 1 by default
 * and Abar under ZOH, de/dA = 0 by default and (dt Abar - e) / A under ZOH (dt^2 / 2 at
 * A == 0, the limit).  With G_n the gradient reaching h_n after step t (time order of the
 * scan):
 *   dy_t   = dout_t * silu(z_t)                     (dout_t without z)
 *   dz_t   = dout_t * y_t * s(z_t) * (1 + z_t (1 - s(z_t))),  s = logistic
 *   G_n   += dy_t * C[n,t];   dC[b,n,t] += dy_t * h_t[n]
 *   du_t   = dy_t * D + sum_n G_n * e * B[n,t]
 *   dD    += dy_t * u_t
 *   ddt_t  = sum_n G_n * (h_{t-1}[n] * Abar * A[n] + de/ddt * u_t * B[n,t])
 *   dA[n] += G_n * (h_{t-1}[n] * Abar * dt_t + de/dA * u_t * B[n,t])
 *   dB[b,n,t] += G_n * e * u_t
 *   G_n    = G_n * Abar                             (on to h_{t-1})
 *   ddelta_t = ddt_t * s(x_t)   (softplus' = logistic);  dbias += ddelta_t
 *   dh0 = G after step 0 of the scan order.
 * Outputs: du, ddelta : [Bsz,Dm,L]; dz : [Bsz,Dm,L] (only when z is given);
 * dA : [Dm,N]; dB, dC : [Bsz,N,L]; dD, dbias : [Dm] (may be NULL); dh0 : [Bsz,Dm,N]
 * (may be NULL).  Sums over channels and batch rows are taken in a fixed order. */
int oracle_scan_bwd_f64(int64_t Bsz, int64_t Dm, int64_t N, int64_t L,
                        const double* u, const double* delta, const double* A,
                        const double* Bm, const double* Cm, const double* Dv,
                        const double* z, const double* bias, const double* h0,
                        const double* dout, const double* dfs,
                        double* du, double* ddelta, double* dA, double* dB, double* dC,
                        double* dD, double* dz, double* dbias, double* dh0,
                        int flags, int nthreads) {
  if (Bsz < 0 || Dm < 0 || N <= 0 || L < 0) return -1;
  if (!u || !delta || !A || !Bm || !Cm || !dout || !du || !ddelta || !dA || !dB || !dC) return -1;
  if (z && !dz) return -1;
  const int zoh = (flags & ORACLE_ZOH) != 0;
  const int64_t rows = Bsz * Dm;
  const int nt = team_size(nthreads);
  (void)nt;  /* unused without OpenMP */
  /* per-row contributions to the channel and batch sums, reduced afterwards in row order */
  double* rA = (double*)calloc((size_t)(rows * N), sizeof(double));
  double* rD = (double*)calloc((size_t)rows, sizeof(double));
  double* rb = (double*)calloc((size_t)rows, sizeof(double));
  if (!rA || !rD || !rb) { free(rA); free(rD); free(rb); return -1; }
  for (int64_t i = 0; i < Bsz * N * L; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
  int bad = 0;
  /* channels are taken in fixed chunks of CH; each chunk sums its channels' dB/dC
   * contributions in channel order into its own slab, and the slabs are added in chunk
   * order, so the result does not depend on the number of threads */
  const int64_t CH = 64;
  const int64_t nch = (Dm + CH - 1) / CH;
  double* slab = (double*)malloc((size_t)(nch > 0 ? nch : 1) * (size_t)(2 * N * (L > 0 ? L : 1)) * sizeof(double));
  if (!slab) { free(rA); free(rD); free(rb); return -1; }
  for (int64_t b = 0; b < Bsz && !bad; ++b) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t c = 0; c < nch; ++c) {
      double* sB = slab + c * 2 * N * L;
      double* sC = sB + N * L;
      for (int64_t i = 0; i < N * L; ++i) { sB[i] = 0.0; sC[i] = 0.0; }
      double* hs = (double*)malloc((size_t)((L + 1) * N) * sizeof(double)); /* state before each step */
      double* ys = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
      double* G = (double*)malloc((size_t)N * sizeof(double));
      if (!hs || !ys || !G) { bad = 1; free(hs); free(ys); free(G); continue; }
      for (int64_t d = c * CH; d < Dm && d < (c + 1) * CH; ++d) {
        const int64_t r = b * Dm + d;
        const double* ur = u + r * L;
        const double* dr = delta + r * L;
        const double* zr = z ? z + r * L : NULL;
        const double* Ab = Bm + b * N * L;
        const double* Cb = Cm + b * N * L;
        const double bd = bias ? bias[d] : 0.0;
        const double Dd = Dv ? Dv[d] : 0.0;
        /* forward, keeping every state: hs[s*N + n] is the state before scan step s */
        for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[r * N + n] : 0.0;
        for (int64_t s = 0; s < L; ++s) {
          const int64_t t = (flags & ORACLE_REVERSE) ? (L - 1 - s) : s;
          const double dt = softplus_f64(dr[t] + bd);
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            const double an = A[d * N + n];
            const double a = exp(dt * an);
            const double e = (zoh && an != 0.0) ? expm1(dt * an) / an : dt;
            const double h = a * hs[s * N + n] + e * Ab[n * L + t] * ur[t];
            hs[(s + 1) * N + n] = h;
            acc += Cb[n * L + t] * h;
          }
          ys[t] = acc + Dd * ur[t];
        }
        /* backward in reverse scan order */
        for (int64_t n = 0; n < N; ++n) G[n] = dfs ? dfs[r * N + n] : 0.0;
        double accD = 0.0, accb = 0.0;
        for (int64_t s = L - 1; s >= 0; --s) {
          const int64_t t = (flags & ORACLE_REVERSE) ? (L - 1 - s) : s;
          const double x = dr[t] + bd;
          const double dt = softplus_f64(x);
          double dy = dout[r * L + t];
          if (zr) {
            const double sg = 1.0 / (1.0 + exp(-zr[t]));
            dz[r * L + t] = dout[r * L + t] * ys[t] * sg * (1.0 + zr[t] * (1.0 - sg));
            dy = dout[r * L + t] * silu_f64(zr[t]);
          }
          double dut = dy * Dd;
          double ddt = 0.0;
          accD += dy * ur[t];
          for (int64_t n = 0; n < N; ++n) {
            const double an = A[d * N + n];
            const double a = exp(dt * an);
            const double hp = hs[s * N + n];
            const double e = (zoh && an != 0.0) ? expm1(dt * an) / an : dt;  /* B_bar / B */
            const double e_dt = zoh ? a : 1.0;                             /* de/ddt */
            const double e_dA = !zoh ? 0.0 : zoh_e_dA_f64(dt, an, a, e);
            G[n] += dy * Cb[n * L + t];
            sC[n * L + t] += dy * hs[(s + 1) * N + n];
            dut += G[n] * e * Ab[n * L + t];
            ddt += G[n] * (hp * a * an + e_dt * ur[t] * Ab[n * L + t]);
            rA[r * N + n] += G[n] * (hp * a * dt + e_dA * ur[t] * Ab[n * L + t]);
            sB[n * L + t] += G[n] * e * ur[t];
            G[n] *= a;
          }
          du[r * L + t] = dut;
          const double dx = ddt / (1.0 + exp(-x));
          ddelta[r * L + t] = dx;
          accb += dx;
        }
        rD[r] = accD;
        rb[r] = accb;
        if (dh0)
          for (int64_t n = 0; n < N; ++n) dh0[r * N + n] = G[n];
      }
      free(hs); free(ys); free(G);
    }
    if (!bad)
      for (int64_t c = 0; c < nch; ++c) {
        const double* sB = slab + c * 2 * N * L;
        const double* sC = sB + N * L;
        for (int64_t i = 0; i < N * L; ++i) {
          dB[b * N * L + i] += sB[i];
          dC[b * N * L + i] += sC[i];
        }
      }
  }
  free(slab);
  if (!bad) {
    for (int64_t d = 0; d < Dm; ++d) {
      for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        for (int64_t b = 0; b < Bsz; ++b) s += rA[(b * Dm + d) * N + n];
        dA[d * N + n] = s;
      }
      double sD = 0.0, sb = 0.0;
      for (int64_t b = 0; b < Bsz; ++b) { sD += rD[b * Dm + d]; sb += rb[b * Dm + d]; }
      if (dD) dD[d] = sD;
      if (dbias) dbias[d] = sb;
    }
  }
  free(rA); free(rD); free(rb);
  return bad ? -1 : 0;
}
