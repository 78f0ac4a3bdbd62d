/*
 * Plain fp64 CPU oracle for the selective scan (S6): TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg may load this file's library. The GPU path never calls it and shares no
 * code with it.
 *
 * Forward: the reference function `selective_scan_ref` on the page "Vision
 * Mamba structure and principle / code implementation" (freeymw.com, section 2):
 *   delta <- delta + delta_bias ; delta <- softplus(delta) when requested
 *   h <- 0 ; for every step t:  h[n] <- exp(delta_t*A[d,n])*h[n] + delta_t*B[g,n,t]*u_t
 *                               y_t  <- sum_n C[g,n,t]*h[n]
 *   out <- y + D*u ; out <- out*silu(z) when z is given
 * with channel d reading B/C group g = d / (dim/ngroups) (the "B G N L -> B (G H) N L"
 * repeat in that function).  Everything is carried out in double precision, one
 * row (b, d) at a time, in the order of the definition.
 *
 * Backward: the exact gradient of that forward map, obtained by running the
 * adjoint (reverse) recurrence in fp64; its inputs and outputs follow the
 * `SelectiveScanFn.backward` call on the same page (du, ddelta, dA, dB, dC, dD,
 * ddelta_bias, dz), with ddelta taken w.r.t. the raw delta (before bias and
 * softplus) and dA/dD/ddelta_bias summed over the batch.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>

static double softplus_exact(double x) {
  /* log(1 + e^x) written so that it neither overflows nor loses digits */
  return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * sigmoid(x); }

/* Forward over all rows. Layouts (dense, last index fastest):
 *   u, delta, z, out : (batch, dim, seqlen)
 *   A                : (dim, dstate)
 *   Bm, Cm           : (batch, ngroups, dstate, seqlen)
 *   Dskip, delta_bias: (dim)            (may be NULL)
 *   last_state       : (batch, dim, dstate)   (may be NULL)
 *   ypre             : (batch, dim, seqlen) y + D*u before the gate (may be NULL) */
void oracle_ss_fwd(const double* u, const double* delta, const double* A, const double* Bm,
                   const double* Cm, const double* Dskip, const double* z, const double* delta_bias,
                   int delta_softplus, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                   int64_t ngroups, double* out, double* last_state, double* ypre) {
  const int64_t per_group = dim / ngroups;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t row = 0; row < batch * dim; ++row) {
    const int64_t b = row / dim, d = row % dim, g = d / per_group;
    double* h = (double*)calloc((size_t)dstate, sizeof(double));
    const double* ur = u + row * seqlen;
    const double* dr = delta + row * seqlen;
    const double* Bg = Bm + (b * ngroups + g) * dstate * seqlen;
    const double* Cg = Cm + (b * ngroups + g) * dstate * seqlen;
    for (int64_t t = 0; t < seqlen; ++t) {
      double dt = dr[t];
      if (delta_bias) dt += delta_bias[d];
      if (delta_softplus) dt = softplus_exact(dt);
      double y = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        const double a = exp(dt * A[d * dstate + n]);
        h[n] = a * h[n] + dt * Bg[n * seqlen + t] * ur[t];
        y += Cg[n * seqlen + t] * h[n];
      }
      if (Dskip) y += Dskip[d] * ur[t];
      if (ypre) ypre[row * seqlen + t] = y;
      if (z) y *= silu(z[row * seqlen + t]);
      out[row * seqlen + t] = y;
    }
    if (last_state)
      for (int64_t n = 0; n < dstate; ++n) last_state[row * dstate + n] = h[n];
    free(h);
  }
}

/* Backward.  Gradient outputs (all overwritten, never accumulated into):
 *   du, ddelta, dz      : (batch, dim, seqlen)       (dz only when z != NULL)
 *   dA                  : (dim, dstate)
 *   dBm, dCm            : (batch, ngroups, dstate, seqlen)
 *   dDskip, ddelta_bias : (dim)                       (when the input exists)
 * Parallel over (b, g) so that the sums over the channels of a group (dB, dC)
 * and over the batch (dA, dD, ddelta_bias) are formed without races: each
 * (b, g) task writes its own slice of per-batch partials, summed at the end. */
void oracle_ss_bwd(const double* u, const double* delta, const double* A, const double* Bm,
                   const double* Cm, const double* Dskip, const double* z, const double* delta_bias,
                   int delta_softplus, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                   int64_t ngroups, const double* dout, double* du, double* ddelta, double* dA,
                   double* dBm, double* dCm, double* dDskip, double* dz, double* ddelta_bias) {
  const int64_t per_group = dim / ngroups;
  const int64_t L = seqlen, N = dstate;
  double* dA_part = (double*)calloc((size_t)(batch * dim * N), sizeof(double));
  double* dD_part = (double*)calloc((size_t)(batch * dim), sizeof(double));
  double* db_part = (double*)calloc((size_t)(batch * dim), sizeof(double));
  memset(dBm, 0, sizeof(double) * (size_t)(batch * ngroups * N * L));
  memset(dCm, 0, sizeof(double) * (size_t)(batch * ngroups * N * L));
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bg = 0; bg < batch * ngroups; ++bg) {
    const int64_t b = bg / ngroups, g = bg % ngroups;
    const double* Bg = Bm + bg * N * L;
    const double* Cg = Cm + bg * N * L;
    double* dBg = dBm + bg * N * L;
    double* dCg = dCm + bg * N * L;
    double* H = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N)); /* H[(t+1)*N+n] = h_t, H[n] = h_{-1} = 0 */
    double* dts = (double*)malloc(sizeof(double) * (size_t)L);
    double* ypre = (double*)malloc(sizeof(double) * (size_t)L);
    double* lam = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t d = g * per_group; d < (g + 1) * per_group; ++d) {
      const int64_t row = b * dim + d;
      const double* ur = u + row * L;
      const double* dr = delta + row * L;
      const double* Ad = A + d * N;
      /* forward again, keeping every state */
      for (int64_t n = 0; n < N; ++n) H[n] = 0.0;
      for (int64_t t = 0; t < L; ++t) {
        double dt = dr[t];
        if (delta_bias) dt += delta_bias[d];
        if (delta_softplus) dt = softplus_exact(dt);
        dts[t] = dt;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double h = exp(dt * Ad[n]) * H[t * N + n] + dt * Bg[n * L + t] * ur[t];
          H[(t + 1) * N + n] = h;
          y += Cg[n * L + t] * h;
        }
        if (Dskip) y += Dskip[d] * ur[t];
        ypre[t] = y;
      }
      /* reverse (adjoint) recurrence */
      for (int64_t n = 0; n < N; ++n) lam[n] = 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const double g_out = dout[row * L + t];
        double dy;
        if (z) {
          const double zz = z[row * L + t];
          const double s = sigmoid(zz);
          dy = g_out * zz * s;                                 /* d out / d ypre = silu(z) */
          dz[row * L + t] = g_out * ypre[t] * s * (1.0 + zz * (1.0 - s));  /* silu'(z) */
        } else {
          dy = g_out;
        }
        const double dt = dts[t];
        double lamB = 0.0, ddt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          /* lambda_t = C_t dy_t + a_{t+1} lambda_{t+1}; lam[] holds a_{t+1} lambda_{t+1} */
          const double l = lam[n] + Cg[n * L + t] * dy;
          const double a = exp(dt * Ad[n]);
          const double hprev = H[t * N + n];
          lamB += l * Bg[n * L + t];
          ddt += l * (Ad[n] * a * hprev + Bg[n * L + t] * ur[t]);
          dA_part[row * N + n] += l * a * hprev * dt;
          dBg[n * L + t] += l * dt * ur[t];
          dCg[n * L + t] += dy * H[(t + 1) * N + n];
          lam[n] = a * l;
        }
        du[row * L + t] = dt * lamB + (Dskip ? Dskip[d] * dy : 0.0);
        dD_part[row] += dy * ur[t];
        double draw = ddt;
        if (delta_softplus) {
          double v = dr[t] + (delta_bias ? delta_bias[d] : 0.0);
          draw *= sigmoid(v); /* softplus' = logistic */
        }
        ddelta[row * L + t] = draw;
        db_part[row] += draw;
      }
    }
    free(H); free(dts); free(ypre); free(lam);
  }
  for (int64_t d = 0; d < dim; ++d) {
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      for (int64_t b = 0; b < batch; ++b) s += dA_part[(b * dim + d) * N + n];
      dA[d * N + n] = s;
    }
    double sd = 0.0, sb = 0.0;
    for (int64_t b = 0; b < batch; ++b) { sd += dD_part[b * dim + d]; sb += db_part[b * dim + d]; }
    if (dDskip) dDskip[d] = sd;
    if (ddelta_bias) ddelta_bias[d] = sb;
  }
  free(dA_part); free(dD_part); free(db_part);
}
