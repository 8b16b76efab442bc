/*
 * Plain fp64 CPU oracle of the Mamba-2 SSD scan (state-space duality layer's
 * recurrence with a scalar decay per head).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product (the HIP
 * library) never calls it, links it or shares code with it.
 *
 * What it computes (niverel-mamba 0.1.0 PKG-INFO, "The weight contract": per
 * head one dt_bias, one A_log and one D; heads of headdim 64; B and C shared
 * by the ngroups groups of heads; "What is *not* promised": the chunked
 * evaluation decays by exp(cs_l - cs_s) over a cumulative sum of the step's
 * log-decay; "Autoregressive decoding": step returns the new state). Per batch
 * row b and head h (group g = h / (nheads / ngroups)), with a state matrix
 * S[p][n] (headdim x d_state):
 *   delta   = softplus(dt[b,t,h] + dt_bias[h])
 *   S[p][n] = exp(delta * A[h]) * S[p][n] + delta * x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] * S[p][n] + D[h] * x[b,t,h,p]
 * i.e. the selective-scan recurrence of calm-mamba 0.1.4 PKG-INFO ("Mamba
 * operator", step 5: decay exp(delta A), input delta B x, readout C.h + D x)
 * with A a scalar per head and x a headdim-vector. S starts from the given
 * state (zeros when absent) and its final value is returned.
 *
 * Evaluated sequentially in t, in double precision, with the C library's
 * exp/log1p; there is no chunking, fusion or reordering.
 *
 * Layouts (row-major, all double):
 *   x, y        [batch][seqlen][nheads][headdim]
 *   dt          [batch][seqlen][nheads]
 *   Bm, Cm      [batch][seqlen][ngroups][d_state]
 *   dt_bias, A, Dskip   [nheads]
 *   state       [batch][nheads][headdim][d_state]
 *
 * Packed documents (oracle_ssd_fwd_seq): a change of the document id resets
 * the state (niverel-mamba 0.1.0 PKG-INFO, "seq_idx strict reset").
 *
 * Pins (tests/test_ssd_oracle.py): the quadratic dual form written with numpy
 * (y_t = sum_{s<=t} (C_t.B_s) exp(sum_{s<r<=t} delta_r A) delta_s x_s + D x_t,
 * non-recursive); A = 0 reduces to a prefix sum; delta = 0 to y = C.S0 + D x;
 * a one-head, one-state case against scipy.signal.lfilter; step^L == fwd;
 * split/resume; packed documents == each document run on its own; and planted
 * mistakes in copies of this file that must fail.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(v) = log(1 + e^v) = max(v,0) + log1p(e^-|v|). */
static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

int oracle_ssd_abi_version(void) { return 1; }

/* Whole sequence, optionally over packed documents: with seq_idx
   ([batch][seqlen] document ids) the state restarts from zero before every
   step whose id differs from the previous step's (niverel-mamba 0.1.0
   PKG-INFO, "seq_idx strict reset"). state_in / state_out may be NULL (zeros /
   not written). Returns 0, or -1 when the shape is invalid. */
static int ssd_fwd_impl(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                        int64_t ngroups, const double* x, const double* dt, const double* Bm, const double* Cm,
                        const int32_t* seq_idx, const double* dt_bias, const double* A, const double* Dskip,
                        const double* state_in, double* y, double* state_out, int nthreads) {
  if (batch < 1 || seqlen < 0 || nheads < 1 || headdim < 1 || d_state < 1 || ngroups < 1 ||
      nheads % ngroups != 0)
    return -1;
  const int64_t HP = nheads * headdim, GN = ngroups * d_state, PN = headdim * d_state;
  const int64_t heads_per_group = nheads / ngroups;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < nheads; ++h) {
      const int64_t g = h / heads_per_group;
      double* S = (double*)malloc((size_t)PN * sizeof(double));
      const double* s0 = state_in ? state_in + (b * nheads + h) * PN : NULL;
      for (int64_t i = 0; i < PN; ++i) S[i] = s0 ? s0[i] : 0.0;
      for (int64_t t = 0; t < seqlen; ++t) {
        if (seq_idx && t > 0 && seq_idx[b * seqlen + t] != seq_idx[b * seqlen + t - 1]) {
          for (int64_t i = 0; i < PN; ++i) S[i] = 0.0;
        }
        const double delta = softplus(dt[(b * seqlen + t) * nheads + h] + dt_bias[h]);
        const double decay = exp(delta * A[h]);
        const double* xt = x + (b * seqlen + t) * HP + h * headdim;
        const double* Bt = Bm + (b * seqlen + t) * GN + g * d_state;
        const double* Ct = Cm + (b * seqlen + t) * GN + g * d_state;
        double* yt = y + (b * seqlen + t) * HP + h * headdim;
        for (int64_t p = 0; p < headdim; ++p) {
          double* Sp = S + p * d_state;
          double acc = 0.0;
          for (int64_t n = 0; n < d_state; ++n) {
            Sp[n] = decay * Sp[n] + delta * xt[p] * Bt[n];
            acc += Ct[n] * Sp[n];
          }
          yt[p] = acc + Dskip[h] * xt[p];
        }
      }
      if (state_out) memcpy(state_out + (b * nheads + h) * PN, S, (size_t)PN * sizeof(double));
      free(S);
    }
  }
  return 0;
}

int oracle_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                   int64_t ngroups, const double* x, const double* dt, const double* Bm, const double* Cm,
                   const double* dt_bias, const double* A, const double* Dskip, const double* state_in,
                   double* y, double* state_out, int nthreads) {
  return ssd_fwd_impl(batch, seqlen, nheads, headdim, d_state, ngroups, x, dt, Bm, Cm, NULL, dt_bias, A, Dskip,
                      state_in, y, state_out, nthreads);
}

int oracle_ssd_fwd_seq(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                       int64_t ngroups, const double* x, const double* dt, const double* Bm, const double* Cm,
                       const int32_t* seq_idx, const double* dt_bias, const double* A, const double* Dskip,
                       const double* state_in, double* y, double* state_out, int nthreads) {
  if (!seq_idx) return -1;
  return ssd_fwd_impl(batch, seqlen, nheads, headdim, d_state, ngroups, x, dt, Bm, Cm, seq_idx, dt_bias, A, Dskip,
                      state_in, y, state_out, nthreads);
}

/* One token per batch row: x [batch][nheads][headdim], dt [batch][nheads],
   Bm, Cm [batch][ngroups][d_state]; state_in and state_out are required and
   may be the same array. Written separately from oracle_ssd_fwd, so that a
   chain of steps reproducing the sequence is a test, not a tautology. */
int oracle_ssd_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t d_state, int64_t ngroups,
                    const double* x, const double* dt, const double* Bm, const double* Cm, const double* dt_bias,
                    const double* A, const double* Dskip, const double* state_in, double* y, double* state_out) {
  if (batch < 1 || nheads < 1 || headdim < 1 || d_state < 1 || ngroups < 1 || nheads % ngroups != 0 ||
      !state_in || !state_out)
    return -1;
  const int64_t per_group = nheads / ngroups;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < nheads; ++h) {
      const double v = dt[b * nheads + h] + dt_bias[h];
      const double step = v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
      const double keep = exp(A[h] * step);
      const double* Bv = Bm + (b * ngroups + h / per_group) * d_state;
      const double* Cv = Cm + (b * ngroups + h / per_group) * d_state;
      for (int64_t p = 0; p < headdim; ++p) {
        const double xv = x[(b * nheads + h) * headdim + p];
        const int64_t base = ((b * nheads + h) * headdim + p) * d_state;
        double out = Dskip[h] * xv;
        for (int64_t n = 0; n < d_state; ++n) {
          const double s_new = keep * state_in[base + n] + step * Bv[n] * xv;
          state_out[base + n] = s_new;
          out += Cv[n] * s_new;
        }
        y[(b * nheads + h) * headdim + p] = out;
      }
    }
  }
  return 0;
}
