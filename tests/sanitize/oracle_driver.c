/*
 * Sanitizer driver for the fp64 oracle (test infrastructure): runs every
 * oracle entry point on small shapes, including the edge cases (one step,
 * fewer steps than the conv history, no incoming states, packed documents,
 * rejected arguments), under AddressSanitizer and UndefinedBehaviorSanitizer.
 * It checks nothing numerically (the pins do that); it exits 0 when every
 * call returned the expected status, and the sanitizers abort on any memory
 * or undefined-behaviour error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
               const double*, const double*, const double*, const double*, const double*, const double*,
               const double*, const double*, const double*, double*, double*, double*, int);
int oracle_fwd_seq(int64_t, int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                   const double*, const double*, const double*, const double*, const double*, const double*,
                   const double*, const int32_t*, const double*, const double*, double*, double*, double*, int);
int oracle_step(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*, const double*,
                const double*, const double*, const double*, const double*, const double*, const double*,
                const double*, const double*, double*, double*, double*);
int oracle_bwd(int64_t, int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
               const double*, const double*, const double*, const double*, const double*, const double*,
               const double*, const double*, const double*, const double*, double*, double*, double*, double*,
               double*, double*, double*, double*, double*, double*, int);
int oracle_ssd_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double*, const double*,
                   const double*, const double*, const double*, const double*, const double*, const double*,
                   double*, double*, int);
int oracle_ssd_fwd_seq(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double*, const double*,
                       const double*, const double*, const int32_t*, const double*, const double*, const double*,
                       const double*, double*, double*, int);
int oracle_ssd_step(int64_t, int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                    const double*, const double*, const double*, const double*, const double*, double*, double*);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* uniform in [-1, 1), a 64-bit LCG */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_state >> 11) / (double)(1ull << 52) - 1.0;
}
static double* arr(size_t n, double scale, double shift) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = shift + scale * urand();
  return p;
}

static int fails = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++fails;
  }
}

static void mamba1(int64_t B, int64_t L, int64_t D, int64_t N, int with_states) {
  const size_t bld = (size_t)(B * L * D), bln = (size_t)(B * L * N);
  double *x = arr(bld, 1, 0), *dt = arr(bld, 0.1, 0), *z = arr(bld, 1, 0), *Bm = arr(bln, 1, 0), *Cm = arr(bln, 1, 0);
  double *w = arr((size_t)D * 4, 0.5, 0), *cb = arr((size_t)D, 0.1, 0), *db = arr((size_t)D, 1, -4);
  double *Dk = arr((size_t)D, 0.5, 1), *A = arr((size_t)(D * N), 3, -4);
  double *cs = with_states ? arr((size_t)(B * D * 3), 1, 0) : NULL, *ss = with_states ? arr((size_t)(B * D * N), 1, 0) : NULL;
  double *y = arr(bld, 0, 0), *cso = arr((size_t)(B * D * 3), 0, 0), *sso = arr((size_t)(B * D * N), 0, 0);
  expect(oracle_fwd(B, L, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, cs, ss, y, cso, sso, 2), 0, "fwd");
  int32_t* sq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * L));
  for (int64_t i = 0; i < B * L; ++i) sq[i] = (int32_t)((i % L) / 3);
  expect(oracle_fwd_seq(B, L, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, sq, cs, ss, y, cso, sso, 2), 0, "fwd_seq");
  expect(oracle_fwd_seq(B, L, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, NULL, cs, ss, y, cso, sso, 2), -1,
         "fwd_seq without ids");
  /* one step from the prefill's states, in place */
  expect(oracle_step(B, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, cso, sso, y, cso, sso), 0, "step");
  expect(oracle_step(B, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, NULL, sso, y, cso, sso), -1, "step without state");
  double *dy = arr(bld, 1, 0), *g[10];
  const size_t gs[10] = {bld, bld, bld, bln, bln, (size_t)D * 4, (size_t)D, (size_t)D, (size_t)D, (size_t)(D * N)};
  for (int i = 0; i < 10; ++i) g[i] = arr(gs[i], 0, 0);
  expect(oracle_bwd(B, L, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, cs, ss, dy, g[0], g[1], g[2], g[3], g[4], g[5],
                    g[6], g[7], g[8], g[9], 2), 0, "bwd");
  expect(oracle_fwd(0, L, D, N, 4, x, dt, z, Bm, Cm, w, cb, db, Dk, A, cs, ss, y, cso, sso, 2), -1, "fwd batch 0");
  for (int i = 0; i < 10; ++i) free(g[i]);
  free(dy); free(sq);
  free(x); free(dt); free(z); free(Bm); free(Cm); free(w); free(cb); free(db); free(Dk); free(A);
  free(cs); free(ss); free(y); free(cso); free(sso);
}

static void mamba2(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int with_state) {
  const size_t bx = (size_t)(B * L * H * P), bbc = (size_t)(B * L * G * N), st = (size_t)(B * H * P * N);
  double *x = arr(bx, 1, 0), *dt = arr((size_t)(B * L * H), 0.1, 0), *Bm = arr(bbc, 1, 0), *Cm = arr(bbc, 1, 0);
  double *db = arr((size_t)H, 1, -4), *A = arr((size_t)H, 3, -4), *Dk = arr((size_t)H, 0.5, 1);
  double *s0 = with_state ? arr(st, 1, 0) : NULL, *y = arr(bx, 0, 0), *so = arr(st, 0, 0);
  expect(oracle_ssd_fwd(B, L, H, P, N, G, x, dt, Bm, Cm, db, A, Dk, s0, y, so, 2), 0, "ssd_fwd");
  int32_t* sq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * L));
  for (int64_t i = 0; i < B * L; ++i) sq[i] = (int32_t)((i % L) / 2);
  expect(oracle_ssd_fwd_seq(B, L, H, P, N, G, x, dt, Bm, Cm, sq, db, A, Dk, s0, y, so, 2), 0, "ssd_fwd_seq");
  expect(oracle_ssd_step(B, H, P, N, G, x, dt, Bm, Cm, db, A, Dk, so, y, so), 0, "ssd_step");
  expect(oracle_ssd_step(B, H, P, N, G, x, dt, Bm, Cm, db, A, Dk, NULL, y, so), -1, "ssd_step without state");
  free(sq); free(x); free(dt); free(Bm); free(Cm); free(db); free(A); free(Dk); free(s0); free(y); free(so);
}

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 16}, {2, 2, 3, 8}, {1, 3, 5, 16}, {3, 7, 4, 1}, {2, 40, 6, 16}};
  for (int i = 0; i < 5; ++i)
    for (int s = 0; s < 2; ++s) mamba1(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], s);
  mamba2(1, 1, 1, 1, 1, 1, 0);
  mamba2(2, 5, 4, 3, 6, 2, 1);
  mamba2(1, 300, 2, 4, 8, 1, 1);
  if (fails) return 1;
  printf("oracle driver ok\n");
  return 0;
}
