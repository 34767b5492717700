/*
 * Runs every entry point of the fp64 oracle on small random problems (all
 * cells, all Jacobian variants, forward and reverse scans, lsim) and on bad
 * arguments, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.
 * Test infrastructure: built and run by tests/test_sanitizers.py.
 */
#include <stdio.h>

#include "../../oracle/oracle.c"

static unsigned long long g_state = 0x9e3779b97f4a7c15ULL;
static double urand(void) {  /* uniform in [-1, 1) */
  g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(g_state >> 11) / 4503599627370496.0 - 1.0;
}
static double *vec(size_t n, double scale) {
  double *v = (double *)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; i++) v[i] = scale * urand();
  return v;
}

static int run_cell(int cell, int B, int T, int d, int n) {
  const int G = (cell == ORC_GRU || cell == ORC_GRU_DIAG || cell == ORC_LSTM) ? 3 : 1;
  const int S = cell == ORC_LSTM ? 2 * n : n;
  const int dense = cell == ORC_TANH_RNN || cell == ORC_GRU || cell == ORC_LINEAR;
  double *Wx = vec((size_t)G * n * d, 0.7), *bx = vec((size_t)G * n, 0.3);
  double *Wh = vec(dense ? (size_t)G * n * n : (size_t)G * n, 0.5), *bh = vec((size_t)G * n, 0.3);
  double *peep = cell == ORC_LSTM ? vec((size_t)2 * n, 0.5) : NULL;
  orc_model m = {cell, B, T, d, n, Wx, bx, Wh, bh, peep};
  double *x = vec((size_t)B * T * d, 1.0), *h0 = vec((size_t)B * S, 0.5), *g = vec((size_t)B * T * S, 1.0);
  double *h = vec((size_t)B * T * S, 0.0), *h2 = vec((size_t)B * T * S, 0.0);
  double *lam = vec((size_t)B * T * S, 0.0), *dx = vec((size_t)B * T * d, 0.0), *dh0 = vec((size_t)B * S, 0.0);
  double *dWx = vec((size_t)G * n * d, 0.0), *dbx = vec((size_t)G * n, 0.0);
  double *dWh = vec(dense ? (size_t)G * n * n : (size_t)G * n, 0.0), *dbh = vec((size_t)G * n, 0.0);
  double *dpeep = vec((size_t)2 * n, 0.0), deltas[64];
  double *f = vec((size_t)S, 0.0), *J = vec((size_t)S * S * 4, 0.0), *ds = vec((size_t)S, 0.0), *dU = vec((size_t)G * n, 0.0);
  int it = 0, st = 0, bad = 0;
  bad |= orc_cell(&m, h0, x, f, J) != ORC_OK;
  bad |= orc_cell_vjp(&m, h0, x, g, ds, dU) != ORC_OK;
  bad |= orc_rollout(&m, x, h0, h) != ORC_OK;
  for (int a = 0; a < 3; a++) bad |= orc_deer_approx(&m, a, x, h0, 1e-9, T, h2, &it, &st, deltas, 64) != ORC_OK;
  bad |= orc_deer(&m, x, h0, 0.0, 3, h2, &it, &st, deltas, 64) != ORC_OK;
  bad |= orc_adjoint(&m, x, h0, h, g, lam, dx, dh0, dWx, dbx, dWh, dbh, cell == ORC_LSTM ? dpeep : NULL) != ORC_OK;
  bad |= orc_adjoint(&m, x, NULL, h, g, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != ORC_OK;
  for (int k = 0; k < 3; k++) {
    const double lam_k = k == 0 ? 0.0 : k == 1 ? 0.3 : 4.0;
    bad |= orc_elk(&m, lam_k, x, h0, 1e-9, 6, h2, &it, &st, deltas, 64) != ORC_OK;
    bad |= orc_elk_full(&m, lam_k, x, h0, 1e-9, 6, h2, &it, &st, deltas, 64) != ORC_OK;
  }
  /* bad arguments are refused */
  bad |= orc_elk_full(&m, -1.0, x, h0, 1e-9, 6, h2, &it, &st, deltas, 64) != ORC_EINVAL;
  bad |= orc_deer_approx(&m, 0, x, h0, 1e-9, 0, h2, &it, &st, deltas, 64) != ORC_EINVAL;
  orc_model broken = m;
  broken.cell = 9;
  bad |= orc_rollout(&broken, x, h0, h) != ORC_EINVAL;
  free(Wx); free(bx); free(Wh); free(bh); free(peep); free(x); free(h0); free(g); free(h); free(h2); free(lam);
  free(dx); free(dh0); free(dWx); free(dbx); free(dWh); free(dbh); free(dpeep); free(f); free(J); free(ds); free(dU);
  if (bad) fprintf(stderr, "cell %d failed\n", cell);
  return bad;
}

static int run_scans(void) {
  int bad = 0;
  const int B = 2, T = 37, n = 3;
  for (int kind = 0; kind < 3; kind++) {
    const size_t na = kind == ORC_DENSE ? (size_t)n * n : kind == ORC_DIAG ? (size_t)n : (size_t)n * 4;
    const size_t nb = kind == ORC_BLOCK2 ? (size_t)n * 2 : (size_t)n;
    double *A = vec((size_t)B * T * na, 0.5), *b = vec((size_t)B * T * nb, 1.0), *y = vec((size_t)B * T * nb, 0.0);
    for (int rev = 0; rev < 2; rev++) bad |= orc_affine_solve(kind, B, T, n, rev, A, b, y) != ORC_OK;
    free(A); free(b); free(y);
  }
  const int nx = 3, mi = 2, p = 2;
  double *Ad = vec(nx * nx, 0.4), *Bd = vec(nx * mi, 1.0), *C = vec(p * nx, 1.0), *D = vec(p * mi, 1.0);
  double *U = vec((size_t)B * T * mi, 1.0), *x0 = vec(B * nx, 1.0), *x = vec((size_t)B * T * nx, 0.0),
         *y = vec((size_t)B * T * p, 0.0);
  bad |= orc_lsim_discrete(B, T, nx, mi, p, Ad, Bd, C, D, U, x0, x, y) != ORC_OK;
  bad |= orc_lsim_discrete(B, T, nx, mi, p, Ad, Bd, C, D, U, NULL, x, y) != ORC_OK;
  free(Ad); free(Bd); free(C); free(D); free(U); free(x0); free(x); free(y);
  if (bad) fprintf(stderr, "scans failed\n");
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run_cell(ORC_TANH_RNN, 2, 9, 3, 4);
  bad |= run_cell(ORC_GRU, 2, 11, 2, 3);
  bad |= run_cell(ORC_LINEAR, 1, 7, 2, 2);
  bad |= run_cell(ORC_GRU_DIAG, 3, 13, 4, 5);
  bad |= run_cell(ORC_LSTM, 2, 10, 3, 4);
  bad |= run_cell(ORC_GRU, 1, 1, 1, 1);
  bad |= run_scans();
  printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
  return bad;
}
