/*
 * fp64 CPU oracle for Newton (DEER) / quasi-Newton (quasi-DEER) evaluation of
 * nonlinear RNNs over the sequence length.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or run
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant with the HIP
 * library; both sides see the same seeded inputs and nothing else.
 *
 * What it computes, and where the pages state it:
 *  - orc_rollout: the plain sequential evaluation h_t = f(h_{t-1}, x_t) that
 *    DEER is measured against ("Parallelizing non-linear sequential models
 *    over the sequence length", Key results and Measured effects: sequential
 *    GRU evaluation; ParaRNN abstract: the plain one-step-at-a-time baseline).
 *  - orc_deer / orc_deer_approx: Newton on the residual system F(h)_t = h_t - f(h_{t-1}, x_t) = 0
 *    (ParaRNN abstract: the recurrences cast as one system of equations solved
 *    with Newton's iterations; Gonzalez et al. abstract: the states as the
 *    solution of a fixed-point problem; Para-Seq README, Background: linearise
 *    and solve the resulting linear recurrence).  Each sweep evaluates the cell
 *    and its Jacobian at every step, solves dh_t = J_t dh_{t-1} + r_t, and
 *    updates.  The linear recurrence is solved here by its plain sequential
 *    definition, not by a scan.  orc_deer_approx replaces the Jacobian by its
 *    diagonal (quasi-DEER) or by zero (Jacobi iteration) (Gonzalez et al.
 *    abstract: quasi-Newton approximations; Para-Seq README, Main features).  Stopping uses the single tolerance
 *    hyperparameter of DEER (DEER summary, Limitations) on max |dh|.
 *  - orc_adjoint: the gradient of L = sum_t <g_t, h_t> by reverse-mode
 *    differentiation through the recurrence at a given trajectory (textbook
 *    backpropagation through time).  At a converged trajectory this equals
 *    the single reverse linear solve lambda_t = g_t + J_{t+1}^T lambda_{t+1}
 *    that the DEER summary describes (Surprising findings: the backward pass
 *    costs a single extra linear solve; Para-Seq README, Main
 *    features: reverse adjoint scans).
 *  - orc_affine_solve: y_t = A_t y_{t-1} + b_t (or the reverse-time recurrence)
 *    by its definition, for the dense, diagonal and 2x2-block operators that
 *    the Para-Seq README lists (Main features: src.utils scans).
 *  - orc_elk: quasi-ELK, the Levenberg-Marquardt-damped quasi-Newton sweep
 *    solved as a Kalman smoother (Gonzalez et al. abstract: ELK connects
 *    Levenberg-Marquardt with Kalman smoothing to stabilise DEER; Para-Seq
 *    README, Main features: ELK and quasi-ELK solvers), with the textbook
 *    Kalman filter and Rauch-Tung-Striebel smoother run sequentially.
 *  - orc_elk_full: ELK, the same damped step with the cell's own Jacobian
 *    (dense for the tanh RNN, GRU and linear cells, 2x2 blocks per channel
 *    for the LSTM, diagonal for the diagonal GRU), the Kalman filter and
 *    smoother run with full covariance matrices, sequentially.
 *  - orc_lsim_discrete: the sampled linear state-space simulation behind the
 *    README's lsim (Main features: ODE solvers; Example: lsim(A, B, C, D, U,
 *    t)) once the system is discretised: x_0 = x0, y_k = C x_k + D u_k,
 *    x_{k+1} = Ad x_k + Bd u_k, sequentially.  The discretisation (zero-order
 *    hold: Ad = exp(A dt), Bd = int_0^dt exp(A s) ds B) is done by the Python
 *    front end with a library matrix exponential.
 *
 * The pages never print the cell equations.  The cells follow the PyTorch
 * conventions that Para-Seq keeps (README intro: the standard RNN/GRU/LSTM
 * interface); the CIFG/peephole ParaLSTM (README, Main features) is read as:
 *   f = sigm(U_f + w_f h + p_f c + b_f),  g = tanh(U_g + w_g h + b_g),
 *   c' = f c + (1-f) g,  o = sigm(U_o + w_o h + p_o c' + b_o),  h' = o tanh(c').
 * Every operation runs in double precision, built without contraction of
 * multiplies and adds into fused operations.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_TANH_RNN = 0, ORC_GRU = 1, ORC_GRU_DIAG = 2, ORC_LSTM = 3, ORC_LINEAR = 4 };
enum { ORC_DENSE = 0, ORC_DIAG = 1, ORC_BLOCK2 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -4, ORC_NOT_CONVERGED = 1, ORC_NONFINITE = 2 };

typedef struct {
  int cell, B, T, d, n;
  const double *Wx;   /* [G*n, d] */
  const double *bx;   /* [G*n] or NULL */
  const double *Wh;   /* dense cells [G*n, n]; diagonal cells [G*n] */
  const double *bh;   /* [G*n] or NULL */
  const double *peep; /* LSTM [2n] = p_f | p_o, else NULL */
} orc_model;

static int n_gates(int cell) { return (cell == ORC_GRU || cell == ORC_GRU_DIAG || cell == ORC_LSTM) ? 3 : 1; }
static int swidth(const orc_model *m) { return m->cell == ORC_LSTM ? 2 * m->n : m->n; }
static int jkind(int cell) {
  if (cell == ORC_GRU_DIAG) return ORC_DIAG;
  if (cell == ORC_LSTM) return ORC_BLOCK2;
  return ORC_DENSE;
}
/* number of doubles one step's Jacobian occupies in its own structure */
static size_t jsize(const orc_model *m) {
  int k = jkind(m->cell), S = swidth(m);
  if (k == ORC_DENSE) return (size_t)S * S;
  if (k == ORC_DIAG) return (size_t)S;
  return (size_t)m->n * 4;
}
static double sigm(double a) { return 1.0 / (1.0 + exp(-a)); }
static double bias(const double *b, int i) { return b ? b[i] : 0.0; }

/* U = W_x x_t + b_x : the input transform of a standard RNN layer. */
static void input_proj(const orc_model *m, const double *xt, double *U) {
  int Gn = n_gates(m->cell) * m->n;
  for (int j = 0; j < Gn; j++) {
    double a = bias(m->bx, j);
    for (int k = 0; k < m->d; k++) a += m->Wx[(size_t)j * m->d + k] * xt[k];
    U[j] = a;
  }
}

/* Dense row-vector product (W s)_i for the rows [row0, row0+n) of W [*, n]. */
static double rowdot(const double *W, int row, int n, const double *s) {
  double a = 0.0;
  for (int k = 0; k < n; k++) a += W[(size_t)row * n + k] * s[k];
  return a;
}

/*
 * One cell step: f = f(s, U) and, when J != NULL, J = df/ds in the cell's own
 * structure (dense S x S row-major; diagonal S; 2x2 blocks [n][2][2] with rows
 * (c', h') and columns (c, h)).
 */
static void cell_fwd(const orc_model *m, const double *s, const double *U, double *f, double *J) {
  int n = m->n;
  switch (m->cell) {
  case ORC_TANH_RNN:
  case ORC_LINEAR:
    for (int i = 0; i < n; i++) {
      double a = U[i] + rowdot(m->Wh, i, n, s) + bias(m->bh, i);
      double fi = m->cell == ORC_TANH_RNN ? tanh(a) : a;
      f[i] = fi;
      if (J) {
        double da = m->cell == ORC_TANH_RNN ? 1.0 - fi * fi : 1.0;
        for (int k = 0; k < n; k++) J[(size_t)i * n + k] = da * m->Wh[(size_t)i * n + k];
      }
    }
    break;
  case ORC_GRU:
    for (int i = 0; i < n; i++) {
      double r = sigm(U[i] + rowdot(m->Wh, i, n, s) + bias(m->bh, i));
      double z = sigm(U[n + i] + rowdot(m->Wh, n + i, n, s) + bias(m->bh, n + i));
      double q = rowdot(m->Wh, 2 * n + i, n, s) + bias(m->bh, 2 * n + i);
      double c = tanh(U[2 * n + i] + r * q);
      f[i] = (1.0 - z) * c + z * s[i];
      if (J) {
        double al = (s[i] - c) * z * (1.0 - z);            /* through z          */
        double be = (1.0 - z) * (1.0 - c * c);             /* through c          */
        for (int k = 0; k < n; k++) {
          double whr = m->Wh[(size_t)i * n + k];
          double whz = m->Wh[(size_t)(n + i) * n + k];
          double whn = m->Wh[(size_t)(2 * n + i) * n + k];
          double v = al * whz + be * (r * whn + q * r * (1.0 - r) * whr);
          if (k == i) v += z;
          J[(size_t)i * n + k] = v;
        }
      }
    }
    break;
  case ORC_GRU_DIAG:
    for (int i = 0; i < n; i++) {
      double ar = m->Wh[i], az = m->Wh[n + i], an = m->Wh[2 * n + i];
      double r = sigm(U[i] + ar * s[i] + bias(m->bh, i));
      double z = sigm(U[n + i] + az * s[i] + bias(m->bh, n + i));
      double q = an * s[i] + bias(m->bh, 2 * n + i);
      double c = tanh(U[2 * n + i] + r * q);
      f[i] = (1.0 - z) * c + z * s[i];
      if (J) J[i] = z + (s[i] - c) * z * (1.0 - z) * az + (1.0 - z) * (1.0 - c * c) * (r * an + q * r * (1.0 - r) * ar);
    }
    break;
  case ORC_LSTM:
    for (int i = 0; i < n; i++) {
      double c = s[2 * i], h = s[2 * i + 1];
      double wf = m->Wh[i], wg = m->Wh[n + i], wo = m->Wh[2 * n + i];
      double pf = m->peep[i], po = m->peep[n + i];
      double fg = sigm(U[i] + wf * h + pf * c + bias(m->bh, i));
      double g = tanh(U[n + i] + wg * h + bias(m->bh, n + i));
      double cn = fg * c + (1.0 - fg) * g;
      double o = sigm(U[2 * n + i] + wo * h + po * cn + bias(m->bh, 2 * n + i));
      double tc = tanh(cn);
      f[2 * i] = cn;
      f[2 * i + 1] = o * tc;
      if (J) {
        double dcc = fg + (c - g) * fg * (1.0 - fg) * pf;
        double dch = (c - g) * fg * (1.0 - fg) * wf + (1.0 - fg) * (1.0 - g * g) * wg;
        double dhdcn = o * (1.0 - tc * tc) + tc * o * (1.0 - o) * po;
        double *Jb = J + (size_t)4 * i;
        Jb[0] = dcc;
        Jb[1] = dch;
        Jb[2] = dhdcn * dcc;
        Jb[3] = tc * o * (1.0 - o) * wo + dhdcn * dch;
      }
    }
    break;
  }
}

/* Size of the gradient of W_h (dense cells [G n, n], diagonal cells [G n]). */
static size_t wh_size(const orc_model *m) {
  int Gn = n_gates(m->cell) * m->n;
  return (m->cell == ORC_GRU_DIAG || m->cell == ORC_LSTM) ? (size_t)Gn : (size_t)Gn * m->n;
}

/*
 * Reverse-mode step through one cell by the chain rule: given the output
 * gradient lam (S) at (s, U), return ds = (df/ds)^T lam, dU = (df/dU)^T lam, and
 * add the parameter gradients of W_h, b_h and the peepholes.
 */
static void cell_vjp(const orc_model *m, const double *s, const double *U, const double *lam,
                     double *ds, double *dU, double *dWh, double *dbh, double *dpeep) {
  int n = m->n;
  switch (m->cell) {
  case ORC_TANH_RNN:
  case ORC_LINEAR: {
    for (int k = 0; k < n; k++) ds[k] = 0.0;
    for (int i = 0; i < n; i++) {
      double a = U[i] + rowdot(m->Wh, i, n, s) + bias(m->bh, i);
      double da = lam[i];
      if (m->cell == ORC_TANH_RNN) { double fi = tanh(a); da *= 1.0 - fi * fi; }
      dU[i] = da;
      dbh[i] += da;
      for (int k = 0; k < n; k++) {
        dWh[(size_t)i * n + k] += da * s[k];
        ds[k] += da * m->Wh[(size_t)i * n + k];
      }
    }
    break;
  }
  case ORC_GRU: {
    for (int k = 0; k < n; k++) ds[k] = 0.0;
    for (int i = 0; i < n; i++) {
      double r = sigm(U[i] + rowdot(m->Wh, i, n, s) + bias(m->bh, i));
      double z = sigm(U[n + i] + rowdot(m->Wh, n + i, n, s) + bias(m->bh, n + i));
      double q = rowdot(m->Wh, 2 * n + i, n, s) + bias(m->bh, 2 * n + i);
      double c = tanh(U[2 * n + i] + r * q);
      double dc = lam[i] * (1.0 - z);
      double dz = lam[i] * (s[i] - c);
      double daz = dz * z * (1.0 - z);
      double dan = dc * (1.0 - c * c);
      double dq = dan * r;
      double dar = dan * q * r * (1.0 - r);
      ds[i] += lam[i] * z;
      dU[i] = dar; dU[n + i] = daz; dU[2 * n + i] = dan;
      dbh[i] += dar; dbh[n + i] += daz; dbh[2 * n + i] += dq;
      for (int k = 0; k < n; k++) {
        dWh[(size_t)i * n + k] += dar * s[k];
        dWh[(size_t)(n + i) * n + k] += daz * s[k];
        dWh[(size_t)(2 * n + i) * n + k] += dq * s[k];
        ds[k] += dar * m->Wh[(size_t)i * n + k] + daz * m->Wh[(size_t)(n + i) * n + k] +
                 dq * m->Wh[(size_t)(2 * n + i) * n + k];
      }
    }
    break;
  }
  case ORC_GRU_DIAG:
    for (int i = 0; i < n; i++) {
      double ar = m->Wh[i], az = m->Wh[n + i], an = m->Wh[2 * n + i];
      double r = sigm(U[i] + ar * s[i] + bias(m->bh, i));
      double z = sigm(U[n + i] + az * s[i] + bias(m->bh, n + i));
      double q = an * s[i] + bias(m->bh, 2 * n + i);
      double c = tanh(U[2 * n + i] + r * q);
      double dc = lam[i] * (1.0 - z);
      double dz = lam[i] * (s[i] - c);
      double daz = dz * z * (1.0 - z);
      double dan = dc * (1.0 - c * c);
      double dq = dan * r;
      double dar = dan * q * r * (1.0 - r);
      ds[i] = lam[i] * z + dar * ar + daz * az + dq * an;
      dU[i] = dar; dU[n + i] = daz; dU[2 * n + i] = dan;
      dbh[i] += dar; dbh[n + i] += daz; dbh[2 * n + i] += dq;
      dWh[i] += dar * s[i]; dWh[n + i] += daz * s[i]; dWh[2 * n + i] += dq * s[i];
    }
    break;
  case ORC_LSTM:
    for (int i = 0; i < n; i++) {
      double c = s[2 * i], h = s[2 * i + 1];
      double wf = m->Wh[i], wg = m->Wh[n + i], wo = m->Wh[2 * n + i];
      double pf = m->peep[i], po = m->peep[n + i];
      double fg = sigm(U[i] + wf * h + pf * c + bias(m->bh, i));
      double g = tanh(U[n + i] + wg * h + bias(m->bh, n + i));
      double cn = fg * c + (1.0 - fg) * g;
      double o = sigm(U[2 * n + i] + wo * h + po * cn + bias(m->bh, 2 * n + i));
      double tc = tanh(cn);
      double lc = lam[2 * i], lh = lam[2 * i + 1];
      double dao = lh * tc * o * (1.0 - o);
      double dcn = lc + lh * o * (1.0 - tc * tc) + dao * po;
      double daf = dcn * (c - g) * fg * (1.0 - fg);
      double dag = dcn * (1.0 - fg) * (1.0 - g * g);
      ds[2 * i] = dcn * fg + daf * pf;
      ds[2 * i + 1] = daf * wf + dag * wg + dao * wo;
      dU[i] = daf; dU[n + i] = dag; dU[2 * n + i] = dao;
      dbh[i] += daf; dbh[n + i] += dag; dbh[2 * n + i] += dao;
      dWh[i] += daf * h; dWh[n + i] += dag * h; dWh[2 * n + i] += dao * h;
      dpeep[i] += daf * c; dpeep[n + i] += dao * cn;
    }
    break;
  }
}

static int model_ok(const orc_model *m) {
  if (m->cell < 0 || m->cell > 4) return 0;
  if (m->B < 0 || m->T < 0 || m->d < 1 || m->n < 1) return 0;
  if (!m->Wx || !m->Wh) return 0;
  if (m->cell == ORC_LSTM && !m->peep) return 0;
  return 1;
}

/* ---------------------------------------------------------------------- */
/* Exported API                                                            */
/* ---------------------------------------------------------------------- */

/* One cell step (f and its structured Jacobian) at s_prev, x_t. */
int orc_cell(const orc_model *m, const double *s_prev, const double *xt, double *f, double *J) {
  if (!model_ok(m)) return ORC_EINVAL;
  int Gn = n_gates(m->cell) * m->n;
  double *U = (double *)malloc(sizeof(double) * Gn);
  if (!U) return ORC_ENOMEM;
  input_proj(m, xt, U);
  cell_fwd(m, s_prev, U, f, J);
  free(U);
  return ORC_OK;
}

/* One reverse-mode cell step: ds = J^T lam and dU = (df/dU)^T lam. */
int orc_cell_vjp(const orc_model *m, const double *s_prev, const double *xt, const double *lam,
                 double *ds, double *dU) {
  if (!model_ok(m)) return ORC_EINVAL;
  int Gn = n_gates(m->cell) * m->n;
  double *U = (double *)malloc(sizeof(double) * Gn);
  double *dWh = (double *)calloc(wh_size(m), sizeof(double));
  double *dbh = (double *)calloc(Gn, sizeof(double));
  double *dp = (double *)calloc(2 * m->n, sizeof(double));
  if (!U || !dWh || !dbh || !dp) { free(U); free(dWh); free(dbh); free(dp); return ORC_ENOMEM; }
  input_proj(m, xt, U);
  cell_vjp(m, s_prev, U, lam, ds, dU, dWh, dbh, dp);
  free(U); free(dWh); free(dbh); free(dp);
  return ORC_OK;
}

/* Sequential rollout h_t = f(h_{t-1}, x_t), h_{-1} = h0 (NULL = 0).  h: [B,T,S]. */
int orc_rollout(const orc_model *m, const double *x, const double *h0, double *h) {
  if (!model_ok(m)) return ORC_EINVAL;
  int S = swidth(m), Gn = n_gates(m->cell) * m->n, err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int b = 0; b < m->B; b++) {
    double *U = (double *)malloc(sizeof(double) * Gn);
    double *s = (double *)malloc(sizeof(double) * S);
    if (!U || !s) { err |= 1; free(U); free(s); continue; }
    for (int i = 0; i < S; i++) s[i] = h0 ? h0[(size_t)b * S + i] : 0.0;
    for (int t = 0; t < m->T; t++) {
      const double *xt = x + ((size_t)b * m->T + t) * m->d;
      double *ht = h + ((size_t)b * m->T + t) * S;
      input_proj(m, xt, U);
      cell_fwd(m, s, U, ht, NULL);
      memcpy(s, ht, sizeof(double) * S);
    }
    free(U); free(s);
  }
  return err ? ORC_ENOMEM : ORC_OK;
}

/* y = A y_prev + b for one step of an operator of the given structure. */
static void affine_step(int kind, int n, const double *A, const double *yprev, const double *b, double *y) {
  if (kind == ORC_DENSE) {
    for (int i = 0; i < n; i++) {
      double a = b[i];
      for (int k = 0; k < n; k++) a += A[(size_t)i * n + k] * yprev[k];
      y[i] = a;
    }
  } else if (kind == ORC_DIAG) {
    for (int i = 0; i < n; i++) y[i] = A[i] * yprev[i] + b[i];
  } else { /* n channels, 2x2 blocks, state interleaved */
    for (int i = 0; i < n; i++) {
      const double *Ab = A + (size_t)4 * i;
      double y0 = yprev[2 * i], y1 = yprev[2 * i + 1];
      y[2 * i] = Ab[0] * y0 + Ab[1] * y1 + b[2 * i];
      y[2 * i + 1] = Ab[2] * y0 + Ab[3] * y1 + b[2 * i + 1];
    }
  }
}

/*
 * The linear recurrence by its definition, per sequence b:
 *   forward:  y_t = A_t y_{t-1} + b_t,  y_{-1} = 0;
 *   reverse:  y_t = A_t y_{t+1} + b_t,  y_T = 0.
 * kind DENSE: A [B,T,n,n], b,y [B,T,n]; DIAG: A,b,y [B,T,n];
 * BLOCK2: A [B,T,n,2,2], b,y [B,T,n,2].
 */
int orc_affine_solve(int kind, int B, int T, int n, int reverse, const double *A, const double *bv, double *y) {
  if (kind < 0 || kind > 2 || B < 0 || T < 0 || n < 1) return ORC_EINVAL;
  int S = kind == ORC_BLOCK2 ? 2 * n : n;
  size_t js = kind == ORC_DENSE ? (size_t)n * n : (kind == ORC_DIAG ? (size_t)n : (size_t)4 * n);
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int b = 0; b < B; b++) {
    double *zero = (double *)calloc(S, sizeof(double));
    if (!zero) { err |= 1; continue; }
    for (int s = 0; s < T; s++) {
      int t = reverse ? T - 1 - s : s;
      const double *yp = s == 0 ? zero : y + ((size_t)b * T + (reverse ? t + 1 : t - 1)) * S;
      affine_step(kind, n, A + ((size_t)b * T + t) * js, yp, bv + ((size_t)b * T + t) * S,
                  y + ((size_t)b * T + t) * S);
    }
    free(zero);
  }
  return err ? ORC_ENOMEM : ORC_OK;
}

/*
 * Which Jacobian the linear solve of a sweep uses (Gonzalez et al. abstract:
 * quasi-Newton approximations of DEER; Para-Seq README, Main features: the
 * Jacobi, quasi-DEER and DEER solvers):
 *   ORC_NEWTON  the cell's own Jacobian (DEER);
 *   ORC_QUASI   its diagonal only: the entries J[i][i] of a dense Jacobian,
 *               the two diagonal entries of each 2x2 block; a diagonal
 *               Jacobian is kept whole (quasi-DEER);
 *   ORC_JACOBI  zero: the sweep sets h_t to f(h_{t-1}, x_t) of the previous
 *               iterate (Jacobi / Picard iteration).
 * All three have the rollout as their fixed point and reproduce it exactly
 * on steps t < k after k sweeps, so a solve also ends after sweep T.
 */
enum { ORC_NEWTON = 0, ORC_QUASI = 1, ORC_JACOBI = 2 };

/* Apply the approximation to one step's Jacobian, stored in the cell's structure. */
static void approx_jac(const orc_model *m, int approx, double *J) {
  int kind = jkind(m->cell), S = swidth(m);
  size_t js = jsize(m);
  if (approx == ORC_JACOBI) {
    for (size_t e = 0; e < js; e++) J[e] = 0.0;
  } else if (approx == ORC_QUASI && kind == ORC_DENSE) {
    for (int i = 0; i < S; i++)
      for (int k = 0; k < S; k++)
        if (k != i) J[(size_t)i * S + k] = 0.0;
  } else if (approx == ORC_QUASI && kind == ORC_BLOCK2) {
    for (int c = 0; c < m->n; c++) {
      J[(size_t)4 * c + 1] = 0.0; /* d c' / d h */
      J[(size_t)4 * c + 2] = 0.0; /* d h' / d c */
    }
  }
}

/*
 * CPU DEER.  h: [B,T,S] output (the last iterate); iters, status out;
 * deltas: [hist_cap] history of delta_k = max |dh| (entry k-1 for sweep k).
 *
 * Sweep k, for every sequence:
 *   1. for every t: s_prev = (t == 0 ? h0 : h_{t-1}) of the current iterate;
 *      f_t, J_t = cell(s_prev, U_t);  r_t = f_t - h_t;  J_t approximated as
 *      `approx` says;
 *   2. dh_0-1 = 0;  for t = 0..T-1: dh_t = J_t dh_{t-1} + r_t  (sequential);
 *   3. h_t += dh_t.
 * delta_k is the max over the whole batch.  Stop rule: non-finite delta ->
 * NONFINITE; tol > 0 and delta < tol -> OK; k == T -> OK (every variant is
 * exact after T sweeps); k == max_iters -> NOT_CONVERGED (OK when tol <= 0).
 */
int orc_deer_approx(const orc_model *m, int approx, const double *x, const double *h0, double tol, int max_iters,
                    double *h, int *iters, int *status, double *deltas, int hist_cap) {
  if (!model_ok(m) || max_iters < 1 || approx < ORC_NEWTON || approx > ORC_JACOBI) return ORC_EINVAL;
  int S = swidth(m), Gn = n_gates(m->cell) * m->n, T = m->T;
  size_t js = jsize(m);
  int kind = jkind(m->cell);
  memset(h, 0, sizeof(double) * (size_t)m->B * T * S); /* initial guess: zeros */
  *iters = 0;
  *status = ORC_OK;
  if (T == 0 || m->B == 0) return ORC_OK;
  for (int k = 1; k <= max_iters; k++) {
    double delta = 0.0;
    int err = 0, nonfin = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : delta) reduction(| : err, nonfin)
    for (int b = 0; b < m->B; b++) {
      double *U = (double *)malloc(sizeof(double) * Gn);
      double *F = (double *)malloc(sizeof(double) * (size_t)T * S);
      double *R = (double *)malloc(sizeof(double) * (size_t)T * S);
      double *D = (double *)malloc(sizeof(double) * (size_t)T * S);
      double *Jb = (double *)malloc(sizeof(double) * (size_t)T * js);
      double *zero = (double *)calloc(S, sizeof(double));
      if (!U || !F || !R || !D || !Jb || !zero) {
        err |= 1;
      } else {
        double *hb = h + (size_t)b * T * S;
        /* 1. cell, Jacobian and residual at every step (the parallel part). */
        for (int t = 0; t < T; t++) {
          const double *sp = t == 0 ? (h0 ? h0 + (size_t)b * S : zero) : hb + (size_t)(t - 1) * S;
          input_proj(m, x + ((size_t)b * T + t) * m->d, U);
          cell_fwd(m, sp, U, F + (size_t)t * S, Jb + (size_t)t * js);
          approx_jac(m, approx, Jb + (size_t)t * js);
          for (int i = 0; i < S; i++) R[(size_t)t * S + i] = F[(size_t)t * S + i] - hb[(size_t)t * S + i];
        }
        /* 2. the linear recurrence, sequentially. */
        for (int t = 0; t < T; t++)
          affine_step(kind, m->n, Jb + (size_t)t * js, t == 0 ? zero : D + (size_t)(t - 1) * S,
                      R + (size_t)t * S, D + (size_t)t * S);
        /* 3. update and convergence measure. */
        for (size_t e = 0; e < (size_t)T * S; e++) {
          hb[e] += D[e];
          double a = fabs(D[e]);
          if (!isfinite(a)) nonfin = 1;
          else if (a > delta) delta = a;
        }
      }
      free(U); free(F); free(R); free(D); free(Jb); free(zero);
    }
    if (err) return ORC_ENOMEM;
    if (nonfin) delta = NAN;
    if (deltas && k <= hist_cap) deltas[k - 1] = delta;
    *iters = k;
    if (!isfinite(delta)) { *status = ORC_NONFINITE; return ORC_OK; }
    if (tol > 0.0 && delta < tol) { *status = ORC_OK; return ORC_OK; }
    if (k == T) { *status = ORC_OK; return ORC_OK; }
  }
  *status = tol > 0.0 ? ORC_NOT_CONVERGED : ORC_OK;
  return ORC_OK;
}

/* DEER with the cell's own Jacobian. */
int orc_deer(const orc_model *m, const double *x, const double *h0, double tol, int max_iters, double *h,
             int *iters, int *status, double *deltas, int hist_cap) {
  return orc_deer_approx(m, ORC_NEWTON, x, h0, tol, max_iters, h, iters, status, deltas, hist_cap);
}

/*
 * Gradient of L = sum_{b,t} <g_t, h_t> through the recurrence at the given
 * trajectory h (reverse-mode, t = T-1 .. 0):
 *   lam_t = g_t + carry;  (carry, dU_t, dtheta) = cell_vjp at (h_{t-1}, U_t, lam_t).
 * Outputs (each may be NULL): lam [B,T,S]; dx [B,T,d]; dh0 [B,S]; dWx [Gn,d];
 * dbx [Gn]; dWh (dense [Gn,n] / diag [Gn]); dbh [Gn]; dpeep [2n].
 * Parameter gradients are summed per sequence and then over b in order.
 */
int orc_adjoint(const orc_model *m, const double *x, const double *h0, const double *h, const double *g,
                double *lam, double *dx, double *dh0, double *dWx, double *dbx, double *dWh, double *dbh,
                double *dpeep) {
  if (!model_ok(m)) return ORC_EINVAL;
  int S = swidth(m), Gn = n_gates(m->cell) * m->n, T = m->T, B = m->B, d = m->d, n = m->n;
  size_t nwx = (size_t)Gn * d, nwh = wh_size(m);
  size_t per = nwx + Gn + nwh + Gn + 2 * (size_t)n;
  double *acc = (double *)calloc((size_t)(B > 0 ? B : 1) * per, sizeof(double));
  if (!acc) return ORC_ENOMEM;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int b = 0; b < B; b++) {
    double *A = acc + (size_t)b * per;
    double *aWx = A, *abx = A + nwx, *aWh = abx + Gn, *abh = aWh + nwh, *ap = abh + Gn;
    double *U = (double *)malloc(sizeof(double) * Gn);
    double *dU = (double *)malloc(sizeof(double) * Gn);
    double *carry = (double *)calloc(S, sizeof(double));
    double *ds = (double *)malloc(sizeof(double) * S);
    double *lt = (double *)malloc(sizeof(double) * S);
    double *zero = (double *)calloc(S, sizeof(double));
    if (!U || !dU || !carry || !ds || !lt || !zero) {
      err |= 1;
    } else {
      for (int t = T - 1; t >= 0; t--) {
        const double *xt = x + ((size_t)b * T + t) * d;
        const double *sp = t == 0 ? (h0 ? h0 + (size_t)b * S : zero) : h + ((size_t)b * T + t - 1) * S;
        for (int i = 0; i < S; i++) lt[i] = g[((size_t)b * T + t) * S + i] + carry[i];
        if (lam) memcpy(lam + ((size_t)b * T + t) * S, lt, sizeof(double) * S);
        input_proj(m, xt, U);
        cell_vjp(m, sp, U, lt, ds, dU, aWh, abh, ap);
        for (int j = 0; j < Gn; j++) {
          abx[j] += dU[j];
          for (int k = 0; k < d; k++) aWx[(size_t)j * d + k] += dU[j] * xt[k];
        }
        if (dx)
          for (int k = 0; k < d; k++) {
            double a = 0.0;
            for (int j = 0; j < Gn; j++) a += m->Wx[(size_t)j * d + k] * dU[j];
            dx[((size_t)b * T + t) * d + k] = a;
          }
        memcpy(carry, ds, sizeof(double) * S);
      }
      if (dh0) memcpy(dh0 + (size_t)b * S, carry, sizeof(double) * S);
    }
    free(U); free(dU); free(carry); free(ds); free(lt); free(zero);
  }
  if (!err) {
    double *outs[5] = {dWx, dbx, dWh, dbh, dpeep};
    size_t off[5] = {0, nwx, nwx + Gn, nwx + Gn + nwh, nwx + Gn + nwh + Gn};
    size_t cnt[5] = {nwx, (size_t)Gn, nwh, (size_t)Gn, 2 * (size_t)n};
    for (int o = 0; o < 5; o++) {
      if (!outs[o]) continue;
      if (o == 4 && m->cell != ORC_LSTM) continue;
      for (size_t e = 0; e < cnt[o]; e++) {
        double a = 0.0;
        for (int b = 0; b < B; b++) a += acc[(size_t)b * per + off[o] + e];
        outs[o][e] = a;
      }
    }
  }
  free(acc);
  return err ? ORC_ENOMEM : ORC_OK;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Sampled linear state-space system, per sequence b, by its definition:
 *   x_0 = x0 (0 if NULL);  for k = 0..T-1: y_k = C x_k + D u_k;
 *   x_{k+1} = Ad x_k + Bd u_k.
 * Ad [nx,nx], Bd [nx,m], C [p,nx], D [p,m] row-major; U [B,T,m]; x0 [B,nx];
 * outputs x [B,T,nx] (x_k, the state before input k) and y [B,T,p].
 */
int orc_lsim_discrete(int B, int T, int nx, int m, int p, const double *Ad, const double *Bd, const double *C,
                      const double *D, const double *U, const double *x0, double *x, double *y) {
  if (B < 0 || T < 0 || nx < 1 || m < 1 || p < 1) return ORC_EINVAL;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int b = 0; b < B; b++) {
    double *s = (double *)calloc(nx, sizeof(double)), *sn = (double *)calloc(nx, sizeof(double));
    if (!s || !sn) { err |= 1; free(s); free(sn); continue; }
    if (x0)
      for (int i = 0; i < nx; i++) s[i] = x0[(size_t)b * nx + i];
    for (int k = 0; k < T; k++) {
      const double *u = U + ((size_t)b * T + k) * m;
      for (int i = 0; i < nx; i++) x[((size_t)b * T + k) * nx + i] = s[i];
      for (int o = 0; o < p; o++) {
        double v = 0.0;
        for (int i = 0; i < nx; i++) v += C[(size_t)o * nx + i] * s[i];
        for (int j = 0; j < m; j++) v += D[(size_t)o * m + j] * u[j];
        y[((size_t)b * T + k) * p + o] = v;
      }
      for (int i = 0; i < nx; i++) {
        double v = 0.0;
        for (int l = 0; l < nx; l++) v += Ad[(size_t)i * nx + l] * s[l];
        for (int j = 0; j < m; j++) v += Bd[(size_t)i * m + j] * u[j];
        sn[i] = v;
      }
      for (int i = 0; i < nx; i++) s[i] = sn[i];
    }
    free(s);
    free(sn);
  }
  return err ? ORC_ENOMEM : ORC_OK;
}

/*
 * Quasi-ELK.  Each sweep takes the Levenberg-Marquardt step of the residual
 * system with the Jacobian's diagonal d_t (as ORC_QUASI) and damping lambda:
 *   dh = argmin sum_t ||dh_t - d_t dh_{t-1} - r_t||^2 + lambda sum_t ||dh_t||^2,
 * dh_{-1} = 0, which is the posterior mean of the linear-Gaussian model
 *   dh_t = d_t dh_{t-1} + r_t + w_t,  w_t ~ N(0, 1);  0 = dh_t + v_t,
 *   v_t ~ N(0, 1 / lambda),
 * computed per state entry by the Kalman filter and the Rauch-Tung-Striebel
 * smoother.  lambda = 0 gives the quasi-DEER step.  Then h += dh and the stop
 * rule of orc_deer_approx.
 */
int orc_elk(const orc_model *m, double lambda, const double *x, const double *h0, double tol, int max_iters,
            double *h, int *iters, int *status, double *deltas, int hist_cap) {
  if (!model_ok(m) || max_iters < 1 || !(lambda >= 0.0)) return ORC_EINVAL;
  int S = swidth(m), Gn = n_gates(m->cell) * m->n, T = m->T;
  size_t js = jsize(m);
  int kind = jkind(m->cell);
  memset(h, 0, sizeof(double) * (size_t)m->B * T * S);
  *iters = 0;
  *status = ORC_OK;
  if (T == 0 || m->B == 0) return ORC_OK;
  for (int k = 1; k <= max_iters; k++) {
    double delta = 0.0;
    int err = 0, nonfin = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : delta) reduction(| : err, nonfin)
    for (int b = 0; b < m->B; b++) {
      double *U = (double *)malloc(sizeof(double) * Gn);
      double *F = (double *)malloc(sizeof(double) * (size_t)T * S);
      double *D = (double *)malloc(sizeof(double) * (size_t)T * S);  /* d_t: the Jacobian's diagonal */
      double *R = (double *)malloc(sizeof(double) * (size_t)T * S);
      double *J = (double *)malloc(sizeof(double) * js);
      double *Pp = (double *)malloc(sizeof(double) * T), *Mp = (double *)malloc(sizeof(double) * T);
      double *Pf = (double *)malloc(sizeof(double) * T), *Mf = (double *)malloc(sizeof(double) * T);
      double *Ms = (double *)malloc(sizeof(double) * T);
      double *zero = (double *)calloc(S, sizeof(double));
      if (!U || !F || !D || !R || !J || !Pp || !Mp || !Pf || !Mf || !Ms || !zero) {
        err |= 1;
      } else {
        double *hb = h + (size_t)b * T * S;
        for (int t = 0; t < T; t++) {
          const double *sp = t == 0 ? (h0 ? h0 + (size_t)b * S : zero) : hb + (size_t)(t - 1) * S;
          input_proj(m, x + ((size_t)b * T + t) * m->d, U);
          cell_fwd(m, sp, U, F + (size_t)t * S, J);
          for (int i = 0; i < S; i++) {
            double di;
            if (kind == ORC_DENSE) di = J[(size_t)i * S + i];
            else if (kind == ORC_DIAG) di = J[i];
            else di = J[(size_t)4 * (i / 2) + ((i & 1) ? 3 : 0)]; /* dc'/dc, dh'/dh */
            D[(size_t)t * S + i] = di;
            R[(size_t)t * S + i] = F[(size_t)t * S + i] - hb[(size_t)t * S + i];
          }
        }
        for (int i = 0; i < S; i++) {
          /* Kalman filter: predicted (Pp, Mp) and filtered (Pf, Mf) moments */
          double P = 0.0, Mn = 0.0;
          for (int t = 0; t < T; t++) {
            const double d = D[(size_t)t * S + i], r = R[(size_t)t * S + i];
            const double pp = d * d * P + 1.0, mp = d * Mn + r;
            const double K = lambda * pp / (lambda * pp + 1.0);  /* gain for an observation of variance 1/lambda */
            Pp[t] = pp;
            Mp[t] = mp;
            P = (1.0 - K) * pp;
            Mn = (1.0 - K) * mp;
            Pf[t] = P;
            Mf[t] = Mn;
          }
          /* Rauch-Tung-Striebel smoother */
          Ms[T - 1] = Mf[T - 1];
          for (int t = T - 2; t >= 0; t--) {
            const double G = Pf[t] * D[(size_t)(t + 1) * S + i] / Pp[t + 1];
            Ms[t] = Mf[t] + G * (Ms[t + 1] - Mp[t + 1]);
          }
          for (int t = 0; t < T; t++) {
            hb[(size_t)t * S + i] += Ms[t];
            const double a = fabs(Ms[t]);
            if (!isfinite(a)) nonfin = 1;
            else if (a > delta) delta = a;
          }
        }
      }
      free(U); free(F); free(D); free(R); free(J); free(Pp); free(Mp); free(Pf); free(Mf); free(Ms); free(zero);
    }
    if (err) return ORC_ENOMEM;
    if (nonfin) delta = NAN;
    if (deltas && k <= hist_cap) deltas[k - 1] = delta;
    *iters = k;
    if (!isfinite(delta)) { *status = ORC_NONFINITE; return ORC_OK; }
    if (tol > 0.0 && delta < tol) { *status = ORC_OK; return ORC_OK; }
    if (k == T) { *status = ORC_OK; return ORC_OK; }
  }
  *status = tol > 0.0 ? ORC_NOT_CONVERGED : ORC_OK;
  return ORC_OK;
}

/*
 * Small dense linear algebra for orc_elk_full (q x q row-major, q <= a few
 * dozen).  chol_solve: X = A^{-1} Bm for symmetric positive definite A and a
 * q x nc right-hand side, by the Cholesky factorisation A = L L^T and two
 * triangular solves.  Returns 0, or -1 if A is not positive definite.
 */
static int chol_solve(int q, const double *A, const double *Bm, int nc, double *X, double *L) {
  for (int i = 0; i < q; i++) {
    for (int j = 0; j <= i; j++) {
      double v = A[(size_t)i * q + j];
      for (int k = 0; k < j; k++) v -= L[(size_t)i * q + k] * L[(size_t)j * q + k];
      if (i == j) {
        if (!(v > 0.0)) return -1;
        L[(size_t)i * q + i] = sqrt(v);
      } else {
        L[(size_t)i * q + j] = v / L[(size_t)j * q + j];
      }
    }
  }
  for (int c = 0; c < nc; c++) {
    for (int i = 0; i < q; i++) {  /* L y = b */
      double v = Bm[(size_t)i * nc + c];
      for (int k = 0; k < i; k++) v -= L[(size_t)i * q + k] * X[(size_t)k * nc + c];
      X[(size_t)i * nc + c] = v / L[(size_t)i * q + i];
    }
    for (int i = q - 1; i >= 0; i--) {  /* L^T x = y */
      double v = X[(size_t)i * nc + c];
      for (int k = i + 1; k < q; k++) v -= L[(size_t)k * q + i] * X[(size_t)k * nc + c];
      X[(size_t)i * nc + c] = v / L[(size_t)i * q + i];
    }
  }
  return 0;
}

/*
 * ELK.  Each sweep takes the Levenberg-Marquardt step of the residual system
 * with the cell's own Jacobian J_t and damping lambda:
 *   dh = argmin sum_t ||dh_t - J_t dh_{t-1} - r_t||^2 + lambda sum_t ||dh_t||^2,
 * dh_{-1} = 0: the posterior mean of the linear-Gaussian model
 *   dh_t = J_t dh_{t-1} + r_t + w_t,  w_t ~ N(0, I);  0 = dh_t + v_t,
 *   v_t ~ N(0, I / lambda).
 * The Jacobian's structure splits the state into independent blocks (the
 * whole state for dense cells, each channel's (c, h) for the LSTM, each entry
 * for the diagonal GRU); per block the textbook Kalman filter
 *   P^-_t = J_t P_{t-1} J_t^T + I,  m^-_t = J_t m_{t-1} + r_t,
 *   P_t = (lambda P^-_t + I)^{-1} P^-_t,  m_t = (lambda P^-_t + I)^{-1} m^-_t
 * (the gain for an observation of covariance I / lambda), from P_{-1} = 0,
 * m_{-1} = 0, then the Rauch-Tung-Striebel smoother
 *   m^s_{T-1} = m_{T-1},  m^s_t = m_t + G_t (m^s_{t+1} - m^-_{t+1}),
 *   G_t = P_t J_{t+1}^T (P^-_{t+1})^{-1}.
 * lambda = 0 gives the Newton step.  Then h += m^s and the stop rule of
 * orc_deer_approx.
 */
int orc_elk_full(const orc_model *m, double lambda, const double *x, const double *h0, double tol, int max_iters,
                 double *h, int *iters, int *status, double *deltas, int hist_cap) {
  if (!model_ok(m) || max_iters < 1 || !(lambda >= 0.0)) return ORC_EINVAL;
  const int S = swidth(m), Gn = n_gates(m->cell) * m->n, T = m->T, kind = jkind(m->cell);
  const int q = kind == ORC_DENSE ? S : kind == ORC_BLOCK2 ? 2 : 1;  /* block size */
  const int nblk = S / q;
  const size_t js = jsize(m), qq = (size_t)q * q;
  memset(h, 0, sizeof(double) * (size_t)m->B * T * S);
  *iters = 0;
  *status = ORC_OK;
  if (T == 0 || m->B == 0) return ORC_OK;
  for (int k = 1; k <= max_iters; k++) {
    double delta = 0.0;
    int err = 0, nonfin = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : delta) reduction(| : err, nonfin)
    for (int b = 0; b < m->B; b++) {
      double *U = (double *)malloc(sizeof(double) * Gn);
      double *F = (double *)malloc(sizeof(double) * (size_t)T * S);
      double *Jall = (double *)malloc(sizeof(double) * (size_t)T * js);
      double *Jb = (double *)malloc(sizeof(double) * (size_t)T * qq);    /* one block's J_t */
      double *Rb = (double *)malloc(sizeof(double) * (size_t)T * q);     /* its r_t */
      double *Pp = (double *)malloc(sizeof(double) * (size_t)T * qq), *Mp = (double *)malloc(sizeof(double) * (size_t)T * q);
      double *Pf = (double *)malloc(sizeof(double) * (size_t)T * qq), *Mf = (double *)malloc(sizeof(double) * (size_t)T * q);
      double *Ms = (double *)malloc(sizeof(double) * (size_t)T * q);
      double *W1 = (double *)malloc(sizeof(double) * qq), *W2 = (double *)malloc(sizeof(double) * qq);
      double *W3 = (double *)malloc(sizeof(double) * qq), *Lw = (double *)malloc(sizeof(double) * qq);
      double *v1 = (double *)malloc(sizeof(double) * q), *v2 = (double *)malloc(sizeof(double) * q);
      double *zero = (double *)calloc(S, sizeof(double));
      if (!U || !F || !Jall || !Jb || !Rb || !Pp || !Mp || !Pf || !Mf || !Ms || !W1 || !W2 || !W3 || !Lw || !v1 || !v2 ||
          !zero) {
        err |= 1;
      } else {
        double *hb = h + (size_t)b * T * S;
        for (int t = 0; t < T; t++) {
          const double *sp = t == 0 ? (h0 ? h0 + (size_t)b * S : zero) : hb + (size_t)(t - 1) * S;
          input_proj(m, x + ((size_t)b * T + t) * m->d, U);
          cell_fwd(m, sp, U, F + (size_t)t * S, Jall + (size_t)t * js);
        }
        for (int blk = 0; blk < nblk && !err; blk++) {
          /* the block's Jacobians and residuals */
          for (int t = 0; t < T; t++) {
            const double *J = Jall + (size_t)t * js;
            for (int i = 0; i < q; i++) {
              const int gi = blk * q + i;
              for (int j = 0; j < q; j++) {
                double v;
                if (kind == ORC_DENSE) v = J[(size_t)gi * S + blk * q + j];
                else if (kind == ORC_DIAG) v = J[gi];
                else v = J[(size_t)4 * blk + 2 * i + j];
                Jb[(size_t)t * qq + (size_t)i * q + j] = v;
              }
              Rb[(size_t)t * q + i] = F[(size_t)t * S + gi] - hb[(size_t)t * S + gi];
            }
          }
          /* Kalman filter */
          double *P = W3, *mv = v2;
          for (size_t e = 0; e < qq; e++) P[e] = 0.0;
          for (int i = 0; i < q; i++) mv[i] = 0.0;
          for (int t = 0; t < T && !err; t++) {
            const double *J = Jb + (size_t)t * qq;
            double *pp = Pp + (size_t)t * qq, *mp = Mp + (size_t)t * q;
            for (int i = 0; i < q; i++) {            /* W1 = J P */
              for (int j = 0; j < q; j++) {
                double a = 0.0;
                for (int l = 0; l < q; l++) a += J[(size_t)i * q + l] * P[(size_t)l * q + j];
                W1[(size_t)i * q + j] = a;
              }
            }
            for (int i = 0; i < q; i++) {            /* P^- = W1 J^T + I,  m^- = J m + r */
              for (int j = 0; j < q; j++) {
                double a = i == j ? 1.0 : 0.0;
                for (int l = 0; l < q; l++) a += W1[(size_t)i * q + l] * J[(size_t)j * q + l];
                pp[(size_t)i * q + j] = a;
              }
              double a = Rb[(size_t)t * q + i];
              for (int l = 0; l < q; l++) a += J[(size_t)i * q + l] * mv[l];
              mp[i] = a;
            }
            for (size_t e = 0; e < qq; e++) W2[e] = lambda * pp[e];   /* lambda P^- + I */
            for (int i = 0; i < q; i++) W2[(size_t)i * q + i] += 1.0;
            double *pf = Pf + (size_t)t * qq, *mf = Mf + (size_t)t * q;
            if (chol_solve(q, W2, pp, q, pf, Lw) || chol_solve(q, W2, mp, 1, mf, Lw)) { nonfin = 1; break; }
            memcpy(P, pf, sizeof(double) * qq);
            memcpy(mv, mf, sizeof(double) * q);
          }
          /* Rauch-Tung-Striebel smoother */
          memcpy(Ms + (size_t)(T - 1) * q, Mf + (size_t)(T - 1) * q, sizeof(double) * q);
          for (int t = T - 2; t >= 0 && !nonfin; t--) {
            const double *Jn = Jb + (size_t)(t + 1) * qq, *pf = Pf + (size_t)t * qq;
            for (int i = 0; i < q; i++) {            /* W1 = J_{t+1} P_t */
              for (int j = 0; j < q; j++) {
                double a = 0.0;
                for (int l = 0; l < q; l++) a += Jn[(size_t)i * q + l] * pf[(size_t)l * q + j];
                W1[(size_t)i * q + j] = a;
              }
            }
            /* G^T = (P^-_{t+1})^{-1} J_{t+1} P_t  (both covariances symmetric) */
            if (chol_solve(q, Pp + (size_t)(t + 1) * qq, W1, q, W2, Lw)) { nonfin = 1; break; }
            for (int i = 0; i < q; i++) v1[i] = Ms[(size_t)(t + 1) * q + i] - Mp[(size_t)(t + 1) * q + i];
            for (int i = 0; i < q; i++) {
              double a = Mf[(size_t)t * q + i];
              for (int l = 0; l < q; l++) a += W2[(size_t)l * q + i] * v1[l];
              Ms[(size_t)t * q + i] = a;
            }
          }
          for (int t = 0; t < T; t++) {
            for (int i = 0; i < q; i++) {
              const double v = Ms[(size_t)t * q + i];
              hb[(size_t)t * S + blk * q + i] += v;
              const double a = fabs(v);
              if (!isfinite(a)) nonfin = 1;
              else if (a > delta) delta = a;
            }
          }
        }
      }
      free(U); free(F); free(Jall); free(Jb); free(Rb); free(Pp); free(Mp); free(Pf); free(Mf); free(Ms);
      free(W1); free(W2); free(W3); free(Lw); free(v1); free(v2); free(zero);
    }
    if (err) return ORC_ENOMEM;
    if (nonfin) delta = NAN;
    if (deltas && k <= hist_cap) deltas[k - 1] = delta;
    *iters = k;
    if (!isfinite(delta)) { *status = ORC_NONFINITE; return ORC_OK; }
    if (tol > 0.0 && delta < tol) { *status = ORC_OK; return ORC_OK; }
    if (k == T) { *status = ORC_OK; return ORC_OK; }
  }
  *status = tol > 0.0 ? ORC_NOT_CONVERGED : ORC_OK;
  return ORC_OK;
}
