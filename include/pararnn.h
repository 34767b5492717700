/*
 * pararnn.h -- C ABI of the MI355X (gfx950) library for Newton (DEER) and
 * quasi-Newton (quasi-DEER) evaluation of nonlinear RNNs over the sequence
 * length, and for the adjoint gradient of that evaluation.
 *
 * The method: the T recurrences h_t = f(h_{t-1}, x_t) are one nonlinear system
 * of equations (ParaRNN abstract; Gonzalez et al. abstract: the states are the
 * solution of a fixed-point problem).  Each Newton sweep evaluates the cell
 * and its Jacobian J_t = df/dh at every step, forms r_t = f_t - h_t, solves the
 * linear recurrence dh_t = J_t dh_{t-1} + r_t with a parallel associative
 * prefix scan, and updates h += dh ("Parallelizing non-linear sequential models
 * over the sequence length", Approach).  Jacobians are dense (full DEER),
 * diagonal (quasi-DEER / ParaGRU) or 2x2 block-diagonal (ParaLSTM) (Para-Seq
 * README, Main features).  The gradient needs one reverse linear solve with the
 * transposed Jacobians (DEER summary, Surprising findings).
 *
 * Conventions for every entry point
 *  - All array arguments are device pointers to caller-owned memory, row-major,
 *    batch-first ([B, T, ...]).  The library never allocates device memory;
 *    all scratch lives in the caller's workspace.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is ordered
 *    on it.  pararnn_solve returns after it has read the iteration count back
 *    (host-synchronous on `stream`); the other calls are asynchronous.
 *  - Negative return values are errors (outputs undefined); positive values
 *    are soft failures whose outputs are valid.  Arguments are validated before
 *    any HIP call, so PR_EINVAL / PR_EWORKSPACE / PR_EUNSUPPORTED never touch
 *    the device.  pararnn_last_error() gives a message for the calling thread.
 *  - Calls on the same workspace must not overlap; distinct workspaces may be
 *    used concurrently.
 *
 * Co-residency.  Some kernels chain the tiles of a sequence with a decoupled
 * look-back: a tile waits until its predecessors have published their
 * aggregates.  They run as persistent grids sized to the blocks the device
 * holds at once, and assume every block of the grid is resident: the
 * scalar-state sweep and adjoint (n = d = 1), the time-parallel sweep and
 * adjoint of the small dense cells (n <= 8), and pararnn_affine_scan.  The
 * channel-parallel passes (GRU_DIAG, LSTM_CIFG_DIAG), the dense n = 64 GRU,
 * quasi-ELK and lsim have no waits between blocks.  If kernels on other
 * streams keep compute units busy while such a grid runs, its blocks start
 * late, and a wait that sees no progress for 2^16 polls (tens of
 * milliseconds) gives up: the tile's carry becomes NaN, which makes every
 * later state of that sequence NaN, and a fault flag is set in the
 * workspace.  pararnn_solve checks the flag at each poll and then returns
 * PR_ELOOKBACK; the asynchronous calls cannot return it, and their outputs
 * hold the NaNs.  Two such grids on two streams at once can both give up.
 *
 * Run-to-run reproducibility.  How many predecessor aggregates a look-back
 * composes depends on timing, so the kernels listed above can round
 * differently from run to run (fp32 rounding of the carried state: up to a
 * few units in the last place per composed tile; differences below 1e-6 on
 * the scalar GRU at length 2^20).  The stop sweep can then differ between
 * runs only where a delta lies within that distance of tol.  Every other
 * kernel combines in a fixed order and is bitwise reproducible.
 */
#ifndef PARARNN_H
#define PARARNN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- cells (the standard RNN cells Para-Seq keeps, README intro) --------- */
/* f = tanh(W_x x + b_x + W_h h + b_h)                              G = 1, S = n */
#define PR_CELL_TANH_RNN 0
/* PyTorch GRU, gate order r|z|n, b_hn inside r*(.), h' = (1-z) c + z h.  G = 3 */
#define PR_CELL_GRU 1
/* The same GRU with diagonal recurrent weights W_h = [a_r | a_z | a_n] (each [n])
 * (ParaGRU, Para-Seq README Main features).                        G = 3, S = n */
#define PR_CELL_GRU_DIAG 2
/* CIFG ParaLSTM with peepholes, per channel state (c, h) stored interleaved:
 *   f = sigm(U_f + w_f h + p_f c + b_f), g = tanh(U_g + w_g h + b_g),
 *   c' = f c + (1-f) g, o = sigm(U_o + w_o h + p_o c' + b_o), h' = o tanh(c').
 * W_h = [w_f | w_g | w_o] (each [n]); peep = [p_f | p_o].       G = 3, S = 2n */
#define PR_CELL_LSTM_CIFG_DIAG 3
/* f = W_x x + b_x + W_h h + b_h: a linear state-space recurrence; Newton is
 * exact after one update.                                          G = 1, S = n */
#define PR_CELL_LINEAR 4

/* ---- Jacobian used by the linear solve of each sweep --------------------- */
/* The cell's own structure gives Newton (DEER).  A simpler one gives a
 * quasi-Newton sweep with the same fixed point (Gonzalez et al. abstract:
 * quasi-Newton approximations converge comparably, use less memory and are
 * faster; Para-Seq README, Main features: Jacobi, quasi-DEER and DEER
 * solvers): every variant reproduces the sequential evaluation exactly on
 * the first k steps after k sweeps, so a solve still ends by sweep T.  Only
 * the solve changes; residuals, updates and pararnn_adjoint use the cell's
 * exact Jacobian whatever jac the solve used.                                */
#define PR_JAC_DENSE 0   /* n x n per step: Newton for TANH_RNN, GRU, LINEAR     */
#define PR_JAC_DIAG 1    /* the diagonal: Newton for GRU_DIAG (and dense cells with
                            n == 1); quasi-DEER for the other cells (the LSTM
                            keeps dc'/dc and dh'/dh of each 2x2 block)           */
#define PR_JAC_BLOCK2 2  /* 2x2 per channel: Newton for LSTM_CIFG_DIAG           */
#define PR_JAC_ZERO 3    /* none: Jacobi (Picard) sweeps h_t <- f(h_{t-1}, x_t),
                            any cell                                             */

/* ---- storage dtype of x, weights, h0, h, g, lambda, dx, dh0 -------------- */
/* Arithmetic, scan carries and the convergence measure are always fp32.
 * Gradients of the weights (pr_grads) are always fp32.                       */
#define PR_F32 0
#define PR_BF16 1

/* ---- status codes -------------------------------------------------------- */
#define PR_OK 0
#define PR_EINVAL (-1)        /* bad enum, size <= 0, NULL required pointer, max_iters < 1 */
#define PR_EWORKSPACE (-2)    /* workspace NULL or smaller than pararnn_*workspace_bytes   */
#define PR_EHIP (-3)          /* a HIP runtime call failed                                */
#define PR_EUNSUPPORTED (-5)  /* valid problem the library has no kernel for              */
#define PR_ELOOKBACK (-6)     /* a bounded look-back wait gave up (see "Co-residency")     */
#define PR_NOT_CONVERGED 1    /* max_iters sweeps, delta never < tol; h = last iterate   */
#define PR_NONFINITE 2        /* delta became NaN/Inf; h = that iterate                   */

typedef struct {
  int cell;   /* PR_CELL_*                              */
  int jac;    /* PR_JAC_*: the cell's own, DIAG or ZERO  */
  int dtype;  /* PR_F32 or PR_BF16                      */
  int B;      /* batch (independent sequences), >= 1    */
  int T;      /* sequence length, >= 1                  */
  int d;      /* input width, >= 1                      */
  int n;      /* hidden channels, >= 1 (state S = n or 2n) */
} pr_problem;

/* Weights, device pointers in the problem's storage dtype.  G = gate count. */
typedef struct {
  const void *W_x;  /* [G*n, d], required                                   */
  const void *b_x;  /* [G*n] or NULL (= 0)                                  */
  const void *W_h;  /* dense cells [G*n, n]; diagonal cells [G*n]; required */
  const void *b_h;  /* [G*n] or NULL (= 0)                                  */
  const void *peep; /* LSTM: [2n] = p_f | p_o, required; others: ignored    */
} pr_weights;

/* Weight gradients, fp32 device pointers with the shapes of pr_weights; any
 * field may be NULL to skip it.  They are overwritten, not accumulated.      */
typedef struct {
  float *W_x;
  float *b_x;
  float *W_h;
  float *b_h;
  float *peep;
} pr_grads;

/* Bytes of workspace pararnn_solve (with_adjoint = 0) or both pararnn_solve
 * and pararnn_adjoint (with_adjoint = 1) need; 0 for an invalid problem. */
size_t pararnn_workspace_bytes(const pr_problem *p, int with_adjoint);

/*
 * Newton (or, per p->jac, quasi-Newton or Jacobi) solve of the recurrence
 * from the initial guess h = 0 everywhere.  Kernels exist for: TANH_RNN, GRU
 * and LINEAR with n <= 8 and d <= 8 (fp32, any jac); GRU and TANH_RNN with
 * any other n <= 64 (fp32; DENSE, DIAG or ZERO); GRU_DIAG and LSTM_CIFG_DIAG
 * (fp32 or bf16, any jac that suits them).  Other problems return
 * PR_EUNSUPPORTED.  A GRU with n < 64 or a tanh RNN outside the first group
 * runs on the n = 64 GRU kernels with its weights, biases and h0 padded with
 * zeros into the front of the workspace (a tanh RNN's as the GRU's
 * candidate gate, with the reset gate held at 1 and the update gate at 0 by
 * input biases of +-1e30): the padded channels stay exactly 0 and couple to
 * nothing, so iterates, deltas, sweep counts and gradients are those of the
 * n-wide problem of the cell itself (pararnn_workspace_bytes includes the
 * padded copies).
 *   x     [B, T, d]                input sequence
 *   h0    [B, S] or NULL (= 0)     state before the first step
 *   tol   stop when delta_k = max over (b, t, i) of |dh| is < tol; tol <= 0
 *         runs exactly max_iters sweeps (fixed-iteration mode)
 *   max_iters >= 1; a solve also stops after sweep T, where Newton is exact
 *   h     [B, T, S] output: the final iterate (it is used as the iterate in
 *         place, so it must not alias x or h0)
 *   iters (host, may be NULL) number of sweeps run, including the one that met tol
 *   delta_hist (host, may be NULL) delta_k for k = 1 .. min(iters, hist_cap, 1024)
 * Returns PR_OK, PR_NOT_CONVERGED (tol > 0 and max_iters sweeps done),
 * PR_NONFINITE, or an error.
 */
int pararnn_solve(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                  int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, void *workspace,
                  size_t ws_bytes, void *stream);

/*
 * ELK and quasi-ELK solves (Gonzalez et al. abstract: ELK stabilises DEER
 * through the connection between Levenberg-Marquardt and Kalman smoothing;
 * Para-Seq README, Main features: ELK and quasi-ELK solvers).  Each sweep
 * takes the damped step
 *   dh = argmin sum_t ||dh_t - M_t dh_{t-1} - r_t||^2 + lambda ||dh||^2,
 * the Kalman filter / Rauch-Tung-Striebel smoother mean of
 * dh_t = M_t dh_{t-1} + r_t + N(0, I) observed as 0 with covariance I/lambda,
 * then h += dh.  p->jac chooses M_t: the cell's own Jacobian (ELK: the LSTM's
 * 2x2 blocks with PR_JAC_BLOCK2, the dense cells' full n x n Jacobian with
 * PR_JAC_DENSE) or its diagonal (quasi-ELK, PR_JAC_DIAG; the LSTM's dc'/dc
 * and dh'/dh); PR_JAC_ZERO is refused with PR_EINVAL.  lambda = 0 is Newton's
 * (quasi-DEER's) step; larger lambda shortens the steps
 * (lambda ||dh||^2 <= ||r||^2).  Kernels exist for every problem
 * pararnn_solve supports: the tanh RNN, GRU and linear cell with n <= 8 and
 * d <= 8, the dense GRU and tanh RNN with any other n <= 64 (fp32; ELK there
 * holds three 64 x 64 fp32 blocks per step in the workspace), GRU_DIAG and
 * LSTM_CIFG_DIAG (fp32 or bf16); other problems return PR_EUNSUPPORTED.
 * Arguments and results as
 * pararnn_solve, plus lambda (>= 0, finite); the workspace must hold
 * pararnn_elk_workspace_bytes (which also covers pararnn_adjoint).
 */
size_t pararnn_elk_workspace_bytes(const pr_problem *p);
int pararnn_solve_elk(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float lambda,
                      float tol, int max_iters, void *h, int *iters, float *delta_hist, int hist_cap,
                      void *workspace, size_t ws_bytes, void *stream);

/*
 * Gradient of L = sum_{b,t} <g_t, h_t> at the trajectory h (normally the
 * output of pararnn_solve), by one reverse linear solve
 *   lambda_t = g_t + J_{t+1}^T lambda_{t+1},  lambda_T-1 = g_T-1,
 * with J re-evaluated at h, followed by the chain rule through each cell.
 *   g      [B, T, S]               upstream gradient dL/dh
 *   lambda [B, T, S] or NULL       output: the adjoint state
 *   dx     [B, T, d] or NULL       output: dL/dx
 *   dh0    [B, S] or NULL          output: dL/dh0
 *   dW     NULL or the fp32 weight-gradient outputs (fields may be NULL)
 * The workspace must be at least pararnn_workspace_bytes(p, 1).
 */
int pararnn_adjoint(const pr_problem *p, const pr_weights *w, const void *x, const void *h0,
                    const void *h, const void *g, void *lambda, void *dx, void *dh0, const pr_grads *dW,
                    void *workspace, size_t ws_bytes, void *stream);

/*
 * pararnn_solve followed by pararnn_adjoint at the returned trajectory, in
 * one call (a training step's forward and backward evaluation; DEER summary,
 * Surprising findings: the gradient costs one more linear solve).  Results
 * are those of the two calls; the adjoint reuses the input projection U the
 * solve left in the workspace instead of computing it again.  The adjoint is enqueued right behind the
 * solve's first batch of sweeps, before the host waits for its convergence
 * poll, when that batch is sure to be the last (tol <= 0: a fixed number of
 * sweeps) or, for n = d = 1, when the previous call on the same problem,
 * tol and max_iters converged within it; if the solve then needs more
 * sweeps, its state is restored and the adjoint runs again at the end.
 * Otherwise the adjoint follows the solve's last poll.  Arguments as the two
 * calls (h is the solve's output and the adjoint's trajectory); the
 * workspace must be at least pararnn_workspace_bytes(p, 1).  Returns the
 * solve's error, else the adjoint's error (its arguments are checked when
 * it is enqueued, after the solve has run), else the solve's status (PR_OK,
 * PR_NOT_CONVERGED or PR_NONFINITE; with PR_NONFINITE the adjoint's outputs
 * are unspecified).  The adjoint's outputs are complete once the stream
 * reaches this point.
 */
int pararnn_solve_adjoint(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                          int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, const void *g,
                          void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace, size_t ws_bytes,
                          void *stream);

/*
 * The linear recurrence alone (the Newton inner solve), fp32, per sequence:
 *   reverse = 0:  y_t = A_t y_{t-1} + b_t,  y_{-1} = 0
 *   reverse = 1:  y_t = A_t y_{t+1} + b_t,  y_T = 0
 * PR_JAC_DIAG:   A, b, y [B, T, n]
 * PR_JAC_BLOCK2: A [B, T, n, 2, 2], b, y [B, T, n, 2]
 * PR_JAC_DENSE:  A [B, T, n, n], b, y [B, T, n]   (n <= 8)
 */
size_t pararnn_scan_workspace_bytes(int jac, int B, int T, int n);
int pararnn_affine_scan(int jac, int B, int T, int n, int reverse, const float *A, const float *b,
                        float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * pararnn_affine_scan without a workspace, for callers that cannot allocate
 * device memory at all: code under stream capture, tight serving loops,
 * harnesses that forbid allocation.  The same recurrence, layouts, kernels
 * and results as pararnn_affine_scan (jac, B, T, n, reverse, A, b, y as
 * there).  Its scratch (look-back descriptors and a state record) lives in
 * a static device array of PR_NOALLOC_SCRATCH_BYTES that every device this
 * entry point runs on holds until the process ends; the call itself
 * allocates nothing and makes no allocating runtime call.  A problem whose
 * pararnn_scan_workspace_bytes exceeds PR_NOALLOC_SCRATCH_BYTES returns
 * PR_EWORKSPACE before any HIP call.  `stream` must belong to the current
 * device.  All calls on one device share that device's array, which keeps
 * the last call's contents (each call clears what it needs before its
 * scan): calls that overlap on one device (two streams, or two host
 * threads) race and must be serialised by the caller.  Asynchronous on
 * `stream`.
 */
#define PR_NOALLOC_SCRATCH_BYTES (16u << 20)
int pararnn_affine_scan_noalloc(int jac, int B, int T, int n, int reverse, const float *A, const float *b, float *y,
                                void *stream);

/*
 * Linear state-space simulation (Para-Seq README, Main features: ODE
 * solvers; Example: lsim(A, B, C, D, U, t)): the system dx/dt = A x + B u,
 * y = C x + D u sampled every dt with the input held between samples
 * (zero-order hold), i.e. per sequence
 *   x_0 = x0,  y_k = C x_k + D u_k,  x_{k+1} = Ad x_k + Bd u_k,
 *   Ad = exp(A dt),  Bd = int_0^dt exp(A s) ds B,
 * evaluated with parallel scans over time (no Newton loop).  fp32 storage;
 * the discretisation is computed on the device in fp64.
 *   A [nx, nx], B [nx, m], C [p, nx], D [p, m]   row-major, shared by all sequences
 *   U  [B, T, m]            input samples
 *   x0 [B, nx] or NULL (= 0)
 *   x  [B, T, nx] or NULL   output: x_k, the state at sample k
 *   y  [B, T, p]            output
 * 1 <= nx, m, p <= 8 (else PR_EUNSUPPORTED); dt > 0 and finite.  The
 * workspace (256-byte aligned) must hold pararnn_lsim_workspace_bytes.
 * Asynchronous on `stream`.
 */
size_t pararnn_lsim_workspace_bytes(int B, int T, int nx, int m, int p);
int pararnn_lsim(int B, int T, int nx, int m, int p, const float *A, const float *Bm, const float *C,
                 const float *D, float dt, const float *U, const float *x0, float *x, float *y,
                 void *workspace, size_t ws_bytes, void *stream);

/*
 * Kernel timing for profiling and benchmarks (per calling thread).
 * pararnn_trace(1) clears the counters and starts bracketing, with HIP events
 * on the call's stream, the Newton sweeps and the main kernel of each
 * adjoint; pararnn_trace(0) stops.  Sweeps are bracketed per batch of
 * back-to-back launches (per launch on the dense n = 64 path, whose parts are
 * timed too); launches after the stop rule has fired exit at once and are
 * not counted, their few microseconds stay in the total.
 * pararnn_trace_read waits for pending events and returns the totals (any
 * pointer may be NULL).
 */
int pararnn_trace(int enable);
int pararnn_trace_read(double *sweep_ms, long long *sweep_launches, double *adjoint_ms, long long *adjoint_launches);
/* Totals of one category: 0 Newton sweeps, 1 the adjoint's scan kernel(s),
 * 2 the input projection, 3 the adjoint's products and reductions, 4 the
 * chunk-product kernel of the dense n = 64 path (within its sweeps; with an
 * approximate Jacobian, its chunk-carry kernel), 5 linear state-space
 * simulations. */
#define PR_TRACE_SWEEP 0
#define PR_TRACE_ADJOINT 1
#define PR_TRACE_PROJECTION 2
#define PR_TRACE_ADJOINT_PRODUCTS 3
#define PR_TRACE_DENSE_PRODUCTS 4
#define PR_TRACE_LSIM 5  /* the kernels of each pararnn_lsim call */
int pararnn_trace_kernel(int which, double *ms, long long *launches);

/* Static text for a status code. */
const char *pararnn_strerror(int status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char *pararnn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PARARNN_H */
