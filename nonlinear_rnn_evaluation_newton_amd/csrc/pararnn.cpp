// C ABI of libpararnn: argument validation, workspace planning, the host side
// of the Newton loop (asynchronous sweeps, on-device stop rule, rare polls of
// a 4 KB state record) and dispatch to the kernel families.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

#include "internal.h"
#include "pararnn.h"

using namespace pr;

namespace pr {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

void clear_error() { g_err.clear(); }

}  // namespace pr

namespace {

#define HIPCHK(expr)                                                                          \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(PR_EHIP, "%s: %s", #expr, hipGetErrorString(e_));       \
  } while (0)

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

enum { PATH_NONE = 0, PATH_TIME = 1, PATH_CHAN = 2, PATH_D64 = 3 };

struct Plan {
  int path = PATH_NONE;
  int approx = APX_NEWTON;  // Jacobian of the sweeps' linear solve (the adjoint always uses the cell's)
  int G = 1, S = 1, N = 1, SW = 1;
  int tile = 0, tps = 0, ntiles = 0;
  // scalar-state sweep (n = d = 1, T % 4 == 0): its own tile size
  int scalar_ok = 0, tps_s = 0, ntiles_s = 0, tps_sa = 0, ntiles_sa = 0;
  // channel path: stripes (sequence x channel group), tiles of sweep / adjoint
  int stripes = 0, CH = 0;
  // channel path, streaming sweep passes (tiles of CHAN2_TT steps)
  int tps_2 = 0, ntiles_2 = 0;
  size_t off_state = 0, off_agg = 0, off_incl = 0, off_bnd = 0, off_part = 0;
  size_t off_U = 0, off_dU = 0, off_gws = 0, off_coef = 0;
  size_t off_cb = 0;              // channel path: the projection's fp32 bias (folded recurrent biases) and column scale
  size_t off_wt = 0;              // channel path adjoint: W_x^T
  size_t off_red = 0;             // channel path adjoint: fp64 split sums of the weight partials
  size_t off_tn = 0;              // dense n = 64 adjoint: partials of the K-outer weight products
  // dense n = 64 path
  int cps = 0, nchunks = 0;
  size_t off_gates = 0, off_aggP = 0, off_aggb = 0, off_carry = 0, off_dA = 0, off_hprev = 0, off_csum = 0;
  size_t zero_bytes = 0;     // bytes cleared at the start of each call
  size_t solve_bytes = 0, adjoint_bytes = 0;
};

int gates_of(int cell) { return (cell == PR_CELL_GRU || cell == PR_CELL_GRU_DIAG || cell == PR_CELL_LSTM_CIFG_DIAG) ? 3 : 1; }

// Validates the problem and picks the kernel family.  Returns PR_OK,
// PR_EINVAL or PR_EUNSUPPORTED.
int make_plan(const pr_problem *p, Plan *pl) {
  if (!p) return fail(PR_EINVAL, "problem is NULL");
  if (p->cell < 0 || p->cell > 4) return fail(PR_EINVAL, "unknown cell %d", p->cell);
  if (p->jac < 0 || p->jac > 3) return fail(PR_EINVAL, "unknown jac %d", p->jac);
  if (p->dtype != PR_F32 && p->dtype != PR_BF16) return fail(PR_EINVAL, "unknown dtype %d", p->dtype);
  if (p->B < 1 || p->T < 1 || p->d < 1 || p->n < 1)
    return fail(PR_EINVAL, "sizes must be >= 1 (B=%d T=%d d=%d n=%d)", p->B, p->T, p->d, p->n);
  const bool dense_cell = p->cell == PR_CELL_TANH_RNN || p->cell == PR_CELL_GRU || p->cell == PR_CELL_LINEAR;
  // the cell's own structure is Newton; PR_JAC_DIAG on a dense or block cell
  // keeps the diagonal (quasi-DEER); PR_JAC_ZERO runs Jacobi sweeps
  bool jac_ok = p->jac == PR_JAC_DIAG || p->jac == PR_JAC_ZERO;
  if (dense_cell) jac_ok = jac_ok || p->jac == PR_JAC_DENSE;
  if (p->cell == PR_CELL_LSTM_CIFG_DIAG) jac_ok = jac_ok || p->jac == PR_JAC_BLOCK2;
  if (!jac_ok) return fail(PR_EINVAL, "jac %d does not suit cell %d", p->jac, p->cell);
  if (p->jac == PR_JAC_ZERO) pl->approx = APX_ZERO;
  else if (p->jac == PR_JAC_DIAG && p->cell != PR_CELL_GRU_DIAG && !(dense_cell && p->n == 1)) pl->approx = APX_DIAG;
  if ((double)p->B * p->T * p->n * 2 > 2147483647.0 * 64) return fail(PR_EUNSUPPORTED, "problem too large");
  // rows of the products and row indices are 32-bit
  if ((long long)p->B * p->T > 2147483647LL)
    return fail(PR_EUNSUPPORTED, "B * T = %lld rows exceed 2^31 - 1", (long long)p->B * p->T);

  pl->G = gates_of(p->cell);
  pl->S = p->cell == PR_CELL_LSTM_CIFG_DIAG ? 2 * p->n : p->n;
  if (dense_cell && p->n <= 8 && p->d <= DX_FUSED) {
    if (p->dtype != PR_F32) return fail(PR_EUNSUPPORTED, "dense cells with n <= 8 run in fp32 storage only");
    pl->path = PATH_TIME;
    pl->N = time_padded_n(p->n);
    pl->tile = time_tile(pl->N);
    pl->tps = (p->T + pl->tile - 1) / pl->tile;
    if ((long long)pl->tps * p->B > 2147483647LL) return fail(PR_EUNSUPPORTED, "too many tiles");
    pl->ntiles = pl->tps * p->B;
    const int N = pl->N;
    int nt = pl->ntiles;  // descriptor and boundary slots for either sweep
    // (buffer resources of the scalar sweep address rows, descriptors and
    // boundary states with 31-bit byte offsets)
    if (pl->approx == APX_NEWTON && p->n == 1 && p->d == 1 && p->T % 4 == 0 && (long long)p->T * 4 < (1LL << 31) &&
        (long long)p->B * ((p->T + scalar_adj_tile() - 1) / scalar_adj_tile()) * 16 < (1LL << 31)) {
      pl->scalar_ok = 1;
      pl->tps_s = (p->T + scalar_tile() - 1) / scalar_tile();
      if ((long long)pl->tps_s * p->B > 2147483647LL) return fail(PR_EUNSUPPORTED, "too many tiles");
      pl->ntiles_s = pl->tps_s * p->B;
      pl->tps_sa = (p->T + scalar_adj_tile() - 1) / scalar_adj_tile();
      if ((long long)pl->tps_sa * p->B > 2147483647LL) return fail(PR_EUNSUPPORTED, "too many tiles");
      pl->ntiles_sa = pl->tps_sa * p->B;
      nt = nt > pl->ntiles_s ? nt : pl->ntiles_s;
      nt = nt > pl->ntiles_sa ? nt : pl->ntiles_sa;
    }
    size_t o = 0;
    pl->off_state = o; o = align256(o + sizeof(SolveState));
    pl->off_agg = o; o = align256(o + (size_t)nt * (N * N + N) * 8);
    pl->off_incl = o; o = align256(o + (size_t)nt * N * 8);
    pl->zero_bytes = o;
    pl->off_bnd = o; o = align256(o + (size_t)2 * nt * N * 4);
    pl->off_coef = o; o = align256(o + 64 * 4);
    pl->solve_bytes = o;
    pl->off_part = o; o = align256(o + (size_t)nt * time_part_count(p->cell, N) * 4);
    pl->adjoint_bytes = o;
    return PR_OK;
  }
  if (p->cell == PR_CELL_GRU && p->n == D64_N) {
    if (p->dtype != PR_F32) return fail(PR_EUNSUPPORTED, "the dense n = 64 GRU runs in fp32 storage only");
    pl->path = PATH_D64;
    pl->cps = (p->T + D64_L - 1) / D64_L;
    if ((long long)pl->cps * p->B > 2147483647LL || (long long)p->B * p->T * 320 > (1LL << 62))
      return fail(PR_EUNSUPPORTED, "problem too large");
    pl->nchunks = pl->cps * p->B;
    const size_t rows = (size_t)p->B * p->T;
    size_t o = 0;
    pl->off_state = o; o = align256(o + sizeof(SolveState));
    pl->zero_bytes = o;
    pl->off_U = o; o = align256(o + rows * 192 * 4);
    pl->off_gates = o; o = align256(o + rows * 320 * 4);
    pl->off_aggP = o; o = align256(o + (size_t)pl->nchunks * 4096 * 4);
    pl->off_aggb = o; o = align256(o + (size_t)pl->nchunks * 64 * 4);
    pl->off_carry = o; o = align256(o + (size_t)pl->nchunks * 64 * 4);
    pl->solve_bytes = o;
    pl->off_dU = o; o = align256(o + rows * 192 * 4);
    pl->off_dA = o; o = align256(o + rows * 192 * 4);
    pl->off_hprev = o; o = align256(o + rows * 64 * 4);
    pl->off_csum = o; o = align256(o + (size_t)512 * 192 * 8);
    const int K = (int)(rows < 2147483647ULL ? rows : 2147483647ULL);
    const int s1 = gemm_splits(192, p->d, K), s2 = gemm_splits(192, 64, K);
    const size_t gw = (size_t)(s1 > 1 ? s1 * 192 * p->d : 0) > (size_t)(s2 > 1 ? s2 * 192 * 64 : 0)
                          ? (size_t)(s1 > 1 ? s1 * 192 * p->d : 0)
                          : (size_t)(s2 > 1 ? s2 * 192 * 64 : 0);
    pl->off_gws = o; o = align256(o + gw * 4);
    pl->off_tn = o; o = align256(o + tn_workspace_bytes(K));
    pl->adjoint_bytes = o;
    return PR_OK;
  }
  if (p->cell == PR_CELL_GRU_DIAG || p->cell == PR_CELL_LSTM_CIFG_DIAG) {
    const int kc = p->cell == PR_CELL_GRU_DIAG ? C_GRU_DIAG : C_LSTM;
    pl->path = PATH_CHAN;
    pl->SW = p->cell == PR_CELL_LSTM_CIFG_DIAG ? 2 : 1;
    const ChanGeomInfo g = chan2_geom(kc, p->n);
    pl->CH = g.CH;
    const long long CG = (p->n + g.CH - 1) / g.CH;
    if ((long long)p->B * CG > 2147483647LL) return fail(PR_EUNSUPPORTED, "too many stripes");
    pl->stripes = (int)(p->B * CG);
    const size_t es = p->dtype == PR_BF16 ? 2 : 4;
    // a tile's rows of U (and the load groups just past it) are addressed
    // with 31-bit byte offsets
    if ((long long)(2 * CHAN2_TT) * 3 * p->n * (long long)es >= (1LL << 31))
      return fail(PR_EUNSUPPORTED, "channel count too large");
    pl->tps_2 = (p->T + CHAN2_TT - 1) / CHAN2_TT;
    if ((long long)pl->tps_2 * pl->stripes > 2147483647LL) return fail(PR_EUNSUPPORTED, "too many tiles");
    pl->ntiles_2 = pl->tps_2 * pl->stripes;
    const int SW = pl->SW, AW = SW * SW + SW;
    const size_t nt = (size_t)pl->ntiles_2;
    const size_t rows = (size_t)p->B * p->T;
    size_t o = 0;
    pl->off_state = o; o = align256(o + sizeof(SolveState));
    pl->zero_bytes = o;
    // tile aggregates, carries and each tile's last state (written before
    // they are read in every call, so never cleared)
    pl->off_agg = o; o = align256(o + nt * g.CH * AW * 4);
    pl->off_incl = o; o = align256(o + nt * g.CH * SW * 4);
    pl->off_bnd = o; o = align256(o + (size_t)2 * nt * g.CH * SW * 4);
    pl->off_U = o; o = align256(o + rows * 3 * p->n * es);
    pl->off_cb = o; o = align256(o + (size_t)6 * p->n * 4);
    pl->solve_bytes = o;
    pl->off_dU = o; o = align256(o + rows * 3 * p->n * es);
    pl->off_part = o; o = align256(o + nt * g.CH * 11 * 4);
    pl->off_red = o; o = align256(o + (size_t)CHAN_RED_SPLITS * p->n * 11 * 8);
    const int splits = gemm_splits(3 * p->n, p->d, (int)(rows < 2147483647ULL ? rows : 2147483647ULL),
                                   p->dtype == PR_BF16);
    pl->off_gws = o; o = align256(o + (splits > 1 ? (size_t)splits * 3 * p->n * p->d * 4 : 0));
    pl->off_wt = o; o = align256(o + (size_t)3 * p->n * p->d * es);
    pl->adjoint_bytes = o;
    return PR_OK;
  }
  return fail(PR_EUNSUPPORTED, "no kernel for cell %d jac %d dtype %d n %d d %d", p->cell, p->jac, p->dtype, p->n,
              p->d);
}

// U = x W_x^T + b_x on MFMA ([B*T, d] x [3n, d]^T).  For the per-channel
// cells (cb non-null, 6n floats) the bias also takes the recurrent biases of
// the gates whose pre-activation is a plain sum (the LSTM's three, the GRU's r
// and z), summed in fp32 into cb, and each gate's column is scaled by its
// exp2 factor: the cells then add no bias and multiply no constant per step.
hipError_t input_projection(const pr_problem *p, const pr_weights *w, const void *x, void *U, hipStream_t s,
                            float *cb = nullptr) {
  const bool bf = p->dtype == PR_BF16;
  const size_t es = bf ? 2 : 4;
  GemmArgs g{};
  g.A = x; g.B = w->W_x; g.C = U; g.bias = w->b_x; g.ws = nullptr;
  if (cb) {
    const hipError_t e =
        launch_fold_bias(bf, w->b_x, w->b_h, p->n, p->cell == PR_CELL_LSTM_CIFG_DIAG ? C_LSTM : C_GRU_DIAG, cb, s);
    if (e != hipSuccess) return e;
    g.bias = nullptr;
    g.bias32 = cb;
    g.scale32 = cb + (size_t)3 * p->n;
  }
  g.M = p->B * p->T; g.N = gates_of(p->cell) * p->n; g.K = p->d;
  g.lda = p->d; g.ldb = p->d; g.ldc = g.N; g.splits = 1;
  g.a_kc = true; g.b_kc = true; g.bf16 = bf; g.out_f32 = !bf;
  g.vec_a = ((uintptr_t)x % 16 == 0) && ((size_t)p->d * es) % 16 == 0;
  g.vec_b = ((uintptr_t)w->W_x % 16 == 0) && ((size_t)p->d * es) % 16 == 0;
  return launch_gemm(g, s);
}

// Dense cells the n = 64 GRU kernels run zero-padded (see padded_solve):
// GRUs with n < 64 and tanh RNNs (as GRUs, see pad_inputs) with n <= 64,
// fp32, outside the time-parallel kernels' range (n > 8 or d > 8).
static bool pad_gru(const pr_problem *p) {
  return p && (p->cell == PR_CELL_GRU || p->cell == PR_CELL_TANH_RNN) && p->dtype == PR_F32 && p->B >= 1 &&
         p->T >= 1 && p->d >= 1 && p->n >= 1 &&
         (p->n < D64_N || (p->n == D64_N && p->cell == PR_CELL_TANH_RNN)) && !(p->n <= 8 && p->d <= DX_FUSED) &&
         (p->jac == PR_JAC_DENSE || p->jac == PR_JAC_DIAG || p->jac == PR_JAC_ZERO) &&
         (long long)p->B * p->T <= 2147483647LL;
}
struct PadLayout {
  size_t wx = 0, bx = 0, wh = 0, bh = 0, h0 = 0, h = 0, g = 0, lam = 0, dh0 = 0, dwx = 0, dbx = 0, dwh = 0, dbh = 0;
  size_t bytes = 0;
};
static PadLayout pad_layout(const pr_problem *p, bool adj) {
  PadLayout L;
  size_t o = 0;
  const size_t rows = (size_t)p->B * p->T, N = D64_N, G3 = 3 * N;
  L.wx = o; o = align256(o + G3 * p->d * 4);
  L.bx = o; o = align256(o + G3 * 4);
  L.wh = o; o = align256(o + G3 * N * 4);
  L.bh = o; o = align256(o + G3 * 4);
  L.h0 = o; o = align256(o + (size_t)p->B * N * 4);
  L.h = o; o = align256(o + rows * N * 4);
  if (adj) {
    L.g = o; o = align256(o + rows * N * 4);
    L.lam = o; o = align256(o + rows * N * 4);
    L.dh0 = o; o = align256(o + (size_t)p->B * N * 4);
    L.dwx = o; o = align256(o + G3 * p->d * 4);
    L.dbx = o; o = align256(o + G3 * 4);
    L.dwh = o; o = align256(o + G3 * N * 4);
    L.dbh = o; o = align256(o + G3 * 4);
  }
  L.bytes = o;
  return L;
}
static pr_problem padded(const pr_problem *p) {
  pr_problem q = *p;
  q.cell = PR_CELL_GRU;
  q.n = D64_N;
  return q;
}
static int padded_solve(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                        int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, void *workspace,
                        size_t ws_bytes, void *stream, const float *elk_lambda);
static int padded_adjoint(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                          int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, const void *g,
                          void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace, size_t ws_bytes,
                          void *stream, bool with_solve);
int kcell(int cell) { return cell == PR_CELL_TANH_RNN ? C_TANH : cell == PR_CELL_LINEAR ? C_LINEAR : C_GRU; }

bool al16(const void *q) { return q == nullptr || ((uintptr_t)q & 15) == 0; }

// Host copy of the solve state, one per thread, in pinned device-coherent
// memory: a small kernel stores the state there and then, with a
// system-scope release, the sequence word the host waits on, so a solve's
// stop test needs neither a copy-engine transfer nor an event between the
// sweeps and the work enqueued after them.
struct HostSnap {
  SolveState st;
  unsigned seq;
  unsigned *seq_dev;  // the device's address of seq
  SolveState *st_dev;
  unsigned next;      // sequence value of the next snapshot
};
HostSnap *host_snap() {
  thread_local HostSnap *hs = nullptr;
  thread_local bool tried = false;
  if (!hs && !tried) {
    tried = true;
    HostSnap *q = nullptr;
    if (hipHostMalloc((void **)&q, sizeof(HostSnap), hipHostMallocCoherent | hipHostMallocPortable | hipHostMallocMapped) !=
        hipSuccess)
      return nullptr;
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, q, 0) != hipSuccess) return nullptr;
    q->seq = 0;
    q->next = 1;
    q->st_dev = &((HostSnap *)d)->st;
    q->seq_dev = &((HostSnap *)d)->seq;
    hs = q;
  }
  return hs;
}
// Enqueue a snapshot of the device state at `dev` on s.
hipError_t snapshot_enqueue(HostSnap *hs, const void *dev, hipStream_t s, unsigned *want) {
  *want = hs->next++;
  if (hs->next == 0) hs->next = 1;
  return launch_snapshot(dev, hs->st_dev, sizeof(SolveState), hs->seq_dev, *want, s);
}
// Wait for snapshot `want` (spinning on the host word; the stream is queried
// now and then so that a device error or a lost snapshot ends the wait).
int snapshot_wait(HostSnap *hs, unsigned want, hipStream_t s) {
  for (unsigned long n = 1;; n++) {
    if (__atomic_load_n(&hs->seq, __ATOMIC_ACQUIRE) == want) return PR_OK;
    if ((n & 1023) == 0) {
      const hipError_t e = hipStreamQuery(s);
      if (e == hipSuccess) {  // everything enqueued has finished: the word is there or lost
        if (__atomic_load_n(&hs->seq, __ATOMIC_ACQUIRE) == want) return PR_OK;
        return fail(PR_EHIP, "the solve-state snapshot did not arrive");
      }
      if (e != hipErrorNotReady) return fail(PR_EHIP, "%s", hipGetErrorString(e));
    }
  }
}

// Event timing of the main kernels (pararnn_trace).  Categories: Newton
// sweeps (only launches that did work are counted), the adjoint's scan
// kernel, the input projection, the adjoint's products and reductions.
enum { TR_SWEEP = 0, TR_ADJ = 1, TR_PROJ = 2, TR_AGEMM = 3, TR_DPROD = 4, TR_SWEEP_LSIM = 5, TR_N = 6 };
struct Trace {
  bool on = false;
  bool made = false;
  double ms[TR_N] = {};
  long long cnt[TR_N] = {};
  static constexpr int CAP = 256;
  hipEvent_t sw[2 * CAP] = {};        // per sweep of the current solve
  hipEvent_t swa[2 * CAP] = {};       // per sweep: the dense path's chunk-product kernel
  hipEvent_t ev[TR_N][2 * CAP] = {};  // rings of the other categories
  int pending[TR_N] = {};
  hipError_t make() {
    if (made) return hipSuccess;
    // timing-only events: no system-scope fence (cache write-back and
    // invalidation) when they complete, which would stall the next launch
    const unsigned fl = hipEventDefault | hipEventDisableSystemFence;
    for (int i = 0; i < 2 * CAP; i++) {
      hipError_t e = hipEventCreateWithFlags(&sw[i], fl);
      if (e != hipSuccess) return e;
      e = hipEventCreateWithFlags(&swa[i], fl);
      if (e != hipSuccess) return e;
      for (int c = 1; c < TR_N; c++) {
        e = hipEventCreateWithFlags(&ev[c][i], fl);
        if (e != hipSuccess) return e;
      }
    }
    made = true;
    return hipSuccess;
  }
  hipError_t drain(int cat) {
    for (int i = 0; i < pending[cat]; i++) {
      hipError_t e = hipEventSynchronize(ev[cat][2 * i + 1]);
      if (e != hipSuccess) return e;
      float m = 0.f;
      e = hipEventElapsedTime(&m, ev[cat][2 * i], ev[cat][2 * i + 1]);
      if (e != hipSuccess) return e;
      ms[cat] += m;
      cnt[cat]++;
    }
    pending[cat] = 0;
    return hipSuccess;
  }
  hipError_t drain_all() {
    for (int c = 1; c < TR_N; c++) {
      hipError_t e = drain(c);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // bracket a launch group of category cat (cat != TR_SWEEP); returns the slot or -1
  int begin(int cat, hipStream_t s) {
    if (!on || !made) return -1;
    if (pending[cat] == CAP && drain(cat) != hipSuccess) return -1;
    const int i = pending[cat]++;
    return hipEventRecord(ev[cat][2 * i], s) == hipSuccess ? i : -1;
  }
  void end(int cat, int i, hipStream_t s) {
    if (i >= 0) hipEventRecord(ev[cat][2 * i + 1], s);
  }
};
Trace &trace() {
  thread_local Trace t;
  return t;
}

void poll_schedule(int *first, int *next) {
  *first = 4;
  *next = 2;
  const char *e = getenv("PARARNN_POLL");
  if (e) {
    int a = 0, b = 0;
    if (sscanf(e, "%d,%d", &a, &b) == 2 && a > 0 && b > 0) {
      *first = a;
      *next = b;
    }
  }
}

}  // namespace

extern "C" {

const char *pararnn_strerror(int status) {
  switch (status) {
    case PR_OK: return "ok";
    case PR_EINVAL: return "invalid argument";
    case PR_EWORKSPACE: return "workspace too small";
    case PR_EHIP: return "HIP runtime error";
    case PR_EUNSUPPORTED: return "unsupported problem";
    case PR_ELOOKBACK: return "a look-back wait gave up: the persistent grid's blocks were not all resident";
    case PR_NOT_CONVERGED: return "not converged within max_iters";
    case PR_NONFINITE: return "non-finite Newton update";
  }
  return "unknown status";
}

const char *pararnn_last_error(void) { return g_err.c_str(); }

int pararnn_trace(int enable) {
  Trace &t = trace();
  if (t.on) {
    hipError_t e = t.drain_all();
    if (e != hipSuccess) return fail(PR_EHIP, "trace: %s", hipGetErrorString(e));
  }
  t.on = enable != 0;
  for (int c = 0; c < TR_N; c++) {
    t.ms[c] = 0;
    t.cnt[c] = 0;
  }
  if (t.on) {
    hipError_t e = t.make();
    if (e != hipSuccess) return fail(PR_EHIP, "trace: %s", hipGetErrorString(e));
  }
  return PR_OK;
}

int pararnn_trace_kernel(int which, double *ms, long long *launches) {
  if (which < 0 || which >= TR_N) return fail(PR_EINVAL, "unknown trace category %d", which);
  Trace &t = trace();
  hipError_t e = t.drain_all();
  if (e != hipSuccess) return fail(PR_EHIP, "trace: %s", hipGetErrorString(e));
  if (ms) *ms = t.ms[which];
  if (launches) *launches = t.cnt[which];
  return PR_OK;
}

int pararnn_trace_read(double *sweep_ms, long long *sweep_launches, double *adjoint_ms, long long *adjoint_launches) {
  int rc = pararnn_trace_kernel(TR_SWEEP, sweep_ms, sweep_launches);
  if (rc != PR_OK) return rc;
  return pararnn_trace_kernel(TR_ADJ, adjoint_ms, adjoint_launches);
}

size_t pararnn_workspace_bytes(const pr_problem *p, int with_adjoint) {
  Plan pl;
  if (pad_gru(p)) {
    const pr_problem q = padded(p);
    if (make_plan(&q, &pl) != PR_OK) return 0;
    return pad_layout(p, with_adjoint != 0).bytes + (with_adjoint ? pl.adjoint_bytes : pl.solve_bytes);
  }
  if (make_plan(p, &pl) != PR_OK) return 0;
  return with_adjoint ? pl.adjoint_bytes : pl.solve_bytes;
}

// Quasi-ELK scratch beyond a solve's workspace.  Dense n = 64 GRU: [G | e]
// per step ([d | r] sits in the gates buffer), chunk aggregates and carries.
// Per-channel cells: chunk aggregates, carries and boundary values only.
// ELK with the cell's own Jacobian (full covariances): per step J | r and
// G | e, per (chunk, unit) the filtering elements and carries.
struct ElkLayout {
  size_t off_jr = 0, off_ge = 0, off_r1 = 0, off_pc = 0, off_mc = 0, off_r3 = 0, off_msc = 0;
  size_t off_fagg = 0, off_fcar = 0, off_fsub = 0, off_dr = 0, off_hb = 0;
  size_t off_elem = 0, off_fin = 0, off_rev = 0, off_msin = 0;
  size_t off_A = 0, off_D = 0, off_S = 0, off_f = 0, off_g = 0, off_v = 0, off_x = 0;  // n = 64 ELK
  size_t bytes = 0;
  int cps = 0, nch = 0, cpf = 0, nchf = 0;
  bool full = false;           // the cell's own Jacobian (else its diagonal: quasi-ELK)
  int Nf = 0, units = 0, L = 0, cpu = 0;
};
// Which ELK a problem asks for: the cell's own Jacobian gives ELK, the
// diagonal quasi-ELK.  Where the own Jacobian is diagonal (the diagonal GRU,
// a dense cell with one state entry) the two are the same and the quasi-ELK
// kernels run.
static int elk_kind(const pr_problem *p, const Plan &pl, bool *full) {
  *full = false;
  if (p->jac == PR_JAC_ZERO) return fail(PR_EINVAL, "ELK needs a Jacobian: jac must be the cell's own or PR_JAC_DIAG");
  const bool own = (p->cell == PR_CELL_LSTM_CIFG_DIAG && p->jac == PR_JAC_BLOCK2) ||
                   (pl.path != PATH_CHAN && p->jac == PR_JAC_DENSE && p->n > 1);
  *full = own;
  return PR_OK;
}
static int elk_layout(const pr_problem *p, const Plan &pl, ElkLayout *el) {
  if (pl.path != PATH_D64 && pl.path != PATH_CHAN && pl.path != PATH_TIME)
    return fail(PR_EUNSUPPORTED, "no quasi-ELK kernels for this problem");
  int rc = elk_kind(p, pl, &el->full);
  if (rc != PR_OK) return rc;
  if (el->full && pl.path == PATH_D64) {  // block rows of the normal equations, 64 x 64 each
    const size_t rows = (size_t)p->B * p->T;
    size_t o = pl.solve_bytes;
    el->off_A = o; o = align256(o + rows * 4096 * 4);
    el->off_D = o; o = align256(o + rows * 4096 * 4);
    el->off_S = o; o = align256(o + rows * 4096 * 4);
    el->off_f = o; o = align256(o + rows * 64 * 4);
    el->off_g = o; o = align256(o + rows * 64 * 4);
    el->off_v = o; o = align256(o + rows * 64 * 4);
    el->off_x = o; o = align256(o + rows * 64 * 4);
    el->bytes = o;
    return PR_OK;
  }
  if (el->full) {
    const int N = pl.path == PATH_CHAN ? 2 : pl.N;
    el->Nf = N;
    el->units = pl.path == PATH_CHAN ? p->B * p->n : p->B;
    el->L = elk_full_chunk_len(p->T);
    el->cpu = (p->T + el->L - 1) / el->L;
    if ((long long)el->units * el->cpu > 2147483647LL / 4) return fail(PR_EUNSUPPORTED, "problem too large");
    const size_t steps = (size_t)p->T * el->units, pc = (size_t)el->cpu * el->units, NN = (size_t)N * N;
    size_t o = pl.solve_bytes;
    el->off_jr = o; o = align256(o + steps * (NN + N) * 4);
    el->off_ge = o; o = align256(o + steps * (NN + N) * 4);
    el->off_elem = o; o = align256(o + pc * (3 * NN + 2 * N) * 4);
    el->off_fin = o; o = align256(o + pc * (NN + N) * 4);
    el->off_rev = o; o = align256(o + pc * (NN + N) * 4);
    el->off_msin = o; o = align256(o + pc * N * 4);
    el->bytes = o;
    return PR_OK;
  }
  const size_t rows = (size_t)p->B * p->T, S = (size_t)pl.S;
  const int L = pl.path == PATH_CHAN ? elk_chan_chunk_len(p->cell == PR_CELL_LSTM_CIFG_DIAG ? 2 : 1)
                                      : elk_chunk_len(pl.S);
  el->cps = (p->T + L - 1) / L;
  if ((long long)el->cps * p->B * ((pl.S + 63) / 64) > 2147483647LL / 4 || (long long)p->B * pl.S > 2147483647LL / 4)
    return fail(PR_EUNSUPPORTED, "problem too large");
  el->nch = el->cps * p->B;
  const size_t nch = (size_t)el->nch;
  size_t o = pl.solve_bytes;
  if (pl.path == PATH_D64 || pl.path == PATH_TIME) {
    if (pl.path == PATH_D64) {
      el->off_jr = pl.off_gates;  // [row][320] floats hold [d (64) | r (64)]
    } else {
      el->off_jr = o; o = align256(o + rows * 2 * S * 4);
    }
    el->off_ge = o; o = align256(o + rows * 2 * S * 4);
    el->off_r1 = o; o = align256(o + nch * 7 * S * 4);
    el->off_pc = o; o = align256(o + nch * S * 4);
    el->off_mc = o; o = align256(o + nch * S * 4);
  } else {
    el->cpf = (p->T + 4 * L - 1) / (4 * L);  // filter chunks of 4 apply chunks
    el->nchf = el->cpf * p->B;
    el->off_fagg = o; o = align256(o + (size_t)el->nchf * 7 * S * 4);
    el->off_fcar = o; o = align256(o + (size_t)el->nchf * 2 * S * 4);
    el->off_fsub = o; o = align256(o + nch * 2 * S * 4);
    el->off_dr = o; o = align256(o + nch * 2 * S * 4);
    el->off_hb = o; o = align256(o + nch * S * 4);
  }
  el->off_r3 = o; o = align256(o + nch * 2 * S * 4);
  el->off_msc = o; o = align256(o + nch * S * 4);
  el->bytes = o;
  return PR_OK;
}

// An adjoint that pararnn_solve_adjoint lets the solve enqueue right after
// its first batch of sweeps, before the convergence poll waits: when that
// batch turns out to be the last, the device runs the adjoint with no gap.
struct SpecAdjoint {
  const void *g;
  void *lambda, *dx, *dh0;
  const pr_grads *dW;
  bool done = false;  // out: the adjoint ran at the returned trajectory
  bool ran = false;   // out: an adjoint was enqueued (done or not)
  bool chan_aggs = false;  // out: the last channel pass composed the adjoint's tile aggregates
  int rc = PR_OK;     // out: its status when done
};
// Whether the last combined call on a problem converged within its first
// batch (then the next one speculates on the scalar-state path).
struct SpecMemo {
  pr_problem p{};
  float tol = 0.f;
  int max_iters = 0;
  bool valid = false, first_batch = false;
  bool same(const pr_problem *q, float t, int m) const {
    return valid && p.cell == q->cell && p.jac == q->jac && p.dtype == q->dtype && p.B == q->B && p.T == q->T &&
           p.d == q->d && p.n == q->n && tol == t && max_iters == m;
  }
};
// Event marking a convergence poll's state snapshot (null if it cannot be made).
static SpecMemo &spec_memo() {
  thread_local SpecMemo m;
  return m;
}

static int adjoint_impl(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, const void *h,
                        const void *g, void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace,
                        size_t ws_bytes, void *stream, bool u_ready, bool fresh, bool chan_aggs = false);
// Sweep number of the descriptors of an adjoint that follows its solve
// without clearing: above any sweep count (the scalar-state path has T < 2^29).
constexpr int ADJ_TAG_SWEEP = 1 << 30;

static int solve_impl(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                      int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, void *workspace,
                      size_t ws_bytes, void *stream, const float *elk_lambda, SpecAdjoint *spec = nullptr) {
  g_err.clear();
  Plan pl;
  int rc = make_plan(p, &pl);
  if (rc != PR_OK) return rc;
  ElkLayout el;
  if (elk_lambda) {
    if (!(*elk_lambda >= 0.f) || *elk_lambda > 3.0e38f) return fail(PR_EINVAL, "lambda must be >= 0 and finite");
    rc = elk_layout(p, pl, &el);
    if (rc != PR_OK) return rc;
    // the quasi-ELK producers evaluate the Jacobian's diagonal; ELK on the
    // 64 x 64 GRU takes the gates kernel's factors of the whole Jacobian
    pl.approx = el.full && pl.path == PATH_D64 ? APX_NEWTON : APX_DIAG;
    pl.solve_bytes = el.bytes;
  }
  if (!w || !w->W_x || !w->W_h) return fail(PR_EINVAL, "W_x and W_h are required");
  if (p->cell == PR_CELL_LSTM_CIFG_DIAG && !w->peep) return fail(PR_EINVAL, "the LSTM cell needs peepholes");
  if (!x || !h) return fail(PR_EINVAL, "x and h are required");
  if (max_iters < 1) return fail(PR_EINVAL, "max_iters must be >= 1");
  if (tol != tol) return fail(PR_EINVAL, "tol is NaN");
  if (!workspace || ws_bytes < pl.solve_bytes)
    return fail(PR_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, pl.solve_bytes);
  if (((uintptr_t)workspace & 255) != 0) return fail(PR_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  HostSnap *snap = host_snap();
  if (!snap) return fail(PR_EHIP, "pinned host buffer allocation failed");
  SolveState *hs = &snap->st;

  Trace &tr = trace();
  if (tr.on) HIPCHK(tr.make());
  // n = d = 1 with vector-friendly sizes takes the scalar-state sweep
  const bool scalar = pl.path == PATH_TIME && pl.scalar_ok && al16(h) && al16(x) && !getenv("PARARNN_NO_SCALAR");
  if (scalar)
    HIPCHK(launch_zero_coef(ws, pl.zero_bytes, (const float *)w->W_x, (const float *)w->b_x, (const float *)w->W_h,
                            (const float *)w->b_h, kcell(p->cell), (float *)(ws + pl.off_coef), s));
  else
    HIPCHK(launch_zero(ws, pl.zero_bytes, s));
  const int kmax = max_iters < p->T ? max_iters : p->T;

  TimeArgs a{};
  ChanArgs ca{};
  D64Args da{};
  if (pl.path == PATH_D64) {
    da.U = (const float *)(ws + pl.off_U);
    da.h = (float *)h;
    da.h0 = (const float *)h0;
    da.Wh = (const float *)w->W_h;
    da.bh = (const float *)w->b_h;
    da.gates = (float *)(ws + pl.off_gates);
    da.aggP = (float *)(ws + pl.off_aggP);
    da.aggb = (float *)(ws + pl.off_aggb);
    da.carry = (float *)(ws + pl.off_carry);
    da.B = p->B; da.T = p->T; da.cps = pl.cps; da.nchunks = pl.nchunks;
    da.approx = pl.approx;
    da.tol = tol;
    da.max_iters = max_iters;
    da.st = (SolveState *)(ws + pl.off_state);
    if (((uintptr_t)h % 16) || (h0 && ((uintptr_t)h0 % 16)) || ((uintptr_t)w->W_h % 16))
      return fail(PR_EINVAL, "h, h0 and W_h must be 16-byte aligned for n = 64");
    const int ti = tr.begin(TR_PROJ, s);
    HIPCHK(input_projection(p, w, x, ws + pl.off_U, s));
    tr.end(TR_PROJ, ti, s);
  } else if (pl.path == PATH_TIME) {
    a.x = (const float *)x;
    a.h = (float *)h;
    a.h0 = (const float *)h0;
    a.Wx = (const float *)w->W_x;
    a.bx = (const float *)w->b_x;
    a.Wh = (const float *)w->W_h;
    a.bh = (const float *)w->b_h;
    a.B = p->B; a.T = p->T; a.d = p->d; a.n = p->n;
    a.tol = tol;
    a.max_iters = max_iters;
    a.st = (SolveState *)(ws + pl.off_state);
    a.agg = (unsigned long long *)(ws + pl.off_agg);
    a.incl = (unsigned long long *)(ws + pl.off_incl);
    a.bnd = (float *)(ws + pl.off_bnd);
    a.tiles_per_seq = pl.tps;
    a.ntiles = pl.ntiles;
    a.vec_ok = (al16(h) ? 1 : 0) | (al16(x) ? 2 : 0);
    a.coef = (const float *)(ws + pl.off_coef);
    a.approx = pl.approx;
  } else {
    ca.U = ws + pl.off_U;
    ca.h = h;
    ca.h0 = h0;
    ca.Wh = w->W_h;
    ca.bh = w->b_h;
    ca.peep = p->cell == PR_CELL_LSTM_CIFG_DIAG ? w->peep : nullptr;
    ca.B = p->B; ca.T = p->T; ca.n = p->n; ca.SW = pl.SW;
    ca.tol = tol;
    ca.max_iters = max_iters;
    ca.st = (SolveState *)(ws + pl.off_state);
    ca.agg = (unsigned long long *)(ws + pl.off_agg);
    ca.incl = (unsigned long long *)(ws + pl.off_incl);
    ca.bnd = (float *)(ws + pl.off_bnd);
    ca.stripes = pl.stripes;
    ca.tps = pl.tps_2;
    ca.ntiles = pl.ntiles_2;
    const int ti = tr.begin(TR_PROJ, s);
    HIPCHK(input_projection(p, w, x, ws + pl.off_U, s, (float *)(ws + pl.off_cb)));
    tr.end(TR_PROJ, ti, s);
  }
  const int kc = p->cell == PR_CELL_GRU_DIAG ? C_GRU_DIAG : p->cell == PR_CELL_LSTM_CIFG_DIAG ? C_LSTM : kcell(p->cell);
  if (scalar) {  // its coefficients were computed with the clearing
    a.tiles_per_seq = pl.tps_s;
    a.ntiles = pl.ntiles_s;
  }

  ElkArgs ea{};
  ElkChanArgs eca{};
  ElkFullArgs fa{};
  Elk64Args e64{};
  if (elk_lambda && el.full && pl.path == PATH_D64) {
    e64.gates = da.gates;
    e64.Wh = da.Wh;
    e64.A = (float *)(ws + el.off_A);
    e64.D = (float *)(ws + el.off_D);
    e64.S = (float *)(ws + el.off_S);
    e64.f = (float *)(ws + el.off_f);
    e64.g = (float *)(ws + el.off_g);
    e64.v = (float *)(ws + el.off_v);
    e64.x = (float *)(ws + el.off_x);
    e64.h = (float *)h;
    e64.B = p->B; e64.T = p->T;
    e64.lam = *elk_lambda;
    e64.st = (SolveState *)(ws + pl.off_state);
  } else if (elk_lambda && el.full) {
    fa.jr = (float *)(ws + el.off_jr);
    fa.ge = (float *)(ws + el.off_ge);
    fa.elem = (float *)(ws + el.off_elem);
    fa.fin = (float *)(ws + el.off_fin);
    fa.rev = (float *)(ws + el.off_rev);
    fa.msin = (float *)(ws + el.off_msin);
    fa.h = h;
    fa.U = ws + pl.off_U;
    fa.h0 = h0;
    fa.Wh = w->W_h;
    fa.bh = w->b_h;
    fa.peep = w->peep;
    fa.B = p->B; fa.T = p->T; fa.n = p->n; fa.S = pl.S;
    fa.units = el.units;
    fa.upb = pl.path == PATH_CHAN ? p->n : 1;
    fa.NS = pl.path == PATH_CHAN ? 2 : p->n;
    fa.L = el.L; fa.cpu = el.cpu;
    fa.lam = *elk_lambda;
    fa.tol = tol;
    fa.max_iters = max_iters;
    fa.st = (SolveState *)(ws + pl.off_state);
  } else if (elk_lambda) {
    if (pl.path == PATH_D64 || pl.path == PATH_TIME) {
      ea.jr = (float *)(ws + el.off_jr);
      ea.ge = (float *)(ws + el.off_ge);
      ea.r1 = (float *)(ws + el.off_r1);
      ea.pc = (float *)(ws + el.off_pc);
      ea.mc = (float *)(ws + el.off_mc);
    }
    ea.r3 = (float *)(ws + el.off_r3);
    ea.msc = (float *)(ws + el.off_msc);
    ea.h = h;
    ea.h_bf16 = p->dtype == PR_BF16;
    ea.B = p->B; ea.T = p->T; ea.S = pl.S; ea.cps = el.cps; ea.nch = el.nch;
    ea.L = elk_chunk_len(pl.S);
    ea.sp = elk_lanes_per_chunk(pl.S);
    ea.lam = *elk_lambda;
    ea.tol = tol;
    ea.max_iters = max_iters;
    ea.st = (SolveState *)(ws + pl.off_state);
    if (pl.path == PATH_CHAN) {
      eca.e = ea;
      eca.U = ws + pl.off_U;
      eca.h0 = h0;
      eca.Wh = w->W_h;
      eca.bh = w->b_h;
      eca.peep = p->cell == PR_CELL_LSTM_CIFG_DIAG ? w->peep : nullptr;
      eca.n = p->n;
      eca.fagg = (float *)(ws + el.off_fagg);
      eca.fcar = (float *)(ws + el.off_fcar);
      eca.fsub = (float *)(ws + el.off_fsub);
      eca.cpf = el.cpf;
      eca.nchf = el.nchf;
      eca.dr = (float *)(ws + el.off_dr);
      eca.hb = (float *)(ws + el.off_hb);
    }
  }

  int first, next;
  poll_schedule(&first, &next);
  if (tol <= 0.f) first = kmax;
  // Speculate when the first batch is surely the last (a fixed sweep count),
  // or on the scalar-state path (whose adjoint leaves nothing the later sweeps
  // read besides the solve state, which is restored) when the last call on
  // this problem converged within its first batch.
  const bool speculate = spec && !elk_lambda &&
                         (first >= kmax || (scalar && al16(spec->g) && al16(spec->lambda) && al16(spec->dx) &&
                                            spec_memo().same(p, tol, max_iters) && spec_memo().first_batch));
  bool spec_enqueued = false;
  // channel cells with a fixed sweep count: the last pass composes the
  // adjoint's tile aggregates (it evaluates the cell at the final iterate
  // anyway), so the adjoint skips its own aggregate pass
  const bool fuse_adj = speculate && pl.path == PATH_CHAN && tol <= 0.f && spec->g != nullptr;
  if (fuse_adj) {
    ca.g = spec->g;
    spec->chan_aggs = true;
  }
  int k = 1, out_iters = 0, out_status = PR_OK;
  // Sweep timing: the dense n = 64 path brackets every sweep (its parts are
  // timed too); the others bracket each batch of back-to-back sweeps, so the
  // per-launch figure carries no event overhead between launches.
  const bool per_sweep_events = pl.path == PATH_D64 && !elk_lambda;
  int nbatch = 0, batch_first[Trace::CAP], batch_last[Trace::CAP];
  while (true) {
    const int batch = k == 1 ? first : next;
    int k_last = k + batch - 1;
    if (k_last > kmax) k_last = kmax;
    const bool bev = tr.on && !per_sweep_events && k_last <= Trace::CAP && nbatch < Trace::CAP;
    if (bev) {
      HIPCHK(hipEventRecord(tr.sw[2 * (k - 1)], s));
      batch_first[nbatch] = k;
      batch_last[nbatch] = k_last;
      nbatch++;
    }
    for (int kk = k; kk <= k_last; kk++) {
      a.k = kk;
      const bool ev = tr.on && per_sweep_events && kk <= Trace::CAP;
      if (ev) HIPCHK(hipEventRecord(tr.sw[2 * (kk - 1)], s));
      if (elk_lambda && el.full && pl.path == PATH_D64) {  // the gates, then the normal equations
        da.k = kk;
        HIPCHK(launch_d64_sweep_part(da, 0, s));
        e64.k = kk;
        HIPCHK(launch_elk64_passes(e64, s));
      } else if (elk_lambda && el.full) {  // the damped step with the cell's own Jacobian
        fa.k = kk;
        if (pl.path == PATH_CHAN) HIPCHK(launch_elk_full_lstm(p->dtype == PR_BF16, fa, s));
        else HIPCHK(launch_elk_full_dense(kc, pl.N, a, fa, s));
      } else if (elk_lambda) {  // the damped step with the Jacobian's diagonal
        if (pl.path == PATH_D64) {  // producer of [d | r], then the scans
          da.k = kk;
          HIPCHK(launch_d64_sweep_part(da, 0, s));
          ea.k = kk;
          HIPCHK(launch_elk_sweep(ea, s));
        } else if (pl.path == PATH_TIME) {
          HIPCHK(launch_time_elk_jr(kc, pl.N, a, ea.jr, s));
          ea.k = kk;
          HIPCHK(launch_elk_sweep(ea, s));
        } else {
          eca.e.k = kk;
          HIPCHK(launch_elk_chan_sweep(kc, p->dtype == PR_BF16, eca, s));
        }
      } else if (scalar) {
        HIPCHK(launch_scalar_sweep(kc, a, s));
      } else if (pl.path == PATH_TIME) {
        HIPCHK(launch_time_sweep(kc, pl.N, a, s));
      } else if (pl.path == PATH_D64) {
        da.k = kk;
        HIPCHK(launch_d64_sweep_part(da, 0, s));
        if (ev) HIPCHK(hipEventRecord(tr.swa[2 * (kk - 1)], s));
        HIPCHK(launch_d64_sweep_part(da, 1, s));
        if (ev) HIPCHK(hipEventRecord(tr.swa[2 * (kk - 1) + 1], s));
        HIPCHK(launch_d64_sweep_part(da, 2, s));
      } else {  // channel cells: carry scan, then the pass applying this sweep
        ca.k = kk;
        const bool bf = p->dtype == PR_BF16;
        if (kk == 1) HIPCHK(launch_chan2(kc, pl.approx, bf, ca, CHAN2_FIRST, s));
        HIPCHK(launch_chan2(kc, pl.approx, bf, ca, CHAN2_CARRY, s));
        // the last possible sweep composes no aggregates for a next one (but
        // the adjoint's, when it follows a fixed sweep count)
        const int what = kk < kmax ? CHAN2_APPLY_NEXT : fuse_adj ? CHAN2_APPLY_ADJ : CHAN2_APPLY;
        HIPCHK(launch_chan2(kc, pl.approx, bf, ca, what, s));
      }
      if (ev) HIPCHK(hipEventRecord(tr.sw[2 * (kk - 1) + 1], s));
    }
    if (bev) HIPCHK(hipEventRecord(tr.sw[2 * (k_last - 1) + 1], s));
    unsigned want = 0;
    HIPCHK(snapshot_enqueue(snap, ws + pl.off_state, s, &want));
    // the host waits for the snapshot only: a speculative adjoint enqueued
    // behind it keeps the device busy while the host decides
    if (speculate && k == 1) {
      spec->rc = adjoint_impl(p, w, x, h0, h, spec->g, spec->lambda, spec->dx, spec->dh0, spec->dW, workspace,
                              ws_bytes, stream, true, true, spec->chan_aggs);
      spec_enqueued = spec->rc >= 0;
      spec->ran = spec_enqueued;
    }
    {
      const int rc = snapshot_wait(snap, want, s);
      if (rc != PR_OK) return rc;
    }
    if (hs->fault)
      return fail(PR_ELOOKBACK, "a look-back wait exceeded its bound (the persistent grid was not co-resident)");
    if (hs->stopped) {
      out_iters = hs->iters;
      out_status = hs->status;
      break;
    }
    int status;
    unsigned dbits = 0;
    for (int i = 0; i < PR_DSHARDS; i++) dbits = hs->dslot[k_last & 3][i] > dbits ? hs->dslot[k_last & 3][i] : dbits;
    hs->hist[k_last % PR_HIST] = dbits;
    const float dl = __builtin_bit_cast(float, dbits);
    if (stop_rule(dl, k_last, tol, p->T, max_iters, &status)) {
      out_iters = k_last;
      out_status = status;
      break;
    }
    if (spec_enqueued) {  // the speculative adjoint reset the solve state: put the snapshot back
      HIPCHK(hipMemcpyAsync(ws + pl.off_state, hs, sizeof(SolveState), hipMemcpyHostToDevice, s));
      spec_enqueued = false;
    }
    k = k_last + 1;
  }
  if (spec) {
    spec->done = spec_enqueued;
    SpecMemo &m = spec_memo();
    m.p = *p;
    m.tol = tol;
    m.max_iters = max_iters;
    m.valid = true;
    m.first_batch = out_iters <= first;
  }
  if (tr.on && !per_sweep_events) {
    // a batch's launches past the stop exit at once; count the ones that worked
    // (the host has seen the snapshot written after the batch's end event, but
    // the runtime may not report that event complete yet: wait for it)
    for (int i = 0; i < nbatch && batch_first[i] <= out_iters; i++) {
      float ms = 0.f;
      HIPCHK(hipEventSynchronize(tr.sw[2 * (batch_last[i] - 1) + 1]));
      HIPCHK(hipEventElapsedTime(&ms, tr.sw[2 * (batch_first[i] - 1)], tr.sw[2 * (batch_last[i] - 1) + 1]));
      tr.ms[TR_SWEEP] += ms;
      tr.cnt[TR_SWEEP] += (batch_last[i] < out_iters ? batch_last[i] : out_iters) - batch_first[i] + 1;
    }
  }
  if (tr.on && per_sweep_events) {
    const int m = out_iters < Trace::CAP ? out_iters : Trace::CAP;
    for (int kk = 1; kk <= m; kk++) {
      float ms = 0.f;
      HIPCHK(hipEventSynchronize(tr.sw[2 * (kk - 1) + 1]));
      HIPCHK(hipEventElapsedTime(&ms, tr.sw[2 * (kk - 1)], tr.sw[2 * (kk - 1) + 1]));
      tr.ms[TR_SWEEP] += ms;
      tr.cnt[TR_SWEEP]++;
      if (pl.path == PATH_D64) {
        HIPCHK(hipEventElapsedTime(&ms, tr.swa[2 * (kk - 1)], tr.swa[2 * (kk - 1) + 1]));
        tr.ms[TR_DPROD] += ms;
        tr.cnt[TR_DPROD]++;
      }
    }
  }
  if (iters) *iters = out_iters;
  if (delta_hist) {
    int m = out_iters < hist_cap ? out_iters : hist_cap;
    if (m > PR_HIST) m = PR_HIST;
    for (int kk = 1; kk <= m; kk++) delta_hist[kk - 1] = __builtin_bit_cast(float, hs->hist[kk % PR_HIST]);
  }
  return out_status == ST_NONFINITE ? PR_NONFINITE : out_status == ST_NOT_CONVERGED ? PR_NOT_CONVERGED : PR_OK;
}

int pararnn_solve(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol, int max_iters,
                  void *h, int *iters, float *delta_hist, int hist_cap, void *workspace, size_t ws_bytes,
                  void *stream) {
  if (pad_gru(p))
    return padded_solve(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, workspace, ws_bytes, stream,
                        nullptr);
  return solve_impl(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, workspace, ws_bytes, stream,
                    nullptr);
}

size_t pararnn_elk_workspace_bytes(const pr_problem *p) {
  g_err.clear();
  if (pad_gru(p)) {
    const pr_problem q = padded(p);
    const size_t inner = pararnn_elk_workspace_bytes(&q);
    return inner ? pad_layout(p, true).bytes + inner : 0;
  }
  Plan pl;
  if (make_plan(p, &pl) != PR_OK) return 0;
  ElkLayout el;
  if (elk_layout(p, pl, &el) != PR_OK) return 0;
  return el.bytes > pl.adjoint_bytes ? el.bytes : pl.adjoint_bytes;
}

int pararnn_solve_elk(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float lambda,
                      float tol, int max_iters, void *h, int *iters, float *delta_hist, int hist_cap,
                      void *workspace, size_t ws_bytes, void *stream) {
  if (pad_gru(p))
    return padded_solve(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, workspace, ws_bytes, stream,
                        &lambda);
  return solve_impl(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, workspace, ws_bytes, stream,
                    &lambda);
}

int pararnn_adjoint(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, const void *h,
                    const void *g, void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace,
                    size_t ws_bytes, void *stream) {
  if (pad_gru(p))
    return padded_adjoint(p, w, x, h0, 0.f, 1, (void *)h, nullptr, nullptr, 0, g, lambda, dx, dh0, dW, workspace,
                          ws_bytes, stream, false);
  return adjoint_impl(p, w, x, h0, h, g, lambda, dx, dh0, dW, workspace, ws_bytes, stream, false, false);
}

}  // extern "C"

// The adjoint; u_ready: the workspace already holds this problem's input
// projection U (a solve on the same workspace and inputs has just computed
// it, as in pararnn_solve_adjoint), so it is not recomputed.
// u_ready: the solve of the same call left the input projection in the
// workspace.  fresh: the solve of the same call cleared the workspace (and
// folded the scalar-state coefficients) and no adjoint has run since; the
// scalar-state adjoint then skips its clearing and tags its descriptors with
// a sweep number no solve reaches, so the sweeps' descriptors never match.
static int adjoint_impl(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, const void *h,
                        const void *g, void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace,
                        size_t ws_bytes, void *stream, bool u_ready, bool fresh, bool chan_aggs) {
  g_err.clear();
  Plan pl;
  int rc = make_plan(p, &pl);
  if (rc != PR_OK) return rc;
  if (!w || !w->W_x || !w->W_h) return fail(PR_EINVAL, "W_x and W_h are required");
  if (p->cell == PR_CELL_LSTM_CIFG_DIAG && !w->peep) return fail(PR_EINVAL, "the LSTM cell needs peepholes");
  if (!x || !h || !g) return fail(PR_EINVAL, "x, h and g are required");
  if (!workspace || ws_bytes < pl.adjoint_bytes)
    return fail(PR_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, pl.adjoint_bytes);
  if (((uintptr_t)workspace & 255) != 0) return fail(PR_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  // n = d = 1 with vector-friendly sizes takes the scalar-state adjoint
  const bool scalar = pl.path == PATH_TIME && pl.scalar_ok && al16(h) && al16(x) && al16(g) && al16(lambda) &&
                      al16(dx) && !getenv("PARARNN_NO_SCALAR");
  const bool keep = scalar && fresh;
  if (keep) {
  } else if (scalar) {
    HIPCHK(launch_zero_coef(ws, pl.zero_bytes, (const float *)w->W_x, (const float *)w->b_x, (const float *)w->W_h,
                            (const float *)w->b_h, kcell(p->cell), (float *)(ws + pl.off_coef), s));
  } else {
    HIPCHK(launch_zero(ws, pl.zero_bytes, s));
  }
  if (pl.path == PATH_TIME) {
    TimeArgs a{};
    a.x = (const float *)x;
    a.h = (float *)h;
    a.h0 = (const float *)h0;
    a.Wx = (const float *)w->W_x;
    a.bx = (const float *)w->b_x;
    a.Wh = (const float *)w->W_h;
    a.bh = (const float *)w->b_h;
    a.g = (const float *)g;
    a.lam = (float *)lambda;
    a.dx = (float *)dx;
    a.dh0 = (float *)dh0;
    a.part = (float *)(ws + pl.off_part);
    a.B = p->B; a.T = p->T; a.d = p->d; a.n = p->n;
    a.k = keep ? ADJ_TAG_SWEEP : 1;
    a.st = (SolveState *)(ws + pl.off_state);
    a.agg = (unsigned long long *)(ws + pl.off_agg);
    a.incl = (unsigned long long *)(ws + pl.off_incl);
    a.tiles_per_seq = pl.tps;
    a.ntiles = pl.ntiles;
    a.vec_ok = (al16(h) ? 1 : 0) | (al16(x) ? 2 : 0) | (al16(g) ? 4 : 0) | (al16(lambda) ? 8 : 0);
    if (scalar) {  // its coefficients were computed with the clearing
      a.coef = (const float *)(ws + pl.off_coef);
      a.tiles_per_seq = pl.tps_sa;
      a.ntiles = pl.ntiles_sa;
    }
    Trace &tr = trace();
    const int ti = tr.begin(TR_ADJ, s);
    if (scalar) HIPCHK(launch_scalar_adjoint(kcell(p->cell), a, s));
    else HIPCHK(launch_time_adjoint(kcell(p->cell), pl.N, a, s));
    tr.end(TR_ADJ, ti, s);
    if (dW && (dW->W_x || dW->b_x || dW->W_h || dW->b_h))
      HIPCHK(launch_time_reduce(kcell(p->cell), pl.N, a, a.part, dW->W_x, dW->b_x, dW->W_h, dW->b_h, s));
    return PR_OK;
  }
  if (pl.path == PATH_D64) {
    if (((uintptr_t)h % 16) || (h0 && ((uintptr_t)h0 % 16)) || ((uintptr_t)w->W_h % 16) || ((uintptr_t)g % 16))
      return fail(PR_EINVAL, "h, h0, g and W_h must be 16-byte aligned for n = 64");
    if (!lambda) return fail(PR_EINVAL, "the dense n = 64 adjoint needs the lambda output buffer");
    Trace &tr = trace();
    if (!u_ready) {
      const int tp = tr.begin(TR_PROJ, s);
      HIPCHK(input_projection(p, w, x, ws + pl.off_U, s));
      tr.end(TR_PROJ, tp, s);
    }
    D64Args da{};
    da.U = (const float *)(ws + pl.off_U);
    da.h = (float *)h;
    da.h0 = (const float *)h0;
    da.Wh = (const float *)w->W_h;
    da.bh = (const float *)w->b_h;
    da.gates = (float *)(ws + pl.off_gates);
    da.aggP = (float *)(ws + pl.off_aggP);
    da.aggb = (float *)(ws + pl.off_aggb);
    da.carry = (float *)(ws + pl.off_carry);
    da.g = (const float *)g;
    da.lam = (float *)lambda;
    da.B = p->B; da.T = p->T; da.cps = pl.cps; da.nchunks = pl.nchunks;
    da.approx = pl.approx;
    da.st = (SolveState *)(ws + pl.off_state);
    const int ta = tr.begin(TR_ADJ, s);
    HIPCHK(launch_d64_adjoint_scan(da, s));
    tr.end(TR_ADJ, ta, s);
    const int tg = tr.begin(TR_AGEMM, s);
    D64AdjArgs ea{};
    ea.gates = da.gates; ea.lam = da.lam; ea.h = da.h; ea.h0 = da.h0; ea.Wh = da.Wh;
    ea.dU = (float *)(ws + pl.off_dU);
    ea.dA = (float *)(ws + pl.off_dA);
    ea.hprev = (float *)(ws + pl.off_hprev);
    ea.dh0 = (float *)dh0;
    ea.B = p->B; ea.T = p->T;
    HIPCHK(launch_d64_adjoint_epilogue(ea, s));
    const int rows = p->B * p->T;
    double *csp = (double *)(ws + pl.off_csum);
    // dW_x = dU^T x with db_x = column sums of dU, and dW_h = dA^T h_prev with
    // db_h = column sums of dA, each from one pass over its K-outer operands
    const bool tn_x = dW && (dW->W_x || dW->b_x) && p->d <= 64;
    if (tn_x) HIPCHK(launch_tn_products(ea.dU, (const float *)x, rows, p->d, dW->W_x, dW->b_x, ws + pl.off_tn, s));
    if (dW && (dW->W_h || dW->b_h))
      HIPCHK(launch_tn_products(ea.dA, ea.hprev, rows, 64, dW->W_h, dW->b_h, ws + pl.off_tn, s));
    if (dW && dW->b_x && !tn_x) HIPCHK(launch_colsum(ea.dU, rows, 192, dW->b_x, csp, s));
    if (dx) {  // dx = dU W_x
      GemmArgs gm{};
      gm.A = ea.dU; gm.B = w->W_x; gm.C = dx;
      gm.M = rows; gm.N = p->d; gm.K = 192; gm.lda = 192; gm.ldb = p->d; gm.ldc = p->d; gm.splits = 1;
      gm.a_kc = true; gm.b_kc = false; gm.bf16 = false; gm.out_f32 = true;
      gm.vec_a = true;
      gm.vec_b = ((uintptr_t)w->W_x % 16 == 0) && (p->d % 4) == 0;
      HIPCHK(launch_gemm(gm, s));
    }
    if (dW && dW->W_x && !tn_x) {  // dW_x = dU^T x (input widths past 64)
      GemmArgs gm{};
      gm.A = ea.dU; gm.B = x; gm.C = dW->W_x; gm.ws = (float *)(ws + pl.off_gws);
      gm.M = 192; gm.N = p->d; gm.K = rows; gm.lda = 192; gm.ldb = p->d; gm.ldc = p->d;
      gm.splits = gemm_splits(192, p->d, rows);
      gm.a_kc = false; gm.b_kc = false; gm.bf16 = false; gm.out_f32 = true;
      gm.vec_a = true;
      gm.vec_b = ((uintptr_t)x % 16 == 0) && (p->d % 4) == 0;
      HIPCHK(launch_gemm(gm, s));
    }
    tr.end(TR_AGEMM, tg, s);
    return PR_OK;
  }
  if (pl.path == PATH_CHAN) {
    const bool bf = p->dtype == PR_BF16;
    const size_t es = bf ? 2 : 4;
    const int kc = p->cell == PR_CELL_GRU_DIAG ? C_GRU_DIAG : C_LSTM;
    Trace &tr = trace();
    if (!u_ready) {
      const int tp = tr.begin(TR_PROJ, s);
      HIPCHK(input_projection(p, w, x, ws + pl.off_U, s, (float *)(ws + pl.off_cb)));
      tr.end(TR_PROJ, tp, s);
    }
    ChanArgs ca{};
    ca.U = ws + pl.off_U;
    ca.h = (void *)h;
    ca.h0 = h0;
    ca.Wh = w->W_h;
    ca.bh = w->b_h;
    ca.peep = p->cell == PR_CELL_LSTM_CIFG_DIAG ? w->peep : nullptr;
    ca.g = g;
    ca.lam = lambda;
    ca.dh0 = dh0;
    ca.dU = ws + pl.off_dU;
    ca.part = (float *)(ws + pl.off_part);
    ca.B = p->B; ca.T = p->T; ca.n = p->n; ca.SW = pl.SW;
    ca.k = 1;
    ca.st = (SolveState *)(ws + pl.off_state);
    ca.agg = (unsigned long long *)(ws + pl.off_agg);
    ca.incl = (unsigned long long *)(ws + pl.off_incl);
    ca.stripes = pl.stripes;
    const int ta = tr.begin(TR_ADJ, s);
    ca.tps = pl.tps_2;
    ca.ntiles = pl.ntiles_2;
    HIPCHK(launch_chan2_adjoint(kc, bf, ca, s, chan_aggs));
    tr.end(TR_ADJ, ta, s);
    const int tg = tr.begin(TR_AGEMM, s);
    if (dW && (dW->W_h || dW->b_h || dW->peep || dW->b_x))
      HIPCHK(launch_chan_reduce_tiles(kc, ca, (double *)(ws + pl.off_red), dW->W_h, dW->b_h, dW->peep, dW->b_x, s));
    // dx contracts over U's columns: W_x is read through a transposed copy
    // (small); dW_x contracts over the rows of dU and x, which the GEMM reads
    // K-outer and transposes while staging its tiles.
    const int rows = p->B * p->T, G3 = 3 * p->n;
    if (dx) {  // dx = dU W_x: B operand W_x^T [d, 3n]
      HIPCHK(launch_transpose(w->W_x, ws + pl.off_wt, G3, p->d, (int)es, s));
      GemmArgs gm{};
      gm.A = ws + pl.off_dU; gm.B = ws + pl.off_wt; gm.C = dx; gm.bias = nullptr; gm.ws = nullptr;
      gm.M = rows; gm.N = p->d; gm.K = G3; gm.lda = G3; gm.ldb = G3; gm.ldc = p->d; gm.splits = 1;
      gm.a_kc = true; gm.b_kc = true; gm.bf16 = bf; gm.out_f32 = !bf;
      gm.vec_a = ((size_t)G3 * es) % 16 == 0;
      gm.vec_b = gm.vec_a;
      HIPCHK(launch_gemm(gm, s));
    }
    if (dW && dW->W_x) {  // dW_x = dU^T x: dU [rows, 3n] and x [rows, d], both K-outer
      GemmArgs gm{};
      gm.A = ws + pl.off_dU; gm.B = x; gm.C = dW->W_x; gm.bias = nullptr;
      gm.ws = (float *)(ws + pl.off_gws);
      gm.M = G3; gm.N = p->d; gm.K = rows; gm.lda = G3; gm.ldb = p->d; gm.ldc = p->d;
      gm.splits = gemm_splits(G3, p->d, rows, bf);
      gm.a_kc = false; gm.b_kc = false; gm.bf16 = bf; gm.out_f32 = true;
      gm.vec_a = ((size_t)G3 * es) % 16 == 0;
      gm.vec_b = ((uintptr_t)x % 16 == 0) && ((size_t)p->d * es) % 16 == 0;
      HIPCHK(launch_gemm(gm, s));
    }
    tr.end(TR_AGEMM, tg, s);
    return PR_OK;
  }
  return fail(PR_EUNSUPPORTED, "no adjoint kernel for this problem");
}

static int solve_adjoint_core(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                              int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, const void *g,
                              void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace,
                              size_t ws_bytes, void *stream) {
  if (p && workspace && ws_bytes < pararnn_workspace_bytes(p, 1))
    return fail(PR_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, pararnn_workspace_bytes(p, 1));
  SpecAdjoint sa;
  sa.g = g;
  sa.lambda = lambda;
  sa.dx = dx;
  sa.dh0 = dh0;
  sa.dW = dW;
  const int rc = solve_impl(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, workspace, ws_bytes, stream,
                            nullptr, &sa);
  if (rc < 0) return rc;
  if (sa.done) return sa.rc < 0 ? sa.rc : rc;
  if (sa.rc < 0) return sa.rc;  // the speculative enqueue was rejected: the same arguments fail again
  if (rc == PR_NONFINITE) return rc;
  const int ra = adjoint_impl(p, w, x, h0, h, g, lambda, dx, dh0, dW, workspace, ws_bytes, stream, true, !sa.ran);
  return ra < 0 ? ra : rc;
}

namespace {

// ---------------------------------------------------------------------------
// Dense GRUs of other widths on the n = 64 kernels.  Padded with zero
// weights, biases and initial state, the extra channels stay exactly 0 (their
// gates are 1/2 and their candidate tanh(0) = 0) and the Jacobian has no
// entry between them and the real channels, so every sweep's update, the stop
// measure, the sweep count and the adjoint of the real channels are those of
// the unpadded problem.  The padded weights, states and gradients live at the
// front of the workspace; the results are copied back.
// ---------------------------------------------------------------------------
// A tanh RNN runs as the GRU whose reset gate is held at 1 and update gate
// at 0: its weights fill the candidate gate (block 2), the other blocks are
// zero, and the input biases of gates 0 and 1 are +-TANH_AS_GRU_BIAS, so the
// sigmoids give exactly 1 and 0 (exp of the negated argument is 0 or +inf,
// and the reciprocal of +inf is 0).  Then h' = tanh(W_x x + b_x + W_h h +
// b_h), and every Jacobian term through r or z carries r (1 - r) = 0 or
// z (1 - z) = 0, leaving diag(1 - c^2) W_h.
constexpr float TANH_AS_GRU_BIAS = 1e30f;
// The padded weights (and h0) into the workspace; w64 / h0p point at them.
static int pad_inputs(const pr_problem *p, const pr_weights *w, const void *h0, char *ws, const PadLayout &L,
                      pr_weights *w64, const void **h0p, hipStream_t s) {
  if (!w || !w->W_x || !w->W_h) return fail(PR_EINVAL, "W_x and W_h are required");
  const int n = p->n, d = p->d, N = D64_N;
  const bool tanh = p->cell == PR_CELL_TANH_RNN;
  const int gate = tanh ? 2 : -1;  // the source gate block (all three for a GRU)
  *w64 = pr_weights{};
  HIPCHK(launch_pad_gates((const float *)w->W_x, 3, n, d, (float *)(ws + L.wx), N, d, s, gate));
  HIPCHK(launch_pad_gates((const float *)w->W_h, 3, n, n, (float *)(ws + L.wh), N, N, s, gate));
  w64->W_x = ws + L.wx;
  w64->W_h = ws + L.wh;
  if (w->b_x || tanh) {
    if (w->b_x) HIPCHK(launch_pad_gates((const float *)w->b_x, 3, n, 1, (float *)(ws + L.bx), N, 1, s, gate));
    else HIPCHK(launch_pad_gates(nullptr, 3, 0, 1, (float *)(ws + L.bx), N, 1, s));  // zeros
    if (tanh) HIPCHK(launch_gate_consts((float *)(ws + L.bx), n, N, TANH_AS_GRU_BIAS, -TANH_AS_GRU_BIAS, s));
    w64->b_x = ws + L.bx;
  }
  if (w->b_h) {
    HIPCHK(launch_pad_gates((const float *)w->b_h, 3, n, 1, (float *)(ws + L.bh), N, 1, s, gate));
    w64->b_h = ws + L.bh;
  }
  *h0p = nullptr;
  if (h0) {
    HIPCHK(launch_pad_gates((const float *)h0, 1, p->B, n, (float *)(ws + L.h0), p->B, N, s));
    *h0p = ws + L.h0;
  }
  return PR_OK;
}
// [rows, 64] -> [rows, n]
static hipError_t unpad_state(const void *src, long long rows, int n, void *dst, hipStream_t s) {
  return launch_unpad_gates((const float *)src, 1, (int)rows, n, (float *)dst, (int)rows, D64_N, s);
}
// Workspace of the padded problem q for a solve (kind 0), an adjoint (1) or
// an ELK solve (2); returns the plan's error code and message if q has none.
static int padded_inner_bytes(const pr_problem *q, int kind, size_t *bytes) {
  *bytes = 0;
  Plan pl;
  int rc = make_plan(q, &pl);
  if (rc != PR_OK) return rc;
  if (kind == 2) {
    ElkLayout el;
    rc = elk_layout(q, pl, &el);
    if (rc != PR_OK) return rc;
    *bytes = el.bytes > pl.adjoint_bytes ? el.bytes : pl.adjoint_bytes;
  } else {
    *bytes = kind == 1 ? pl.adjoint_bytes : pl.solve_bytes;
  }
  return PR_OK;
}
static int pad_workspace_check(const pr_problem *q, int kind, const PadLayout &L, void *workspace, size_t ws_bytes) {
  size_t inner = 0;
  const int rc = padded_inner_bytes(q, kind, &inner);
  if (rc != PR_OK) return rc;
  if (!workspace || ws_bytes < L.bytes + inner)
    return fail(PR_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, L.bytes + inner);
  if (((uintptr_t)workspace & 255) != 0) return fail(PR_EINVAL, "workspace must be 256-byte aligned");
  return PR_OK;
}

static int padded_solve(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                        int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, void *workspace,
                        size_t ws_bytes, void *stream, const float *elk_lambda) {
  g_err.clear();
  if (!x || !h) return fail(PR_EINVAL, "x and h are required");
  if (max_iters < 1) return fail(PR_EINVAL, "max_iters must be >= 1");
  if (elk_lambda && (!(*elk_lambda >= 0.f) || *elk_lambda > 3.0e38f))
    return fail(PR_EINVAL, "lambda must be >= 0 and finite");
  const pr_problem q = padded(p);
  const PadLayout L = pad_layout(p, elk_lambda != nullptr);
  int rc = pad_workspace_check(&q, elk_lambda ? 2 : 0, L, workspace, ws_bytes);
  if (rc != PR_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  pr_weights w64;
  const void *h0p;
  rc = pad_inputs(p, w, h0, ws, L, &w64, &h0p, s);
  if (rc != PR_OK) return rc;
  rc = solve_impl(&q, &w64, x, h0p, tol, max_iters, ws + L.h, iters, delta_hist, hist_cap, ws + L.bytes,
                  ws_bytes - L.bytes, stream, elk_lambda);
  if (rc < 0) return rc;
  HIPCHK(unpad_state(ws + L.h, (long long)p->B * p->T, p->n, h, s));
  return rc;
}

static int padded_adjoint(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                          int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, const void *g,
                          void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace, size_t ws_bytes,
                          void *stream, bool with_solve) {
  g_err.clear();
  if (!x || !h || !g) return fail(PR_EINVAL, "x, h and g are required");
  if (with_solve && max_iters < 1) return fail(PR_EINVAL, "max_iters must be >= 1");
  const pr_problem q = padded(p);
  const PadLayout L = pad_layout(p, true);
  int rc = pad_workspace_check(&q, 1, L, workspace, ws_bytes);
  if (rc != PR_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  const long long rows = (long long)p->B * p->T;
  const int n = p->n, d = p->d, N = D64_N;
  pr_weights w64;
  const void *h0p;
  rc = pad_inputs(p, w, h0, ws, L, &w64, &h0p, s);
  if (rc != PR_OK) return rc;
  HIPCHK(launch_pad_gates((const float *)g, 1, (int)rows, n, (float *)(ws + L.g), (int)rows, N, s));
  pr_grads g64{};
  if (dW) {
    g64.W_x = dW->W_x ? (float *)(ws + L.dwx) : nullptr;
    g64.b_x = dW->b_x ? (float *)(ws + L.dbx) : nullptr;
    g64.W_h = dW->W_h ? (float *)(ws + L.dwh) : nullptr;
    g64.b_h = dW->b_h ? (float *)(ws + L.dbh) : nullptr;
  }
  void *dh0p = dh0 ? ws + L.dh0 : nullptr;
  if (with_solve) {
    rc = solve_adjoint_core(&q, &w64, x, h0p, tol, max_iters, ws + L.h, iters, delta_hist, hist_cap, ws + L.g,
                            ws + L.lam, dx, dh0p, dW ? &g64 : nullptr, ws + L.bytes, ws_bytes - L.bytes, stream);
    if (rc < 0) return rc;
    HIPCHK(unpad_state(ws + L.h, rows, n, h, s));
    if (rc == PR_NONFINITE) return rc;
  } else {
    HIPCHK(launch_pad_gates((const float *)h, 1, (int)rows, n, (float *)(ws + L.h), (int)rows, N, s));
    rc = adjoint_impl(&q, &w64, x, h0p, ws + L.h, ws + L.g, ws + L.lam, dx, dh0p, dW ? &g64 : nullptr, ws + L.bytes,
                      ws_bytes - L.bytes, stream, false, false);
    if (rc < 0) return rc;
  }
  if (lambda) HIPCHK(unpad_state(ws + L.lam, rows, n, lambda, s));
  if (dh0) HIPCHK(unpad_state(ws + L.dh0, p->B, n, dh0, s));
  // a tanh RNN's gradients are the candidate gate's block
  const int G = p->cell == PR_CELL_TANH_RNN ? 1 : 3, g0 = 3 - G;
  const float *dwx = (const float *)(ws + L.dwx) + (size_t)g0 * N * d, *dbx = (const float *)(ws + L.dbx) + g0 * N;
  const float *dwh = (const float *)(ws + L.dwh) + (size_t)g0 * N * N, *dbh = (const float *)(ws + L.dbh) + g0 * N;
  if (dW && dW->W_x) HIPCHK(launch_unpad_gates(dwx, G, n, d, dW->W_x, N, d, s));
  if (dW && dW->b_x) HIPCHK(launch_unpad_gates(dbx, G, n, 1, dW->b_x, N, 1, s));
  if (dW && dW->W_h) HIPCHK(launch_unpad_gates(dwh, G, n, n, dW->W_h, N, N, s));
  if (dW && dW->b_h) HIPCHK(launch_unpad_gates(dbh, G, n, 1, dW->b_h, N, 1, s));
  return rc;
}

}  // namespace

extern "C" {

int pararnn_solve_adjoint(const pr_problem *p, const pr_weights *w, const void *x, const void *h0, float tol,
                          int max_iters, void *h, int *iters, float *delta_hist, int hist_cap, const void *g,
                          void *lambda, void *dx, void *dh0, const pr_grads *dW, void *workspace, size_t ws_bytes,
                          void *stream) {
  if (pad_gru(p))
    return padded_adjoint(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, g, lambda, dx, dh0, dW,
                          workspace, ws_bytes, stream, true);
  return solve_adjoint_core(p, w, x, h0, tol, max_iters, h, iters, delta_hist, hist_cap, g, lambda, dx, dh0, dW,
                            workspace, ws_bytes, stream);
}

static bool lsim_sizes_ok(int B, int T, int nx, int m, int p) {
  return B >= 1 && T >= 1 && nx >= 1 && nx <= 8 && m >= 1 && m <= 8 && p >= 1 && p <= 8 &&
         (long long)B * ((T + lsim_chunk_len(m) - 1) / lsim_chunk_len(m)) < (1LL << 31) &&
         (long long)B * T < (1LL << 40);
}

size_t pararnn_lsim_workspace_bytes(int B, int T, int nx, int m, int p) {
  if (!lsim_sizes_ok(B, T, nx, m, p)) return 0;
  const size_t nchunks = (size_t)B * ((T + lsim_chunk_len(m) - 1) / lsim_chunk_len(m));
  return align256((size_t)lsim_table_floats() * 4) + 2 * align256(nchunks * 8 * 4);
}

int pararnn_lsim(int B, int T, int nx, int m, int p, const float *A, const float *Bm, const float *Cm,
                 const float *Dm, float dt, const float *U, const float *x0, float *x, float *y, void *workspace,
                 size_t ws_bytes, void *stream) {
  g_err.clear();
  if (B < 1 || T < 1 || nx < 1 || m < 1 || p < 1) return fail(PR_EINVAL, "sizes must be >= 1");
  if (nx > 8 || m > 8 || p > 8) return fail(PR_EUNSUPPORTED, "state, input and output widths are limited to 8");
  if (!lsim_sizes_ok(B, T, nx, m, p)) return fail(PR_EUNSUPPORTED, "problem too large");
  if (!A || !Bm || !Cm || !Dm || !U || !y) return fail(PR_EINVAL, "A, B, C, D, U and y are required");
  if (!(dt > 0.f) || dt != dt || dt > 3.0e38f) return fail(PR_EINVAL, "dt must be positive and finite");
  const size_t need = pararnn_lsim_workspace_bytes(B, T, nx, m, p);
  if (!workspace || ws_bytes < need) return fail(PR_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (((uintptr_t)workspace & 255) != 0) return fail(PR_EINVAL, "workspace must be 256-byte aligned");
  char *ws = (char *)workspace;
  const size_t nchunks = (size_t)B * ((T + lsim_chunk_len(m) - 1) / lsim_chunk_len(m));
  LsimArgs a{};
  a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dm = Dm; a.dt = dt;
  a.U = U; a.x0 = x0; a.x = x; a.y = y;
  a.table = (float *)ws;
  a.agg = (float *)(ws + align256((size_t)lsim_table_floats() * 4));
  a.carry = (float *)(ws + align256((size_t)lsim_table_floats() * 4) + align256(nchunks * 8 * 4));
  a.B = B; a.T = T; a.nx = nx; a.m = m; a.p = p;
  hipStream_t s = (hipStream_t)stream;
  Trace &tr = trace();
  if (tr.on) HIPCHK(tr.make());
  const int ti = tr.begin(TR_SWEEP_LSIM, s);
  HIPCHK(launch_lsim(a, s));
  tr.end(TR_SWEEP_LSIM, ti, s);
  return PR_OK;
}

size_t pararnn_scan_workspace_bytes(int jac, int B, int T, int n) {
  if (B < 1 || T < 1 || n < 1) return 0;
  if (jac == PR_JAC_DENSE) {
    const int N = time_padded_n(n);
    if (!N) return 0;
    const size_t nt = (size_t)B * ((T + time_tile(N) - 1) / time_tile(N));
    return align256(sizeof(SolveState)) + align256(nt * (N * N + N) * 8) + align256(nt * N * 8);
  }
  if (jac == PR_JAC_DIAG || jac == PR_JAC_BLOCK2) {
    const int SW = jac == PR_JAC_BLOCK2 ? 2 : 1;
    const ChanGeomInfo gi = chan_geom(SW == 2 ? C_LSTM : C_GRU_DIAG, n);
    const size_t nt = (size_t)B * ((n + gi.CH - 1) / gi.CH) * ((T + gi.TT - 1) / gi.TT);
    return align256(sizeof(SolveState)) + align256(nt * gi.CH * (SW * SW + SW) * 8) + align256(nt * gi.CH * SW * 8);
  }
  return 0;
}

int pararnn_affine_scan(int jac, int B, int T, int n, int reverse, const float *A, const float *b, float *y,
                        void *workspace, size_t ws_bytes, void *stream) {
  g_err.clear();
  return affine_scan_run(jac, B, T, n, reverse, A, b, y, workspace, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"

namespace pr {

int affine_scan_run(int jac, int B, int T, int n, int reverse, const float *A, const float *b, float *y, void *workspace,
                    size_t ws_bytes, hipStream_t s) {
  if (jac < 0 || jac > 2) return fail(PR_EINVAL, "unknown jac %d", jac);
  if (B < 1 || T < 1 || n < 1) return fail(PR_EINVAL, "sizes must be >= 1");
  if (!A || !b || !y) return fail(PR_EINVAL, "A, b and y are required");
  const size_t need = pararnn_scan_workspace_bytes(jac, B, T, n);
  if (need == 0) return fail(PR_EUNSUPPORTED, "no scan kernel for jac %d n %d", jac, n);
  if (!workspace || ws_bytes < need) return fail(PR_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (((uintptr_t)workspace & 255) != 0) return fail(PR_EINVAL, "workspace must be 256-byte aligned");
  char *ws = (char *)workspace;
  HIPCHK(launch_zero(ws, need, s));
  if (jac != PR_JAC_DENSE) {
    const int SW = jac == PR_JAC_BLOCK2 ? 2 : 1;
    const ChanGeomInfo gi = chan_geom(SW == 2 ? C_LSTM : C_GRU_DIAG, n);
    ChanArgs ca{};
    ca.A = A; ca.b = b; ca.y = y;
    ca.B = B; ca.T = T; ca.n = n; ca.SW = SW; ca.reverse = reverse ? 1 : 0;
    ca.stripes = B * ((n + gi.CH - 1) / gi.CH);
    ca.tps = (T + gi.TT - 1) / gi.TT;
    ca.ntiles = ca.stripes * ca.tps;
    ca.st = (SolveState *)ws;
    ca.agg = (unsigned long long *)(ws + align256(sizeof(SolveState)));
    ca.incl = (unsigned long long *)(ws + align256(sizeof(SolveState)) +
                                     align256((size_t)ca.ntiles * gi.CH * (SW * SW + SW) * 8));
    HIPCHK(launch_chan_scan(SW, ca, s));
    return PR_OK;
  }
  const int N = time_padded_n(n);
  ScanArgs a{};
  a.A = A; a.b = b; a.y = y;
  a.B = B; a.T = T; a.n = n; a.reverse = reverse ? 1 : 0;
  a.tiles_per_seq = (T + time_tile(N) - 1) / time_tile(N);
  a.ntiles = a.tiles_per_seq * B;
  a.st = (SolveState *)ws;
  a.agg = (unsigned long long *)(ws + align256(sizeof(SolveState)));
  a.incl = (unsigned long long *)(ws + align256(sizeof(SolveState)) + align256((size_t)a.ntiles * (N * N + N) * 8));
  HIPCHK(launch_time_scan(N, a, s));
  return PR_OK;
}

}  // namespace pr
