// Host-side interface between the ABI layer (pararnn.cpp) and the kernel
// files.  Every launch_* returns a hipError_t and validates nothing: the ABI
// layer checks shapes, pointers and workspace sizes before it calls them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace pr {

constexpr int DX_FUSED = 8;  // largest input width folded into the time-parallel kernels

// ---------------- time-parallel path (dense state, n <= 8) -----------------
struct TimeArgs {
  const float *x;   // [B,T,d]
  float *h;         // [B,T,n] iterate, updated in place (read-only in the adjoint)
  const float *h0;  // [B,n] or null
  const float *Wx, *bx, *Wh, *bh;
  const float *g;   // adjoint: [B,T,n]
  float *lam, *dx, *dh0;  // adjoint outputs (may be null)
  float *part;            // adjoint: per-tile parameter-gradient partials
  int B, T, d, n;
  int k;
  float tol;
  int max_iters;
  SolveState *st;
  unsigned long long *agg, *incl;  // look-back descriptors
  float *bnd;                      // [2][ntiles][N] boundary states
  int tiles_per_seq, ntiles, vec_ok;
  int nparts;  // adjoint: blocks that wrote weight partials (set by the launcher)
  const float *coef;  // scalar-state sweep: cell coefficients folded from the weights
  int approx;         // sweep: APX_NEWTON, APX_DIAG or APX_ZERO (not the scalar-state sweep)
};

int time_tile(int N);               // elements per tile for padded width N
int time_padded_n(int n);           // N for a given n (0 if unsupported)
int time_part_count(int cell, int N);  // floats per tile of gradient partials
hipError_t launch_time_sweep(int cell, int N, const TimeArgs &a, hipStream_t s);
hipError_t launch_time_adjoint(int cell, int N, TimeArgs &a, hipStream_t s);
// Scalar-state sweep (n = d = 1, T % 4 == 0, x and h 16-byte aligned); same
// tile geometry as the generic sweep at N = 1.
int scalar_tile();      // steps per tile of the scalar sweep
int scalar_adj_tile();  // steps per tile of the scalar adjoint
hipError_t launch_zero_coef(void *p, size_t bytes, const float *Wx, const float *bx, const float *Wh,
                            const float *bh, int cell, float *coef, hipStream_t s);
hipError_t launch_scalar_sweep(int cell, const TimeArgs &a, hipStream_t s);
hipError_t launch_scalar_adjoint(int cell, TimeArgs &a, hipStream_t s);  // sets a.nparts
hipError_t launch_time_elk_jr(int cell, int N, const TimeArgs &a, float *jr, hipStream_t s);
hipError_t launch_time_reduce(int cell, int N, const TimeArgs &a, const float *part, float *dWx, float *dbx,
                              float *dWh, float *dbh, hipStream_t s);

struct ScanArgs {
  const float *A, *b;
  float *y;
  int B, T, n, reverse;
  unsigned long long *agg, *incl;
  SolveState *st;
  int tiles_per_seq, ntiles;
};
hipError_t launch_time_scan(int N, const ScanArgs &a, hipStream_t s);

// ---------------- channel-parallel path (diagonal / 2x2-block Jacobian) ----
struct ChanArgs {
  const void *U;        // [B,T,3n] input projection (storage dtype)
  void *h;              // [B,T,S] iterate, updated in place
  const void *h0;       // [B,S] or null
  const void *Wh, *bh, *peep;
  const void *g;        // adjoint: [B,T,S]
  void *lam, *dh0;      // adjoint outputs (may be null)
  void *dU;             // adjoint: [B,T,3n] gate gradients (storage dtype)
  float *part;          // adjoint: weight-gradient partials
  const float *A, *b;   // standalone scan
  float *y;
  int B, T, n, SW;
  int k;
  float tol;
  int max_iters;
  SolveState *st;
  // standalone scan: tagged look-back descriptors; sweep and adjoint passes:
  // fp32 tile aggregates [ntiles][CH][SW*SW+SW] and carries [ntiles][CH][SW]
  unsigned long long *agg, *incl;
  float *bnd;           // [2][ntiles][CH*SW] each tile's last state, per sweep parity
  int stripes, tps, ntiles;
  int reverse;
};
struct ChanGeomInfo {
  int CPL, TW, CH, TT;
};
ChanGeomInfo chan_geom(int cell, int n);  // tiles of the standalone scan
// streaming sweep passes (no chain between tiles): tiles of CHAN2_TT steps,
// one wavefront each; per sweep a carry scan then a pass that applies the
// sweep and composes the next sweep's tile aggregates
constexpr int CHAN2_TT = 64;
// CHAN2_APPLY_ADJ: the last pass of a fixed sweep count followed by an
// adjoint (a.g set): it composes the adjoint's tile aggregates at the final
// iterate; the adjoint then runs with fused = true
enum { CHAN2_FIRST = 0, CHAN2_CARRY = 1, CHAN2_APPLY_NEXT = 2, CHAN2_APPLY = 3, CHAN2_APPLY_ADJ = 4 };
ChanGeomInfo chan2_geom(int cell, int n);
// apx: APX_NEWTON, APX_DIAG (LSTM) or APX_ZERO
hipError_t launch_chan2(int cell, int apx, bool bf16, const ChanArgs &a, int what, hipStream_t s);
// adjoint as streaming passes on the same tiles (aggregates, reverse carry
// scan, apply); per-tile weight partials [tiles][CH][11]
// fused: the tile aggregates were composed by a CHAN2_APPLY_ADJ pass (all but
// each tile's first step) and only the carry and the applying pass run
hipError_t launch_chan2_adjoint(int cell, bool bf16, const ChanArgs &a, hipStream_t s, bool fused = false);
// weight gradients from per-tile partials: CHAN_RED_SPLITS fp64 partial sums
// per (channel, slot) in `red`, then their sum in order
constexpr int CHAN_RED_SPLITS = 32;
hipError_t launch_chan_reduce_tiles(int cell, ChanArgs &a, double *red, float *dWh, float *dbh, float *dpeep,
                                   float *dbx, hipStream_t s);
hipError_t launch_chan_scan(int SW, ChanArgs &a, hipStream_t s);

// ---------------- dense n = 64 path (MFMA scan) ----------------------------
constexpr int D64_N = 64, D64_L = 64;  // state width, steps per chunk
struct D64Args {
  const float *U;       // [B*T, 192] input projection
  float *h;             // [B*T, 64] iterate (read-only in the adjoint)
  const float *h0;      // [B, 64] or null
  const float *Wh, *bh; // [192, 64], [192] or null
  float *gates;         // [B*T, 5, 64]: z, alpha, beta, gamma, and res (sweep) or eta (adjoint)
  float *aggP;          // [nchunks, 64, 64] chunk products
  float *aggb;          // [nchunks, 64] chunk offsets
  float *carry;         // [nchunks, 64] state entering each chunk
  const float *g;       // adjoint: [B*T, 64]
  float *lam;           // adjoint: [B*T, 64]
  int B, T, cps, nchunks;  // chunks per sequence, total chunks
  int k;
  float tol;
  int max_iters;
  SolveState *st;
  int adjoint;          // reverse-time scan with transposed Jacobians
  int approx;           // sweep: APX_NEWTON (dense chunk products) or APX_DIAG / APX_ZERO (per-channel scan)
};
// one sweep = part 0 (gates), part 1 (chunk products), part 2 (carries + replay);
// with a.approx != APX_NEWTON: part 0 (gates, diagonal Jacobian, chunk
// aggregates), part 1 (carries), part 2 (apply)
hipError_t launch_d64_sweep_part(D64Args &a, int part, hipStream_t s);
hipError_t launch_d64_adjoint_scan(D64Args &a, hipStream_t s);
struct D64AdjArgs {
  const float *gates, *lam, *h, *h0, *Wh;
  float *dU;            // [B*T, 192] gate pre-activation gradients
  float *dA;            // [B*T, 192] gradients of the recurrent pre-activations
  float *hprev;         // [B*T, 64] state entering each step
  float *dh0;           // [B, 64] or null
  int B, T;
};
hipError_t launch_d64_adjoint_epilogue(const D64AdjArgs &a, hipStream_t s);
// column sums of X [rows, cols] (cols <= 256 per pass), fp64 partials [512][cols] in `part`
hipError_t launch_colsum(const float *X, int rows, int cols, float *out, double *part, hipStream_t s);

// ---------------- MFMA GEMM ------------------------------------------------
struct GemmArgs {
  const void *A, *B;    // A: [M,K] (a_kc) or [K,M]; B: [N,K] (b_kc) or [K,N]
  void *C;              // [M,N] row stride ldc
  const void *bias;     // [N] or null (input dtype)
  const float *bias32;  // [N] fp32 or null: used instead of bias when set
  const float *scale32; // [N] fp32 or null: C = scale * (A B^T) + bias per column
  float *ws;            // split-K workspace [splits][M][N]
  int M, N, K, lda, ldb, ldc, splits;
  bool a_kc, b_kc, bf16, out_f32, vec_a, vec_b;
};
// K splits of a long-K product; big: sized for the 256 x 256 bf16 kernel
// (used when M and N reach a block tile)
int gemm_splits(int M, int N, int K, bool big = false);
// C[192,N] = A^T B and csum = column sums of A for K-outer fp32 A [K,192],
// B [K,N] (N <= 64); C or csum may be null; ws of tn_workspace_bytes(K)
size_t tn_workspace_bytes(int K);
hipError_t launch_tn_products(const float *A, const float *B, int K, int N, float *C, float *csum, void *ws,
                              hipStream_t s);
hipError_t launch_gemm(const GemmArgs &g, hipStream_t s);

// ---------------- utilities ------------------------------------------------
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
// Gate-blocked zero padding (fp32): src [G*n, cols] -> dst [G*np, cols_p],
// row g*np + j = row g*n + j of src for j < n (first cols columns), zeros
// elsewhere; with only_gate >= 0, src is one gate [n, cols] placed in block
// only_gate and the other blocks are zero.  unpad copies back (cols <=
// cols_p).  A state array [rows, n] padded to [rows, np] is the case G = 1,
// n = np = rows, cols = n, cols_p = np.
hipError_t launch_pad_gates(const float *src, int G, int n, int cols, float *dst, int np, int cols_p, hipStream_t s,
                            int only_gate = -1);
hipError_t launch_unpad_gates(const float *src, int G, int n, int cols, float *dst, int np, int cols_p, hipStream_t s);
// dst[j] = v0, dst[np + j] = v1 for j < n (the first two gate blocks of a bias)
hipError_t launch_gate_consts(float *dst, int n, int np, float v0, float v1, hipStream_t s);
// copy `bytes` (a multiple of 4) from device memory to host-coherent memory,
// then store val to *seq with a system-scope release (one block)
hipError_t launch_snapshot(const void *src, void *dst, size_t bytes, unsigned *seq, unsigned val, hipStream_t s);
// Epilogue of the per-channel cells' input projection, fp32 [6n]: [0, 3n) the
// bias, b_x plus the recurrent biases of the gates whose pre-activations are
// plain sums (LSTM f, g, o; GRU r, z), and [3n, 6n) the column scale, each
// gate's chan_gate_scale; the bias is stored scaled.  Either bias may be null
// (= 0).  cell is C_GRU_DIAG or C_LSTM.
hipError_t launch_fold_bias(bool bf16, const void *bx, const void *bh, int n, int cell, float *out, hipStream_t s);
// dst [C, R] = transpose of row-major src [R, C]; elem_bytes 2 or 4
hipError_t launch_transpose(const void *src, void *dst, int R, int C, int elem_bytes, hipStream_t s);

// linear state-space simulation (k_lsim.hip)
struct LsimArgs {
  const float *A, *Bm, *Cm, *Dm;  // [nx,nx], [nx,m], [p,nx], [p,m]
  float dt;
  const float *U;    // [B,T,m]
  const float *x0;   // [B,nx] or null
  float *x;          // [B,T,nx] or null
  float *y;          // [B,T,p]
  float *table;      // lsim_table_floats(): Ad, Bd and power tables
  float *agg, *carry;  // [nchunks][8]
  int B, T, nx, m, p;
  int V, cps, nchunks;  // steps per lane, chunks per sequence, chunks (set by launch_lsim)
};
int lsim_table_floats();
int lsim_chunk_len(int m);  // steps per chunk
hipError_t launch_lsim(LsimArgs &a, hipStream_t s);

// quasi-ELK (k_elk.hip)
struct ElkArgs {
  float *jr;  // [rows][2S]: the Jacobian's diagonal d | residual r (producer output)
  float *ge;  // [rows][2S]: smoother gains G | offsets e
  float *r1, *pc, *mc, *r3, *msc;  // per chunk: filter maps [7][S], entering P [S] and m [S],
                                   // reverse maps [2][S], m^s from the right [S]
  void *h;    // [rows][S] iterate (storage dtype)
  int h_bf16;
  int B, T, S, cps, nch;
  int L, sp;  // steps per chunk, lanes per chunk (the dense-family scans)
  float lam;
  int k;
  float tol;
  int max_iters;
  SolveState *st;
};
struct ElkChanArgs {  // per-channel cells (the smoother's e.r3 and e.msc are shared)
  ElkArgs e;
  const void *U, *h0, *Wh, *bh, *peep;
  float *fagg, *fcar;  // per filter chunk (4 apply chunks): filter maps [7][S], (P, m) entering [2][S]
  float *fsub;         // per apply chunk (e.cps per sequence): (P, m) entering [2][S]
  float *dr, *hb;      // per apply chunk: d, r at the next chunk's first step [2][S], state at the last step [S]
  int n;
  int cpf, nchf;       // filter chunks per sequence and in all
};
// ELK with the cell's own Jacobian (full covariances per unit of N state
// entries: each LSTM channel's (c, h), N = 2; a small dense cell's state, N =
// n padded).  Per step [t][unit][N*N + N]: J_t | r_t (jr), then G_t | e_t (ge);
// per (chunk, unit): the filtering element [3N^2 + 2N], (m, P) entering
// [N + N^2], the reverse map Mr | vr [N^2 + N], m^s from the right [N].
struct ElkFullArgs {
  float *jr, *ge, *elem, *fin, *rev, *msin;
  void *h;                              // iterate [B, T, S] (storage dtype)
  const void *U, *h0, *Wh, *bh, *peep;  // the LSTM producer's inputs
  int B, T, n, S;
  int units, upb, NS;  // units, units per sequence, state entries per unit
  int L, cpu;          // steps per chunk, chunks per unit
  float lam;
  int k;
  float tol;
  int max_iters;
  SolveState *st;
};
// ELK with the full 64 x 64 Jacobian of the dense GRU: the damped step's
// normal equations eliminated by block cyclic reduction (k_elk64.hip).
struct Elk64Args {
  const float *gates;      // [B*T, 5, 64] from the gates kernel: z, alpha, beta, gamma, res
  const float *Wh;         // [192, 64]
  float *A, *D, *S;        // [B*T, 64, 64] block rows (A, D become P, Q at elimination)
  float *f, *g, *v, *x;    // [B*T, 64]
  float *h;                // [B*T, 64] iterate
  int B, T;
  float lam;
  int k;
  SolveState *st;
};
hipError_t launch_elk64_passes(const Elk64Args &a, hipStream_t s);
int elk_full_chunk_len(int T);
hipError_t launch_elk_full_lstm(bool bf16, const ElkFullArgs &a, hipStream_t s);
hipError_t launch_elk_full_dense(int cell, int Nv, const TimeArgs &ta, const ElkFullArgs &a, hipStream_t s);
int elk_chunk_len(int S);         // steps per chunk of the dense-family quasi-ELK scans
int elk_lanes_per_chunk(int S);
int elk_chan_chunk_len(int sw);
hipError_t launch_elk_sweep(ElkArgs &a, hipStream_t s);
hipError_t launch_elk_chan_sweep(int cell, bool bf16, ElkChanArgs &a, hipStream_t s);

// ---------------- ABI layer helpers shared across translation units ---------
// Records a message for pararnn_last_error() on the calling thread and
// returns `code`.
int fail(int code, const char *fmt, ...);
void clear_error();
// The linear recurrence of pararnn_affine_scan on a caller-provided scratch
// buffer `ws` (256-byte aligned, ws_bytes long): validates the arguments,
// clears what must start at zero and launches the scan on `s`.
int affine_scan_run(int jac, int B, int T, int n, int reverse, const float *A, const float *b, float *y, void *ws,
                    size_t ws_bytes, hipStream_t s);

}  // namespace pr
