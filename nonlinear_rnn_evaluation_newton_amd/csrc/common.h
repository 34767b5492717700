// Device-side building blocks shared by the gfx950 kernels of libpararnn:
// storage conversion, fast fp32 activations, the affine scan operator and its
// wavefront scan in DPP registers, tagged look-back descriptors, and the
// solve-state record that carries the on-device convergence test.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define PR_HIST 1024  // delta history ring (entries) kept in the solve state

namespace pr {

// ---------------------------------------------------------------------------
// solve state (lives at the start of the workspace)
// ---------------------------------------------------------------------------
// delta_k is accumulated as float bits with atomicMax on |dh| (non-negative
// floats order like their bit patterns; NaN bits sort above +inf) into 64
// shards, so no address takes more than a few dozen atomics per sweep.
constexpr int PR_DSHARDS = 64;
struct SolveState {
  unsigned int stopped;      // sticky: a sweep saw the stop rule hold
  int iters;                 // sweep count at the stop
  int status;                // PR_OK / PR_NOT_CONVERGED / PR_NONFINITE
  unsigned int fault;        // a look-back wait exceeded PR_SPIN_LIMIT (grid not co-resident)
  unsigned int pad[12];
  unsigned int dslot[4][PR_DSHARDS];  // shards of delta_k for sweep k % 4
  unsigned int hist[PR_HIST];         // delta_k (slot k % PR_HIST), finalised by sweep k + 1 or the host
};

enum { ST_OK = 0, ST_NOT_CONVERGED = 1, ST_NONFINITE = 2 };

// kernel-side cell codes (same values as the ABI's PR_CELL_*)
enum { C_TANH = 0, C_GRU = 1, C_GRU_DIAG = 2, C_LSTM = 3, C_LINEAR = 4 };

// The Jacobian a sweep's linear solve uses: the cell's own (Newton, DEER),
// its diagonal (quasi-DEER), or zero (Jacobi) (Gonzalez et al. abstract:
// quasi-Newton approximations; Para-Seq README, Main features: Jacobi,
// quasi-DEER and DEER solvers).  Only the solve changes: the residual, the
// update and the adjoint use the cell itself.
enum { APX_NEWTON = 0, APX_DIAG = 1, APX_ZERO = 2 };
// Channel kernels take the approximation in the cell template argument:
// cell code + 16 * approximation.
constexpr int cell_code(int CELL) { return CELL & 15; }
constexpr int cell_apx(int CELL) { return CELL >> 4; }
__host__ __device__ constexpr int cell_gates(int cell) {
  return (cell == C_GRU || cell == C_GRU_DIAG || cell == C_LSTM) ? 3 : 1;
}

// The stop rule after sweep k with measure delta (same on host and device):
// non-finite -> NONFINITE; tol > 0 and delta < tol -> OK; k == T -> OK (Newton
// is exact after T sweeps); k == max_iters -> NOT_CONVERGED (OK if tol <= 0).
__host__ __device__ inline bool stop_rule(float delta, int k, float tol, int T, int max_iters, int *status) {
  if (!(delta <= 3.402823466e38f)) { *status = ST_NONFINITE; return true; }  // NaN or +inf
  if (tol > 0.f && delta < tol) { *status = ST_OK; return true; }
  if (k >= T) { *status = ST_OK; return true; }
  if (k >= max_iters) { *status = tol > 0.f ? ST_NOT_CONVERGED : ST_OK; return true; }
  return false;
}

// ---------------------------------------------------------------------------
// atomics at agent scope (coherent across the XCDs' L2 caches)
// ---------------------------------------------------------------------------
__device__ inline unsigned ld_agent(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bound on the retries of a look-back wait.  A healthy wait needs a few
// hundred at most; past the bound the waiter records a fault in the solve
// state and gives up (its results are then undefined), so a grid that is not
// co-resident ends with an error instead of hanging the device.
constexpr int PR_SPIN_LIMIT = 1 << 16;
__device__ inline void spin_fault(SolveState *st) {
  if (st) st_agent(&st->fault, 1u);
}
__device__ inline unsigned long long ld_agent64(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent64(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned add_agent(unsigned *p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void max_agent(unsigned *p, unsigned v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Look-back descriptors are arrays of 64-bit words (tag << 32 | float bits).
// Each word is single-copy atomic, so a reader accepts a payload only when
// every word carries the expected tag; no fences are needed.  Tags: 2k for a
// tile aggregate, 2k+1 for an inclusive prefix, k = sweep number >= 1; the
// arrays are zeroed at the start of each call.
__device__ inline unsigned tag_agg(int k) { return 2u * (unsigned)k; }
__device__ inline unsigned tag_incl(int k) { return 2u * (unsigned)k + 1u; }
__device__ inline void desc_put(unsigned long long *p, unsigned tag, float v) {
  st_agent64(p, ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v));
}
template <int W>
__device__ inline bool desc_get(const unsigned long long *p, unsigned tag, float *out) {
#pragma unroll
  for (int i = 0; i < W; i++) {
    unsigned long long v = ld_agent64(p + i);
    if ((unsigned)(v >> 32) != tag) return false;
    out[i] = __uint_as_float((unsigned)v);
  }
  return true;
}

// ---------------------------------------------------------------------------
// storage conversion
// ---------------------------------------------------------------------------
__device__ inline float bf2f(uint16_t b) { return __uint_as_float((unsigned)b << 16); }
// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
__device__ inline uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ inline float ldf(const float *p, size_t i) { return p[i]; }
__device__ inline float ldf(const uint16_t *p, size_t i) { return bf2f(p[i]); }
__device__ inline void stf(float *p, size_t i, float v) { p[i] = v; }
__device__ inline void stf(uint16_t *p, size_t i, float v) { p[i] = f2bf(v); }

// ---------------------------------------------------------------------------
// fp32 activations on the hardware exp2 / reciprocal units
// ---------------------------------------------------------------------------
__device__ inline float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float fsigm(float a) { return frcp(1.f + fexp(-a)); }
__device__ inline float ftanh(float a) {
  return 1.f - 2.f * frcp(1.f + __builtin_amdgcn_exp2f(a * (2.f * 1.4426950408889634f)));
}

// ---------------------------------------------------------------------------
// The affine operator y -> A y + b (dense N x N) and its composition.
// compose(later, earlier) = (A_l A_e, A_l b_e + b_l): apply `earlier` first.
// ---------------------------------------------------------------------------
template <int N>
struct Op {
  float A[N * N];
  float b[N];
};

template <int N>
__device__ inline Op<N> op_identity() {
  Op<N> o;
#pragma unroll
  for (int i = 0; i < N; i++) {
#pragma unroll
    for (int j = 0; j < N; j++) o.A[i * N + j] = i == j ? 1.f : 0.f;
    o.b[i] = 0.f;
  }
  return o;
}

template <int N>
__device__ inline Op<N> compose(const Op<N> &l, const Op<N> &e) {
  Op<N> o;
#pragma unroll
  for (int i = 0; i < N; i++) {
#pragma unroll
    for (int j = 0; j < N; j++) {
      float a = l.A[i * N] * e.A[j];
#pragma unroll
      for (int k = 1; k < N; k++) a = fmaf(l.A[i * N + k], e.A[k * N + j], a);
      o.A[i * N + j] = a;
    }
    float bb = l.b[i];
#pragma unroll
    for (int k = 0; k < N; k++) bb = fmaf(l.A[i * N + k], e.b[k], bb);
    o.b[i] = bb;
  }
  return o;
}

// y = A c + b
template <int N>
__device__ inline void op_apply(const Op<N> &o, const float *c, float *y) {
#pragma unroll
  for (int i = 0; i < N; i++) {
    float a = o.b[i];
#pragma unroll
    for (int k = 0; k < N; k++) a = fmaf(o.A[i * N + k], c[k], a);
    y[i] = a;
  }
}

// Move an operator across lanes with DPP; lanes without a source (or masked
// off) receive the identity operator.
template <int CTRL, int ROW_MASK, int N>
__device__ inline Op<N> dpp_op(const Op<N> &v) {
  Op<N> o;
#pragma unroll
  for (int i = 0; i < N * N; i++) {
    const int idv = (i / N == i % N) ? (int)0x3f800000 : 0;
    o.A[i] = __int_as_float(__builtin_amdgcn_update_dpp(idv, __float_as_int(v.A[i]), CTRL, ROW_MASK, 0xf, false));
  }
#pragma unroll
  for (int i = 0; i < N; i++)
    o.b[i] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v.b[i]), CTRL, ROW_MASK, 0xf, false));
  return o;
}

// Inclusive scan of the (non-commutative) affine operator over the 64 lanes
// of a wavefront, lane order = application order: row shifts 1, 2, 4, 8 inside
// 16-lane rows, then row broadcasts of lane 15 and lane 31.
template <int N>
__device__ inline Op<N> wave_scan_incl(Op<N> x) {
  x = compose(x, dpp_op<0x111, 0xf>(x));  // row_shr:1
  x = compose(x, dpp_op<0x112, 0xf>(x));  // row_shr:2
  x = compose(x, dpp_op<0x114, 0xf>(x));  // row_shr:4
  x = compose(x, dpp_op<0x118, 0xf>(x));  // row_shr:8
  x = compose(x, dpp_op<0x142, 0xa>(x));  // row_bcast:15 -> rows 1, 3
  x = compose(x, dpp_op<0x143, 0xc>(x));  // row_bcast:31 -> rows 2, 3
  return x;
}

// Value of lane (l - 1), identity for lane 0 (wave_shr:1).
template <int N>
__device__ inline Op<N> wave_shift1(const Op<N> &x) {
  return dpp_op<0x138, 0xf>(x);
}

// Read lane 63's value into every lane.
template <int N>
__device__ inline Op<N> wave_last(const Op<N> &x) {
  Op<N> o;
#pragma unroll
  for (int i = 0; i < N * N; i++) o.A[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x.A[i]), 63));
#pragma unroll
  for (int i = 0; i < N; i++) o.b[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x.b[i]), 63));
  return o;
}

__device__ inline unsigned wave_max_u32(unsigned v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    unsigned o = (unsigned)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// v of the lane the DPP control names (0 where there is none, or where the
// row mask leaves the row out)
template <int CTRL, int ROWS>
__device__ inline unsigned dpp_or0(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
// Sum and maximum over the wavefront's 64 lanes (all active), returned to every lane: an
// inclusive scan by row shifts (1, 2, 4, 8) and row broadcasts (15, 31),
// whose last lane holds the total.  A fixed order, and no LDS round trip per
// level as a shuffle butterfly has.
__device__ inline float wave_total(float v) {
  v += __uint_as_float(dpp_or0<0x111, 0xf>(__float_as_uint(v)));
  v += __uint_as_float(dpp_or0<0x112, 0xf>(__float_as_uint(v)));
  v += __uint_as_float(dpp_or0<0x114, 0xf>(__float_as_uint(v)));
  v += __uint_as_float(dpp_or0<0x118, 0xf>(__float_as_uint(v)));
  v += __uint_as_float(dpp_or0<0x142, 0xa>(__float_as_uint(v)));
  v += __uint_as_float(dpp_or0<0x143, 0xc>(__float_as_uint(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline unsigned wave_max_dpp(unsigned v) {
  v = max(v, dpp_or0<0x111, 0xf>(v));
  v = max(v, dpp_or0<0x112, 0xf>(v));
  v = max(v, dpp_or0<0x114, 0xf>(v));
  v = max(v, dpp_or0<0x118, 0xf>(v));
  v = max(v, dpp_or0<0x142, 0xa>(v));
  v = max(v, dpp_or0<0x143, 0xc>(v));
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace pr

namespace pr {

// Start-of-sweep control shared by every kernel that opens a sweep: apply the
// stop rule to the previous sweep's measure (k >= 2); block 0 finalises the
// history entry and clears the shards sweep k + 1 will use.  Returns true
// (to every thread of the block) when the solve has stopped.
__device__ inline bool sweep_open(SolveState *st, int k, float tol, int T, int max_iters, int *s_stop) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int stop = ld_agent(&st->stopped) != 0;
    if (!stop && k >= 2) {
      unsigned d = ld_agent(&st->dslot[(k - 1) & 3][lane]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        unsigned o = (unsigned)__shfl_xor((int)d, off, 64);
        d = d > o ? d : o;
      }
      int status;
      if (stop_rule(__uint_as_float(d), k - 1, tol, T, max_iters, &status)) {
        stop = 1;
        if (blockIdx.x == 0 && lane == 0) {
          st_agent((unsigned *)&st->iters, (unsigned)(k - 1));
          st_agent((unsigned *)&st->status, (unsigned)status);
          st_agent(&st->stopped, 1u);
        }
      }
      if (blockIdx.x == 0 && lane == 0) st_agent(&st->hist[(k - 1) % PR_HIST], d);
    }
    if (!stop && blockIdx.x == 0) st_agent(&st->dslot[(k + 1) & 3][lane], 0u);
    if (lane == 0) *s_stop = stop;
  }
  __syncthreads();
  return *s_stop != 0;
}

// Later kernels of a sweep only test the sticky flag.
__device__ inline bool sweep_is_stopped(const SolveState *st, int *s_stop) {
  if (threadIdx.x == 0) *s_stop = ld_agent(&st->stopped) != 0;
  __syncthreads();
  return *s_stop != 0;
}

// Block barrier that orders LDS accesses only: waits for this wavefront's
// LDS operations, then s_barrier.  Unlike __syncthreads it does not wait for
// outstanding global loads and stores, so loads prefetched for later steps
// stay in flight across it.  Global memory written before it is not
// guaranteed visible to other wavefronts after it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Blocks of `kernel` that fit on the device at once: the grid of a
// persistent kernel (every block resident, so an in-order tile walk cannot
// deadlock).
inline int device_cu_count() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  return cus;
}

template <auto KERN, int THREADS = 256>
int resident_blocks() {
  static int cached = 0;  // one per kernel instantiation
  if (cached) return cached;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERN, THREADS, 0) != hipSuccess || per_cu < 1) return 0;
  cached = per_cu * device_cu_count();
  return cached;
}

template <auto KERN, int THREADS = 256>
int persistent_grid(int ntiles) {
  const int r = resident_blocks<KERN, THREADS>();
  if (r <= 0) return 0;
  return ntiles < r ? ntiles : r;
}

}  // namespace pr
