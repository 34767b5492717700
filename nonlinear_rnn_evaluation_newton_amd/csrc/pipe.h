// Tile pipeline shared by the sweep and adjoint kernels of the scalar-state
// path: a persistent grid of blocks of 11 compute wavefronts
// and one look-back wavefront (three wavefronts per SIMD, one block per CU).  A block computes tile N while the tile before
// it waits for its carry (two register sets alternate; the loads of the tile
// after N are in flight during N); the look-back wavefront resolves carries
// alone, so its waits on the tile descriptors never queue behind the bulk
// loads and stores of the compute wavefronts.  All memory access of the tile
// loop goes through buffer instructions whose range check drops out-of-range
// lanes, so no load or store sits under a branch (see below).
//
// A policy type supplies the work of one tile (Raw inputs, computed Tile,
// LDS, accumulators, constants, look-back) through static members (load
// with tile id -1 must move no data: it stands for the tile after a block's
// last), and
// WPE, the wavefronts per SIMD its register budget is sized for; see
// k_scalar.hip.
#pragma once

#include "k_time_impl.h"

namespace pr {

constexpr int SC_CW = 11;                      // compute wavefronts per block
constexpr int SC_THREADS = 64 * (SC_CW + 1);  // + the look-back wavefront (a multiple of 4 wavefronts)
constexpr int SC_LB = SC_CW;                  // wavefront id of the look-back wavefront

__device__ inline float rdlane(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// lane l receives v of lane l - 1; lane 0 receives first
__device__ inline float shift_in(float first, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(v), 0x138, 0xf, 0xf, false));
}
// lane l receives v of lane l + 1; lane 63 receives last
__device__ inline float shift_out(float last, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(last), __float_as_int(v), 0x130, 0xf, 0xf, false));
}

// Memory access goes through buffer instructions on per-row buffer
// resources: the hardware range check returns zero for loads outside a
// resource and drops stores outside it (offset SC_OOB is outside every
// resource; a null base gets an empty resource), so every load and store in
// the tile loop is unconditional.  That keeps the compiler's count of memory
// operations in flight exact: loads and stores share one in-order counter on
// this architecture, and a memory instruction under a branch would make later
// waits conservative, draining recent stores before prefetched data can be
// used.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr unsigned SC_OOB = 0x80000000u;
constexpr int SC_SC1 = 16;  // cache policy: device-scope coherent access

__device__ inline Rsrc sc_rsrc(const void *base, unsigned bytes) {
  // raw buffer, stride 0, 32-bit data format in the fourth descriptor word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, base ? (int)bytes : 0, 0x00020000);
}
__device__ inline float4 ld4(Rsrc r, unsigned off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ inline float ld1(Rsrc r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void st4(Rsrc r, unsigned off, float a, float b, float c, float d) {
  u32x4 v;
  v.x = __float_as_uint(a); v.y = __float_as_uint(b); v.z = __float_as_uint(c); v.w = __float_as_uint(d);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
// Non-temporal store (cache policy NT) for outputs nothing in the call reads
// back: the lines are not kept in the caches, which are left to the inputs.
constexpr int SC_NT = 2;
__device__ inline void st4_nt(Rsrc r, unsigned off, float a, float b, float c, float d) {
  u32x4 v;
  v.x = __float_as_uint(a); v.y = __float_as_uint(b); v.z = __float_as_uint(c); v.w = __float_as_uint(d);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SC_NT);
}
__device__ inline void st1(Rsrc r, unsigned off, float a) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, off, 0, 0);
}
// byte offset of step t in a row of floats, or SC_OOB when t is outside [0, T)
__device__ inline unsigned toff(int t, int T) { return (t >= 0 && t < T) ? (unsigned)t * 4u : SC_OOB; }

__device__ inline unsigned short ld_u16(Rsrc r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ inline unsigned ld_u32(Rsrc r, unsigned off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ inline void st_u16(Rsrc r, unsigned off, unsigned short v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ inline void st_u32(Rsrc r, unsigned off, unsigned v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0); }

template <class Pol>
__device__ inline void pipe_compute_any(const typename Pol::Args &a, const typename Pol::Consts &K, int id,
                                        const typename Pol::Raw &R, typename Pol::Tile &Tl,
                                        typename Pol::Shared &sh, typename Pol::Lds &lds, int buf) {
  if (Pol::full(a, id)) Pol::template compute<true>(a, K, id, R, Tl, sh, lds, buf);
  else Pol::template compute<false>(a, K, id, R, Tl, sh, lds, buf);
}

// One stage of the compute wavefronts: issue the loads of the tile after N,
// compute N into buffer bufN, block barrier (the look-back wavefront has left
// the carries entering P's wavefronts in LDS buffer bufN ^ 1), update P.
template <class Pol>
__device__ inline void pipe_stage(const typename Pol::Args &a, const typename Pol::Consts &K, int idP,
                                  const typename Pol::Tile &TP, int idN, const typename Pol::Raw &RN,
                                  typename Pol::Raw &Rnext, typename Pol::Tile &TN, typename Pol::Shared &sh,
                                  typename Pol::Lds &lds, int bufN, typename Pol::Acc &acc) {
  const int nt = Pol::ntiles(a);
  const int nn = idN + (int)gridDim.x < nt ? idN + (int)gridDim.x : -1;  // -1: an empty load
  Pol::load(a, nn, Rnext);
  pipe_compute_any<Pol>(a, K, idN, RN, TN, sh, lds, bufN);
  __syncthreads();
  Pol::apply(a, K, idP, TP, sh, lds, bufN ^ 1, acc);
}

// Persistent grid (every block resident, grid <= tile count); block g takes
// tiles g, g + grid, ... in order.  Stage s of a block computes its tile s
// (compute wavefronts) while the look-back wavefront resolves tile s - 1;
// after the stage's barrier the compute wavefronts update tile s - 1.  Every
// look-back needs only aggregates of tiles computed in an earlier or the same
// stage of resident blocks and published before their look-backs wait, so the
// grid cannot deadlock.  The two wavefront roles run separate loops with the
// same number of barriers (tiles + 1).
template <class Pol>
__global__ __launch_bounds__(SC_THREADS, Pol::WPE) void k_pipe(const typename Pol::Args a) {
  __shared__ typename Pol::Shared sh;
  __shared__ typename Pol::Lds lds;
  // the wavefront id through readfirstlane: the compiler then knows the role
  // branch is uniform, so each wavefront runs exactly one role's loop (and
  // its barriers) instead of both under an execution mask
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, nt = Pol::ntiles(a);
  typename Pol::Acc acc;
  Pol::acc_init(acc);
  if (wid == SC_LB) {
    if (lane == 0) Pol::shared_init(sh);
    if (Pol::open(a, sh)) return;
    __syncthreads();  // end of stage 0
    for (int id = blockIdx.x; id < nt; id += G) {
      Pol::lookback_tile(a, id, sh, ((id - (int)blockIdx.x) / G) & 1);
      __syncthreads();
    }
  } else {
    // constants (weights folded per call) before any other load: a vector
    // load inside the tile loop would wait behind the prefetched tile
    typename Pol::Consts K;
    Pol::consts(a, K);
    typename Pol::Raw R0, R1;
    typename Pol::Tile T0, T1;
    int id = blockIdx.x;
    Pol::load(a, id, R0);  // overlaps the stop check
    if (Pol::open(a, sh)) return;
    // stage 0: compute the first tile
    Pol::load(a, id + G < nt ? id + G : -1, R1);
    pipe_compute_any<Pol>(a, K, id, R0, T0, sh, lds, 0);
    __syncthreads();
    int idP = id;
    id += G;
    int last = 0;  // register set of the final pending tile
    while (true) {
      if (id >= nt) { last = 0; break; }
      pipe_stage<Pol>(a, K, idP, T0, id, R1, R0, T1, sh, lds, 1, acc);
      idP = id;
      id += G;
      if (id >= nt) { last = 1; break; }
      pipe_stage<Pol>(a, K, idP, T1, id, R0, R1, T0, sh, lds, 0, acc);
      idP = id;
      id += G;
    }
    __syncthreads();  // final stage: the look-back wavefront has resolved the last tile
    if (last == 0) Pol::apply(a, K, idP, T0, sh, lds, 0, acc);
    else Pol::apply(a, K, idP, T1, sh, lds, 1, acc);
  }
  Pol::finish(a, acc, sh);
}

// Launch on a persistent grid; *grid_out receives the block count.
template <class Pol>
hipError_t pipe_launch(const typename Pol::Args &a, hipStream_t s, int *grid_out = nullptr) {
  const int grid = persistent_grid<k_pipe<Pol>, SC_THREADS>(Pol::ntiles(a));
  if (grid <= 0) return hipErrorInvalidConfiguration;
  if (grid_out) *grid_out = grid;
  hipLaunchKernelGGL((k_pipe<Pol>), dim3(grid), dim3(SC_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace pr
