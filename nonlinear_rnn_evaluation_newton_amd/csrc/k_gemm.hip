// MFMA GEMM for the dense contractions of the path: the input projection
// U = x W_x^T + b_x, done once per solve, and the adjoint's dx = dU W_x and
// dW_x = dU^T x.  C[M,N] = sum_k A[m,k] B[n,k] with either operand stored
// K-contiguous or M/N-contiguous, bf16 inputs on v_mfma_f32_32x32x16_bf16 or
// fp32 inputs on v_mfma_f32_32x32x2_f32, fp32 accumulation.
//
// Tiling: 128 x 128 block tile, K step 32, 4 wavefronts of 64 x 64 (2 x 2
// MFMA tiles of 32 x 32), LDS double buffer holding both operands
// K-contiguous so every lane reads its MFMA operand with one vector load.
// Long-K products (dW_x) split K over blocks into an fp32 workspace that a
// second kernel sums in a fixed order.
#include "internal.h"

namespace pr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

template <typename T>
struct Mfma;
template <>
struct Mfma<uint16_t> {
  static constexpr int KSTEP = 16, VEC = 8;
  __device__ static inline f32x16_t mma(const uint16_t *a, const uint16_t *b, f32x16_t c) {
    bf16x8_t va = *reinterpret_cast<const bf16x8_t *>(a);
    bf16x8_t vb = *reinterpret_cast<const bf16x8_t *>(b);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, c, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  static constexpr int KSTEP = 2, VEC = 1;
  __device__ static inline f32x16_t mma(const float *a, const float *b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(*a, *b, c, 0, 0, 0);
  }
};

constexpr int GBM = 128, GBN = 128, GBK = 32;

template <typename T>
struct GemmLds {
  static constexpr int PAD = 16 / sizeof(T);  // keeps row starts off one bank
  static constexpr int LD = GBK + PAD;
};

// Load one 128 x 32 operand tile (rows r0.., k0..) from global into registers:
// KC: element (r, k) at P[r * ld + k]; else at P[k * ld + r].
template <typename T, bool KC>
struct TileLoader {
  static constexpr int VE = 16 / sizeof(T);                 // elements per 16-byte vector
  static constexpr int NV = GBM * GBK / VE / 256;           // vectors per thread
  uint4 v[NV];
  __device__ inline void load(const T *P, int ld, int rows, int K, int r0, int k0, bool vec) {
#pragma unroll
    for (int q = 0; q < NV; q++) {
      const int e = threadIdx.x + q * 256;
      int r, k;
      if (KC) { r = e / (GBK / VE); k = (e % (GBK / VE)) * VE; }
      else { k = e / (GBM / VE); r = (e % (GBM / VE)) * VE; }
      const int gr = r0 + r, gk = k0 + k;
      T tmp[VE];
      const bool full = KC ? (gr < rows && gk + VE <= K) : (gk < K && gr + VE <= rows);
      if (vec && full) {
        v[q] = *reinterpret_cast<const uint4 *>(KC ? P + (size_t)gr * ld + gk : P + (size_t)gk * ld + gr);
        continue;
      }
#pragma unroll
      for (int i = 0; i < VE; i++) {
        const int rr = KC ? gr : gr + i, kk = KC ? gk + i : gk;
        tmp[i] = (rr < rows && kk < K) ? (KC ? P[(size_t)rr * ld + kk] : P[(size_t)kk * ld + rr]) : (T)0;
      }
      v[q] = *reinterpret_cast<const uint4 *>(tmp);
    }
  }
  __device__ inline void store(T *S) const {
#pragma unroll
    for (int q = 0; q < NV; q++) {
      const int e = threadIdx.x + q * 256;
      if (KC) {
        const int r = e / (GBK / VE), k = (e % (GBK / VE)) * VE;
        *reinterpret_cast<uint4 *>(S + r * GemmLds<T>::LD + k) = v[q];
      } else {
        const int k = e / (GBM / VE), r = (e % (GBM / VE)) * VE;
        const T *t = reinterpret_cast<const T *>(&v[q]);
#pragma unroll
        for (int i = 0; i < VE; i++) S[(r + i) * GemmLds<T>::LD + k] = t[i];
      }
    }
  }
};

template <typename TO>
__device__ inline void store_out(TO *p, float v);
template <>
__device__ inline void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ inline void store_out<uint16_t>(uint16_t *p, float v) { *p = f2bf(v); }

// C (or the split-K workspace slice) = A B^T over K range [kb, ke).
template <typename T, bool AKC, bool BKC, typename TO>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs g) {
  using MF = Mfma<T>;
  constexpr int LD = GemmLds<T>::LD;
  __shared__ __attribute__((aligned(16))) T sA[2][GBM * LD];
  __shared__ __attribute__((aligned(16))) T sB[2][GBN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int m0 = (tile / tiles_n) * GBM, n0 = (tile % tiles_n) * GBN;
  const int kchunk = ((g.K + g.splits - 1) / g.splits + GBK - 1) / GBK * GBK;
  const int kb = split * kchunk;
  const int ke = min(g.K, kb + kchunk);
  const T *A = (const T *)g.A, *B = (const T *)g.B;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  TileLoader<T, AKC> la;
  TileLoader<T, BKC> lb;
  int buf = 0;
  if (kb < ke) {
    la.load(A, g.lda, g.M, ke, m0, kb, g.vec_a);
    lb.load(B, g.ldb, g.N, ke, n0, kb, g.vec_b);
    la.store(sA[0]);
    lb.store(sB[0]);
  }
  __syncthreads();
  for (int k0 = kb; k0 < ke; k0 += GBK) {
    const bool more = k0 + GBK < ke;
    if (more) {
      la.load(A, g.lda, g.M, ke, m0, k0 + GBK, g.vec_a);
      lb.load(B, g.ldb, g.N, ke, n0, k0 + GBK, g.vec_b);
    }
    const T *cA = sA[buf], *cB = sB[buf];
#pragma unroll
    for (int ks = 0; ks < GBK; ks += MF::KSTEP) {
      const int kk = ks + (lane >> 5) * MF::VEC;
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = MF::mma(cA + (wm * 64 + i * 32 + (lane & 31)) * LD + kk,
                              cB + (wn * 64 + j * 32 + (lane & 31)) * LD + kk, acc[i][j]);
    }
    if (more) {
      la.store(sA[buf ^ 1]);
      lb.store(sB[buf ^ 1]);
    }
    __syncthreads();
    buf ^= 1;
  }

  // epilogue: 32x32 MFMA result, lane holds column (lane & 31) of rows
  // 8*(r/4) + 4*(lane/32) + (r%4)
  const TO *dummy = nullptr;
  (void)dummy;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= g.N) continue;
      const float bias = split != 0 ? 0.f : g.bias32 ? g.bias32[col] : g.bias ? ldf((const T *)g.bias, col) : 0.f;
      const float scale = g.scale32 ? g.scale32[col] : 1.f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        const float v = fmaf(acc[i][j][r], scale, bias);
        if (g.splits > 1) g.ws[((size_t)split * g.M + row) * g.N + col] = v;
        else store_out<TO>((TO *)g.C + (size_t)row * g.ldc + col, v);
      }
    }
}

// Sums the split partials in split order (a fixed order: the result does not
// depend on scheduling).  Four adjacent elements per thread when rows are
// whole 16-byte groups, else one.
template <typename TO>
__global__ void k_gemm_splitk_sum(const GemmArgs g) {
  const size_t MN = (size_t)g.M * g.N;
  const bool vec = (g.N % 4) == 0 && (g.ldc % 4) == 0 && ((uintptr_t)g.C % 16) == 0 && sizeof(TO) == 4;
  if (vec) {
    const size_t e = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e >= MN) return;
    float4 s = *reinterpret_cast<const float4 *>(g.ws + e);
    for (int q = 1; q < g.splits; q++) {
      const float4 v = *reinterpret_cast<const float4 *>(g.ws + (size_t)q * MN + e);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const size_t row = e / g.N, col = e % g.N;
    *reinterpret_cast<float4 *>((float *)g.C + row * g.ldc + col) = s;
    return;
  }
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= MN) return;
  float s = 0.f;
  for (int q = 0; q < g.splits; q++) s += g.ws[(size_t)q * MN + e];
  const size_t row = e / g.N, col = e % g.N;
  store_out<TO>((TO *)g.C + row * g.ldc + col, s);
}
template <typename TO>
static unsigned splitk_sum_blocks(const GemmArgs &g) {
  const size_t tot = (size_t)g.M * g.N;
  const bool vec = (g.N % 4) == 0 && (g.ldc % 4) == 0 && ((uintptr_t)g.C % 16) == 0 && sizeof(TO) == 4;
  return (unsigned)(((vec ? (tot + 3) / 4 : tot) + 255) / 256);
}

// ---------------------------------------------------------------------------
// Large bf16 products with both operands K-contiguous (the input projection
// and the adjoint's dx and dW_x at channel widths of hundreds and more).
//
// 256 x 256 block tile, K step 64, 8 wavefronts of 128 (M) x 64 (N) each:
// per 16-wide K slice a wavefront reads 6 operand fragments from LDS for 8
// MFMAs, half the LDS traffic per MFMA of a 64 x 64 wavefront tile, which
// saturates LDS bandwidth before the matrix cores.  Operands are staged
// global -> registers -> LDS (rows padded by 16 B, so the 16-byte fragment
// reads of 8 consecutive rows fall in distinct banks), double-buffered.
// The MFMA takes the B fragment as its first operand, so a lane's results
// are 4 adjacent columns of one output row (8- or 16-byte stores).
// Loads go through buffer resources on the block's rows: rows past M or N
// and K chunks past the split's end read as zero.
// Tile order: blocks are dealt round-robin over the 8 XCDs, so block ids are
// regrouped to give each XCD a contiguous range of tiles, walked in groups
// of 8 tile rows; concurrently running tiles of one XCD share operand rows
// in its L2.
constexpr int BT = 256, BK = 64, BLD = BK + 8;

typedef __amdgpu_buffer_rsrc_t GRsrc;
__device__ inline GRsrc g_rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
typedef unsigned int gu32x4 __attribute__((ext_vector_type(4)));

#ifndef PR_GEMM_WGM
#define PR_GEMM_WGM 2
#define PR_GEMM_WGN 4
#endif
// wavefront grid WGM x WGN over the 256 x 256 tile; each wavefront holds
// FM x FN MFMA tiles of 32 x 32
constexpr int WGM = PR_GEMM_WGM, WGN = PR_GEMM_WGN, FM = BT / 32 / WGM, FN = BT / 32 / WGN;
constexpr int GT = 64 * WGM * WGN;  // threads per block
constexpr int GQ = BT * (BK / 8) / GT;  // 16-byte staging chunks per operand per thread

// KO = true: both operands stored K-outer (A [K, lda], B [K, ldb]; the
// products over the time rows).  Each thread loads a 4 (k) x 8 (m) block as
// four 16-byte row pieces, transposes it with byte permutes and writes eight
// 8-byte k-runs, so the tiles land K-contiguous as in the other layout.  Two
// unpadded rows (64 k each) share a 256-byte line of 16 chunks of 8 k, and
// chunk ((m & 1) << 3 | k / 8) of line L = m / 2 sits at slot chunk ^ g(L),
// g(L) = ((L >> 2) ^ 2 (L & 3)) & 15: each 32-lane phase of the 8-byte
// writes (16 m-groups, both k-row parities) and each 16-lane phase of the
// 16-byte fragment reads (16 consecutive rows) then covers all 64 banks once.
__device__ inline int ko_slot(int m, int chunk) {
  const int L = m >> 1;
  return ((((m & 1) << 3) | chunk) ^ ((L >> 2) ^ ((L & 3) << 1))) & 15;
}
__device__ inline int ko_index(int m, int chunk) { return (m >> 1) * 128 + ko_slot(m, chunk) * 8; }
constexpr int BKO = BK;  // elements per row of the K-outer layout

template <typename TO, bool KO>
__global__ __launch_bounds__(GT, 1) void k_gemm_bf16_nt(const GemmArgs g, int tiles_m, int tiles_n) {
  constexpr int LDW = KO ? BKO : BLD;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BT * LDW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BT * LDW];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int tiles = tiles_m * tiles_n;
  int id = blockIdx.x;
  if (tiles % 8 == 0) id = (id % 8) * (tiles / 8) + id / 8;
  constexpr int GM = 8;
  const int width = GM * tiles_n, fm = (id / width) * GM;
  const int gm = min(tiles_m - fm, GM);
  const int tm = fm + (id % width) % gm, tn = (id % width) / gm;
  const int m0 = tm * BT, n0 = tn * BT;
  const int split = blockIdx.y;
  const int kchunk = ((g.K + g.splits - 1) / g.splits + BK - 1) / BK * BK;
  const int kb = split * kchunk, ke = min(g.K, kb + kchunk);

  const uint16_t *A = (const uint16_t *)g.A + (KO ? (size_t)m0 : (size_t)m0 * g.lda);
  const uint16_t *B = (const uint16_t *)g.B + (KO ? (size_t)n0 : (size_t)n0 * g.ldb);
  // K-outer: the resource spans the rows up to K from the block's first
  // column; columns past M (N) and rows past the split's K range read zero
  // through the offsets (M, N, lda, ldb are multiples of 8)
  const GRsrc ra = g_rsrc(A, KO ? (unsigned)(((size_t)g.K * g.lda - m0) * 2) : (unsigned)(min(BT, g.M - m0) * g.lda * 2));
  const GRsrc rb = g_rsrc(B, KO ? (unsigned)(((size_t)g.K * g.ldb - n0) * 2) : (unsigned)(min(BT, g.N - n0) * g.ldb * 2));

  // staging: GQ chunks of 8 elements per operand per thread; K-contiguous:
  // 8 K-consecutive elements of one row; K-outer: 8 columns (m-group tid %
  // 32) of K rows 4 (tid / 32) + q
  int srow[GQ], skc[GQ];
#pragma unroll
  for (int q = 0; q < GQ; q++) {
    const int e = tid + q * GT;
    srow[q] = e >> 3;
    skc[q] = (e & 7) * 8;
  }
  // K-outer staging: m-group (8 columns) and first of 4 K rows; a
  // wavefront's even lanes take one K row group, odd lanes the next
  const int ko_mg = (tid & 63) >> 1, ko_k = ((tid >> 6) * 2 + (tid & 1)) * 4;
  const bool ko_ina = m0 + ko_mg * 8 < g.M, ko_inb = n0 + ko_mg * 8 < g.N;
  gu32x4 va[GQ], vb[GQ];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < GQ; q++) {
      if constexpr (KO) {
        const int k = k0 + ko_k + q;
        va[q] = __builtin_amdgcn_raw_buffer_load_b128(
            ra, (k < ke && ko_ina) ? (unsigned)(k * g.lda + ko_mg * 8) * 2u : 0x80000000u, 0, 0);
        vb[q] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, (k < ke && ko_inb) ? (unsigned)(k * g.ldb + ko_mg * 8) * 2u : 0x80000000u, 0, 0);
      } else {
        const bool in = k0 + skc[q] < ke;
        va[q] = __builtin_amdgcn_raw_buffer_load_b128(
            ra, in ? (unsigned)(srow[q] * g.lda + k0 + skc[q]) * 2u : 0x80000000u, 0, 0);
        vb[q] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, in ? (unsigned)(srow[q] * g.ldb + k0 + skc[q]) * 2u : 0x80000000u, 0, 0);
      }
    }
  };
  // K-outer: column c of the 4 x 8 block becomes the 4-element k-run of row
  // 8 mg + c (two dwords: rows 0-1 and 2-3 of the block, low halves for even
  // c, high halves for odd)
  auto ko_store = [&](uint16_t *dst, const gu32x4 (&v)[GQ]) {
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
      const unsigned lo = __builtin_amdgcn_perm(v[1][c >> 1], v[0][c >> 1], sel);
      const unsigned hi = __builtin_amdgcn_perm(v[3][c >> 1], v[2][c >> 1], sel);
      const int idx = ko_index(ko_mg * 8 + c, ko_k >> 3) + (ko_k & 7);
      *reinterpret_cast<unsigned long long *>(&dst[idx]) = ((unsigned long long)hi << 32) | lo;
    }
  };
  auto lstore = [&](int buf) {
    if constexpr (KO) {
      ko_store(sA[buf], va);
      ko_store(sB[buf], vb);
    } else {
#pragma unroll
      for (int q = 0; q < GQ; q++) {
        *reinterpret_cast<gu32x4 *>(&sA[buf][srow[q] * BLD + skc[q]]) = va[q];
        *reinterpret_cast<gu32x4 *>(&sB[buf][srow[q] * BLD + skc[q]]) = vb[q];
      }
    }
  };

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int j = 0; j < FN; j++)
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[j][i][r] = 0.f;

  int buf = 0;
  if (kb < ke) {
    gload(kb);
    lstore(0);
  }
  __syncthreads();
  const int arow = wm * (FM * 32) + (lane & 31), brow = wn * (FN * 32) + (lane & 31), kl = (lane >> 5) * 8;
  // Per K step: the next step's operands are requested from global memory
  // (past the range they read zero and are never used); the fragments of
  // 16-wide K slice q + 1 are read from LDS while slice q's MFMAs run, and
  // the staged next step is written to the other LDS buffer during the last
  // slice's MFMAs, so LDS traffic overlaps the matrix cores instead of
  // alternating with them between barriers.
  constexpr int NQ = BK / 16;
  for (int k0 = kb; k0 < ke; k0 += BK) {
    gload(k0 + BK);
    const uint16_t *cA = sA[buf], *cB = sB[buf];
    bf16x8_t a[2][FM], b[2][FN];
    auto frag = [&](int h, int ks) {
      if constexpr (KO) {
        const int kc = (ks + kl) >> 3;
#pragma unroll
        for (int i = 0; i < FM; i++)
          a[h][i] = *reinterpret_cast<const bf16x8_t *>(cA + ko_index(arow + i * 32, kc));
#pragma unroll
        for (int j = 0; j < FN; j++)
          b[h][j] = *reinterpret_cast<const bf16x8_t *>(cB + ko_index(brow + j * 32, kc));
      } else {
#pragma unroll
        for (int i = 0; i < FM; i++)
          a[h][i] = *reinterpret_cast<const bf16x8_t *>(cA + (arow + i * 32) * BLD + ks + kl);
#pragma unroll
        for (int j = 0; j < FN; j++)
          b[h][j] = *reinterpret_cast<const bf16x8_t *>(cB + (brow + j * 32) * BLD + ks + kl);
      }
    };
    frag(0, 0);
    // the global loads first, then the first slice's fragment reads
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * GQ, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      if (q + 1 < NQ) frag((q + 1) & 1, (q + 1) * 16);
      else lstore(buf ^ 1);
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int i = 0; i < FM; i++)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[q & 1][j], a[q & 1][i], acc[j][i], 0, 0, 0);
      if (q + 1 < NQ) {  // one fragment read after each MFMA, then the remaining MFMAs
#pragma unroll
        for (int r = 0; r < FM + FN; r++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      } else if constexpr (KO) {  // two LDS stores after each MFMA
#pragma unroll
        for (int r = 0; r < 2 * GQ; r++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - 2 * GQ, 0);
      } else {  // one LDS store after each MFMA
#pragma unroll
        for (int r = 0; r < 2 * GQ; r++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - 2 * GQ, 0);
      }
    }
    __syncthreads();
    buf ^= 1;
  }

  // lane holds rows m = (lane & 31) of each 32 x 32 tile and, per group of 4
  // registers, the 4 adjacent columns 8 * (r / 4) + 4 * (lane / 32) + (0..3)
  const bool vec_c = g.splits == 1 && (g.ldc % 4) == 0 && ((uintptr_t)g.C % 16) == 0;
  // the bias of this lane's columns, loaded once (they do not depend on the row)
  float bias[FN][4][4], scale[FN][4][4];
#pragma unroll
  for (int j = 0; j < FN; j++)
#pragma unroll
    for (int rg = 0; rg < 4; rg++) {
      const int n = n0 + wn * (FN * 32) + j * 32 + 8 * rg + 4 * (lane >> 5);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        bias[j][rg][c] = (split != 0 || n + c >= g.N) ? 0.f
                         : g.bias32 ? g.bias32[n + c]
                         : g.bias ? bf2f(((const uint16_t *)g.bias)[n + c]) : 0.f;
        scale[j][rg][c] = (g.scale32 && n + c < g.N) ? g.scale32[n + c] : 1.f;
      }
    }
#pragma unroll
  for (int i = 0; i < FM; i++) {
    const int m = m0 + wm * (FM * 32) + i * 32 + (lane & 31);
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int rg = 0; rg < 4; rg++) {
        const int n = n0 + wn * (FN * 32) + j * 32 + 8 * rg + 4 * (lane >> 5);
        if (n >= g.N) continue;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; c++) v[c] = fmaf(acc[j][i][4 * rg + c], scale[j][rg][c], bias[j][rg][c]);
        if (g.splits > 1) {
          float *w = g.ws + ((size_t)split * g.M + m) * g.N + n;
          if (n + 4 <= g.N && (g.N % 4) == 0) *reinterpret_cast<float4 *>(w) = make_float4(v[0], v[1], v[2], v[3]);
          else
            for (int c = 0; c < 4 && n + c < g.N; c++) w[c] = v[c];
          continue;
        }
        TO *o = (TO *)g.C + (size_t)m * g.ldc + n;
        if (vec_c && n + 4 <= g.N) {
          if constexpr (sizeof(TO) == 2) {
            uint2 u;
            u.x = (unsigned)f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16);
            u.y = (unsigned)f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16);
            *reinterpret_cast<uint2 *>(o) = u;
          } else {
            *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
          }
        } else {
          for (int c = 0; c < 4 && n + c < g.N; c++) store_out<TO>(o + c, v[c]);
        }
      }
  }
}

// Direct staging for K-contiguous operands: each 16-byte buffer load writes
// LDS straight from memory (buffer_load ... lds: lane l of an instruction
// fills bytes 16 l .. 16 l + 15 of a 1 KB run whose base is wavefront-
// uniform), so operands take no registers and no LDS store instructions on
// their way in.  Two stages of one 64-wide K step each; the loads of step
// j + 1 are issued at the start of step j.  The layout is set by which chunk
// each lane fetches: tile rows are 64 k (128 bytes) unpadded, and 8-element
// chunk c of row r sits at slot c ^ ((r >> 1) & 7), which spreads each
// 16-lane phase of the fragment reads (16 consecutive rows, one chunk) over
// all 64 banks.  Out-of-range offsets write zeros, as the register path
// reads them.
//
// Wavefront grid DWM x DWN over the 256 x 256 tile: 2 x 4 wavefronts of
// 128 x 64, two per SIMD, so one wavefront's waits overlap the other's MFMAs
// (2 x 2 wavefronts of 128 x 128, one per SIMD, read a third less LDS per
// MFMA but ran 25% slower: nothing hides a lone wavefront's waits).
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ inline int dl_off(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 3); }

// Wait until this wavefront's direct loads have landed and its LDS reads are
// done, then meet the other wavefronts.  Empty asm statements with a memory
// clobber keep every memory access on its side of the barrier.
__device__ inline void dl_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

#ifndef PR_DWM
#define PR_DWM 2
#define PR_DWN 4
#endif
constexpr int DWM = PR_DWM, DWN = PR_DWN, DFM = BT / 32 / DWM, DFN = BT / 32 / DWN, DGT = 64 * DWM * DWN;
constexpr int DQ = BT * BK / 8 / DGT;  // direct loads per operand per thread and K step

template <typename TO>
__global__ __launch_bounds__(DGT, 1) void k_gemm_bf16_dl(const GemmArgs g, int tiles_m, int tiles_n) {
  // one array per stage (A tile, then B tile), so the compiler can tell the
  // stage being loaded from the one being read
  __shared__ __attribute__((aligned(1024))) uint16_t s0[2 * BT * BK], s1[2 * BT * BK];
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / DWN, wn = wid % DWN;
  const int tiles = tiles_m * tiles_n;
  int id = blockIdx.x;
  if (tiles % 8 == 0) id = (id % 8) * (tiles / 8) + id / 8;
  constexpr int GM = 8;
  const int width = GM * tiles_n, fm = (id / width) * GM;
  const int gm = min(tiles_m - fm, GM);
  const int tm = fm + (id % width) % gm, tn = (id % width) / gm;
  const int m0 = tm * BT, n0 = tn * BT;
  const int split = blockIdx.y;
  const int kchunk = ((g.K + g.splits - 1) / g.splits + BK - 1) / BK * BK;
  const int kb = split * kchunk, ke = min(g.K, kb + kchunk);

  const uint16_t *A = (const uint16_t *)g.A + (size_t)m0 * g.lda;
  const uint16_t *B = (const uint16_t *)g.B + (size_t)n0 * g.ldb;
  const GRsrc ra = g_rsrc(A, (unsigned)(min(BT, g.M - m0) * g.lda * 2));
  const GRsrc rb = g_rsrc(B, (unsigned)(min(BT, g.N - n0) * g.ldb * 2));
  // instruction q of wavefront w fills slots 64 (DQ w + q) + lane: row
  // r = 8 (DQ w + q) + lane / 8, physical slot lane % 8, so the chunk swizzle
  // (r >> 1) & 7 = 4 (q & 1) + lane / 16 (DQ is even) takes two values per
  // lane; the row's wavefront-uniform part goes in the scalar offset
  static_assert(DQ % 2 == 0, "even number of direct loads");
  const int rl = lane >> 3, kce = ((lane & 7) ^ (lane >> 4)) * 8, kco = ((lane & 7) ^ (4 | (lane >> 4))) * 8;
  const unsigned va_e = (unsigned)(rl * g.lda + kce) * 2u, va_o = (unsigned)(rl * g.lda + kco) * 2u;
  const unsigned vb_e = (unsigned)(rl * g.ldb + kce) * 2u, vb_o = (unsigned)(rl * g.ldb + kco) * 2u;
  auto dload = [&](uint16_t *d, int k0) {
#pragma unroll
    for (int q = 0; q < DQ; q++) {
      const int kc = (q & 1) ? kco : kce;
      const bool in = k0 + kc < ke;
      const int u = wid * DQ + q;
      const unsigned sa = (unsigned)(u * 8 * g.lda + k0) * 2u, sb = (unsigned)(u * 8 * g.ldb + k0) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)&d[u * 512], 16,
                                               in ? ((q & 1) ? va_o : va_e) : 0x80000000u, sa, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)&d[BT * BK + u * 512], 16,
                                               in ? ((q & 1) ? vb_o : vb_e) : 0x80000000u, sb, 0, 0);
    }
  };

  f32x16_t acc[DFN][DFM];
#pragma unroll
  for (int j = 0; j < DFN; j++)
#pragma unroll
    for (int i = 0; i < DFM; i++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[j][i][r] = 0.f;

  if (kb < ke) dload(s0, kb);
  dl_sync();
  const int arow = wm * (DFM * 32) + (lane & 31), brow = wn * (DFN * 32) + (lane & 31), kl = lane >> 5;
  // Per K step: the next step's loads go straight to the other stage (read
  // by every wavefront before the previous barrier) and have the whole step's
  // MFMAs to land; fragments of slice q + 1 are read while slice q's MFMAs
  // run.  The loop is unrolled over the two stages.
  constexpr int NQ = BK / 16;
  auto step = [&](const uint16_t *cA, uint16_t *nx, int k0) {
    const uint16_t *cB = cA + BT * BK;
    if (k0 + BK < ke) dload(nx, k0 + BK);
    bf16x8_t a[2][DFM], b[2][DFN];
    auto frag = [&](int h, int q) {
      const int c = 2 * q + kl;
#pragma unroll
      for (int i = 0; i < DFM; i++) a[h][i] = *reinterpret_cast<const bf16x8_t *>(cA + dl_off(arow + i * 32, c));
#pragma unroll
      for (int j = 0; j < DFN; j++) b[h][j] = *reinterpret_cast<const bf16x8_t *>(cB + dl_off(brow + j * 32, c));
    };
    frag(0, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * DQ, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DFM + DFN, 0);
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      if (q + 1 < NQ) frag((q + 1) & 1, q + 1);
#pragma unroll
      for (int j = 0; j < DFN; j++)
#pragma unroll
        for (int i = 0; i < DFM; i++)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[q & 1][j], a[q & 1][i], acc[j][i], 0, 0, 0);
      if (q + 1 < NQ) {
#pragma unroll
        for (int r = 0; r < DFM + DFN; r++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, DFM * DFN - (DFM + DFN), 0);
      }
    }
    dl_sync();
  };
  // whole pairs of steps, then an odd last one (no join of the accumulators
  // inside the loop)
  int k0 = kb;
  for (; k0 + BK < ke; k0 += 2 * BK) {
    step(s0, s1, k0);
    step(s1, s0, k0 + BK);
  }
  if (k0 < ke) step(s0, s1, k0);

  // lane holds rows m = (lane & 31) of each 32 x 32 tile and, per group of 4
  // registers, the 4 adjacent columns 8 * (r / 4) + 4 * (lane / 32) + (0..3)
  const bool vec_c = g.splits == 1 && (g.ldc % 4) == 0 && ((uintptr_t)g.C % 16) == 0;
#pragma unroll
  for (int j = 0; j < DFN; j++) {
    // the bias and scale of this lane's columns (they do not depend on the row)
    float bias[4][4], scale[4][4];
#pragma unroll
    for (int rg = 0; rg < 4; rg++) {
      const int n = n0 + wn * (DFN * 32) + j * 32 + 8 * rg + 4 * (lane >> 5);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        bias[rg][c] = (split != 0 || n + c >= g.N) ? 0.f
                      : g.bias32 ? g.bias32[n + c]
                      : g.bias ? bf2f(((const uint16_t *)g.bias)[n + c]) : 0.f;
        scale[rg][c] = (g.scale32 && n + c < g.N) ? g.scale32[n + c] : 1.f;
      }
    }
#pragma unroll
    for (int i = 0; i < DFM; i++) {
      const int m = m0 + wm * (DFM * 32) + i * 32 + (lane & 31);
      if (m >= g.M) continue;
#pragma unroll
      for (int rg = 0; rg < 4; rg++) {
        const int n = n0 + wn * (DFN * 32) + j * 32 + 8 * rg + 4 * (lane >> 5);
        if (n >= g.N) continue;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; c++) v[c] = fmaf(acc[j][i][4 * rg + c], scale[rg][c], bias[rg][c]);
        if (g.splits > 1) {
          float *w = g.ws + ((size_t)split * g.M + m) * g.N + n;
          if (n + 4 <= g.N && (g.N % 4) == 0) *reinterpret_cast<float4 *>(w) = make_float4(v[0], v[1], v[2], v[3]);
          else
            for (int c = 0; c < 4 && n + c < g.N; c++) w[c] = v[c];
          continue;
        }
        TO *o = (TO *)g.C + (size_t)m * g.ldc + n;
        if (vec_c && n + 4 <= g.N) {
          if constexpr (sizeof(TO) == 2) {
            uint2 u;
            u.x = (unsigned)f2bf(v[0]) | ((unsigned)f2bf(v[1]) << 16);
            u.y = (unsigned)f2bf(v[2]) | ((unsigned)f2bf(v[3]) << 16);
            *reinterpret_cast<uint2 *>(o) = u;
          } else {
            *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
          }
        } else {
          for (int c = 0; c < 4 && n + c < g.N; c++) store_out<TO>(o + c, v[c]);
        }
      }
    }
  }
}

// The large-tile kernel takes bf16 products with both operands K-contiguous,
// 16-byte rows (K, lda, ldb multiples of 8, aligned bases), both output
// extents of at least one block tile, and 256 rows of either operand within
// the 31-bit reach of a buffer offset.
static bool big_nt(const GemmArgs &g) {
  return g.bf16 && g.a_kc && g.b_kc && g.vec_a && g.vec_b && g.K % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         g.M >= BT && g.N >= BT && (long long)BT * g.lda * 2 < (1LL << 31) && (long long)BT * g.ldb * 2 < (1LL << 31);
}
// both operands K-outer: whole 16-byte column pieces and 32-bit row offsets
static bool big_tn(const GemmArgs &g) {
  return g.bf16 && !g.a_kc && !g.b_kc && g.vec_a && g.vec_b && g.M % 8 == 0 && g.N % 8 == 0 && g.lda % 8 == 0 &&
         g.ldb % 8 == 0 && g.lda >= g.M && g.ldb >= g.N && g.M >= BT && g.N >= BT &&
         (long long)g.K * g.lda * 2 < (1LL << 31) && (long long)g.K * g.ldb * 2 < (1LL << 31);
}

template <typename TO, bool KO = false>
static hipError_t gemm_big_launch(const GemmArgs &g, hipStream_t s) {
  const int tm = (g.M + BT - 1) / BT, tn = (g.N + BT - 1) / BT;
  if constexpr (KO) hipLaunchKernelGGL((k_gemm_bf16_nt<TO, KO>), dim3(tm * tn, g.splits), dim3(GT), 0, s, g, tm, tn);
  else hipLaunchKernelGGL((k_gemm_bf16_dl<TO>), dim3(tm * tn, g.splits), dim3(DGT), 0, s, g, tm, tn);
  if (g.splits > 1) {
    hipLaunchKernelGGL((k_gemm_splitk_sum<TO>), dim3(splitk_sum_blocks<TO>(g)), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

template <typename T, bool AKC, bool BKC, typename TO>
static hipError_t gemm_launch(const GemmArgs &g, hipStream_t s) {
  const int tiles = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
  hipLaunchKernelGGL((k_gemm<T, AKC, BKC, TO>), dim3(tiles, g.splits), dim3(256), 0, s, g);
  if (g.splits > 1) {
    hipLaunchKernelGGL((k_gemm_splitk_sum<TO>), dim3(splitk_sum_blocks<TO>(g)), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Long-K fp32 products with both operands stored K-outer and a small output,
// as the dense n = 64 adjoint's weight gradients: C[M,N] = sum_k A[k,m] B[k,n]
// (A [K,M], B [K,N] row-major, M = 192, N <= 64), with the column sums of A
// (bias gradients) from the same reads.  Each block takes 1024 rows of K in
// LDS chunks of 32 and accumulates on v_mfma_f32_32x32x2_f32 (4 wavefronts,
// 3 of the 12 32x32 output tiles each); the per-block partials are summed in
// fp64, in block order, by k_tn_final.
constexpr int TN_M = 192, TN_N = 64, TN_KS = 1024, TN_KC = 32;

__global__ __launch_bounds__(256) void k_tn_part(const float *__restrict__ A, const float *__restrict__ B, int K,
                                                 int N, float *__restrict__ part, float *__restrict__ cpart) {
  __shared__ float sA[TN_KC][TN_M];
  __shared__ float sB[TN_KC][TN_N];
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k0 = blockIdx.x * TN_KS, k1 = min(K, k0 + TN_KS);
  f32x16_t acc[3];
#pragma unroll
  for (int t = 0; t < 3; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.f;
  float csum = 0.f;
  for (int kc = k0; kc < k1; kc += TN_KC) {
    // A chunk: 32 rows x 192 = 1536 float4, 6 per thread; B chunk: 32 x N
#pragma unroll
    for (int q = 0; q < 6; q++) {
      const int e = tid + 256 * q, r = e / (TN_M / 4), c4 = (e % (TN_M / 4)) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (kc + r < k1) v = *reinterpret_cast<const float4 *>(A + (size_t)(kc + r) * TN_M + c4);
      *reinterpret_cast<float4 *>(&sA[r][c4]) = v;
    }
    for (int e = tid; e < TN_KC * TN_N; e += 256) {
      const int r = e / TN_N, c = e % TN_N;
      sB[r][c] = (kc + r < k1 && c < N) ? B[(size_t)(kc + r) * N + c] : 0.f;
    }
    __syncthreads();
    if (tid < TN_M) {
#pragma unroll 8
      for (int r = 0; r < TN_KC; r++) csum += sA[r][tid];
    }
#pragma unroll 4
    for (int k2 = 0; k2 < TN_KC; k2 += 2) {
      const int kr = k2 + (lane >> 5);
#pragma unroll
      for (int t = 0; t < 3; t++) {
        const int tile = wid + 4 * t, tm = tile >> 1, tn = tile & 1;
        const float a = sA[kr][tm * 32 + (lane & 31)], b = sB[kr][tn * 32 + (lane & 31)];
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // lane holds column n = tn*32 + (lane & 31) of rows 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
  for (int t = 0; t < 3; t++) {
    const int tile = wid + 4 * t, tm = tile >> 1, tn = tile & 1;
    const int n = tn * 32 + (lane & 31);
    if (n >= N) continue;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int m = tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      part[((size_t)blockIdx.x * TN_M + m) * N + n] = acc[t][r];
    }
  }
  if (tid < TN_M) cpart[(size_t)blockIdx.x * TN_M + tid] = csum;
}

__global__ __launch_bounds__(256) void k_tn_final(const float *__restrict__ part, const float *__restrict__ cpart,
                                                  int nblk, int N, float *C, float *csum) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < TN_M * N && C) {
    double s = 0.0;
    for (int q = 0; q < nblk; q++) s += (double)part[(size_t)q * TN_M * N + e];
    C[e] = (float)s;
  }
  if (e < TN_M && csum) {
    double s = 0.0;
    for (int q = 0; q < nblk; q++) s += (double)cpart[(size_t)q * TN_M + e];
    csum[e] = (float)s;
  }
}

size_t tn_workspace_bytes(int K) {
  const size_t nblk = (size_t)((K + TN_KS - 1) / TN_KS);
  return nblk * TN_M * TN_N * 4 + nblk * TN_M * 4;
}

hipError_t launch_tn_products(const float *A, const float *B, int K, int N, float *C, float *csum, void *ws,
                              hipStream_t s) {
  if (N < 1 || N > TN_N) return hipErrorInvalidValue;
  const int nblk = (K + TN_KS - 1) / TN_KS;
  float *part = (float *)ws, *cpart = part + (size_t)nblk * TN_M * TN_N;
  hipLaunchKernelGGL(k_tn_part, dim3(nblk), dim3(256), 0, s, A, B, K, N, part, cpart);
  hipLaunchKernelGGL(k_tn_final, dim3((TN_M * N + 255) / 256), dim3(256), 0, s, (const float *)part,
                     (const float *)cpart, nblk, N, C, csum);
  return hipGetLastError();
}

// Split K until the grid covers the device about twice (long-K products
// such as dW = dU^T x have few output tiles; every split writes a full fp32
// partial of C), keeping at least 8 K tiles per split.
int gemm_splits(int M, int N, int K, bool big) {
  if (big && M >= BT && N >= BT) {
    // The large-tile kernel runs one block per CU, so a grid of t tiles x s
    // splits takes ceil(t s / 256) rounds of 1/s of the full-K block time;
    // each split beyond one adds a fp32 partial of C written and summed.
    // Rates (measured): a 256 x 256 block at ~3.7 TFLOP/s, partials moved at
    // ~5 TB/s.  The split count with the smallest estimate, K chunks of at
    // least 512.
    const int tiles = ((M + BT - 1) / BT) * ((N + BT - 1) / BT);
    const double full = 2.0 * BT * BT * (double)K / 3.7e12;
    double best = 1e30;
    int bs = 1;
    for (int s = 1; s <= 32 && (s == 1 || K / s >= 8 * BK); s++) {
      const double t = (double)((tiles * s + 255) / 256) * full / s +
                       (s > 1 ? ((double)s * 8.0 + 4.0) * M * N / 5e12 : 0.0);
      if (t < best * 0.999) {
        best = t;
        bs = s;
      }
    }
    return bs;
  }
  const int tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  int s = 1;
  while (tiles * s < 512 && K / (s * 2) >= 8 * GBK && s < 512) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  const bool bf = g.bf16;
  if (big_nt(g) && !getenv("PARARNN_SMALL_GEMM"))
    return g.out_f32 ? gemm_big_launch<float>(g, s) : gemm_big_launch<uint16_t>(g, s);
  if (big_tn(g) && !getenv("PARARNN_SMALL_GEMM"))
    return g.out_f32 ? gemm_big_launch<float, true>(g, s) : gemm_big_launch<uint16_t, true>(g, s);
#define PR_G(AKC, BKC)                                                                        \
  if (g.a_kc == AKC && g.b_kc == BKC) {                                                       \
    if (bf) return g.out_f32 ? gemm_launch<uint16_t, AKC, BKC, float>(g, s)                   \
                             : gemm_launch<uint16_t, AKC, BKC, uint16_t>(g, s);               \
    return gemm_launch<float, AKC, BKC, float>(g, s);                                         \
  }
  PR_G(true, true)
  PR_G(true, false)
  PR_G(false, true)
  PR_G(false, false)
#undef PR_G
  return hipErrorInvalidValue;
}

}  // namespace pr
