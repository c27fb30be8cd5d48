// Rank-k residual compression by subspace iteration with INT4 factors.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion notes), Key designs / Low-rank strategy for
// extreme compression: approximate the residual X by U V^T, found by subspace
// iteration instead of an SVD, and send U, V quantised to INT4 so that more
// rank fits the same bandwidth. Overall framework and Error feedback give the
// recurrence: the sender keeps e_t = r - U V^T and both sides add U V^T to
// their reconstruction.
//
// Per tensor (n = rows, m = cols, k = rank), with Q0 given:
//   R = bf16(a_t - ahat)                          (fused into the first product)
//   repeat iters times:
//     P = R * bf16(Q)        bf16 MFMA, fp32 accumulate            [lr_rq_kernel]
//     P = CQR(CQR(P))        CholeskyQR2 of the n x k panel        [lr_gram_reduce_kernel,
//                                                                    lr_chol_kernel, lr_solve_kernel]
//     Q = R^T * bf16(P)      bf16 MFMA, R transposed through LDS   [lr_rtp_kernel]
//   U = P, V = Q; per-column absmax INT4                          [lr_int4_kernel]
//   c = Uq Vq^T (fp32 MFMA), e = r - c, ahat += c                 [lr_recon_kernel]
// CQR(P): G = P^T P (fp32 MFMA on 64-row tiles, tile partials summed in tile
// order), G = L L^T (one wave, left-looking, in registers), P <- P L^{-T} as
// the product P (L^{-1})^T (fp32 MFMA).
// A pivot <= 2^-23 * max(trace G, k * FLT_MIN) marks a dead column, whose P
// column is zeroed, so zero or rank-deficient residuals never produce NaN.
// Rank 8 runs 16 wide with start columns 8 .. 15 zero (dead in every pass, k in
// the pivot threshold is the rank asked for); only 8 columns are sent.
//
// MFMA register layouts (gfx950):
//   v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8(l/16) .. +7],
//     B lane l holds B[8(l/16) .. +7][l%16], D lane l holds D[4(l/16) + t][l%16];
//   v_mfma_f32_16x16x4_f32: A[l%16][l/16], B[l/16][l%16], same D.
// ds_read_b64_tr_b16: within each 16-lane group, lanes 4k..4k+3 point at four
// consecutive 16-bit elements of "row k" (16 elements per row), and lane t of
// the group receives element t of rows 0..3 (a 4 x 16 transpose).
// A contraction index may be permuted freely as long as both operands use the
// same permutation; the kernels use that to give each lane longer contiguous
// runs of memory.
#include <float.h>

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "lr_layout.hpp"

namespace rc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kTile = 64;  // rows per panel tile

// Gram partial of a 64 x K tile held in LDS (row stride LD): G[a][b] for the
// upper tile pairs (16-column blocks ta <= tb), fp32 MFMA over the 64 rows in
// order, written to out[K][K] (entries of lower tile pairs are left untouched).
template <int K, int LD>
__device__ __forceinline__ void tile_gram(const float* T, float* out, int nwaves) {
  constexpr int NT = K / 16;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  int pair = 0;
  for (int ta = 0; ta < NT; ++ta)
    for (int tb = ta; tb < NT; ++tb, ++pair) {
      if (pair % nwaves != w) continue;
      // every operand is read from LDS before the first MFMA, so the chain of
      // 16 MFMAs waits for the reads once instead of after each pair of them
      float va[kTile / 4], vb[kTile / 4];
#pragma unroll
      for (int s = 0; s < kTile / 4; ++s) {
        const float* row = T + (4 * s + lk) * LD;
        va[s] = row[16 * ta + lr];
        vb[s] = row[16 * tb + lr];
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kTile / 4; ++s) acc = mfma_f32(va[s], vb[s], acc);
#pragma unroll
      for (int t = 0; t < 4; ++t) out[(16 * ta + 4 * lk + t) * K + 16 * tb + lr] = acc[t];
    }
}

__device__ __forceinline__ void load16_bf16(const uint16_t* p, F8& lo, F8& hi) {
  load8<uint16_t>(p, lo);
  load8<uint16_t>(p + 8, hi);
}
__device__ __forceinline__ u32x4 pack_r(const F8& x, const F8& h) {
  u32x4 v;
  v.x = bf16_rne(x.v[0] - h.v[0]) | (bf16_rne(x.v[1] - h.v[1]) << 16);
  v.y = bf16_rne(x.v[2] - h.v[2]) | (bf16_rne(x.v[3] - h.v[3]) << 16);
  v.z = bf16_rne(x.v[4] - h.v[4]) | (bf16_rne(x.v[5] - h.v[5]) << 16);
  v.w = bf16_rne(x.v[6] - h.v[6]) | (bf16_rne(x.v[7] - h.v[7]) << 16);
  return v;
}

// ---------------------------------------------------------------- P = R * Q
// Block: 64 rows of one tensor, walked in steps of 128 columns. Each step's
// 64 x 128 bf16 tile of R is staged in LDS: wave w loads rows 16w .. 16w+15,
// 32 lanes per row with 4 consecutive columns each, so every wave-wide load
// covers two contiguous row runs (256 B of R or a_t, 512 B of ahat). The next
// step's rows are loaded while the current tile is multiplied. For the MFMAs
// wave w takes the step's columns [32 w, +32) over all 64 rows: lane group
// g = l/16 owns columns [8 g, +8) of that quarter, one 16-byte LDS read per
// 16-row fragment, with the bf16 Q^T operand read the same way from global
// memory (each B operand serves the 4 row fragments). The four waves' partial
// tiles are summed through LDS as (w0 + w2) + (w1 + w3).
// FROM_A: R = bf16(a_t - ahat) is formed while staging and written out for the
// later passes. The block of tile 0 clears the tensor's INT4 absmax slots, which the
// iteration's last solve (U) and last R^T P pass (V) fill.
constexpr int kRqStep = 128;        // columns per step
constexpr int kRqLd = kRqStep + 8;  // bf16 per staged row (272 B)

template <typename IN, bool FROM_A, int K>
__global__ __launch_bounds__(256) void lr_rq_kernel(const IN* __restrict__ a,
                                                    const float* __restrict__ ahat,
                                                    uint16_t* __restrict__ R,
                                                    const uint16_t* __restrict__ Qtb,
                                                    float* __restrict__ P, float* __restrict__ gpart,
                                                    uint32_t* __restrict__ amax, int n, int m,
                                                    int ntiles) {
  constexpr int NT = K / 16;
  constexpr int LD = K + 1;
  constexpr int kStageF = kTile * kRqLd / 2;  // floats spanned by the staged tile
  constexpr int kRedF = 2 * kTile * LD;       // floats of the two reduction tiles
  __shared__ __attribute__((aligned(16))) float lds[kStageF > kRedF ? kStageF : kRedF];
  uint16_t* sR = reinterpret_cast<uint16_t*>(lds);
  float* red0 = lds;
  float* red1 = lds + kTile * LD;
  const int lin = xcd_contiguous(blockIdx.x + ntiles * blockIdx.y, ntiles * gridDim.y);
  const int b = lin / ntiles, tile = lin % ntiles, row0 = tile * kTile;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const uint16_t* Qb = Qtb + (size_t)b * K * m;
  if (tile == 0 && threadIdx.x < 2 * K) amax[(size_t)b * 2 * K + threadIdx.x] = 0u;

  // staging: lane covers row 16w + 2i + (lane >> 5), columns 4 (lane & 31) .. +3
  using Raw = typename std::conditional<std::is_same<IN, uint16_t>::value, u32x2, f32x4>::type;
  struct Stage {
    Raw x[8];
    f32x4 h[8];  // FROM_A: a_t (as loaded) and ahat
    u32x2 r[8];  // otherwise: R
  };
  const int srow = 16 * w + (lane >> 5), scol = 4 * (lane & 31);
  // offsets of staged row i in a_t / ahat (row-major) and in R (tiled); rows
  // past n reread row n-1
  // R: this block's tile of column chunk c0/128 starts at rbase + (c0/128) * cstride
  const size_t rbase = (size_t)(b * ntiles + tile) * 8192;
  const size_t cstride = (size_t)gridDim.y * ntiles * 8192;
  auto soff = [&](int c0, int i) -> size_t {
    const int row = min(row0 + srow + 2 * i, n - 1);
    return ((size_t)b * n + row) * m + (c0 + scol < m ? c0 + scol : 0);
  };
  auto roff = [&](int c0, int i) -> size_t {
    const int r = min(row0 + srow + 2 * i, n - 1) - row0;
    return (size_t)(c0 >> 7) * cstride + rbase + (size_t)(r * 128 + (c0 + scol < m ? scol : 0));
  };
  auto gload = [&](int c0, Stage& S) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (FROM_A) {
        const size_t off = soff(c0, i);
        S.x[i] = __builtin_nontemporal_load(reinterpret_cast<const Raw*>(a + off));
        S.h[i] = load4<float>(ahat + off);
      } else {
        S.r[i] = *reinterpret_cast<const u32x2*>(R + roff(c0, i));
      }
    }
  };
  auto put = [&](int c0, const Stage& S) {
    const bool col_ok = c0 + scol < m;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x2 v;
      if constexpr (FROM_A) {
        f32x4 x;
        if constexpr (std::is_same<IN, uint16_t>::value)
          x = f32x4{bf16_lo(S.x[i].x), bf16_hi(S.x[i].x), bf16_lo(S.x[i].y), bf16_hi(S.x[i].y)};
        else
          x = S.x[i];
        v.x = bf16_rne(x[0] - S.h[i][0]) | (bf16_rne(x[1] - S.h[i][1]) << 16);
        v.y = bf16_rne(x[2] - S.h[i][2]) | (bf16_rne(x[3] - S.h[i][3]) << 16);
        // non-temporal: R is read again three times, and the later passes read
        // it half as fast when its lines are still dirty in the caches
        if (col_ok && row0 + srow + 2 * i < n)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(R + roff(c0, i)));
      } else {
        v = S.r[i];
      }
      if (!col_ok) v = u32x2{0u, 0u};  // columns past m multiply as zeros
      *reinterpret_cast<u32x2*>(&sR[(srow + 2 * i) * kRqLd + scol]) = v;
    }
  };

  f32x4 acc[4][NT];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < NT; ++g) acc[f][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  // R alone (2 B per element) is prefetched a step ahead; a_t and ahat (6 B per
  // element) are loaded at the top of their own step, which keeps the register
  // count low enough for more resident waves to cover the latency instead.
  // The Q^T operands of a step are loaded before any later load is issued, and
  // neither is behind a branch: waits on loads complete in issue order, so the
  // MFMAs then wait for Q^T alone, not for the prefetch behind it. (A wave
  // whose columns lie past m reads column 0 of Q^T against staged zeros.)
  auto bload = [&](int c0, u32x4 (&B)[NT]) {
    const int kc = c0 + 32 * w < m ? c0 + 32 * w : 0;
#pragma unroll
    for (int g = 0; g < NT; ++g)
      B[g] = *reinterpret_cast<const u32x4*>(Qb + g32(16 * g + lr, kc + 8 * lk, K));
  };
  Stage S;
  auto step = [&](int c0, auto prefetch) {
    u32x4 B[NT];
    if constexpr (FROM_A) {
      bload(c0, B);
      __builtin_amdgcn_sched_barrier(0);  // keep the Q^T loads first
      gload(c0, S);
    }
    __syncthreads();  // the previous tile has been read
    put(c0, S);
    __syncthreads();
    if constexpr (!FROM_A) {
      bload(c0, B);
      __builtin_amdgcn_sched_barrier(0);  // keep the Q^T loads first
      if constexpr (decltype(prefetch)::value) gload(c0 + kRqStep, S);
      __builtin_amdgcn_sched_barrier(0);  // and the prefetch before the MFMAs
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const u32x4 A = *reinterpret_cast<const u32x4*>(&sR[(16 * f + lr) * kRqLd + 32 * w + 8 * lk]);
#pragma unroll
      for (int g = 0; g < NT; ++g) acc[f][g] = mfma_bf16(A, B[g], acc[f][g]);
    }
  };
  if constexpr (!FROM_A) gload(0, S);
  int c0 = 0;
  for (; c0 + kRqStep < m; c0 += kRqStep) step(c0, std::true_type{});
  step(c0, std::false_type{});

  // (w0 + w2) + (w1 + w3), rows past n zeroed, tile kept in red1
  auto store_acc = [&](float* dst) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < NT; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) dst[(16 * f + 4 * lk + t) * LD + 16 * g + lr] = acc[f][g][t];
  };
  auto add_acc = [&](const float* src) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < NT; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[f][g][t] += src[(16 * f + 4 * lk + t) * LD + 16 * g + lr];
  };
  __syncthreads();  // the staged tile is no longer needed
  if (w >= 2) store_acc(w == 2 ? red0 : red1);
  __syncthreads();
  if (w < 2) add_acc(w == 0 ? red0 : red1);
  __syncthreads();
  if (w == 1) store_acc(red0);
  __syncthreads();
  if (w == 0) {
    add_acc(red0);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (row0 + 16 * f + 4 * lk + t >= n)
#pragma unroll
          for (int g = 0; g < NT; ++g) acc[f][g][t] = 0.f;
    store_acc(red1);
  }
  __syncthreads();
  const float* T = red1;
  // P rows of the tile: 4 consecutive entries per lane and pass, all LDS reads
  // of the lane before its stores
  constexpr int kPIt = kTile * K / 4 / 256;
  static_assert(kTile * K % (4 * 256) == 0, "P tile must split evenly over the block");
  f32x4 pv[kPIt];
#pragma unroll
  for (int it = 0; it < kPIt; ++it) {
    const int q = it * 256 + (int)threadIdx.x, r = (4 * q) / K, j = (4 * q) % K;
#pragma unroll
    for (int t = 0; t < 4; ++t) pv[it][t] = T[r * LD + j + t];
  }
#pragma unroll
  for (int it = 0; it < kPIt; ++it) {
    const int q = it * 256 + (int)threadIdx.x, r = (4 * q) / K, j = (4 * q) % K;
    if (row0 + r < n) *reinterpret_cast<f32x4*>(P + ((size_t)b * n + row0 + r) * K + j) = pv[it];
  }
  tile_gram<K, LD>(T, gpart + ((size_t)b * ntiles + tile) * K * K, 4);
}

// ---------------------------------------------------------------- Gram sum
// gsum[b] = sum of the tile partials, in tile order (four interleaved running
// sums, combined as (s0 + s1) + (s2 + s3)); one lane per entry.
template <int K>
__global__ __launch_bounds__(256) void lr_gram_reduce_kernel(const float* __restrict__ gpart,
                                                             float* __restrict__ gsum, int ntiles) {
  const int b = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= K * K) return;
  const float* gp = gpart + (size_t)b * ntiles * K * K + idx;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  int p = 0;
  for (; p + 16 <= ntiles; p += 16) {  // 16 loads in flight, same summation order
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = gp[(size_t)(p + q) * K * K];
#pragma unroll
    for (int q = 0; q < 16; ++q) s[q & 3] += v[q];
  }
  for (; p + 4 <= ntiles; p += 4)
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += gp[(size_t)(p + q) * K * K];
  for (int q = 0; p < ntiles; ++p, ++q) s[q] += gp[(size_t)p * K * K];
  gsum[(size_t)b * K * K + idx] = (s[0] + s[1]) + (s[2] + s[3]);
}

// ---------------------------------------------------------------- Cholesky
// One wave per tensor, no LDS and no barriers: lane i holds row i of G (from
// the upper triangle of gsum) and builds row i of L by the left-looking
// recurrence; lane c builds column c of L^{-1} by forward substitution. Step j
// of both needs row j of L up to column j-1, which lives in lane j's
// registers: each entry is broadcast with one readlane and feeds both dot
// products, which run as independent chains. Dead columns (pivot <= 2^-23 *
// max(trace G, K * FLT_MIN)) get L[j][j] = 1, a zero column below the diagonal
// and a zero row j of L^{-1}, so x = L^{-1} p has x_j = 0 there and the other
// entries are those of the forward substitution. Both dot products are fused
// multiply-add chains in index order; divisions by L[j][j] are products with
// its correctly rounded reciprocal.
__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <int K, int KP>
__global__ __launch_bounds__(64) void lr_chol_kernel(const float* __restrict__ gsum,
                                                     float* __restrict__ linv,
                                                     uint32_t* __restrict__ dead) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float* gs = gsum + (size_t)b * K * K;
  float* out = linv + (size_t)b * K * K + lane;  // column `lane` of L^{-1}
  float g[K], L[K], y[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    g[j] = (lane < K && j <= lane) ? gs[j * K + lane] : 0.f;  // G[lane][j] = G[j][lane]
    L[j] = 0.f;
  }
  float tr = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) tr += lane_f32(g[j], j);
  const float tol = ldexpf(fmaxf(tr, (float)KP * FLT_MIN), -23);  // KP: the rank asked for
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float s = g[j];                     // G[lane][j] - sum_p L[lane][p] L[j][p]
    float t = (j == lane) ? 1.f : 0.f;  // e_lane[j] - sum_p L[j][p] y[p]
#pragma unroll
    for (int p = 0; p < j; ++p) {
      const float ljp = lane_f32(L[p], j);  // L[j][p]
      s = fmaf(-L[p], ljp, s);
      t = fmaf(-ljp, y[p], t);
    }
    const float piv = lane_f32(s, j);
    const bool dj = !(piv > tol);
    const float ljj = dj ? 1.0f : sqrtf(piv);
    const float inv = 1.0f / ljj;
    L[j] = lane == j ? ljj : (lane > j && !dj ? s * inv : 0.f);
    y[j] = dj ? 0.f : t * inv;
    if (lane < K) out[(size_t)j * K] = y[j];  // stored here, so the chain is not deferred to the end
    if (dead && dj && j < KP && lane == 0) atomicAdd(dead, 1u);  // debug report of sent columns
  }
}

// ---------------------------------------------------------------- P <- P L^-T
// One 64-row tile per block of 4 waves: X = T L^{-T} with fp32 MFMA (T = the
// tile of P), wave w producing rows 16w .. 16w+15. All global loads (L^{-1}
// and the tile) are issued before the first LDS store. A wave reads only its
// own 16 rows of T, so it writes X over them in place.
// GRAM: also write the Gram partial of the solved tile (next CQR pass).
// FINAL: also write the bf16 transposed panel used by the R^T P product
// (rows n .. rows_pad-1 written as 0) and fold the column absmax of the tile
// into amax[b][0][*] (the INT4 scales of U).
template <int K, bool GRAM, bool FINAL>
__global__ __launch_bounds__(256) void lr_solve_kernel(float* __restrict__ P,
                                                       const float* __restrict__ linv,
                                                       float* __restrict__ gpart,
                                                       uint16_t* __restrict__ Pbt,
                                                       uint32_t* __restrict__ amax, int n,
                                                       int ntiles, int rows_pad) {
  constexpr int NT = K / 16;
  constexpr int LD = K + 4;  // 16-B aligned rows; MFMA operand reads hit 64 distinct banks
  constexpr int V4 = K / 4;  // f32x4 per row
  constexpr int LI_IT = (K * V4 + 255) / 256;
  constexpr int T_IT = kTile * V4 / 256;
  static_assert(kTile * V4 % 256 == 0, "tile must split evenly over the block");
  __shared__ __attribute__((aligned(16))) float Li[K * LD];
  __shared__ __attribute__((aligned(16))) float T[kTile * LD];
  const int b = blockIdx.y, tile = blockIdx.x, row0 = tile * kTile;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lk = lane >> 4;
  const float* li = linv + (size_t)b * K * K;
  float* Pb = P + (size_t)b * n * K;
  f32x4 lv[LI_IT], tv[T_IT];
#pragma unroll
  for (int i = 0; i < LI_IT; ++i) {
    const int idx = tid + 256 * i;
    lv[i] = idx < K * V4 ? *reinterpret_cast<const f32x4*>(li + 4 * idx) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < T_IT; ++i) {
    const int idx = tid + 256 * i, r = idx / V4, j = 4 * (idx % V4);
    tv[i] = row0 + r < n ? *reinterpret_cast<const f32x4*>(Pb + (size_t)(row0 + r) * K + j)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < LI_IT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < K * V4) *reinterpret_cast<f32x4*>(Li + (idx / V4) * LD + 4 * (idx % V4)) = lv[i];
  }
#pragma unroll
  for (int i = 0; i < T_IT; ++i) {
    const int idx = tid + 256 * i;
    *reinterpret_cast<f32x4*>(T + (idx / V4) * LD + 4 * (idx % V4)) = tv[i];
  }
  __syncthreads();
  // X[r][i] = sum_c T[r][c] Linv[i][c]: A = T (rows r), B[c][i] = Linv[i][c]
  f32x4 acc[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
  float* Tw = T + 16 * w * LD;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4) {
    const float a = Tw[lr * LD + k0 + lk];
#pragma unroll
    for (int it = 0; it < NT; ++it) acc[it] = mfma_f32(a, Li[(16 * it + lr) * LD + k0 + lk], acc[it]);
  }
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int t = 0; t < 4; ++t) Tw[(4 * lk + t) * LD + 16 * it + lr] = acc[it][t];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < T_IT; ++i) {
    const int idx = tid + 256 * i, r = idx / V4, j = 4 * (idx % V4);
    if (row0 + r < n)
      *reinterpret_cast<f32x4*>(Pb + (size_t)(row0 + r) * K + j) =
          *reinterpret_cast<const f32x4*>(T + r * LD + j);
  }
  if constexpr (FINAL) {
    // lane = row of the tile (rows past n are zero in X); wave w writes
    // columns w, w + 4, ...
    const int row = row0 + lane;
    uint16_t* dst = Pbt + (size_t)b * K * rows_pad;
#pragma unroll
    for (int j = w; j < K; j += 4) dst[g32(j, row, K)] = (uint16_t)bf16_rne(T[lane * LD + j]);
    __shared__ float cm[4 * K];
    if (lane < K) {
      float mx = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(Tw[r * LD + lane]));
      cm[w * K + lane] = mx;
    }
    __syncthreads();
    if (tid < K) {
      const float mx = fmaxf(fmaxf(cm[tid], cm[K + tid]), fmaxf(cm[2 * K + tid], cm[3 * K + tid]));
      atomicMax(amax + (size_t)b * 2 * K + tid, __float_as_uint(mx));
    }
  }
  if constexpr (GRAM) tile_gram<K, LD>(T, gpart + ((size_t)b * ntiles + tile) * K * K, 4);
}

// ---------------------------------------------------------------- Q = R^T P
// Block: 128 columns of one tensor over all of its rows, in two halves of 4
// waves: half h walks rows [h * rows_pad/2, (h+1) * rows_pad/2), and at the end
// half 1's sums are added to half 0's through LDS (one fixed order). Within a
// half, wave w owns columns 32w .. 32w+31 (two 16-column MFMA tiles). Per step
// of 32 rows the R tile [32 x 128] and the matching P^T chunk [K x 32] are
// staged through LDS (double buffered per half, one barrier per step). R is
// read back transposed with ds_read_b64_tr_b16 (A[c][i] = R[i][c]); each P^T
// fragment read from LDS feeds both column tiles of the wave. A last block of
// 64 columns (cols % 128 == 64) computes its missing half from reread valid
// columns and stores only the valid ones.
// The two halves matter where the grid is small: the video-like share has 15
// column blocks per tensor and 30 tensors, 450 blocks on 256 CUs, and twice
// the waves per block run it 5 % faster (the flux-like grid, 1368 blocks, is
// unchanged).
// The block writes its columns of Q^T itself. Before the last iteration Q is
// needed only as the bf16 operand of the next product (Qtb); after it, only as
// V: Qt in fp32 and the column absmax of V folded into amax[b][1][j] (FINAL).
// Splitting the rows over several blocks (and summing the splits in a second
// kernel) was measured slower on both low-rank workloads: the products gain
// less from the larger grid than the sum costs.
constexpr int kRtpCols = 128;
constexpr int kRtpLd = kRtpCols + 8;  // bf16 per staged R row (272 B)
constexpr int kRtpPld = 32 + 8;       // bf16 per staged P^T row (80 B)
constexpr int kRtpHalves = 2;         // row halves per block, 256 threads each

template <int K, bool FINAL>
__global__ __launch_bounds__(256 * kRtpHalves) void lr_rtp_kernel(const uint16_t* __restrict__ R,
                                                     const uint16_t* __restrict__ Pbt,
                                                     float* __restrict__ Qt,
                                                     uint16_t* __restrict__ Qtb,
                                                     uint32_t* __restrict__ amax, int n, int m,
                                                     int rows_pad) {
  constexpr int NT = K / 16;
  constexpr int PCH = K * 4;  // 16-byte chunks of a [K x 32] bf16 P^T block
  __shared__ __attribute__((aligned(16))) uint16_t sRh[kRtpHalves][2][32 * kRtpLd];
  __shared__ __attribute__((aligned(16))) uint16_t sPh[kRtpHalves][2][K * kRtpPld];
  const int tid = threadIdx.x & 255, half = threadIdx.x >> 8;
  auto sR = sRh[half];
  auto sP = sPh[half];
  // Logical blocks (column block fastest, then tensor) are spread over the
  // XCDs in contiguous ranges, so the column blocks that share a P^T chunk
  // share an L2. Tensors are taken in the reverse of that order: every XCD's
  // range of the R*Q pass before this one ran forwards, so the tensors this
  // pass starts with are the ones that pass read last and are still in the
  // device's last-level cache (the next forward pass finds this pass's in turn).
  const int nblk = gridDim.x * gridDim.y;
  const int lin = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, nblk);
  const int cb = lin % gridDim.x;
  const int b = gridDim.y - 1 - lin / gridDim.x;
  const int c0 = cb * kRtpCols;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lk = lane >> 4;
  // R staging: each wave-wide load covers 4 whole 256-byte row pieces (16 lanes
  // x 16 bytes per row); loads q = 0, 1 take rows ld_row and ld_row + 16
  const int ld_row = tid >> 4, ld_col = (tid & 15) * 8;
  const bool col_ok = c0 + ld_col < m;
  // this half's rows (rows_pad is a multiple of 64, so both halves hold the
  // same whole number of 32-row steps and meet every barrier together)
  const int i_begin = half * (rows_pad / kRtpHalves);
  const int i_end = i_begin + rows_pad / kRtpHalves;
  const int batch = gridDim.y, bands = rows_pad >> 6;
  const uint16_t* Pb = Pbt + (size_t)b * K * rows_pad;
  const int tr_off = (8 * lk + (lr >> 2)) * kRtpLd + 32 * w + 4 * (lr & 3);

  // Two steps are in flight while one is multiplied: the loop is unrolled by two
  // so each step's registers keep their role, and every load is unconditional
  // (past the last step the addresses are clamped to it, which the cache
  // serves), so waits count only the older step's loads.
  struct Stage { u32x4 r0, r1, p; };
  const int last = i_end - 32;
  auto gload = [&](int i0) {
    i0 = min(i0, last);
    Stage st;
    const int row0 = min(i0 + ld_row, n - 1), row1 = min(i0 + ld_row + 16, n - 1);
    // columns past m reread column c0; output row c of the product depends on
    // column c of R alone, and rows past m are never stored
    const int col = c0 + (col_ok ? ld_col : 0);
    // R is read non-temporally here and with ordinary loads in R*Q. An R*Q
    // pass leaves the part of R it read last in the device's last-level
    // cache, where the R^T*P pass after it still finds it, and non-temporal
    // reads keep this pass from displacing other cached data: the three passes
    // that read R alone took 242 / 311 us together this way against 254 / 333
    // us with ordinary loads in all of them (flux / video, one stream). The
    // cache policy changes no value.
    st.r0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(R + r_index(b, row0, col, batch, bands)));
    st.r1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(R + r_index(b, row1, col, batch, bands)));
    // lanes past the P^T chunk count reread chunk 0 and never store it
    const int t = tid < PCH ? tid : 0;
    st.p = *reinterpret_cast<const u32x4*>(Pb + g32(t >> 2, i0 + 8 * (t & 3), K));
    return st;
  };
  f32x4 acc[2][NT];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int g = 0; g < NT; ++g) acc[ct][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto put = [&](const Stage& st, int buf) {
    *reinterpret_cast<u32x4*>(&sR[buf][ld_row * kRtpLd + ld_col]) = st.r0;
    *reinterpret_cast<u32x4*>(&sR[buf][(ld_row + 16) * kRtpLd + ld_col]) = st.r1;
    if (tid < PCH)
      *reinterpret_cast<u32x4*>(&sP[buf][(tid >> 2) * kRtpPld + 8 * (tid & 3)]) = st.p;
  };
  auto compute = [&](int buf) {
    u32x4 A[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int o = tr_off + 16 * ct;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)&sR[buf][o]);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)&sR[buf][o + 4 * kRtpLd]);
      A[ct].x = (uint32_t)(uint16_t)lo.x | ((uint32_t)(uint16_t)lo.y << 16);
      A[ct].y = (uint32_t)(uint16_t)lo.z | ((uint32_t)(uint16_t)lo.w << 16);
      A[ct].z = (uint32_t)(uint16_t)hi.x | ((uint32_t)(uint16_t)hi.y << 16);
      A[ct].w = (uint32_t)(uint16_t)hi.z | ((uint32_t)(uint16_t)hi.w << 16);
    }
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const u32x4 Bv = *reinterpret_cast<const u32x4*>(&sP[buf][(16 * g + lr) * kRtpPld + 8 * lk]);
      acc[0][g] = mfma_bf16(A[0], Bv, acc[0][g]);
      acc[1][g] = mfma_bf16(A[1], Bv, acc[1][g]);
    }
  };

  // LDS double buffer, one barrier per step: a buffer is refilled two steps
  // after it was read, and every wave has passed the barrier in between.
  Stage s0 = gload(i_begin), s1 = gload(i_begin + 32);
  int i0 = i_begin;
  for (; i0 + 32 < i_end; i0 += 64) {
    put(s0, 0);
    __syncthreads();
    s0 = gload(i0 + 64);
    compute(0);
    put(s1, 1);
    __syncthreads();
    s1 = gload(i0 + 96);
    compute(1);
  }
  if (i0 < i_end) {  // an odd number of steps
    put(s0, 0);
    __syncthreads();
    compute(0);
  }
  // half 1's sums into half 0's (the staging buffers are free after the barrier)
  static_assert(2 * (K / 16) * 256 * 16 <= sizeof(sRh), "R staging too small for the half sums");
  __syncthreads();
  f32x4* hsum = reinterpret_cast<f32x4*>(&sRh[0][0][0]);
  if (half == 1)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int g = 0; g < NT; ++g) hsum[(ct * NT + g) * 256 + tid] = acc[ct][g];
  __syncthreads();
  if (half == 0)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int g = 0; g < NT; ++g) {
        const f32x4 o = hsum[(ct * NT + g) * 256 + tid];
        acc[ct][g] = f32x4{acc[ct][g].x + o.x, acc[ct][g].y + o.y, acc[ct][g].z + o.z,
                           acc[ct][g].w + o.w};
      }
  // D[c][j]: lane holds c = c0 + 32w + 16ct + 4lk + t, j = 16g + lr (half 0 stores)
  float mx[NT];
#pragma unroll
  for (int g = 0; g < NT; ++g) mx[g] = 0.f;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c = c0 + 32 * w + 16 * ct + 4 * lk;
    if (c < m && half == 0) {
#pragma unroll
      for (int g = 0; g < NT; ++g) {
        const f32x4 v = acc[ct][g];
        const size_t o = ((size_t)b * K + 16 * g + lr) * m + c;
        if constexpr (FINAL) {
          *reinterpret_cast<f32x4*>(Qt + o) = v;
          mx[g] = fmaxf(mx[g], fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        } else {
          uint2 hb;
          hb.x = bf16_rne(v.x) | (bf16_rne(v.y) << 16);
          hb.y = bf16_rne(v.z) | (bf16_rne(v.w) << 16);
          *reinterpret_cast<uint2*>(Qtb + (size_t)b * K * m + g32(16 * g + lr, c, K)) = hb;
        }
      }
    }
  }
  if constexpr (FINAL) {
    // column j's maximum over the wave's 32 columns, then over the 4 waves
    __shared__ float cm[4 * K];
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 16));
      mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 32));
      if (lk == 0 && half == 0) cm[w * K + 16 * g + lr] = mx[g];
    }
    __syncthreads();
    const int j = threadIdx.x;
    if (j < K) {
      const float v = fmaxf(fmaxf(cm[j], cm[K + j]), fmaxf(cm[2 * K + j], cm[3 * K + j]));
      atomicMax(amax + ((size_t)b * 2 + 1) * K + j, __float_as_uint(v));
    }
  }
}

// ---------------------------------------------------------------- INT4 factors
// One lane per factor row: rows 0..n-1 are U (= P, [n][K]), rows n..n+m-1 are V
// (= Q, stored as Qt [K][m]). Per column j: s_j = absmax_j / 7,
// q = clamp(rint_even(x / s_j), -7, 7) (0 when s_j = 0), packed row-major,
// element t in nibble t (even t low), two's complement. Block 0 writes the
// scale sections and zeroes the section padding. Sender and receiver both
// reconstruct from these packed bytes (q * s_j, in the reconstruct kernel).
template <int K, int KP>
__global__ __launch_bounds__(256) void lr_int4_kernel(const float* __restrict__ P,
                                                      const float* __restrict__ Qt,
                                                      const uint32_t* __restrict__ amax,
                                                      uint8_t* __restrict__ packed, Layout L) {
  __shared__ float sc[2 * K];
  const int b = blockIdx.y;
  const int n = (int)L.rows, m = (int)L.cols;
  uint8_t* pk = packed + (size_t)b * L.tstride;
  if (threadIdx.x < 2 * K) sc[threadIdx.x] = __uint_as_float(amax[(size_t)b * 2 * K + threadIdx.x]) / 7.0f;
  __syncthreads();
  if (blockIdx.x == 0) {
    float* su = reinterpret_cast<float*>(pk + L.sec_off[2]);
    float* sv = reinterpret_cast<float*>(pk + L.sec_off[3]);
    if (threadIdx.x < KP) su[threadIdx.x] = sc[threadIdx.x];
    else if (threadIdx.x >= K && threadIdx.x < K + KP) sv[threadIdx.x - K] = sc[threadIdx.x];
    for (int s = 0; s < L.nsec; ++s) {
      const int64_t start = L.sec_off[s] + L.sec_len[s];
      const int64_t end = (s + 1 < L.nsec) ? L.sec_off[s + 1] : L.tstride;
      for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) pk[i] = 0;
    }
  }
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n + m) return;
  const bool isV = r >= n;
  const int i = isV ? r - n : r;
  const float* s = sc + (isV ? K : 0);
  // the whole factor row (its KP sent columns) is loaded before any of it is quantised
  float x[KP];
  if (isV) {
    const float* src = Qt + (size_t)b * K * m + i;
#pragma unroll
    for (int j = 0; j < KP; ++j) x[j] = src[(size_t)j * m];
  } else {
    const f32x4* src = reinterpret_cast<const f32x4*>(P + ((size_t)b * n + i) * K);
#pragma unroll
    for (int j = 0; j < KP / 4; ++j) {
      const f32x4 v = src[j];
      x[4 * j] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
    }
  }
  uint32_t words[KP / 8];
#pragma unroll
  for (int q = 0; q < KP / 8; ++q) words[q] = 0;
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    int qi = 0;
    if (s[j] > 0.f) qi = (int)fminf(fmaxf(rintf(x[j] / s[j]), -7.f), 7.f);
    words[j / 8] |= ((uint32_t)qi & 0xFu) << (4 * (j % 8));
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(pk + (isV ? L.sec_off[1] : L.sec_off[0]) + (size_t)i * (KP / 2));
#pragma unroll
  for (int q = 0; q < KP / 8; ++q) dst[q] = words[q];
}

// ---------------------------------------------------------------- bf16 factors
// The factor-precision alternative: U and V sent as bf16 (round to nearest
// even), row-major, no scales. One lane per factor row as above; sender and
// receiver reconstruct from the bf16 values.
template <int K, int KP>
__global__ __launch_bounds__(256) void lr_bf16f_kernel(const float* __restrict__ P,
                                                       const float* __restrict__ Qt,
                                                       uint8_t* __restrict__ packed, Layout L) {
  const int b = blockIdx.y;
  const int n = (int)L.rows, m = (int)L.cols;
  uint8_t* pk = packed + (size_t)b * L.tstride;
  if (blockIdx.x == 0) {
    for (int s = 0; s < L.nsec; ++s) {
      const int64_t start = L.sec_off[s] + L.sec_len[s];
      const int64_t end = (s + 1 < L.nsec) ? L.sec_off[s + 1] : L.tstride;
      for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) pk[i] = 0;
    }
  }
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n + m) return;
  const bool isV = r >= n;
  const int i = isV ? r - n : r;
  const float* src = isV ? Qt + (size_t)b * K * m + i : P + ((size_t)b * n + i) * K;
  const size_t stride = isV ? (size_t)m : 1;
  uint32_t* dst = reinterpret_cast<uint32_t*>(pk + (isV ? L.sec_off[1] : L.sec_off[0]) + (size_t)i * KP * 2);
#pragma unroll
  for (int j = 0; j < KP; j += 2) dst[j / 2] = bf16_rne(src[j * stride]) | (bf16_rne(src[(j + 1) * stride]) << 16);
}

// ---------------------------------------------------------------- reconstruct
// c = Uq Vq^T with fp32 MFMA, read straight from the packed factors (INT4 codes
// times their column scale, or bf16), applied to the state arrays. A block owns
// CW columns (CW = 256 or 128: four strips of CW/4 columns, one per wave) of a
// chunk of rows of one tensor of one peer and walks it in 16-row tiles:
//   * once: each wave's V operands (CW/64 MFMA column tiles x K) in registers;
//   * per tile: each wave computes its 16 x CW/4 piece of c^T = Vq Uq^T with
//     MFMAs and writes it to an LDS tile (two buffers, one barrier per tile);
//     then wave w applies rows 4w .. 4w+3 of the tile, each lane owning 4
//     consecutive columns, so every global access of a wave covers whole
//     CW-column row pieces (one 1 KiB run, or two 512 B runs):
//     r = a - ahat, e = r - c, ahat += c (SENDER) or ahat += c.
//     The next tile's U operands and state rows are loaded before the current
//     tile's MFMAs; the last tile has no successor to load.
// MFMA step (j, i), j < K/16, i < 4: lane group g = l/16 covers contraction
// index 16 j + 4 g + i, so both operands come from 4 consecutive factor
// entries of one row (2 bytes of INT4 codes or 8 bytes of bf16). The M index mi
// of column tile p is strip column 32 (p/2) + 8 (mi/4) + 4 (p%2) + mi%4, so each
// lane's results are runs of 8 columns of one row. Sender and receiver run the
// same MFMA sequence on the same packed bytes, so both get the same c bit for
// bit (the column width changes which block computes an entry, not how).
// Strips and lanes past m (m a multiple of 64) compute and store nothing.
// Grid z = peer * batch + tensor.

// Factor entries (row, k0 .. k0+3) as the encoder defined them: INT4 code times
// the column scale (scale4 = the 4 scales of k0 .. k0+3), or the bf16 value.
// Rows hold KP entries; columns k0 >= KP are not sent and are zero.
// The raw bytes (factor_raw: 4 INT4 codes in the low 16 bits, or 4 bf16) are
// loaded first and decoded at use (factor_decode), so loads in flight hold as
// few registers as possible.
template <bool BF16F>
using FactorRaw = typename std::conditional<BF16F, u32x2, uint32_t>::type;

template <int KP, bool BF16F>
__device__ __forceinline__ FactorRaw<BF16F> factor_raw(const uint8_t* sec, int row, int k0) {
  if constexpr (BF16F) {
    if (k0 >= KP) return u32x2{0u, 0u};
    return *reinterpret_cast<const u32x2*>(sec + ((size_t)row * KP + k0) * 2);
  } else {
    if (k0 >= KP) return 0u;
    return *reinterpret_cast<const uint16_t*>(sec + ((size_t)row * KP + k0) / 2);
  }
}

template <bool BF16F>
__device__ __forceinline__ f32x4 factor_decode(const FactorRaw<BF16F>& w, const f32x4& scale4) {
  if constexpr (BF16F) {
    return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  } else {
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = (int)((w >> (4 * i)) & 15u);
      v[i] = (float)(q >= 8 ? q - 16 : q) * scale4[i];
    }
    return v;
  }
}

template <int KP, bool BF16F>
__device__ __forceinline__ f32x4 factor4(const uint8_t* sec, const f32x4& scale4, int row, int k0) {
  return factor_decode<BF16F>(factor_raw<KP, BF16F>(sec, row, k0), scale4);
}

// a_t as loaded (bf16 pairs or fp32), widened to fp32 at use.
template <typename IN>
using InRaw = typename std::conditional<std::is_same<IN, uint16_t>::value, u32x2, f32x4>::type;

template <typename IN>
__device__ __forceinline__ InRaw<IN> load_raw4(const IN* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const InRaw<IN>*>(p));
}

template <typename IN>
__device__ __forceinline__ f32x4 widen4(const InRaw<IN>& w) {
  if constexpr (std::is_same<IN, uint16_t>::value)
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
  else
    return w;
}

template <typename IN, bool SENDER, int K, int KP, bool BF16F, int CW>
__global__ __launch_bounds__(256) void lr_recon_kernel(const IN* __restrict__ a,
                                                       float* __restrict__ e, PeerSet peers,
                                                       int batch, Layout L, int chunk_rows) {
  static_assert(CW == 256 || CW == 128, "column width");
  constexpr int KJ = K / 16;
  constexpr int SW = CW / 4;       // strip columns per wave
  constexpr int NP = SW / 16;      // MFMA column tiles per wave
  constexpr int LPR = CW / 4;      // lanes per row when applying
  constexpr int RPI = 64 / LPR;    // rows per wave-wide access
  constexpr int NI = 4 / RPI;      // accesses per wave per tile
  constexpr int LDSW = CW + 4;     // LDS row stride, floats
  __shared__ float tile[2][16 * LDSW];
  const int n = (int)L.rows, m = (int)L.cols;
  const int peer = blockIdx.z / batch, b = blockIdx.z % batch;
  float* __restrict__ ahat = peers.state[peer];
  const uint8_t* pk = peers.packed[peer] + (size_t)b * L.tstride;
  const uint8_t* usec = pk + L.sec_off[0];
  const uint8_t* vsec = pk + L.sec_off[1];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const int cb = blockIdx.x * CW;
  const int c0 = cb + SW * w;
  const bool strip_ok = c0 < m;
  const int lc = 4 * (lane % LPR), ri = lane / LPR;  // apply: lane's columns and row in an access
  const bool col_ok = cb + lc < m;
  const int rbeg = blockIdx.y * chunk_rows;
  const int rend = min(n, rbeg + chunk_rows);

  f32x4 su[KJ], sv[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    if constexpr (BF16F) {
      su[j] = sv[j] = f32x4{1.f, 1.f, 1.f, 1.f};
    } else if (16 * j + 4 * lk >= KP) {
      su[j] = sv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      su[j] = *reinterpret_cast<const f32x4*>(pk + L.sec_off[2] + 4 * (16 * j + 4 * lk));
      sv[j] = *reinterpret_cast<const f32x4*>(pk + L.sec_off[3] + 4 * (16 * j + 4 * lk));
    }
  }
  f32x4 av[NP][KJ];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int col = (strip_ok ? c0 : 0) + 32 * (p >> 1) + 8 * (lr >> 2) + 4 * (p & 1) + (lr & 3);
#pragma unroll
    for (int j = 0; j < KJ; ++j) av[p][j] = factor4<KP, BF16F>(vsec, sv[j], col, 16 * j + 4 * lk);
  }
  const size_t tb = (size_t)b * n * m + (size_t)(col_ok ? cb + lc : 0);

  // The receiver keeps the next tile's U operands as packed bytes until use
  // (fewer registers: one more block per CU for k 48); the sender decodes them
  // as they arrive (measured faster there).
  using URow = typename std::conditional<SENDER, f32x4, FactorRaw<BF16F>>::type;
  struct Rows {
    URow u[KJ];              // U operands of the tile's 16 rows
    f32x4 h[NI];             // ahat of this lane's rows and 4 columns
    InRaw<IN> x[NI];         // a_t of the same, as loaded (SENDER)
  };
  // Rows past the chunk reread its last row and are never stored.
  auto load = [&](int r0, Rows& R) {
    const int ru = min(r0 + lr, rend - 1);
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      if constexpr (SENDER)
        R.u[j] = factor4<KP, BF16F>(usec, su[j], ru, 16 * j + 4 * lk);
      else
        R.u[j] = factor_raw<KP, BF16F>(usec, ru, 16 * j + 4 * lk);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const size_t off = tb + (size_t)min(r0 + 4 * w + RPI * i + ri, rend - 1) * m;
      R.h[i] = load4<float>(ahat + off);
      if constexpr (SENDER) R.x[i] = load_raw4<IN>(a + off);
    }
  };
  auto apply = [&](int r0, int it, const Rows& T) {
    f32x4 acc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (strip_ok) {
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        f32x4 u;
        if constexpr (SENDER)
          u = T.u[j];
        else
          u = factor_decode<BF16F>(T.u[j], su[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int p = 0; p < NP; ++p) acc[p] = mfma_f32(av[p][j][i], u[i], acc[p]);
      }
    }
    float* S = tile[it & 1];
#pragma unroll
    for (int p = 0; p < NP; ++p)
      *reinterpret_cast<f32x4*>(&S[lr * LDSW + SW * w + 32 * (p >> 1) + 8 * lk + 4 * (p & 1)]) = acc[p];
    __syncthreads();
    // every row's ahat, then (sender) every row's e: one array at a time
    f32x4 hn[NI], ev[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tr = 4 * w + RPI * i + ri;
      const f32x4 c = *reinterpret_cast<const f32x4*>(&S[tr * LDSW + lc]);
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if constexpr (SENDER) x = widen4<IN>(T.x[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        hn[i][t] = T.h[i][t] + c[t];
        if constexpr (SENDER) ev[i][t] = (x[t] - T.h[i][t]) - c[t];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = r0 + 4 * w + RPI * i + ri;
      if (row < rend && col_ok) store4(ahat + tb + (size_t)row * m, hn[i]);
    }
    if constexpr (SENDER) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = r0 + 4 * w + RPI * i + ri;
        if (row < rend && col_ok) store4(e + tb + (size_t)row * m, ev[i]);
      }
    }
  };

  Rows cur, nxt;
  load(rbeg, cur);
  int it = 0, r0 = rbeg;
  for (; r0 + 16 < rend; r0 += 16, ++it) {
    load(r0 + 16, nxt);
    apply(r0, it, cur);
    cur = nxt;
  }
  apply(r0, it, cur);
}

// Column width of the reconstruct blocks. 256 (1 KiB row runs) is faster on
// whole blocks (flux 57 x 1152 x 3072: 503 us against 534 us at rank 32); where
// the last 256-column block would be at most half used (m % 256 == 64 or 128),
// 128-column blocks waste less (video 30 x 4444 x 1920: 634 us against 667 us).
inline int rc_col_width(int m) {
  const int tail = m % 256;
  return (tail == 64 || tail == 128) ? 128 : 256;
}

// Grid of the reconstruct kernel: CW-column blocks x row chunks x tensors.
// Short chunks keep the blocks that run together on neighbouring rows and
// leave a short tail; the V operands are loaded once per block, which longer
// chunks amortise. Measured on the flux (k 32) and video (k 48) shapes: the
// sender is fastest at 32 / 48 rows (against 64 / 128: -4 % / -2 %), the
// receiver at 48 / 128 rows.
struct RcGrid {
  dim3 grid;
  int chunk_rows;
  int cw;
};
inline RcGrid rc_grid(int n, int m, int B, int k, bool sender) {
  const int chunk_rows = sender ? (k <= 32 ? 32 : 48) : (k <= 32 ? 48 : 128);
  const int cw = rc_col_width(m);
  return RcGrid{dim3((unsigned)((m + cw - 1) / cw), (unsigned)((n + chunk_rows - 1) / chunk_rows),
                     (unsigned)B),
                chunk_rows, cw};
}

// One reconstruct launch with the column width chosen at run time.
template <typename IN, bool SENDER, int K, int KP, bool BF16F>
void launch_recon(const RcGrid& g, hipStream_t s, const IN* a, float* e, const PeerSet& peers,
                  int batch, const Layout& L) {
  if (g.cw == 128)
    hipLaunchKernelGGL((lr_recon_kernel<IN, SENDER, K, KP, BF16F, 128>), g.grid, dim3(256), 0, s, a, e,
                       peers, batch, L, g.chunk_rows);
  else
    hipLaunchKernelGGL((lr_recon_kernel<IN, SENDER, K, KP, BF16F, 256>), g.grid, dim3(256), 0, s, a, e,
                       peers, batch, L, g.chunk_rows);
}

// ---------------------------------------------------------------- start matrices
// Q0t[b][j][c] = bf16(q0[b][c][j]) for j < kp, 0 for kp <= j < rank. One lane
// per (tensor, column); from the caller's fp32 q0, or drawn from the seed as
// the public header defines (SplitMix64 outputs, Box-Muller normals in fp64,
// rounded to fp32 and then to bf16).
__device__ __forceinline__ uint64_t sm64(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ double sm64_unit(uint64_t key, uint64_t i) {
  return ((double)(sm64(key, i) >> 11) + 0.5) * 0x1p-53;
}

__global__ __launch_bounds__(256) void lr_q0_kernel(const float* __restrict__ q0, uint64_t seed,
                                                    uint16_t* __restrict__ Q0t, int batch, int cols,
                                                    int kp, int rank) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * cols) return;
  const int b = (int)(idx / cols), c = (int)(idx % cols);
  const uint64_t key = sm64(sm64(sm64(seed, 7), (uint64_t)b), 0);
  uint16_t* dst = Q0t + (size_t)b * rank * cols;
  for (int j = 0; j < rank; ++j) {
    float v = 0.f;
    if (j < kp) {
      if (q0) {
        v = q0[((size_t)b * cols + c) * kp + j];
      } else {
        const uint64_t i = (uint64_t)c * kp + j, p = i >> 1;
        const double rad = sqrt(-2.0 * log(sm64_unit(key, 2 * p)));
        const double ang = 6.283185307179586476925286766559 * sm64_unit(key, 2 * p + 1);
        v = (float)((i & 1) ? rad * sin(ang) : rad * cos(ang));
      }
    }
    dst[g32(j, c, rank)] = (uint16_t)bf16_rne(v);
  }
}

hipError_t launch_lr_q0(const float* q0, uint64_t seed, uint16_t* Q0t, int batch, int cols, int kp,
                        int rank, hipStream_t s) {
  const int64_t n = (int64_t)batch * cols;
  hipLaunchKernelGGL(lr_q0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, q0, seed, Q0t,
                     batch, cols, kp, rank);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
namespace {

template <int K, int KP>
void cqr_pass(const LowRankWork& w, int n, int B, bool final_pass, hipStream_t s) {
  const int nt = (int)w.ntiles, rp = (int)w.rows_pad;
  hipLaunchKernelGGL((lr_gram_reduce_kernel<K>), dim3((K * K + 255) / 256, B), dim3(256), 0, s,
                     w.gpart, w.gsum, nt);
  hipLaunchKernelGGL((lr_chol_kernel<K, KP>), dim3(B), dim3(64), 0, s, w.gsum, w.linv, w.dead);
  if (final_pass)
    hipLaunchKernelGGL((lr_solve_kernel<K, false, true>), dim3(nt, B), dim3(256), 0, s, w.P, w.linv,
                       w.gpart, w.Pbt, w.amax, n, nt, rp);
  else
    hipLaunchKernelGGL((lr_solve_kernel<K, true, false>), dim3(nt, B), dim3(256), 0, s, w.P, w.linv,
                       w.gpart, w.Pbt, w.amax, n, nt, rp);
}

template <int K, int KP>
hipError_t lr_compress_k(bool bf16, const void* a, float* ahat, float* e, uint8_t* packed, int B,
                         const Layout& L, const LowRankWork& w, hipStream_t s) {
  const int n = (int)L.rows, m = (int)L.cols;
  const int nt = (int)w.ntiles, rp = (int)w.rows_pad;
  const dim3 tiles(nt, B);
  for (int it = 0; it < w.iters; ++it) {
    if (it == 0) {
      if (bf16)
        hipLaunchKernelGGL((lr_rq_kernel<uint16_t, true, K>), tiles, dim3(256), 0, s,
                           static_cast<const uint16_t*>(a), ahat, w.R, w.Q0t, w.P, w.gpart, w.amax,
                           n, m, nt);
      else
        hipLaunchKernelGGL((lr_rq_kernel<float, true, K>), tiles, dim3(256), 0, s,
                           static_cast<const float*>(a), ahat, w.R, w.Q0t, w.P, w.gpart, w.amax,
                           n, m, nt);
    } else {
      hipLaunchKernelGGL((lr_rq_kernel<uint16_t, false, K>), tiles, dim3(256), 0, s,
                         (const uint16_t*)nullptr, (const float*)nullptr, w.R, w.Qtb, w.P, w.gpart,
                         w.amax, n, m, nt);
    }
    cqr_pass<K, KP>(w, n, B, false, s);
    cqr_pass<K, KP>(w, n, B, true, s);
    const dim3 rtp_grid((m + kRtpCols - 1) / kRtpCols, B);
    if (it + 1 == w.iters)
      hipLaunchKernelGGL((lr_rtp_kernel<K, true>), rtp_grid, dim3(256 * kRtpHalves), 0, s, w.R, w.Pbt, w.Qt,
                         w.Qtb, w.amax, n, m, rp);
    else
      hipLaunchKernelGGL((lr_rtp_kernel<K, false>), rtp_grid, dim3(256 * kRtpHalves), 0, s, w.R, w.Pbt, w.Qt,
                         w.Qtb, w.amax, n, m, rp);
  }
  if (w.bf16_factors)
    hipLaunchKernelGGL((lr_bf16f_kernel<K, KP>), dim3((n + m + 255) / 256, B), dim3(256), 0, s, w.P,
                       w.Qt, packed, L);
  else
    hipLaunchKernelGGL((lr_int4_kernel<K, KP>), dim3((n + m + 255) / 256, B), dim3(256), 0, s, w.P,
                       w.Qt, w.amax, packed, L);
  PeerSet self{};
  self.packed[0] = packed;
  self.state[0] = ahat;
  self.count = 1;
  const RcGrid g = rc_grid(n, m, B, K, true);
  if (bf16 && w.bf16_factors)
    launch_recon<uint16_t, true, K, KP, true>(g, s, static_cast<const uint16_t*>(a), e, self, B, L);
  else if (bf16)
    launch_recon<uint16_t, true, K, KP, false>(g, s, static_cast<const uint16_t*>(a), e, self, B, L);
  else if (w.bf16_factors)
    launch_recon<float, true, K, KP, true>(g, s, static_cast<const float*>(a), e, self, B, L);
  else
    launch_recon<float, true, K, KP, false>(g, s, static_cast<const float*>(a), e, self, B, L);
  return hipGetLastError();
}

// Receiver: every peer's tensors in one launch (grid z = peer * batch + tensor),
// split into several launches only if that exceeds the grid's z limit.
template <int K, int KP>
hipError_t lr_decompress_k(const PeerSet& peers, int B, const Layout& L, const LowRankWork& w,
                           hipStream_t s) {
  const int n = (int)L.rows, m = (int)L.cols;
  RcGrid g = rc_grid(n, m, B, K, false);
  const int per_launch = B * peers.count <= 65535 ? peers.count : 1;
  for (int p0 = 0; p0 < peers.count; p0 += per_launch) {
    PeerSet sub{};
    sub.count = per_launch < peers.count - p0 ? per_launch : peers.count - p0;
    for (int q = 0; q < sub.count; ++q) {
      sub.packed[q] = peers.packed[p0 + q];
      sub.state[q] = peers.state[p0 + q];
    }
    g.grid.z = (unsigned)(B * sub.count);
    if (w.bf16_factors)
      launch_recon<float, false, K, KP, true>(g, s, nullptr, nullptr, sub, B, L);
    else
      launch_recon<float, false, K, KP, false>(g, s, nullptr, nullptr, sub, B, L);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lr_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, const LowRankWork& w,
                              hipStream_t s) {
  if (L.cols % 64) return hipErrorInvalidValue;
  switch (w.rank) {
    case 16:
      return w.pay_rank == 8 ? lr_compress_k<16, 8>(bf16_input, a, ahat, e, packed, batch, L, w, s)
                             : lr_compress_k<16, 16>(bf16_input, a, ahat, e, packed, batch, L, w, s);
    case 32: return lr_compress_k<32, 32>(bf16_input, a, ahat, e, packed, batch, L, w, s);
    case 48: return lr_compress_k<48, 48>(bf16_input, a, ahat, e, packed, batch, L, w, s);
    case 64: return lr_compress_k<64, 64>(bf16_input, a, ahat, e, packed, batch, L, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_lr_decompress(const PeerSet& peers, int batch, const Layout& L,
                                const LowRankWork& w, hipStream_t s) {
  if (L.cols % 64) return hipErrorInvalidValue;
  switch (w.rank) {
    case 16:
      return w.pay_rank == 8 ? lr_decompress_k<16, 8>(peers, batch, L, w, s)
                             : lr_decompress_k<16, 16>(peers, batch, L, w, s);
    case 32: return lr_decompress_k<32, 32>(peers, batch, L, w, s);
    case 48: return lr_decompress_k<48, 48>(peers, batch, L, w, s);
    case 64: return lr_decompress_k<64, 64>(peers, batch, L, w, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rc
