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
//     Q = R^T * bf16(P)      bf16 MFMA, R transposed through LDS   [lr_rtp_kernel, lr_qfinish_kernel]
//   U = P, V = Q; per-column absmax INT4                          [lr_int4_kernel]
//   c = Uq Vq^T (fp32 MFMA), e = r - c, ahat += c                 [lr_recon_kernel]
// CQR(P): G = P^T P (fp32 MFMA on 64-row tiles, tile partials summed in tile
// order), G = L L^T (one wave, left-looking), P <- P L^{-T} (one lane per row).
// A pivot <= 2^-23 * max(trace G, k * FLT_MIN) marks a dead column, whose P
// column is zeroed, so zero or rank-deficient residuals never produce NaN.
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

#include "device_common.hpp"
#include "launch.hpp"

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
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kTile / 4; ++s) {
        const float* row = T + (4 * s + lk) * LD;
        acc = mfma_f32(row[16 * ta + lr], row[16 * tb + lr], acc);
      }
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
// Block: 64 rows of one tensor (4 row fragments of 16); the 4 waves split the
// 64-column K-steps (interleaved) and their products are summed through LDS
// in a fixed order. In a K-step lane group g = l/16 owns columns
// [64 ks + 16 g, +16): one 32-byte bf16 run that feeds two MFMAs (its first
// and second 8 columns), so every row is read as whole 128-byte lines.
// FROM_A: R is formed here from a_t and ahat and written out for later passes.
// Block (0, b) clears the tensor's INT4 absmax slots, which the last solve and
// the last Q sum of the iteration fill.
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
  __shared__ float red[2][kTile * LD];
  const int b = blockIdx.y, tile = blockIdx.x, row0 = tile * kTile;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const int nks = m / 64;
  const uint16_t* Qb = Qtb + (size_t)b * K * m;
  if (tile == 0 && threadIdx.x < 2 * K) amax[(size_t)b * 2 * K + threadIdx.x] = 0u;

  f32x4 acc[4][NT];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < NT; ++g) acc[f][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ks = w; ks < nks; ks += 4) {
    const int c0 = ks * 64 + lk * 16;
    u32x4 A0[4], A1[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int row = row0 + 16 * f + lr;
      const int rcl = row < n ? row : n - 1;
      const size_t off = ((size_t)b * n + rcl) * m + c0;
      if constexpr (FROM_A) {
        F8 x0, x1, h0, h1;
        load8<IN>(a + off, x0);
        load8<IN>(a + off + 8, x1);
        load8<float>(ahat + off, h0);
        load8<float>(ahat + off + 8, h1);
        A0[f] = pack_r(x0, h0);
        A1[f] = pack_r(x1, h1);
        if (row < n) {
          reinterpret_cast<u32x4*>(R + off)[0] = A0[f];
          reinterpret_cast<u32x4*>(R + off)[1] = A1[f];
        }
      } else {
        A0[f] = reinterpret_cast<const u32x4*>(R + off)[0];
        A1[f] = reinterpret_cast<const u32x4*>(R + off)[1];
      }
    }
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const u32x4* q = reinterpret_cast<const u32x4*>(Qb + (size_t)(16 * g + lr) * m + c0);
      const u32x4 B0 = q[0], B1 = q[1];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        acc[f][g] = mfma_bf16(A0[f], B0, acc[f][g]);
        acc[f][g] = mfma_bf16(A1[f], B1, acc[f][g]);
      }
    }
  }

  // (w0 + w2) + (w1 + w3), rows past n zeroed, tile kept in red[1]
  auto put = [&](float* dst) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < NT; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) dst[(16 * f + 4 * lk + t) * LD + 16 * g + lr] = acc[f][g][t];
  };
  auto add = [&](const float* src) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < NT; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[f][g][t] += src[(16 * f + 4 * lk + t) * LD + 16 * g + lr];
  };
  if (w >= 2) put(red[w - 2]);
  __syncthreads();
  if (w < 2) add(red[w]);
  __syncthreads();
  if (w == 1) put(red[0]);
  __syncthreads();
  if (w == 0) {
    add(red[0]);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (row0 + 16 * f + 4 * lk + t >= n)
#pragma unroll
          for (int g = 0; g < NT; ++g) acc[f][g][t] = 0.f;
    put(red[1]);
  }
  __syncthreads();
  const float* T = red[1];
  for (int idx = threadIdx.x; idx < kTile * K; idx += blockDim.x) {
    const int r = idx / K, j = idx % K;
    if (row0 + r < n) P[((size_t)b * n + row0 + r) * K + j] = T[r * LD + j];
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
  for (; p + 4 <= ntiles; p += 4)
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += gp[(size_t)(p + q) * K * K];
  for (int q = 0; p < ntiles; ++p, ++q) s[q] += gp[(size_t)p * K * K];
  gsum[(size_t)b * K * K + idx] = (s[0] + s[1]) + (s[2] + s[3]);
}

// ---------------------------------------------------------------- Cholesky
// One wave per tensor: left-looking Cholesky of G (upper triangle of gsum),
// lane i owns row i, with the dead-column rule. Output chol[K][K+1]: L (lower
// triangle; L[j][j] = 1 for dead j) and, in column K, 1.0 for dead columns.
template <int K>
__global__ __launch_bounds__(64) void lr_chol_kernel(const float* __restrict__ gsum,
                                                     float* __restrict__ chol) {
  constexpr int LD = K + 1;
  __shared__ float G[K * LD];
  __shared__ float L[K * LD];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float* gs = gsum + (size_t)b * K * K;
  for (int idx = lane; idx < K * K; idx += 64) {
    const int i = idx / K, j = idx % K;
    G[i * LD + j] = gs[i <= j ? idx : j * K + i];
  }
  for (int idx = lane; idx < K * LD; idx += 64) L[idx] = 0.f;
  __syncthreads();
  float tr = lane < K ? G[lane * LD + lane] : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tr += __shfl_xor(tr, o);
  const float tol = ldexpf(fmaxf(tr, (float)K * FLT_MIN), -23);
  uint64_t dead = 0;
  for (int j = 0; j < K; ++j) {
    float s = 0.f;
    if (lane >= j && lane < K) {
      s = G[lane * LD + j];
      for (int p = 0; p < j; ++p) s -= L[lane * LD + p] * L[j * LD + p];
    }
    const float piv = __shfl(s, j);
    const bool dj = !(piv > tol);
    const float ljj = dj ? 1.0f : sqrtf(piv);
    if (lane == j) L[j * LD + j] = ljj;
    if (lane > j && lane < K) L[lane * LD + j] = dj ? 0.f : s / ljj;
    if (dj) dead |= (uint64_t)1 << j;
    __syncthreads();
  }
  if (lane < K) L[lane * LD + K] = ((dead >> lane) & 1) ? 1.f : 0.f;
  __syncthreads();
  float* out = chol + (size_t)b * K * LD;
  for (int idx = lane; idx < K * LD; idx += 64) out[idx] = L[idx];
}

// ---------------------------------------------------------------- P <- P L^-T
// One wave per 64-row tile, one lane per row: forward substitution x L^T = p.
// GRAM: also write the Gram partial of the solved tile (next CQR pass).
// FINAL: also write the bf16 transposed panel used by the R^T P product
// (rows n .. rows_pad-1 written as 0) and fold the column absmax of the tile
// into amax[b][0][*] (the INT4 scales of U).
template <int K, bool GRAM, bool FINAL>
__global__ __launch_bounds__(64) void lr_solve_kernel(float* __restrict__ P,
                                                      const float* __restrict__ chol,
                                                      float* __restrict__ gpart,
                                                      uint16_t* __restrict__ Pbt,
                                                      uint32_t* __restrict__ amax, int n,
                                                      int ntiles, int rows_pad) {
  constexpr int LD = K + 1;
  __shared__ float Ls[K * LD];
  __shared__ float T[kTile * LD];
  const int b = blockIdx.y, tile = blockIdx.x;
  const int lane = threadIdx.x;
  const float* src = chol + (size_t)b * K * LD;
  for (int idx = lane; idx < K * LD; idx += 64) Ls[idx] = src[idx];
  __syncthreads();
  const int row = tile * kTile + lane;
  const bool valid = row < n;
  float x[K];
  float* prow = P + ((size_t)b * n + (valid ? row : 0)) * K;
#pragma unroll
  for (int j = 0; j < K; j += 4) {
    const f32x4 v = valid ? *reinterpret_cast<const f32x4*>(prow + j) : f32x4{0.f, 0.f, 0.f, 0.f};
    x[j] = v.x; x[j + 1] = v.y; x[j + 2] = v.z; x[j + 3] = v.w;
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float s = x[j];
#pragma unroll
    for (int q = 0; q < j; ++q) s -= Ls[j * LD + q] * x[q];
    x[j] = (Ls[j * LD + K] != 0.f) ? 0.f : s / Ls[j * LD + j];
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < K; j += 4) *reinterpret_cast<f32x4*>(prow + j) = f32x4{x[j], x[j + 1], x[j + 2], x[j + 3]};
  }
#pragma unroll
  for (int j = 0; j < K; ++j) T[lane * LD + j] = x[j];  // x = 0 for rows past n
  __syncthreads();
  if constexpr (FINAL) {
    if (row < rows_pad) {
      uint16_t* dst = Pbt + (size_t)b * K * rows_pad + row;
#pragma unroll
      for (int j = 0; j < K; ++j) dst[(size_t)j * rows_pad] = valid ? (uint16_t)bf16_rne(x[j]) : (uint16_t)0;
    }
    if (lane < K) {
      float mx = 0.f;
      for (int r = 0; r < kTile; ++r) mx = fmaxf(mx, fabsf(T[r * LD + lane]));
      atomicMax(amax + (size_t)b * 2 * K + lane, __float_as_uint(mx));
    }
  }
  if constexpr (GRAM) tile_gram<K, LD>(T, gpart + ((size_t)b * ntiles + tile) * K * K, 1);
}

// ---------------------------------------------------------------- Q = R^T P
// Block: 64 columns x one row split of one tensor; each wave owns 16 columns.
// Per step of 32 rows the R tile [32 x 64] is staged through LDS (double
// buffered, one barrier per step) and read back transposed with
// ds_read_b64_tr_b16 to form the MFMA A operand A[c][i] = R[i][c]. The split's
// partial Q^T goes to qpart; lr_qfinish_kernel sums the splits.
constexpr int kRtpCols = 64;
constexpr int kRtpLd = kRtpCols + 8;  // bf16 elements per LDS row (144 B)

template <int K>
__global__ __launch_bounds__(256) void lr_rtp_kernel(const uint16_t* __restrict__ R,
                                                     const uint16_t* __restrict__ Pbt,
                                                     float* __restrict__ qpart, int n, int m,
                                                     int rows_pad, int nsplit, int split_rows) {
  constexpr int NT = K / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sR[2][32 * kRtpLd];
  const int b = blockIdx.z, split = blockIdx.y, c0 = blockIdx.x * kRtpCols;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const int ld_row = threadIdx.x >> 3, ld_col = (threadIdx.x & 7) * 8;
  const int i_begin = split * split_rows;
  const int i_end = min(rows_pad, i_begin + split_rows);
  const uint16_t* Rb = R + (size_t)b * n * m;
  const uint16_t* Pb = Pbt + (size_t)b * K * rows_pad;
  // transposed-read address of this lane inside a staged tile: group lk,
  // row 8 lk + (lr / 4) (+4 for the second read), columns 16 w + 4 (lr % 4)
  const int tr_off = (8 * lk + (lr >> 2)) * kRtpLd + 16 * w + 4 * (lr & 3);

  auto gload = [&](int i0) {
    int row = i0 + ld_row;
    row = row < n ? row : n - 1;
    return *reinterpret_cast<const u32x4*>(Rb + (size_t)row * m + c0 + ld_col);
  };
  f32x4 acc[NT];
#pragma unroll
  for (int g = 0; g < NT; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 next = gload(i_begin);
  int buf = 0;
  for (int i0 = i_begin; i0 < i_end; i0 += 32, buf ^= 1) {
    *reinterpret_cast<u32x4*>(&sR[buf][ld_row * kRtpLd + ld_col]) = next;
    __syncthreads();
    if (i0 + 32 < i_end) next = gload(i0 + 32);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)&sR[buf][tr_off]);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)&sR[buf][tr_off + 4 * kRtpLd]);
    u32x4 A;
    A.x = (uint32_t)(uint16_t)lo.x | ((uint32_t)(uint16_t)lo.y << 16);
    A.y = (uint32_t)(uint16_t)lo.z | ((uint32_t)(uint16_t)lo.w << 16);
    A.z = (uint32_t)(uint16_t)hi.x | ((uint32_t)(uint16_t)hi.y << 16);
    A.w = (uint32_t)(uint16_t)hi.z | ((uint32_t)(uint16_t)hi.w << 16);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const u32x4 Bv = *reinterpret_cast<const u32x4*>(Pb + (size_t)(16 * g + lr) * rows_pad + i0 + 8 * lk);
      acc[g] = mfma_bf16(A, Bv, acc[g]);
    }
  }
  // D[c][j]: lane holds c = c0 + 16w + 4lk + t, j = 16g + lr
  const int c = c0 + 16 * w + 4 * lk;
  float* qp = qpart + ((size_t)b * nsplit + split) * K * m;
#pragma unroll
  for (int g = 0; g < NT; ++g) *reinterpret_cast<f32x4*>(qp + (size_t)(16 * g + lr) * m + c) = acc[g];
}

// Sum the row splits in split order: Qt (fp32, V of the factorisation), Qtb
// (bf16 operand of the next product), and the column absmax of V folded into
// amax[b][1][j]. Block: one j, 1024 columns (4 per lane).
template <int K>
__global__ __launch_bounds__(256) void lr_qfinish_kernel(const float* __restrict__ qpart,
                                                         float* __restrict__ Qt,
                                                         uint16_t* __restrict__ Qtb,
                                                         uint32_t* __restrict__ amax, int m,
                                                         int nsplit) {
  const int b = blockIdx.z, j = blockIdx.x;
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  float mx = 0.f;
  if (c < m) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nsplit; ++sp)
      s += *reinterpret_cast<const f32x4*>(qpart + (((size_t)b * nsplit + sp) * K + j) * m + c);
    const size_t o = ((size_t)b * K + j) * m + c;
    *reinterpret_cast<f32x4*>(Qt + o) = s;
    uint2 hb;
    hb.x = bf16_rne(s.x) | (bf16_rne(s.y) << 16);
    hb.y = bf16_rne(s.z) | (bf16_rne(s.w) << 16);
    *reinterpret_cast<uint2*>(Qtb + o) = hb;
    mx = fmaxf(fmaxf(fabsf(s.x), fabsf(s.y)), fmaxf(fabsf(s.z), fabsf(s.w)));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) atomicMax(amax + ((size_t)b * 2 + 1) * K + j, __float_as_uint(mx));
}

// ---------------------------------------------------------------- INT4 factors
// One lane per factor row: rows 0..n-1 are U (= P, [n][K]), rows n..n+m-1 are V
// (= Q, stored as Qt [K][m]). Per column j: s_j = absmax_j / 7,
// q = clamp(rint_even(x / s_j), -7, 7) (0 when s_j = 0), packed row-major,
// element t in nibble t (even t low), two's complement. Block 0 writes the
// scale sections and zeroes the section padding.
template <int K>
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
    if (threadIdx.x < K) su[threadIdx.x] = sc[threadIdx.x];
    else if (threadIdx.x < 2 * K) sv[threadIdx.x - K] = sc[threadIdx.x];
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
  const float* src = isV ? Qt + (size_t)b * K * m + i : P + ((size_t)b * n + i) * K;
  const size_t stride = isV ? (size_t)m : 1;
  uint32_t words[K / 8];
#pragma unroll
  for (int q = 0; q < K / 8; ++q) words[q] = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float qv = 0.f;
    if (s[j] > 0.f) qv = fminf(fmaxf(rintf(src[j * stride] / s[j]), -7.f), 7.f);
    words[j / 8] |= ((uint32_t)((int)qv) & 0xFu) << (4 * (j % 8));
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(pk + (isV ? L.sec_off[1] : L.sec_off[0]) + (size_t)i * (K / 2));
#pragma unroll
  for (int q = 0; q < K / 8; ++q) dst[q] = words[q];
}

// ---------------------------------------------------------------- reconstruct
// c = Uq Vq^T on a 64 x 64 tile with fp32 MFMA. The INT4 factors of the tile
// are decoded into LDS (Us[64][K], Vs[64][K]); wave w computes rows 16w..16w+15
// as c^T = Vq Uq^T, so each lane ends with 8 consecutive columns of one row in
// each half of the tile (the MFMA M index is mapped to columns so that the two
// 16-column MFMA tiles of a half interleave in groups of 4).
// SENDER: r = a - ahat, e = r - c, ahat += c. Receiver: ahat += c. Both run
// this same code, so both get the same c bit for bit.
constexpr int kRc = 64;

__device__ __forceinline__ float int4_at(const uint8_t* nib, int64_t t) {
  const uint32_t byte = nib[t >> 1];
  const int v = (t & 1) ? (int)(byte >> 4) : (int)(byte & 15u);
  return (float)(v >= 8 ? v - 16 : v);
}

template <typename IN, bool SENDER, int K>
__global__ __launch_bounds__(256) void lr_recon_kernel(const IN* __restrict__ a,
                                                       float* __restrict__ ahat,
                                                       float* __restrict__ e,
                                                       const uint8_t* __restrict__ packed,
                                                       Layout L) {
  constexpr int LD = K + 1;
  __shared__ float Us[kRc * LD];
  __shared__ float Vs[kRc * LD];
  const int b = blockIdx.y;
  const int n = (int)L.rows, m = (int)L.cols;
  const int ncol_tiles = m / kRc;
  const int r0 = (blockIdx.x / ncol_tiles) * kRc, c0 = (blockIdx.x % ncol_tiles) * kRc;
  const uint8_t* pk = packed + (size_t)b * L.tstride;
  const uint8_t* un = pk + L.sec_off[0];
  const uint8_t* vn = pk + L.sec_off[1];
  const float* su = reinterpret_cast<const float*>(pk + L.sec_off[2]);
  const float* sv = reinterpret_cast<const float*>(pk + L.sec_off[3]);
  for (int idx = threadIdx.x; idx < kRc * K; idx += blockDim.x) {
    const int r = idx / K, j = idx % K;
    const int row = r0 + r;
    Us[r * LD + j] = row < n ? int4_at(un, (int64_t)row * K + j) * su[j] : 0.f;
    Vs[r * LD + j] = int4_at(vn, (int64_t)(c0 + r) * K + j) * sv[j];
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  f32x4 acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  // MFMA tile p covers local columns 32 (p/2) + 8 (m/4) + 4 (p%2) + m%4, m = 0..15
  int vcol[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) vcol[p] = 32 * (p >> 1) + 8 * (lr >> 2) + 4 * (p & 1) + (lr & 3);
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) {
    const float bu = Us[(16 * w + lr) * LD + k0 + lk];
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[p] = mfma_f32(Vs[vcol[p] * LD + k0 + lk], bu, acc[p]);
  }
  const int row = r0 + 16 * w + lr;
  if (row >= n) return;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int col = c0 + 32 * half + 8 * lk;
    const size_t off = ((size_t)b * n + row) * m + col;
    const f32x4 cl = acc[2 * half], ch = acc[2 * half + 1];
    const float c[8] = {cl.x, cl.y, cl.z, cl.w, ch.x, ch.y, ch.z, ch.w};
    F8 h;
    load8<float>(ahat + off, h);
    if constexpr (SENDER) {
      F8 x, ev;
      load8<IN>(a + off, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = x.v[i] - h.v[i];
        ev.v[i] = r - c[i];
        h.v[i] = h.v[i] + c[i];
      }
      store8_nt(e + off, ev);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) h.v[i] = h.v[i] + c[i];
    }
    store8(ahat + off, h);
  }
}

// ---------------------------------------------------------------- launchers
namespace {

template <int K>
void cqr_pass(const LowRankWork& w, int n, int B, bool final_pass, hipStream_t s) {
  const int nt = (int)w.ntiles, rp = (int)w.rows_pad;
  hipLaunchKernelGGL((lr_gram_reduce_kernel<K>), dim3((K * K + 255) / 256, B), dim3(256), 0, s,
                     w.gpart, w.gsum, nt);
  hipLaunchKernelGGL((lr_chol_kernel<K>), dim3(B), dim3(64), 0, s, w.gsum, w.chol);
  if (final_pass)
    hipLaunchKernelGGL((lr_solve_kernel<K, false, true>), dim3(nt, B), dim3(64), 0, s, w.P, w.chol,
                       w.gpart, w.Pbt, w.amax, n, nt, rp);
  else
    hipLaunchKernelGGL((lr_solve_kernel<K, true, false>), dim3(nt, B), dim3(64), 0, s, w.P, w.chol,
                       w.gpart, w.Pbt, w.amax, n, nt, rp);
}

template <int K>
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
    cqr_pass<K>(w, n, B, false, s);
    cqr_pass<K>(w, n, B, true, s);
    hipLaunchKernelGGL((lr_rtp_kernel<K>), dim3(m / kRtpCols, w.nsplit, B), dim3(256), 0, s, w.R,
                       w.Pbt, w.qpart, n, m, rp, w.nsplit, w.split_rows);
    hipLaunchKernelGGL((lr_qfinish_kernel<K>), dim3(K, (m + 1023) / 1024, B), dim3(256), 0, s,
                       w.qpart, w.Qt, w.Qtb, w.amax, m, w.nsplit);
  }
  hipLaunchKernelGGL((lr_int4_kernel<K>), dim3((n + m + 255) / 256, B), dim3(256), 0, s, w.P, w.Qt,
                     w.amax, packed, L);
  const int ntile_rc = ((n + kRc - 1) / kRc) * (m / kRc);
  if (bf16)
    hipLaunchKernelGGL((lr_recon_kernel<uint16_t, true, K>), dim3(ntile_rc, B), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a), ahat, e, (const uint8_t*)packed, L);
  else
    hipLaunchKernelGGL((lr_recon_kernel<float, true, K>), dim3(ntile_rc, B), dim3(256), 0, s,
                       static_cast<const float*>(a), ahat, e, (const uint8_t*)packed, L);
  return hipGetLastError();
}

template <int K>
hipError_t lr_decompress_k(const uint8_t* packed, float* ahat, int B, const Layout& L, hipStream_t s) {
  const int n = (int)L.rows, m = (int)L.cols;
  const int ntile_rc = ((n + kRc - 1) / kRc) * (m / kRc);
  hipLaunchKernelGGL((lr_recon_kernel<float, false, K>), dim3(ntile_rc, B), dim3(256), 0, s,
                     (const float*)nullptr, ahat, (float*)nullptr, packed, L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lr_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, const LowRankWork& w,
                              hipStream_t s) {
  if (L.cols % 64) return hipErrorInvalidValue;
  switch (w.rank) {
    case 16: return lr_compress_k<16>(bf16_input, a, ahat, e, packed, batch, L, w, s);
    case 32: return lr_compress_k<32>(bf16_input, a, ahat, e, packed, batch, L, w, s);
    case 48: return lr_compress_k<48>(bf16_input, a, ahat, e, packed, batch, L, w, s);
    case 64: return lr_compress_k<64>(bf16_input, a, ahat, e, packed, batch, L, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_lr_decompress(const uint8_t* packed, float* ahat, int batch, const Layout& L,
                                int rank, hipStream_t s) {
  if (L.cols % 64) return hipErrorInvalidValue;
  switch (rank) {
    case 16: return lr_decompress_k<16>(packed, ahat, batch, L, s);
    case 32: return lr_decompress_k<32>(packed, ahat, batch, L, s);
    case 48: return lr_decompress_k<48>(packed, ahat, batch, L, s);
    case 64: return lr_decompress_k<64>(packed, ahat, batch, L, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rc
