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
//   R = bf16(a_t - ahat)                                (fused into the 1st product)
//   repeat iters times:
//     P = R * bf16(Q)          bf16 MFMA, fp32 accumulate       [lr_rq_kernel]
//     P = CQR(CQR(P))          CholeskyQR2 of the n x k panel   [lr_chol_kernel, lr_solve_kernel]
//     Q = R^T * bf16(P)        bf16 MFMA via an LDS transpose   [lr_rtp_kernel]
//   U = P, V = Q; per-column absmax INT4                       [lr_int4_kernel]
//   c = Uq Vq^T (fp32 FMA chain, k ascending), e = r - c, ahat += c  [lr_recon_kernel]
// CQR(P): G = P^T P (fp32 MFMA on 64-row tiles, partials summed in tile order),
// G = L L^T (one wave, left-looking), P <- P L^{-T} (one lane per row). A pivot
// <= 2^-23 * max(trace G, k * FLT_MIN) marks a dead column, whose P column is
// zeroed, so zero or rank-deficient residuals never produce NaN.
//
// All MFMA operand layouts follow the gfx950 register layout of
// v_mfma_f32_16x16x32_bf16 (A: lane l holds A[l%16][8(l/16) .. +7], B: lane l
// holds B[8(l/16) .. +7][l%16], D: lane l holds D[4(l/16) + t][l%16]) and of
// v_mfma_f32_16x16x4_f32 (A[l%16][l/16], B[l/16][l%16], same D).
#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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
// Waves of the block share the tile pairs.
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

// ---------------------------------------------------------------- P = R * Q
// Block: 64 rows of one tensor; 4 waves split the K-steps (32 columns each,
// interleaved) and their partial products are summed through LDS in a fixed
// order. FROM_A: R is formed here from a_t and ahat and written out for the
// later passes.
template <typename IN, bool FROM_A, int K>
__global__ __launch_bounds__(256) void lr_rq_kernel(const IN* __restrict__ a,
                                                    const float* __restrict__ ahat,
                                                    uint16_t* __restrict__ R,
                                                    const uint16_t* __restrict__ Qtb,
                                                    float* __restrict__ P, float* __restrict__ gpart,
                                                    int n, int m, int ntiles) {
  constexpr int NT = K / 16;
  constexpr int LD = K + 1;
  __shared__ float red[2][kTile * LD];
  const int b = blockIdx.y, tile = blockIdx.x, row0 = tile * kTile;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const int nks = m / 32;
  const uint16_t* Qb = Qtb + (size_t)b * K * m;

  f32x4 acc[4][NT];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < NT; ++g) acc[f][g] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ks = w; ks < nks; ks += 4) {
    const int c0 = ks * 32 + lk * 8;
    u32x4 A[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int row = row0 + 16 * f + lr;
      const int rcl = row < n ? row : n - 1;
      const size_t off = ((size_t)b * n + rcl) * m + c0;
      if constexpr (FROM_A) {
        F8 x, h;
        load8<IN>(a + off, x);
        load8<float>(ahat + off, h);
        u32x4 v;
        v.x = bf16_rne(x.v[0] - h.v[0]) | (bf16_rne(x.v[1] - h.v[1]) << 16);
        v.y = bf16_rne(x.v[2] - h.v[2]) | (bf16_rne(x.v[3] - h.v[3]) << 16);
        v.z = bf16_rne(x.v[4] - h.v[4]) | (bf16_rne(x.v[5] - h.v[5]) << 16);
        v.w = bf16_rne(x.v[6] - h.v[6]) | (bf16_rne(x.v[7] - h.v[7]) << 16);
        if (row < n) *reinterpret_cast<u32x4*>(R + off) = v;
        A[f] = v;
      } else {
        A[f] = *reinterpret_cast<const u32x4*>(R + off);
      }
    }
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const u32x4 Bv = *reinterpret_cast<const u32x4*>(Qb + (size_t)(16 * g + lr) * m + c0);
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[f][g] = mfma_bf16(A[f], Bv, acc[f][g]);
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

// ---------------------------------------------------------------- Cholesky
// One block per tensor: sum the tile partials of G in tile order, then the
// left-looking Cholesky on one wave (lane i owns row i), with the dead-column
// rule. Output chol[K][K+1]: L (lower triangle; L[j][j] = 1 for dead j) and,
// in column K, 1.0 for dead columns.
template <int K>
__global__ __launch_bounds__(256) void lr_chol_kernel(const float* __restrict__ gpart,
                                                      float* __restrict__ chol, int ntiles) {
  constexpr int LD = K + 1;
  __shared__ float G[K * LD];
  __shared__ float L[K * LD];
  const int b = blockIdx.x;
  const float* gp = gpart + (size_t)b * ntiles * K * K;
  for (int idx = threadIdx.x; idx < K * K; idx += blockDim.x) {
    const int i = idx / K, j = idx % K;
    if (i > j) continue;
    float s = 0.f;
    for (int p = 0; p < ntiles; ++p) s += gp[(size_t)p * K * K + idx];
    G[i * LD + j] = s;
    G[j * LD + i] = s;
  }
  for (int idx = threadIdx.x; idx < K * LD; idx += blockDim.x) L[idx] = 0.f;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
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
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __builtin_amdgcn_wave_barrier();
    }
    if (lane < K) L[lane * LD + K] = ((dead >> lane) & 1) ? 1.f : 0.f;
  }
  __syncthreads();
  float* out = chol + (size_t)b * K * LD;
  for (int idx = threadIdx.x; idx < K * LD; idx += blockDim.x) out[idx] = L[idx];
}

// ---------------------------------------------------------------- P <- P L^-T
// One wave per 64-row tile, one lane per row: forward substitution x L^T = p.
// GRAM: also write the Gram partial of the solved tile (next CQR pass).
// FINAL: also write the bf16 transposed panel used by the R^T P product
// (rows n .. rows_pad-1 written as 0).
template <int K, bool GRAM, bool FINAL>
__global__ __launch_bounds__(64) void lr_solve_kernel(float* __restrict__ P,
                                                      const float* __restrict__ chol,
                                                      float* __restrict__ gpart,
                                                      uint16_t* __restrict__ Pbt, int n,
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
  if constexpr (FINAL) {
    if (row < rows_pad) {
      uint16_t* dst = Pbt + (size_t)b * K * rows_pad + row;
#pragma unroll
      for (int j = 0; j < K; ++j) dst[(size_t)j * rows_pad] = valid ? (uint16_t)bf16_rne(x[j]) : (uint16_t)0;
    }
  }
  if constexpr (GRAM) {
#pragma unroll
    for (int j = 0; j < K; ++j) T[lane * LD + j] = x[j];  // x = 0 for rows past n
    __syncthreads();
    tile_gram<K, LD>(T, gpart + ((size_t)b * ntiles + tile) * K * K, 1);
  }
}

// ---------------------------------------------------------------- Q = R^T P
// Block: 64 columns of one tensor, all rows; each wave owns 16 columns. Per
// step of 32 rows the R tile [32 x 64] is staged through LDS (double buffered)
// and read back column-wise to form the MFMA A operand (A[c][i] = R[i][c]).
// Output written transposed: Qt[j][c] (fp32, for V) and Qtb (bf16, next product).
constexpr int kRtpCols = 64;
constexpr int kRtpLd = kRtpCols + 8;  // bf16 elements per LDS row

template <int K>
__global__ __launch_bounds__(256) void lr_rtp_kernel(const uint16_t* __restrict__ R,
                                                     const uint16_t* __restrict__ Pbt,
                                                     float* __restrict__ Qt,
                                                     uint16_t* __restrict__ Qtb, int n, int m,
                                                     int rows_pad) {
  constexpr int NT = K / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sR[2][32 * kRtpLd];
  const int b = blockIdx.y, c0 = blockIdx.x * kRtpCols;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const int ld_row = threadIdx.x >> 3, ld_col = (threadIdx.x & 7) * 8;
  const uint16_t* Rb = R + (size_t)b * n * m;
  const uint16_t* Pb = Pbt + (size_t)b * K * rows_pad;

  auto gload = [&](int i0) {
    int row = i0 + ld_row;
    row = row < n ? row : n - 1;
    return *reinterpret_cast<const u32x4*>(Rb + (size_t)row * m + c0 + ld_col);
  };
  f32x4 acc[NT];
#pragma unroll
  for (int g = 0; g < NT; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 next = gload(0);
  int buf = 0;
  for (int i0 = 0; i0 < rows_pad; i0 += 32, buf ^= 1) {
    *reinterpret_cast<u32x4*>(&sR[buf][ld_row * kRtpLd + ld_col]) = next;
    __syncthreads();
    if (i0 + 32 < rows_pad) next = gload(i0 + 32);
    const uint16_t* base = &sR[buf][(8 * lk) * kRtpLd + 16 * w + lr];
    u32x4 A;
    A.x = (uint32_t)base[0 * kRtpLd] | ((uint32_t)base[1 * kRtpLd] << 16);
    A.y = (uint32_t)base[2 * kRtpLd] | ((uint32_t)base[3 * kRtpLd] << 16);
    A.z = (uint32_t)base[4 * kRtpLd] | ((uint32_t)base[5 * kRtpLd] << 16);
    A.w = (uint32_t)base[6 * kRtpLd] | ((uint32_t)base[7 * kRtpLd] << 16);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const u32x4 Bv = *reinterpret_cast<const u32x4*>(Pb + (size_t)(16 * g + lr) * rows_pad + i0 + 8 * lk);
      acc[g] = mfma_bf16(A, Bv, acc[g]);
    }
  }
  // D[c][j]: lane holds c = c0 + 16w + 4lk + t, j = 16g + lr
  const int c = c0 + 16 * w + 4 * lk;
#pragma unroll
  for (int g = 0; g < NT; ++g) {
    const size_t o = ((size_t)b * K + 16 * g + lr) * m + c;
    *reinterpret_cast<f32x4*>(Qt + o) = acc[g];
    uint2 hb;
    hb.x = bf16_rne(acc[g][0]) | (bf16_rne(acc[g][1]) << 16);
    hb.y = bf16_rne(acc[g][2]) | (bf16_rne(acc[g][3]) << 16);
    *reinterpret_cast<uint2*>(Qtb + o) = hb;
  }
}

// ---------------------------------------------------------------- INT4 factors
// Block x = 0: U from P [n][K]; x = 1: V from Qt [K][m]. Per column j:
// s_j = absmax_j / 7, q = clamp(rint_even(x / s_j), -7, 7) (0 when s_j = 0),
// packed row-major, element t in nibble t (even t low), two's complement.
template <int K>
__global__ __launch_bounds__(256) void lr_int4_kernel(const float* __restrict__ P,
                                                      const float* __restrict__ Qt,
                                                      uint8_t* __restrict__ packed, Layout L) {
  __shared__ float red[4][K];
  __shared__ float scale[K];
  const int b = blockIdx.y;
  const bool isV = blockIdx.x == 1;
  const int n = (int)L.rows, m = (int)L.cols;
  const int rows = isV ? m : n;
  const float* Pb = P + (size_t)b * n * K;
  const float* Qb = Qt + (size_t)b * K * m;
  uint8_t* pk = packed + (size_t)b * L.tstride;
  uint8_t* nib = pk + (isV ? L.sec_off[1] : L.sec_off[0]);
  float* sc = reinterpret_cast<float*>(pk + (isV ? L.sec_off[3] : L.sec_off[2]));
  auto val = [&](int i, int j) { return isV ? Qb[(size_t)j * m + i] : Pb[(size_t)i * K + j]; };

  float amax[K];
#pragma unroll
  for (int j = 0; j < K; ++j) amax[j] = 0.f;
  for (int i = threadIdx.x; i < rows; i += blockDim.x)
#pragma unroll
    for (int j = 0; j < K; ++j) amax[j] = fmaxf(amax[j], fabsf(val(i, j)));
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float v = amax[j];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[w][j] = v;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int j = threadIdx.x;
    const float am = fmaxf(fmaxf(red[0][j], red[1][j]), fmaxf(red[2][j], red[3][j]));
    const float s = am / 7.0f;
    scale[j] = s;
    sc[j] = s;
  }
  // zero the section padding of this half (U: gaps after sections 0 and 2; V: 1 and 3)
  for (int sidx = isV ? 1 : 0; sidx < 4; sidx += 2) {
    const int64_t start = L.sec_off[sidx] + L.sec_len[sidx];
    const int64_t end = (sidx + 1 < L.nsec) ? L.sec_off[sidx + 1] : L.tstride;
    for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) pk[i] = 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rows; i += blockDim.x) {
    uint32_t words[K / 8];
#pragma unroll
    for (int q = 0; q < K / 8; ++q) words[q] = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float s = scale[j];
      float qv = 0.f;
      if (s > 0.f) qv = fminf(fmaxf(rintf(val(i, j) / s), -7.f), 7.f);
      const uint32_t code = (uint32_t)((int)qv) & 0xFu;
      words[j / 8] |= code << (4 * (j % 8));
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(nib + (size_t)i * (K / 2));
#pragma unroll
    for (int q = 0; q < K / 8; ++q) dst[q] = words[q];
  }
}

// ---------------------------------------------------------------- reconstruct
// c = Uq Vq^T on a 32 x 128 tile: the INT4 factors of the tile are decoded into
// LDS (Us[32][K], Vt[K][128]), each lane accumulates 2 rows x 8 columns as an
// fp32 FMA chain over k ascending. SENDER: r = a - ahat, e = r - c, ahat += c.
// Receiver: ahat += c. Both run this same code, so both get the same c.
constexpr int kRcRows = 32, kRcCols = 128;

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
  __shared__ float Us[kRcRows][K];
  __shared__ __attribute__((aligned(16))) float Vt[K][kRcCols];
  const int b = blockIdx.y;
  const int n = (int)L.rows, m = (int)L.cols;
  const int ncol_tiles = (m + kRcCols - 1) / kRcCols;
  const int r0 = (blockIdx.x / ncol_tiles) * kRcRows, c0 = (blockIdx.x % ncol_tiles) * kRcCols;
  const uint8_t* pk = packed + (size_t)b * L.tstride;
  const uint8_t* un = pk + L.sec_off[0];
  const uint8_t* vn = pk + L.sec_off[1];
  const float* su = reinterpret_cast<const float*>(pk + L.sec_off[2]);
  const float* sv = reinterpret_cast<const float*>(pk + L.sec_off[3]);
  for (int idx = threadIdx.x; idx < kRcRows * K; idx += blockDim.x) {
    const int r = idx / K, j = idx % K;
    const int row = r0 + r;
    Us[r][j] = row < n ? int4_at(un, (int64_t)row * K + j) * su[j] : 0.f;
  }
  for (int idx = threadIdx.x; idx < kRcCols * K; idx += blockDim.x) {
    const int j = idx / kRcCols, c = idx % kRcCols;
    const int col = c0 + c;
    Vt[j][c] = col < m ? int4_at(vn, (int64_t)col * K + j) * sv[j] : 0.f;
  }
  __syncthreads();
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  float acc[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[s][i] = 0.f;
#pragma unroll 4
  for (int j = 0; j < K; ++j) {
    const float u0 = Us[ty][j], u1 = Us[ty + 16][j];
    const f32x4 va = *reinterpret_cast<const f32x4*>(&Vt[j][8 * tx]);
    const f32x4 vb = *reinterpret_cast<const f32x4*>(&Vt[j][8 * tx + 4]);
    const float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[0][i] = fmaf(u0, v[i], acc[0][i]);
      acc[1][i] = fmaf(u1, v[i], acc[1][i]);
    }
  }
  const int col = c0 + 8 * tx;
  if (col >= m) return;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int row = r0 + ty + 16 * s;
    if (row >= n) continue;
    const size_t off = ((size_t)b * n + row) * m + col;
    F8 h;
    load8<float>(ahat + off, h);
    if constexpr (SENDER) {
      F8 x, ev;
      load8<IN>(a + off, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = x.v[i] - h.v[i];
        ev.v[i] = r - acc[s][i];
        h.v[i] = h.v[i] + acc[s][i];
      }
      store8_nt(e + off, ev);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) h.v[i] = h.v[i] + acc[s][i];
    }
    store8(ahat + off, h);
  }
}

// ---------------------------------------------------------------- launchers
namespace {

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
                           static_cast<const uint16_t*>(a), ahat, w.R, w.Q0t, w.P, w.gpart, n, m, nt);
      else
        hipLaunchKernelGGL((lr_rq_kernel<float, true, K>), tiles, dim3(256), 0, s,
                           static_cast<const float*>(a), ahat, w.R, w.Q0t, w.P, w.gpart, n, m, nt);
    } else {
      hipLaunchKernelGGL((lr_rq_kernel<uint16_t, false, K>), tiles, dim3(256), 0, s,
                         (const uint16_t*)nullptr, (const float*)nullptr, w.R, w.Qtb, w.P, w.gpart,
                         n, m, nt);
    }
    hipLaunchKernelGGL((lr_chol_kernel<K>), dim3(B), dim3(256), 0, s, w.gpart, w.chol, nt);
    hipLaunchKernelGGL((lr_solve_kernel<K, true, false>), tiles, dim3(64), 0, s, w.P, w.chol,
                       w.gpart, w.Pbt, n, nt, rp);
    hipLaunchKernelGGL((lr_chol_kernel<K>), dim3(B), dim3(256), 0, s, w.gpart, w.chol, nt);
    hipLaunchKernelGGL((lr_solve_kernel<K, false, true>), tiles, dim3(64), 0, s, w.P, w.chol,
                       w.gpart, w.Pbt, n, nt, rp);
    hipLaunchKernelGGL((lr_rtp_kernel<K>), dim3(m / kRtpCols, B), dim3(256), 0, s, w.R, w.Pbt,
                       w.Qt, w.Qtb, n, m, rp);
  }
  hipLaunchKernelGGL((lr_int4_kernel<K>), dim3(2, B), dim3(256), 0, s, w.P, w.Qt, packed, L);
  const int ntile_rc = ((n + kRcRows - 1) / kRcRows) * ((m + kRcCols - 1) / kRcCols);
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
  const int ntile_rc = ((n + kRcRows - 1) / kRcRows) * ((m + kRcCols - 1) / kRcCols);
  hipLaunchKernelGGL((lr_recon_kernel<float, false, K>), dim3(ntile_rc, B), dim3(256), 0, s,
                     (const float*)nullptr, ahat, (float*)nullptr, packed, L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lr_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, const LowRankWork& w,
                              hipStream_t s) {
  if (L.cols % kRtpCols) return hipErrorInvalidValue;
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
  switch (rank) {
    case 16: return lr_decompress_k<16>(packed, ahat, batch, L, s);
    case 32: return lr_decompress_k<32>(packed, ahat, batch, L, s);
    case 48: return lr_decompress_k<48>(packed, ahat, batch, L, s);
    case 64: return lr_decompress_k<64>(packed, ahat, batch, L, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rc
