// Device-memory layout helpers of the low-rank products, shared by their
// kernels and by the reference probes that read R in the products' patterns.
#pragma once

#include <stddef.h>

#include <hip/hip_runtime.h>

namespace rc {

// The device hands workgroup L (linear over the grid, x fastest) to XCD L % 8,
// and each XCD has its own L2. This returns a logical index for L such that
// every XCD runs one contiguous range of logical indices, so logical neighbours
// (the blocks of one tensor, which read the same small operand) share an L2.
// A bijection on [0, N): XCD x holds q + (x < r) blocks, q = N / 8, r = N % 8.
__device__ __forceinline__ int xcd_contiguous(int L, int N) {
  const int x = L & 7, i = L >> 3, q = N >> 3, r = N & 7;
  return x * q + min(x, r) + i;
}

// The bf16 operands of the products -- Q^T (start matrix and later iterations)
// and P^T -- are [K][cols] matrices stored as 32-column groups: group c/32
// holds its K rows of 32 consecutive columns contiguously (K x 64 bytes). A
// step of either product reads one or four whole groups, so its operand loads
// are contiguous runs instead of K separate 64-byte pieces.
__device__ __forceinline__ size_t g32(int j, int c, int K) {
  return ((size_t)(c >> 5) * K + j) * 32 + (c & 31);
}

// R, the bf16 residual the products share, lives in the library's own
// workspace in 64 x 128 tiles, each a contiguous 16 KiB row-major block (one
// step of one band of the R*Q pass; its halves are the 32-row steps of the
// R^T*P pass). Tiles are ordered column chunk first, then tensor, then band:
// the blocks of the R*Q passes all work on the same column chunk at the same
// time, so together they write (and read) one contiguous region per step
// instead of a thousand scattered ones. The order is over the tensors of one
// launch (its grid), so a launch over a sub-batch uses its own slice of R.
__device__ __forceinline__ size_t r_index(int b, int row, int col, int batch, int bands) {
  return (((size_t)(col >> 7) * batch + b) * bands + (row >> 6)) * 8192 + (size_t)((row & 63) << 7) +
         (col & 127);
}

}  // namespace rc
