// HBM reference kernels for the roofline: the access patterns of the path's
// streaming kernels with trivial arithmetic, so a measurement shows what this
// device's HBM delivers for each pattern (the practical ceiling next to the
// 8 TB/s peak). Diagnostics only; nothing in the compression path calls them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/librescomp_diag.h"
#include "device_common.hpp"
#include "launch.hpp"
#include "lr_layout.hpp"

namespace rc {
namespace {

constexpr int kProbeBlock = 256;

__global__ __launch_bounds__(kProbeBlock) void probe_copy(const f32x4* __restrict__ a, f32x4* __restrict__ b,
                                                          int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
  if (i < n4) b[i] = a[i];
}

__global__ __launch_bounds__(kProbeBlock) void probe_read(const f32x4* __restrict__ a, float* __restrict__ out,
                                                          int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
  float s = 0.f;
  if (i < n4) {
    const f32x4 v = a[i];
    s = v.x + v.y + v.z + v.w;
  }
  if (s == 1234.5f) out[0] = s;  // keeps the loads; never true for the zero-filled buffer
}

__global__ __launch_bounds__(kProbeBlock) void probe_write(f32x4* __restrict__ b, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
  if (i < n4) b[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// sender-like: per 4 elements read 8 B bf16 + 16 B fp32, write 16 B + 16 B, in
// the lane layout of the sender kernels (4 consecutive elements per lane and
// chunk, kMixChunks chunks a block-width apart, all loads before the first
// store; lanes past the end reread chunk 0 and store nothing).
constexpr int kMixChunks = 4;
constexpr int kRmwChunks = 2;

__global__ __launch_bounds__(kProbeBlock) void probe_mix14(const uint16_t* __restrict__ a,
                                                           float* __restrict__ h, float* __restrict__ e,
                                                           int64_t n4) {
  f32x4 xs[kMixChunks], hs[kMixChunks];
#pragma unroll
  for (int j = 0; j < kMixChunks; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * kMixChunks + j) * kProbeBlock + threadIdx.x;
    const int64_t cc = c < n4 ? c : 0;
    xs[j] = load4<uint16_t>(a + cc * 4);
    hs[j] = load4<float>(h + cc * 4);
  }
  f32x4 evs[kMixChunks], hns[kMixChunks];
#pragma unroll
  for (int j = 0; j < kMixChunks; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = xs[j][i] - hs[j][i];
      evs[j][i] = r;
      hns[j][i] = hs[j][i] + 0.5f * r;
    }
  // the kernels' store order: every chunk's h, then every chunk's e
#pragma unroll
  for (int j = 0; j < kMixChunks; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * kMixChunks + j) * kProbeBlock + threadIdx.x;
    if (c < n4) store4(h + c * 4, hns[j]);
  }
#pragma unroll
  for (int j = 0; j < kMixChunks; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * kMixChunks + j) * kProbeBlock + threadIdx.x;
    if (c < n4) store4(e + c * 4, evs[j]);
  }
}

// receiver-like: read and write back fp32 in place, same lane layout
__global__ __launch_bounds__(kProbeBlock) void probe_rmw8(float* __restrict__ h, int64_t n4) {
  f32x4 hs[kRmwChunks];
#pragma unroll
  for (int j = 0; j < kRmwChunks; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * kRmwChunks + j) * kProbeBlock + threadIdx.x;
    hs[j] = load4<float>(h + (c < n4 ? c : 0) * 4);
  }
#pragma unroll
  for (int j = 0; j < kRmwChunks; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * kRmwChunks + j) * kProbeBlock + threadIdx.x;
    f32x4 hn;
#pragma unroll
    for (int i = 0; i < 4; ++i) hn[i] = hs[j][i] + 1.0f;
    if (c < n4) store4(h + c * 4, hn);
  }
}

// The low-rank products' reads of R alone (bf16, the products' tiled layout),
// with the products' grids, XCD mapping and per-lane access pattern, and no
// MFMA, LDS or epilogue: what HBM delivers for these patterns. `never` is 0
// from the host (the sink keeps the loads alive and is never written).
//
// R*Q pattern: one block per 64-row band of a tensor, walking the 128-column
// chunks; lane rows 16w + (lane >> 5) + 2i, 4 columns each; the next chunk is
// loaded while the current one is consumed; rows past n reread row n-1.
__global__ __launch_bounds__(256) void probe_r_rq(const uint16_t* __restrict__ R, int n, int m,
                                                  int ntiles, uint32_t* __restrict__ sink, int never) {
  const int lin = xcd_contiguous(blockIdx.x + ntiles * blockIdx.y, ntiles * gridDim.y);
  const int b = lin / ntiles, tile = lin % ntiles;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int srow = 16 * w + (lane >> 5), scol = 4 * (lane & 31);
  const size_t rbase = (size_t)(b * ntiles + tile) * 8192;
  const size_t cstride = (size_t)gridDim.y * ntiles * 8192;
  const int rlim = n - 1 - tile * 64;
  const int nchunks = (m + 127) / 128;
  auto load = [&](int cc, u32x2 (&v)[8]) {
    const int col = cc * 128 + scol < m ? scol : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = *reinterpret_cast<const u32x2*>(R + (size_t)cc * cstride + rbase +
                                             (size_t)(min(srow + 2 * i, rlim) * 128 + col));
  };
  u32x2 v[8];
  uint32_t acc = 0;
  load(0, v);
  for (int cc = 0; cc < nchunks; ++cc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i].x ^ v[i].y;
    load(min(cc + 1, nchunks - 1), v);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc ^= v[i].x ^ v[i].y;
  if (never) sink[threadIdx.x] = acc;
}

// R^T*P pattern: one 512-thread block per 128-column block of a tensor, two
// 256-thread halves over the two halves of the (padded) rows; per 32-row step
// each lane reads 16 bytes of two rows (16 lanes per 256-byte row piece), two
// steps in flight; rows past n reread row n-1, columns past m reread column
// block 0.
__global__ __launch_bounds__(512) void probe_r_rtp(const uint16_t* __restrict__ R, int n, int m,
                                                   int rows_pad, uint32_t* __restrict__ sink, int never) {
  const int nblk = gridDim.x * gridDim.y;
  const int lin = xcd_contiguous(blockIdx.x + gridDim.x * blockIdx.y, nblk);
  const int cb = lin % gridDim.x;
  const int b = gridDim.y - 1 - lin / gridDim.x;
  const int batch = gridDim.y, bands = rows_pad >> 6;
  const int tid = threadIdx.x & 255, half = threadIdx.x >> 8;
  const int ld_row = tid >> 4, ld_col = (tid & 15) * 8;
  const int col = cb * 128 + (cb * 128 + ld_col < m ? ld_col : 0);
  const int i_begin = half * (rows_pad / 2), i_end = i_begin + rows_pad / 2;
  auto load = [&](int i0, u32x4& r0, u32x4& r1) {
    i0 = min(i0, i_end - 32);
    r0 = *reinterpret_cast<const u32x4*>(R + r_index(b, min(i0 + ld_row, n - 1), col, batch, bands));
    r1 = *reinterpret_cast<const u32x4*>(R + r_index(b, min(i0 + ld_row + 16, n - 1), col, batch, bands));
  };
  u32x4 a0, a1, b0, b1;
  uint32_t acc = 0;
  load(i_begin, a0, a1);
  load(i_begin + 32, b0, b1);
  for (int i0 = i_begin; i0 < i_end; i0 += 32) {
    acc ^= a0.x ^ a0.y ^ a0.z ^ a0.w ^ a1.x ^ a1.y ^ a1.z ^ a1.w;
    a0 = b0;
    a1 = b1;
    load(i0 + 64, b0, b1);
  }
  if (never) sink[threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_r_probe(int pattern, const uint16_t* R, int n, int m, int batch, int ntiles, int rows_pad,
                          uint32_t* sink, hipStream_t s) {
  if (pattern == 0)
    hipLaunchKernelGGL(probe_r_rq, dim3(ntiles, batch), dim3(256), 0, s, R, n, m, ntiles, sink, 0);
  else if (pattern == 1)
    hipLaunchKernelGGL(probe_r_rtp, dim3((m + 127) / 128, batch), dim3(512), 0, s, R, n, m, rows_pad, sink, 0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rc

extern "C" int rcx_hbm_probe(int kind, const void* a, void* b, void* c, int64_t n, hipStream_t s) {
  using namespace rc;
  if (n <= 0 || n % 8) return (int)hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const unsigned g4 = (unsigned)((n4 + kProbeBlock - 1) / kProbeBlock);
  const unsigned gmix = (unsigned)((n4 + kMixChunks * kProbeBlock - 1) / (kMixChunks * kProbeBlock));
  const unsigned grmw = (unsigned)((n4 + kRmwChunks * kProbeBlock - 1) / (kRmwChunks * kProbeBlock));
  switch (kind) {
    case RCX_PROBE_COPY:
      hipLaunchKernelGGL(probe_copy, dim3(g4), dim3(kProbeBlock), 0, s, (const f32x4*)a, (f32x4*)b, n4);
      break;
    case RCX_PROBE_READ:
      hipLaunchKernelGGL(probe_read, dim3(g4), dim3(kProbeBlock), 0, s, (const f32x4*)a, (float*)c, n4);
      break;
    case RCX_PROBE_WRITE:
      hipLaunchKernelGGL(probe_write, dim3(g4), dim3(kProbeBlock), 0, s, (f32x4*)b, n4);
      break;
    case RCX_PROBE_SENDER_MIX:
      hipLaunchKernelGGL(probe_mix14, dim3(gmix), dim3(kProbeBlock), 0, s, (const uint16_t*)a, (float*)b,
                         (float*)c, n4);
      break;
    case RCX_PROBE_RECEIVER_RMW:
      hipLaunchKernelGGL(probe_rmw8, dim3(grmw), dim3(kProbeBlock), 0, s, (float*)b, n4);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
