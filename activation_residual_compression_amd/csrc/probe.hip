// HBM reference kernels for the roofline: the access patterns of the path's
// streaming kernels with trivial arithmetic, so a measurement shows what this
// device's HBM delivers for each pattern (the practical ceiling next to the
// 8 TB/s peak). Diagnostics only; nothing in the compression path calls them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/librescomp_diag.h"
#include "device_common.hpp"

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

}  // namespace
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
