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

// sender-like: per 8 elements read 16 B bf16 + 32 B fp32, write 32 B + 32 B (2
// chunks per lane). As in the sender kernels, both chunks' loads are issued
// before the first store, unconditionally (lanes past the end reread chunk 0
// and store nothing).
__global__ __launch_bounds__(kProbeBlock) void probe_mix14(const uint16_t* __restrict__ a,
                                                           float* __restrict__ h, float* __restrict__ e,
                                                           int64_t nch) {
  F8 xs[2], hs[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int64_t c = ((int64_t)blockIdx.x * 2 + it) * kProbeBlock + threadIdx.x;
    const int64_t cc = c < nch ? c : 0;
    load8<uint16_t>(a + cc * 8, xs[it]);
    load8<float>(h + cc * 8, hs[it]);
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int64_t c = ((int64_t)blockIdx.x * 2 + it) * kProbeBlock + threadIdx.x;
    const bool valid = c < nch;
    const F8& x = xs[it];
    F8& hv = hs[it];
    F8 ev;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = x.v[i] - hv.v[i];
      ev.v[i] = r;
      hv.v[i] = hv.v[i] + 0.5f * r;
    }
    if (valid) {
      store8(h + c * 8, hv);
      store8_nt(e + c * 8, ev);
    }
  }
}

// receiver-like: read and write back fp32 in place (2 chunks of 8 per lane)
__global__ __launch_bounds__(kProbeBlock) void probe_rmw8(float* __restrict__ h, int64_t nch) {
  F8 hs[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int64_t c = ((int64_t)blockIdx.x * 2 + it) * kProbeBlock + threadIdx.x;
    load8<float>(h + (c < nch ? c : 0) * 8, hs[it]);
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int64_t c = ((int64_t)blockIdx.x * 2 + it) * kProbeBlock + threadIdx.x;
    const bool valid = c < nch;
    F8& hv = hs[it];
#pragma unroll
    for (int i = 0; i < 8; ++i) hv.v[i] = hv.v[i] + 1.0f;
    if (valid) store8(h + c * 8, hv);
  }
}

}  // namespace
}  // namespace rc

extern "C" int rcx_hbm_probe(int kind, const void* a, void* b, void* c, int64_t n, hipStream_t s) {
  using namespace rc;
  if (n <= 0 || n % 8) return (int)hipErrorInvalidValue;
  const int64_t n4 = n / 4, nch = n / 8;
  const unsigned g4 = (unsigned)((n4 + kProbeBlock - 1) / kProbeBlock);
  const unsigned g8 = (unsigned)((nch + 2 * kProbeBlock - 1) / (2 * kProbeBlock));
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
      hipLaunchKernelGGL(probe_mix14, dim3(g8), dim3(kProbeBlock), 0, s, (const uint16_t*)a, (float*)b,
                         (float*)c, nch);
      break;
    case RCX_PROBE_RECEIVER_RMW:
      hipLaunchKernelGGL(probe_rmw8, dim3(g8), dim3(kProbeBlock), 0, s, (float*)b, nch);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
