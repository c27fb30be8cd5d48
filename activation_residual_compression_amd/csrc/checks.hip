// Debug checks behind plan flags (not on the default path): a scan for NaN or
// Inf in the sender's inputs, and a one-word fill used to clear the counters.
#include "device_common.hpp"
#include "launch.hpp"

namespace rc {

constexpr int kCheckThreads = 256;

__device__ __forceinline__ bool finite_bits(uint32_t u) { return (u & 0x7F800000u) != 0x7F800000u; }

// Grid-stride over n elements of a and of ahat; one atomic add per wave.
template <typename IN>
__global__ __launch_bounds__(kCheckThreads) void count_nonfinite_kernel(const IN* __restrict__ a,
                                                                        const float* __restrict__ ahat,
                                                                        int64_t n,
                                                                        uint32_t* __restrict__ count) {
  uint32_t bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kCheckThreads) {
    const uint32_t ua = sizeof(IN) == 2 ? (uint32_t)a[i] << 16 : __float_as_uint((float)a[i]);
    bad += !finite_bits(ua);
    bad += !finite_bits(__float_as_uint(ahat[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bad += __shfl_xor(bad, o);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(count, bad);
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

hipError_t launch_count_nonfinite(const void* a, bool bf16, const float* ahat, int64_t n,
                                  uint32_t* count, hipStream_t s) {
  const int64_t want = (n + kCheckThreads - 1) / kCheckThreads;
  const unsigned blocks = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  if (bf16)
    hipLaunchKernelGGL(count_nonfinite_kernel<uint16_t>, dim3(blocks), dim3(kCheckThreads), 0, s,
                       static_cast<const uint16_t*>(a), ahat, n, count);
  else
    hipLaunchKernelGGL(count_nonfinite_kernel<float>, dim3(blocks), dim3(kCheckThreads), 0, s,
                       static_cast<const float*>(a), ahat, n, count);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, hipStream_t s) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, s, p, v);
  return hipGetLastError();
}

}  // namespace rc
