// rc_compress_lowrank_noalloc: the low-rank sender step without a plan and
// without any allocation, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid it).
// The workspace the plan would own lives in a fixed device array of this file,
// one copy per GPU, held until the process ends. The kernels are the plan's:
// the results equal those of rc_compress on a plan with the same parameters.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/librescomp.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = RC_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Device-side workspace. In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];

// The scratch address on the current device, looked up once per device.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch[dev].store(p, std::memory_order_release);  // same value from any thread
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" rc_status_t rc_compress_lowrank_noalloc(rc_shape_t shape, rc_dtype_t dtype,
                                                   const rc_params_t* params, hipStream_t stream,
                                                   const void* a_t, const rc_state_t* state,
                                                   void* packed_out) {
  rc_status_t st = rc::validate(shape, dtype, RC_LOWRANK, params);
  if (st != RC_OK) return st;
  if (params->flags & ~RC_LR_BF16_FACTORS) return RC_ERR_INVALID_ARG;  // one stream, no checks
  if (!a_t || !state || !state->ahat || !state->e || !packed_out) return RC_ERR_INVALID_ARG;
  const uintptr_t mis = (uintptr_t)a_t | (uintptr_t)state->ahat | (uintptr_t)state->e |
                        (uintptr_t)packed_out;
  if (mis & 15u) return RC_ERR_ALIGNMENT;
  rc::Layout L;
  st = rc::make_layout(shape, dtype, RC_LOWRANK, *params, &L);
  if (st != RC_OK) return st;
  rc::LowRankWork w;
  if ((size_t)rc::carve_lowrank(&w, shape, *params, nullptr) > kScratchBytes) return RC_ERR_UNSUPPORTED;
  void* base = nullptr;
  if (scratch_on_current_device(&base) != hipSuccess) return RC_ERR_HIP;
  rc::carve_lowrank(&w, shape, *params, base);
  // the start matrices are set up on every call (the scratch keeps the last
  // call's contents, which may belong to another shape); nothing else in the
  // workspace needs clearing: every piece is written before it is read
  hipError_t err = rc::launch_lr_q0(static_cast<const float*>(params->q0), params->seed, w.Q0t,
                                    shape.batch, shape.cols, w.pay_rank, w.rank, stream);
  if (err == hipSuccess)
    err = rc::launch_lr_compress(dtype == RC_BF16, a_t, state->ahat, state->e,
                                 static_cast<uint8_t*>(packed_out), shape.batch, L, w, stream);
  return err == hipSuccess ? RC_OK : RC_ERR_HIP;
}
