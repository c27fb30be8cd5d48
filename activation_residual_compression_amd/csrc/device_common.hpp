// Device helpers shared by the librescomp kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rc {

constexpr int kWave = 64;

// ---------------------------------------------------------------- DPP lanes
// Cross-lane moves inside a row of 16 lanes, fused by the compiler into
// v_mov_b32_dpp. The patterns used by the reductions:
//   kQuadXor1  lane i <- i^1           kQuadXor2  lane i <- i^2
//   kHalfMirror lane i <- 7-i (in 8)   kRowMirror lane i <- 15-i (in 16)
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// All-reduce over aligned groups of L lanes (L = 1, 2, 4, 8, 16, 32). Every lane
// of a group ends with the same value: each stage combines a lane with one
// partner and the operations are commutative. Stages inside a row of 16 lanes
// are DPP moves; the 32-lane stage crosses rows with a lane-xor shuffle.
template <int L>
__device__ __forceinline__ double group_sum_f64(double v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "group of 1..32 lanes");
  if constexpr (L >= 2) v += dpp_f64<kQuadXor1>(v);
  if constexpr (L >= 4) v += dpp_f64<kQuadXor2>(v);
  if constexpr (L >= 8) v += dpp_f64<kHalfMirror>(v);
  if constexpr (L >= 16) v += dpp_f64<kRowMirror>(v);
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  return v;
}
template <int L>
__device__ __forceinline__ float group_min(float v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "group of 1..32 lanes");
  if constexpr (L >= 2) v = fminf(v, dpp_f32<kQuadXor1>(v));
  if constexpr (L >= 4) v = fminf(v, dpp_f32<kQuadXor2>(v));
  if constexpr (L >= 8) v = fminf(v, dpp_f32<kHalfMirror>(v));
  if constexpr (L >= 16) v = fminf(v, dpp_f32<kRowMirror>(v));
  if constexpr (L >= 32) v = fminf(v, __shfl_xor(v, 16));
  return v;
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "group of 1..32 lanes");
  if constexpr (L >= 2) v = fmaxf(v, dpp_f32<kQuadXor1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp_f32<kQuadXor2>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp_f32<kHalfMirror>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp_f32<kRowMirror>(v));
  if constexpr (L >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "group of 1..32 lanes");
  if constexpr (L >= 2) v = max(v, dpp_u32<kQuadXor1>(v));
  if constexpr (L >= 4) v = max(v, dpp_u32<kQuadXor2>(v));
  if constexpr (L >= 8) v = max(v, dpp_u32<kHalfMirror>(v));
  if constexpr (L >= 16) v = max(v, dpp_u32<kRowMirror>(v));
  if constexpr (L >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  return v;
}
template <int L>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t v) {
  static_assert(L >= 1 && L <= 32 && (L & (L - 1)) == 0, "group of 1..32 lanes");
  if constexpr (L >= 2) v = min(v, dpp_u32<kQuadXor1>(v));
  if constexpr (L >= 4) v = min(v, dpp_u32<kQuadXor2>(v));
  if constexpr (L >= 8) v = min(v, dpp_u32<kHalfMirror>(v));
  if constexpr (L >= 16) v = min(v, dpp_u32<kRowMirror>(v));
  if constexpr (L >= 32) v = min(v, (uint32_t)__shfl_xor((int)v, 16));
  return v;
}
// Bitwise OR over aligned groups of L lanes (L = 1, 2, 4, 8).
template <int L>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  static_assert(L >= 1 && L <= 8 && (L & (L - 1)) == 0, "group of 1..8 lanes");
  if constexpr (L >= 2) v |= dpp_u32<kQuadXor1>(v);
  if constexpr (L >= 4) v |= dpp_u32<kQuadXor2>(v);
  if constexpr (L >= 8) v |= dpp_u32<kHalfMirror>(v);
  return v;
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- 4-element chunks
// The streaming kernels give each lane 4 consecutive elements per chunk, so one
// wave-wide load or store of a chunk covers a single contiguous run (1 KiB of
// fp32, 512 B of bf16): every instruction fills whole cache lines by itself.
// Every array these kernels touch is streamed once per launch and is far larger
// than the caches, so loads and stores are non-temporal (streaming hint): on
// this device that measurably raises the read/write mix the kernels sustain.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename IN>
__device__ __forceinline__ f32x4 load4(const IN* p);
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
}
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store4(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// ---------------------------------------------------------------- 8-element chunks
// The low-rank kernels give a lane 8 consecutive elements: 16 B of bf16 or 32 B
// of fp32 input, 32 B of each fp32 state array.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct F8 {
  float v[8];
};

template <typename IN>
__device__ __forceinline__ void load8(const IN* p, F8& out);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, F8& out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  out.v[0] = bf16_lo(w.x); out.v[1] = bf16_hi(w.x);
  out.v[2] = bf16_lo(w.y); out.v[3] = bf16_hi(w.y);
  out.v[4] = bf16_lo(w.z); out.v[5] = bf16_hi(w.z);
  out.v[6] = bf16_lo(w.w); out.v[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, F8& out) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
  out.v[0] = a.x; out.v[1] = a.y; out.v[2] = a.z; out.v[3] = a.w;
  out.v[4] = b.x; out.v[5] = b.y; out.v[6] = b.z; out.v[7] = b.w;
}

__device__ __forceinline__ void store8(float* p, const F8& x) {
  f32x4* q = reinterpret_cast<f32x4*>(p);
  q[0] = f32x4{x.v[0], x.v[1], x.v[2], x.v[3]};
  q[1] = f32x4{x.v[4], x.v[5], x.v[6], x.v[7]};
}
// Write-only streams (the error-feedback buffer): non-temporal 128-bit stores.
__device__ __forceinline__ void store8_nt(float* p, const F8& x) {
  f32x4* q = reinterpret_cast<f32x4*>(p);
  __builtin_nontemporal_store(f32x4{x.v[0], x.v[1], x.v[2], x.v[3]}, q);
  __builtin_nontemporal_store(f32x4{x.v[4], x.v[5], x.v[6], x.v[7]}, q + 1);
}

}  // namespace rc
