// 2:16 block sparsifier of the residual with error feedback.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion notes) -- Key designs / System co-design: an N:M
// block sparsifier instead of a TopK, which would need a global sort and
// irregular memory access; Overall framework and Error feedback for the
// recurrence around it.
//
// Selection: in every block of 16 contiguous elements keep the 2 with the
// largest |r|, ties to the lower index. No sort and no shared memory: a block is
// a quad of lanes, each owning 4 consecutive elements (the lane layout of the
// quantiser kernels, so every wave-wide access is one contiguous run). Each lane
// keeps a running top-2 of its 4 elements in registers (strict comparisons in
// index order keep the lower index on ties); the quad then merges lists twice,
// first with the neighbouring lane, then with the neighbouring pair, each time
// through DPP quad moves, so all four lanes end with the block's top-2. |r| is
// compared as the integer bit pattern of the magnitude, which orders
// non-negative floats exactly. Kept values travel as bf16 (round to nearest
// even); dropped positions decode to 0, so e_t = r there and e_t = r - bf16(r)
// at kept positions.
#include "device_common.hpp"
#include "launch.hpp"

namespace rc {

constexpr int kNmBlock = 256;

__device__ __forceinline__ void nm_zero_padding(uint8_t* tensor_base, const Layout& L) {
  for (int s = 0; s < L.nsec; ++s) {
    const int64_t start = L.sec_off[s] + L.sec_len[s];
    const int64_t end = (s + 1 < L.nsec) ? L.sec_off[s + 1] : L.tstride;
    for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) tensor_base[i] = 0;
  }
}

__device__ __forceinline__ float bf16_round_f32(float x) { return __uint_as_float(bf16_rne(x) << 16); }

// Running top-2 of a block: keys are |r| bit patterns, indices 0..15 in the block.
struct Top2 {
  uint32_t k1, k2, i1, i2;
  float v1, v2;
};

__device__ __forceinline__ uint32_t mag_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Top-2 of A and B where every index in A is below every index in B: B only
// wins a comparison when strictly larger. Written with selects only.
__device__ __forceinline__ Top2 merge_top2(const Top2& A, const Top2& B) {
  const bool bfirst = B.k1 > A.k1;
  // runner-up: if B leads, the better of B's second and A's first; else the
  // better of A's second and B's first
  const bool b2 = B.k2 > A.k1, b1 = B.k1 > A.k2;
  Top2 o;
  o.k1 = bfirst ? B.k1 : A.k1;
  o.i1 = bfirst ? B.i1 : A.i1;
  o.v1 = bfirst ? B.v1 : A.v1;
  o.k2 = bfirst ? (b2 ? B.k2 : A.k1) : (b1 ? B.k1 : A.k2);
  o.i2 = bfirst ? (b2 ? B.i2 : A.i1) : (b1 ? B.i1 : A.i2);
  o.v2 = bfirst ? (b2 ? B.v2 : A.v1) : (b1 ? B.v1 : A.v2);
  return o;
}

// Merge this lane's list with the partner lane's (DPP pattern CTRL); `upper`
// says that this lane's indices are the higher ones.
template <int CTRL>
__device__ __forceinline__ Top2 merge_with(const Top2& t, bool upper) {
  const float pv1 = dpp_f32<CTRL>(t.v1), pv2 = dpp_f32<CTRL>(t.v2);
  const uint32_t pidx = dpp_u32<CTRL>(t.i1 | (t.i2 << 8));
  const uint32_t pi1 = pidx & 0xFFu, pi2 = pidx >> 8;
  Top2 A, B;
  A.v1 = upper ? pv1 : t.v1;  B.v1 = upper ? t.v1 : pv1;
  A.v2 = upper ? pv2 : t.v2;  B.v2 = upper ? t.v2 : pv2;
  A.i1 = upper ? pi1 : t.i1;  B.i1 = upper ? t.i1 : pi1;
  A.i2 = upper ? pi2 : t.i2;  B.i2 = upper ? t.i2 : pi2;
  A.k1 = mag_key(A.v1); A.k2 = mag_key(A.v2);
  B.k1 = mag_key(B.v1); B.k2 = mag_key(B.v2);
  return merge_top2(A, B);
}

template <typename IN, int NC>
__global__ __launch_bounds__(kNmBlock) void nm_compress_kernel(const IN* __restrict__ a,
                                                               float* __restrict__ ahat,
                                                               float* __restrict__ e,
                                                               uint8_t* __restrict__ packed,
                                                               Layout L) {
  const int b = blockIdx.y;
  const int64_t n4 = L.n / 4;
  const int64_t base = (int64_t)b * L.n;
  uint8_t* pk = packed + (int64_t)b * L.tstride;
  uint32_t* vals = reinterpret_cast<uint32_t*>(pk);
  uint8_t* idxs = pk + L.sec_off[1];
  if (blockIdx.x == 0) nm_zero_padding(pk, L);
  const uint32_t q = threadIdx.x & 3;  // this lane holds elements 4q .. 4q+3 of its block

  // Every chunk's loads before the first store. Lanes past the end work on
  // chunk 0 and store nothing; quads are valid together (16 | n).
  f32x4 xs[NC], hs[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kNmBlock + threadIdx.x;
    const int64_t off = base + (c < n4 ? c : (int64_t)q) * 4;
    xs[j] = load4<IN>(a + off);
    hs[j] = load4<float>(ahat + off);
  }
  f32x4 evs[NC], hns[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kNmBlock + threadIdx.x;
    const bool valid = c < n4;
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = xs[j][i] - hs[j][i];

    // running top-2 of this lane's 4 elements
    Top2 t;
    t.k1 = mag_key(r[0]); t.k2 = mag_key(r[1]);
    t.i1 = 0; t.i2 = 1; t.v1 = r[0]; t.v2 = r[1];
    if (t.k2 > t.k1) {
      t.k1 = mag_key(r[1]); t.k2 = mag_key(r[0]);
      t.i1 = 1; t.i2 = 0; t.v1 = r[1]; t.v2 = r[0];
    }
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      const uint32_t k = mag_key(r[i]);
      const bool top = k > t.k1, second = !top && k > t.k2;
      t.k2 = top ? t.k1 : (second ? k : t.k2);
      t.i2 = top ? t.i1 : (second ? (uint32_t)i : t.i2);
      t.v2 = top ? t.v1 : (second ? r[i] : t.v2);
      t.k1 = top ? k : t.k1;
      t.i1 = top ? (uint32_t)i : t.i1;
      t.v1 = top ? r[i] : t.v1;
    }
    t.i1 += 4 * q;
    t.i2 += 4 * q;
    t = merge_with<kQuadXor1>(t, q & 1u);
    t = merge_with<kQuadXor2>(t, q & 2u);

    const bool swap = t.i2 < t.i1;
    const uint32_t lo_i = swap ? t.i2 : t.i1, hi_i = swap ? t.i1 : t.i2;
    const uint32_t lo_b = bf16_rne(swap ? t.v2 : t.v1), hi_b = bf16_rne(swap ? t.v1 : t.v2);
    const float lo_c = __uint_as_float(lo_b << 16), hi_c = __uint_as_float(hi_b << 16);

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t g = 4 * q + i;
      const float cv = (g == lo_i) ? lo_c : ((g == hi_i) ? hi_c : 0.0f);
      evs[j][i] = r[i] - cv;
      hns[j][i] = hs[j][i] + cv;
    }
    if (valid && q == 0) {
      vals[c >> 2] = lo_b | (hi_b << 16);
      idxs[c >> 2] = (uint8_t)(lo_i | (hi_i << 4));
    }
  }
  // every chunk's ahat, then every chunk's e (longer runs per array)
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kNmBlock + threadIdx.x;
    if (c < n4) store4(ahat + base + c * 4, hns[j]);
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kNmBlock + threadIdx.x;
    if (c < n4) store4(e + base + c * 4, evs[j]);
  }
}

template <int NC>
__global__ __launch_bounds__(kNmBlock) void nm_decompress_kernel(PeerSet peers, Layout L) {
  const int b = blockIdx.y;
  const uint8_t* __restrict__ packed = peers.packed[blockIdx.z];
  float* __restrict__ ahat = peers.state[blockIdx.z];
  const int64_t n4 = L.n / 4;
  const int64_t base = (int64_t)b * L.n;
  const uint8_t* pk = packed + (int64_t)b * L.tstride;
  const uint32_t* vals = reinterpret_cast<const uint32_t*>(pk);
  const uint8_t* idxs = pk + L.sec_off[1];
  const uint32_t q = threadIdx.x & 3;
  f32x4 hs[NC];
  uint32_t vs[NC], ids[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kNmBlock + threadIdx.x;
    const int64_t cc = c < n4 ? c : 0;
    hs[j] = load4<float>(ahat + base + cc * 4);
    vs[j] = vals[cc >> 2];
    ids[j] = idxs[cc >> 2];
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kNmBlock + threadIdx.x;
    if (c >= n4) continue;
    const uint32_t lo_i = ids[j] & 15u, hi_i = ids[j] >> 4;
    const float lo_c = bf16_lo(vs[j]), hi_c = bf16_hi(vs[j]);
    f32x4 h = hs[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t g = 4 * q + i;
      h[i] = h[i] + ((g == lo_i) ? lo_c : ((g == hi_i) ? hi_c : 0.0f));
    }
    store4(ahat + base + c * 4, h);
  }
}

namespace {
constexpr int kNmChunks = 4;     // chunks per lane, sender
constexpr int kNmDecChunks = 2;  // chunks per lane, receiver
}

hipError_t launch_nm_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, hipStream_t s) {
  const int64_t n4 = L.n / 4;
  const dim3 grid((unsigned)((n4 + kNmBlock * kNmChunks - 1) / (kNmBlock * kNmChunks)), (unsigned)batch);
  if (bf16_input)
    hipLaunchKernelGGL((nm_compress_kernel<uint16_t, kNmChunks>), grid, dim3(kNmBlock), 0, s,
                       static_cast<const uint16_t*>(a), ahat, e, packed, L);
  else
    hipLaunchKernelGGL((nm_compress_kernel<float, kNmChunks>), grid, dim3(kNmBlock), 0, s,
                       static_cast<const float*>(a), ahat, e, packed, L);
  return hipGetLastError();
}

hipError_t launch_nm_decompress(const PeerSet& peers, int batch, const Layout& L, hipStream_t s) {
  const int64_t n4 = L.n / 4;
  const dim3 grid((unsigned)((n4 + kNmBlock * kNmDecChunks - 1) / (kNmBlock * kNmDecChunks)), (unsigned)batch,
                  (unsigned)peers.count);
  hipLaunchKernelGGL((nm_decompress_kernel<kNmDecChunks>), grid, dim3(kNmBlock), 0, s, peers, L);
  return hipGetLastError();
}

}  // namespace rc
