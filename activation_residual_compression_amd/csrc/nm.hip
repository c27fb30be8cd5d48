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
// two lanes (8 elements each, one 128-bit bf16 load). Each lane keeps a running
// top-2 of its 8 elements in registers (strict comparisons in index order keep
// the lower index on ties), the pair exchanges its lists with one DPP quad move
// and both lanes merge them the same way. |r| is compared as the integer bit
// pattern of the magnitude, which orders non-negative floats exactly.
// Kept values travel as bf16 (round to nearest even); dropped positions decode
// to 0, so e_t = r there and e_t = r - bf16(r) at kept positions.
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

template <typename IN, int IT>
__global__ __launch_bounds__(kNmBlock) void nm_compress_kernel(const IN* __restrict__ a,
                                                               float* __restrict__ ahat,
                                                               float* __restrict__ e,
                                                               uint8_t* __restrict__ packed,
                                                               Layout L) {
  const int b = blockIdx.y;
  const int64_t nch = L.n / 8;
  const int64_t base = (int64_t)b * L.n;
  uint8_t* pk = packed + (int64_t)b * L.tstride;
  uint32_t* vals = reinterpret_cast<uint32_t*>(pk);
  uint8_t* idxs = pk + L.sec_off[1];
  if (blockIdx.x == 0) nm_zero_padding(pk, L);
  const bool hi = threadIdx.x & 1;  // odd lane: elements 8..15 of its block

  // every chunk's loads before the first store (see the quantiser kernel)
  F8 xs[IT], hs[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kNmBlock + threadIdx.x;
    const int64_t off = base + (ch < nch ? ch : (ch & 1)) * 8;
    load8<IN>(a + off, xs[it]);
    load8<float>(ahat + off, hs[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kNmBlock + threadIdx.x;
    const bool valid = ch < nch;  // lane pairs are valid together (16 | n)
    const int64_t off = base + (valid ? ch : (ch & 1)) * 8;
    const F8& x = xs[it];
    F8& h = hs[it];
    F8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = x.v[i] - h.v[i];

    // running top-2 of this lane's 8 elements
    uint32_t k1 = __float_as_uint(r.v[0]) & 0x7FFFFFFFu, k2 = __float_as_uint(r.v[1]) & 0x7FFFFFFFu;
    uint32_t i1 = 0, i2 = 1;
    float v1 = r.v[0], v2 = r.v[1];
    if (k2 > k1) {
      const uint32_t tk = k1; k1 = k2; k2 = tk;
      i1 = 1; i2 = 0;
      const float tv = v1; v1 = v2; v2 = tv;
    }
#pragma unroll
    for (int i = 2; i < 8; ++i) {
      const uint32_t k = __float_as_uint(r.v[i]) & 0x7FFFFFFFu;
      const bool top = k > k1, second = !top && k > k2;
      k2 = top ? k1 : (second ? k : k2);
      i2 = top ? i1 : (second ? (uint32_t)i : i2);
      v2 = top ? v1 : (second ? r.v[i] : v2);
      k1 = top ? k : k1;
      i1 = top ? (uint32_t)i : i1;
      v1 = top ? r.v[i] : v1;
    }
    if (hi) { i1 += 8; i2 += 8; }
    // exchange with the partner lane of the block
    const uint32_t pk1 = dpp_u32<kQuadXor1>(k1), pk2 = dpp_u32<kQuadXor1>(k2);
    const uint32_t pidx = dpp_u32<kQuadXor1>(i1 | (i2 << 8));
    const float pv1 = dpp_f32<kQuadXor1>(v1), pv2 = dpp_f32<kQuadXor1>(v2);
    // A = list of the low lane (lower indices), B = list of the high lane
    const uint32_t Ak1 = hi ? pk1 : k1, Ak2 = hi ? pk2 : k2;
    const uint32_t Ai1 = hi ? (pidx & 0xFF) : i1, Ai2 = hi ? (pidx >> 8) : i2;
    const float Av1 = hi ? pv1 : v1, Av2 = hi ? pv2 : v2;
    const uint32_t Bk1 = hi ? k1 : pk1, Bk2 = hi ? k2 : pk2;
    const uint32_t Bi1 = hi ? i1 : (pidx & 0xFF), Bi2 = hi ? i2 : (pidx >> 8);
    const float Bv1 = hi ? v1 : pv1, Bv2 = hi ? v2 : pv2;
    // merge: B only wins a comparison when strictly larger (A has lower indices)
    uint32_t fi, si;
    float fv, sv;
    if (Bk1 > Ak1) {
      fi = Bi1; fv = Bv1;
      const bool b2 = Bk2 > Ak1;
      si = b2 ? Bi2 : Ai1; sv = b2 ? Bv2 : Av1;
    } else {
      fi = Ai1; fv = Av1;
      const bool b1 = Bk1 > Ak2;
      si = b1 ? Bi1 : Ai2; sv = b1 ? Bv1 : Av2;
    }
    const bool swap = si < fi;
    const uint32_t lo_i = swap ? si : fi, hi_i = swap ? fi : si;
    const uint32_t lo_b = bf16_rne(swap ? sv : fv), hi_b = bf16_rne(swap ? fv : sv);
    const float lo_c = __uint_as_float(lo_b << 16), hi_c = __uint_as_float(hi_b << 16);

    F8 ev;
    const uint32_t first = hi ? 8u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t g = first + i;
      const float c = (g == lo_i) ? lo_c : ((g == hi_i) ? hi_c : 0.0f);
      ev.v[i] = r.v[i] - c;
      h.v[i] = h.v[i] + c;
    }
    if (valid) {
      if (!hi) {
        vals[ch >> 1] = lo_b | (hi_b << 16);
        idxs[ch >> 1] = (uint8_t)(lo_i | (hi_i << 4));
      }
      store8(ahat + off, h);
      store8_nt(e + off, ev);
    }
  }
}

template <int IT>
__global__ __launch_bounds__(kNmBlock) void nm_decompress_kernel(const uint8_t* __restrict__ packed,
                                                                 float* __restrict__ ahat, Layout L) {
  const int b = blockIdx.y;
  const int64_t nch = L.n / 8;
  const int64_t base = (int64_t)b * L.n;
  const uint8_t* pk = packed + (int64_t)b * L.tstride;
  const uint32_t* vals = reinterpret_cast<const uint32_t*>(pk);
  const uint8_t* idxs = pk + L.sec_off[1];
  F8 hs[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kNmBlock + threadIdx.x;
    load8<float>(ahat + base + (ch < nch ? ch : 0) * 8, hs[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kNmBlock + threadIdx.x;
    if (ch >= nch) continue;
    const int64_t off = base + ch * 8;
    F8& h = hs[it];
    const uint32_t v = vals[ch >> 1];
    const uint32_t id = idxs[ch >> 1];
    const uint32_t lo_i = id & 15u, hi_i = id >> 4;
    const float lo_c = bf16_lo(v), hi_c = bf16_hi(v);
    const uint32_t first = (ch & 1) ? 8u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t g = first + i;
      h.v[i] = h.v[i] + ((g == lo_i) ? lo_c : ((g == hi_i) ? hi_c : 0.0f));
    }
    store8(ahat + off, h);
  }
}

namespace {
constexpr int kNmIt = 2;
}

hipError_t launch_nm_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, hipStream_t s) {
  const int64_t nch = L.n / 8;
  const dim3 grid((unsigned)((nch + kNmBlock * kNmIt - 1) / (kNmBlock * kNmIt)), (unsigned)batch);
  if (bf16_input)
    hipLaunchKernelGGL((nm_compress_kernel<uint16_t, kNmIt>), grid, dim3(kNmBlock), 0, s,
                       static_cast<const uint16_t*>(a), ahat, e, packed, L);
  else
    hipLaunchKernelGGL((nm_compress_kernel<float, kNmIt>), grid, dim3(kNmBlock), 0, s,
                       static_cast<const float*>(a), ahat, e, packed, L);
  return hipGetLastError();
}

hipError_t launch_nm_decompress(const uint8_t* packed, float* ahat, int batch, const Layout& L,
                                hipStream_t s) {
  const int64_t nch = L.n / 8;
  const dim3 grid((unsigned)((nch + kNmBlock * kNmIt - 1) / (kNmBlock * kNmIt)), (unsigned)batch);
  hipLaunchKernelGGL((nm_decompress_kernel<kNmIt>), grid, dim3(kNmBlock), 0, s, packed, ahat, L);
  return hipGetLastError();
}

}  // namespace rc
