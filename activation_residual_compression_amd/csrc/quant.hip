// 1-bit and 2-bit group quantisation of the residual with error feedback.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion notes) -- Overall framework (residual against the
// receiver's reconstruction, receiver update), Key designs / Error feedback
// (e_t = r - C(r) kept locally), Main experiment table (1-bit 16x, 2-bit 8x).
//
// One fused pass per step on the sender: each lane loads 8 consecutive
// elements of a_t (one 128-bit load of bf16) and of ahat (two 128-bit loads),
// forms r = a_t - ahat, reduces the group statistic across the G/8 lanes of its
// group with DPP row moves, encodes, and writes codes, group metadata, e_t and
// the new ahat. The receiver kernel decodes and accumulates in one pass.
//
// Arithmetic (fp32, one rounding per operation, no contraction):
//   Q1: s = fp32(sum_fp64 |r| / G), bit = (r >= 0), c = bit ? s : -s
//   Q2: mn, mx = group min/max; d = (mx - mn) / 3 (zeros of mn and d stored
//       as +0); if d >= FLT_MIN:
//       inv = 1/d, q = min(3, rint_even((r - mn) * inv)) else q = 0;
//       c = fma(q, d, mn)
//   e = r - c; ahat = ahat + c   (the receiver applies the same c)
#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rc {

constexpr int kBlock = 256;

// Zero the gaps between sections (and after the last) of one tensor's packed
// block, so the stream is fully defined. Each gap is below 256 bytes.
__device__ __forceinline__ void zero_padding(uint8_t* tensor_base, const Layout& L) {
  for (int s = 0; s < L.nsec; ++s) {
    const int64_t start = L.sec_off[s] + L.sec_len[s];
    const int64_t end = (s + 1 < L.nsec) ? L.sec_off[s + 1] : L.tstride;
    for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) tensor_base[i] = 0;
  }
}

template <typename IN, int G, int BITS, int IT>
__global__ __launch_bounds__(kBlock) void q_compress_kernel(const IN* __restrict__ a,
                                                            float* __restrict__ ahat,
                                                            float* __restrict__ e,
                                                            uint8_t* __restrict__ packed, Layout L) {
  constexpr int LANES = G / 8;  // lanes per group
  const int b = blockIdx.y;
  const int64_t nch = L.n / 8;
  const int64_t base = (int64_t)b * L.n;
  uint8_t* pk = packed + (int64_t)b * L.tstride;
  uint8_t* meta = pk + L.sec_off[1];
  if (blockIdx.x == 0) zero_padding(pk, L);

  // All chunks' loads are issued before the first store: the stores go to
  // ahat, so the compiler would otherwise keep each chunk's loads behind the
  // previous chunk's stores.
  F8 xs[IT], hs[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kBlock + threadIdx.x;
    // Lanes past the end work on chunk 0 and store nothing; groups never mix
    // valid and invalid lanes because a tensor holds whole groups.
    const int64_t off = base + (ch < nch ? ch : 0) * 8;
    load8<IN>(a + off, xs[it]);
    load8<float>(ahat + off, hs[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kBlock + threadIdx.x;
    const bool valid = ch < nch;
    const int64_t off = base + (valid ? ch : 0) * 8;
    const F8& x = xs[it];
    F8& h = hs[it];
    F8 c, r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = x.v[i] - h.v[i];

    if constexpr (BITS == 1) {
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += (double)fabsf(r.v[i]);
      s = group_sum_f64<LANES>(s);
      const float scale = (float)(s * (1.0 / G));
      uint32_t byte = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool pos = r.v[i] >= 0.0f;
        byte |= (pos ? 1u : 0u) << i;
        c.v[i] = pos ? scale : -scale;
      }
      if (valid) {
        pk[ch] = (uint8_t)byte;
        if ((ch % LANES) == 0) reinterpret_cast<float*>(meta)[ch / LANES] = scale;
      }
    } else {
      float mn = r.v[0], mx = r.v[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, r.v[i]);
        mx = fmaxf(mx, r.v[i]);
      }
      // zeros of the stored minimum and step are normalised to +0 (x + 0)
      mn = group_min<LANES>(mn) + 0.0f;
      mx = group_max<LANES>(mx);
      const float d = (mx - mn) / 3.0f + 0.0f;
      const bool live = d >= FLT_MIN;
      const float inv = 1.0f / d;
      uint32_t code = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = (r.v[i] - mn) * inv;
        const float q = live ? fminf(rintf(t), 3.0f) : 0.0f;
        code |= ((uint32_t)q) << (2 * i);
        c.v[i] = fmaf(q, d, mn);
      }
      if (valid) {
        reinterpret_cast<uint16_t*>(pk)[ch] = (uint16_t)code;
        if ((ch % LANES) == 0) reinterpret_cast<float2*>(meta)[ch / LANES] = make_float2(mn, d);
      }
    }

    F8 ev;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ev.v[i] = r.v[i] - c.v[i];
      h.v[i] = h.v[i] + c.v[i];
    }
    if (valid) {
      store8(ahat + off, h);
      store8_nt(e + off, ev);
    }
  }
}

template <int G, int BITS, int IT>
__global__ __launch_bounds__(kBlock) void q_decompress_kernel(const uint8_t* __restrict__ packed,
                                                              float* __restrict__ ahat, Layout L) {
  constexpr int LANES = G / 8;
  const int b = blockIdx.y;
  const int64_t nch = L.n / 8;
  const int64_t base = (int64_t)b * L.n;
  const uint8_t* pk = packed + (int64_t)b * L.tstride;
  const uint8_t* meta = pk + L.sec_off[1];
  F8 hs[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kBlock + threadIdx.x;
    load8<float>(ahat + base + (ch < nch ? ch : 0) * 8, hs[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t ch = ((int64_t)blockIdx.x * IT + it) * kBlock + threadIdx.x;
    if (ch >= nch) continue;
    const int64_t off = base + ch * 8;
    F8& h = hs[it];
    if constexpr (BITS == 1) {
      const uint32_t byte = pk[ch];
      const float scale = reinterpret_cast<const float*>(meta)[ch / LANES];
#pragma unroll
      for (int i = 0; i < 8; ++i) h.v[i] = h.v[i] + (((byte >> i) & 1u) ? scale : -scale);
    } else {
      const uint32_t code = reinterpret_cast<const uint16_t*>(pk)[ch];
      const float2 md = reinterpret_cast<const float2*>(meta)[ch / LANES];
#pragma unroll
      for (int i = 0; i < 8; ++i) h.v[i] = h.v[i] + fmaf((float)((code >> (2 * i)) & 3u), md.y, md.x);
    }
    store8(ahat + off, h);
  }
}

namespace {
constexpr int kIt = 2;  // chunks per lane

template <typename IN, int G, int BITS>
hipError_t q_compress_t(const void* a, float* ahat, float* e, uint8_t* packed, int batch,
                        const Layout& L, hipStream_t s) {
  const int64_t nch = L.n / 8;
  const dim3 grid((unsigned)((nch + kBlock * kIt - 1) / (kBlock * kIt)), (unsigned)batch);
  hipLaunchKernelGGL((q_compress_kernel<IN, G, BITS, kIt>), grid, dim3(kBlock), 0, s,
                     static_cast<const IN*>(a), ahat, e, packed, L);
  return hipGetLastError();
}

template <int G, int BITS>
hipError_t q_decompress_t(const uint8_t* packed, float* ahat, int batch, const Layout& L,
                          hipStream_t s) {
  const int64_t nch = L.n / 8;
  const dim3 grid((unsigned)((nch + kBlock * kIt - 1) / (kBlock * kIt)), (unsigned)batch);
  hipLaunchKernelGGL((q_decompress_kernel<G, BITS, kIt>), grid, dim3(kBlock), 0, s, packed, ahat, L);
  return hipGetLastError();
}

template <int BITS>
hipError_t q_compress_g(int group, bool bf16, const void* a, float* ahat, float* e, uint8_t* p,
                        int batch, const Layout& L, hipStream_t s) {
  switch (group) {
    case 32: return bf16 ? q_compress_t<uint16_t, 32, BITS>(a, ahat, e, p, batch, L, s)
                         : q_compress_t<float, 32, BITS>(a, ahat, e, p, batch, L, s);
    case 64: return bf16 ? q_compress_t<uint16_t, 64, BITS>(a, ahat, e, p, batch, L, s)
                         : q_compress_t<float, 64, BITS>(a, ahat, e, p, batch, L, s);
    case 128: return bf16 ? q_compress_t<uint16_t, 128, BITS>(a, ahat, e, p, batch, L, s)
                          : q_compress_t<float, 128, BITS>(a, ahat, e, p, batch, L, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t q_decompress_g(int group, const uint8_t* p, float* ahat, int batch, const Layout& L,
                          hipStream_t s) {
  switch (group) {
    case 32: return q_decompress_t<32, BITS>(p, ahat, batch, L, s);
    case 64: return q_decompress_t<64, BITS>(p, ahat, batch, L, s);
    case 128: return q_decompress_t<128, BITS>(p, ahat, batch, L, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_q_compress(int bits, int group, bool bf16_input, const void* a, float* ahat,
                             float* e, uint8_t* packed, int batch, const Layout& L, hipStream_t s) {
  return bits == 1 ? q_compress_g<1>(group, bf16_input, a, ahat, e, packed, batch, L, s)
                   : q_compress_g<2>(group, bf16_input, a, ahat, e, packed, batch, L, s);
}

hipError_t launch_q_decompress(int bits, int group, const uint8_t* packed, float* ahat, int batch,
                               const Layout& L, hipStream_t s) {
  return bits == 1 ? q_decompress_g<1>(group, packed, ahat, batch, L, s)
                   : q_decompress_g<2>(group, packed, ahat, batch, L, s);
}

}  // namespace rc
