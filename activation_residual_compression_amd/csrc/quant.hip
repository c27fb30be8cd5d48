// 1-bit and 2-bit group quantisation of the residual with error feedback.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion notes) -- Overall framework (residual against the
// receiver's reconstruction, receiver update), Key designs / Error feedback
// (e_t = r - C(r) kept locally), Main experiment table (1-bit 16x, 2-bit 8x).
//
// One fused pass per step on the sender. A lane owns 4 consecutive elements
// per chunk and NC chunks spaced one block-width apart, so each wave-wide access
// is one contiguous run; all chunks are loaded before the first store. The lane
// forms r = a_t - ahat, reduces the group statistic across the G/4 lanes of its
// group (DPP row moves, one lane-xor shuffle for 32 lanes), encodes, gathers
// the codes of 4 (2-bit) or 8 (1-bit) lanes into one 32-bit word, and writes
// codes, group metadata, e_t and the new ahat. The receiver kernel decodes and
// accumulates in one pass with the same lane layout.
//
// Arithmetic (fp32, one rounding per operation, no contraction):
//   Q1: s = the mean of |r| over the group rounded once to fp32 (nearest,
//       ties to even), bit = (r >= 0), c = bit ? s : -s
//   Q2: mn, mx = group min/max; d = (mx - mn) / 3 (zeros of mn and d stored
//       as +0); if d >= FLT_MIN:
//       inv = 1/d, q = min(3, rint_even((r - mn) * inv)) else q = 0;
//       c = fma(q, d, mn)
//   e = r - c; ahat = ahat + c   (the receiver applies the same c)
//
// The exact 1-bit mean. Each nonzero |r| is m * 2^(x - 150) with m < 2^24 and
// x = max(exponent field, 1), an integer multiple of 2^(x_min - 150) for the
// group's smallest x. When the group's exponents span at most 29 - log2(G)
// binades, the sum is below 2^53 such units, so the fp64 sum is exact in any
// order, and s = fp32(sum / G) rounds once (the common case: one fp64 sum over
// the group's lanes). Otherwise (a term smaller than about 2^-22 of the
// largest) the group takes an exact integer path: the magnitudes are added as
// integers in units of 2^-149 into a 288-bit accumulator in LDS (64-bit words
// of 32 live bits, so concurrent lane additions need no carry) and rounded to
// fp32 from its bits.
#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace rc {

constexpr int kBlock = 256;
constexpr int kQ1Words = 9;  // 288-bit exact |r| sum, 32 bits per 64-bit word

// Exact mean of the group's |r| (slow path, see the file header). `acc` and
// `nrm` are this group's kQ1Words-word LDS areas; every lane of the group
// calls this with its 4 residuals and returns the same scale. LDS operations
// of one wave complete in issue order, so the group needs no barrier.
template <int LANES, int LOG2G>
__device__ __forceinline__ float q1_exact_mean(f32x4 r, unsigned long long* acc, uint32_t* nrm) {
  const int lig = threadIdx.x % LANES;  // lane in group
  for (int k = lig; k < kQ1Words; k += LANES) acc[k] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = __float_as_uint(r[i]) & 0x7FFFFFFFu;
    const uint32_t x = u >> 23;
    if (u == 0u || x == 0xFFu) continue;
    const uint32_t pos = (x ? x : 1u) - 1u;                     // lsb of m, in units of 2^-149
    const uint64_t v = (uint64_t)(x ? ((u & 0x7FFFFFu) | 0x800000u) : u) << (pos & 31u);
    atomicAdd(&acc[pos >> 5], v & 0xFFFFFFFFull);
    atomicAdd(&acc[(pos >> 5) + 1], v >> 32);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  uint64_t carry = 0;
  int top = -1;
  for (int k = 0; k < kQ1Words; ++k) {
    const uint64_t t = acc[k] + carry;
    nrm[k] = (uint32_t)t;
    carry = t >> 32;
    if ((uint32_t)t) top = 32 * k + 31 - __clz((uint32_t)t);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (top < 0) return 0.0f;
  // keep 24 significant bits, or the subnormal grid 2^-149 (2^LOG2G units)
  const int drop = max(top - 23, LOG2G);
  const int w0 = drop >> 5;
  const uint64_t win = ((uint64_t)(w0 + 1 < kQ1Words ? nrm[w0 + 1] : 0u) << 32) | nrm[w0];
  uint32_t q = (uint32_t)(win >> (drop & 31));
  const int gp = drop - 1;  // the first dropped bit (drop >= LOG2G >= 1)
  const uint32_t gw = nrm[gp >> 5];
  const bool half = (gw >> (gp & 31)) & 1u;
  bool sticky = (gw & ((1u << (gp & 31)) - 1u)) != 0u;
  for (int k = 0; k < (gp >> 5); ++k) sticky |= nrm[k] != 0u;
  if (half && (sticky || (q & 1u))) ++q;  // nearest, ties to even
  return (float)ldexp((double)q, drop - 149 - LOG2G);  // exact: q <= 2^24
}

// Zero the gaps between sections (and after the last) of one tensor's packed
// block, so the stream is fully defined. Each gap is below 256 bytes.
__device__ __forceinline__ void zero_padding(uint8_t* tensor_base, const Layout& L) {
  for (int s = 0; s < L.nsec; ++s) {
    const int64_t start = L.sec_off[s] + L.sec_len[s];
    const int64_t end = (s + 1 < L.nsec) ? L.sec_off[s + 1] : L.tstride;
    for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) tensor_base[i] = 0;
  }
}

template <typename IN, int G, int BITS, int NC>
__global__ __launch_bounds__(kBlock) void q_compress_kernel(const IN* __restrict__ a,
                                                            float* __restrict__ ahat,
                                                            float* __restrict__ e,
                                                            uint8_t* __restrict__ packed, Layout L) {
  constexpr int LANES = G / 4;  // lanes per group
  constexpr int LOG2G = G == 32 ? 5 : (G == 64 ? 6 : 7);
  static_assert(G == 32 || G == 64 || G == 128, "group");
  // exact |r| sums of the 1-bit slow path, one area per group of the block
  __shared__ unsigned long long q1_acc[BITS == 1 ? kBlock / LANES : 1][kQ1Words];
  __shared__ uint32_t q1_nrm[BITS == 1 ? kBlock / LANES : 1][kQ1Words];
  // 2-bit: the minima, then the steps, of the block's NC * kBlock / LANES groups
  __shared__ float q2_meta[BITS == 2 ? 2 * NC * (kBlock / LANES) : 1];
  const int b = blockIdx.y;
  const int64_t n4 = L.n / 4;
  const int64_t base = (int64_t)b * L.n;
  uint8_t* pk = packed + (int64_t)b * L.tstride;
  uint8_t* meta = pk + L.sec_off[1];
  if (blockIdx.x == 0) zero_padding(pk, L);

  // Lanes past the end work on chunk 0 and store nothing; a group (and the
  // 4 or 8 lanes sharing a code word) never mixes valid and invalid lanes
  // because a tensor holds whole groups.
  f32x4 xs[NC], hs[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kBlock + threadIdx.x;
    const int64_t off = base + (c < n4 ? c : 0) * 4;
    xs[j] = load4<IN>(a + off);
    hs[j] = load4<float>(ahat + off);
  }
  f32x4 evs[NC], hns[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kBlock + threadIdx.x;
    const bool valid = c < n4;
    f32x4 r, cq;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = xs[j][i] - hs[j][i];

    if constexpr (BITS == 1) {
      double s = 0.0;
      uint32_t xmax = 0u, xmin = 0xFFu;  // exponents of the nonzero |r| (subnormals: 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s += (double)fabsf(r[i]);
        const uint32_t u = __float_as_uint(r[i]) & 0x7FFFFFFFu;
        const uint32_t x = max(u >> 23, 1u);
        xmax = u ? max(xmax, x) : xmax;
        xmin = u ? min(xmin, x) : xmin;
      }
      s = group_sum_f64<LANES>(s);
      xmax = group_max_u32<LANES>(xmax);
      xmin = group_min_u32<LANES>(xmin);
      float scale = (float)(s * (1.0 / G));
      if (xmax > xmin + (29u - LOG2G))  // the fp64 sum may have rounded: exact path
        scale = q1_exact_mean<LANES, LOG2G>(r, q1_acc[threadIdx.x / LANES], q1_nrm[threadIdx.x / LANES]);
      uint32_t nib = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool pos = r[i] >= 0.0f;
        nib |= (pos ? 1u : 0u) << i;
        cq[i] = pos ? scale : -scale;
      }
      // word w holds the sign bits of elements 32w .. 32w+31 (8 lanes)
      const uint32_t word = group_or<8>(nib << (4 * (threadIdx.x & 7)));
      if (valid) {
        if ((threadIdx.x & 7) == 0) reinterpret_cast<uint32_t*>(pk)[c >> 3] = word;
        if ((c % LANES) == 0) reinterpret_cast<float*>(meta)[c / LANES] = scale;
      }
    } else {
      float mn = fminf(fminf(r[0], r[1]), fminf(r[2], r[3]));
      float mx = fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]));
      // zeros of the stored minimum and step are normalised to +0 (x + 0)
      mn = group_min<LANES>(mn) + 0.0f;
      mx = group_max<LANES>(mx);
      const float d = (mx - mn) / 3.0f + 0.0f;
      const bool live = d >= FLT_MIN;
      const float inv = 1.0f / d;
      uint32_t code = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t = (r[i] - mn) * inv;
        const float q = live ? fminf(rintf(t), 3.0f) : 0.0f;
        code |= ((uint32_t)q) << (2 * i);
        cq[i] = fmaf(q, d, mn);
      }
      // word w holds the codes of elements 16w .. 16w+15 (4 lanes)
      const uint32_t word = group_or<4>(code << (8 * (threadIdx.x & 3)));
      if (valid && (threadIdx.x & 3) == 0) reinterpret_cast<uint32_t*>(pk)[c >> 2] = word;
      // the group's first lane parks mn and d in LDS; the block writes its
      // groups' (consecutive) minima and steps out together below
      if ((c % LANES) == 0) {
        q2_meta[j * (kBlock / LANES) + threadIdx.x / LANES] = mn;
        q2_meta[NC * (kBlock / LANES) + j * (kBlock / LANES) + threadIdx.x / LANES] = d;
      }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      evs[j][i] = r[i] - cq[i];
      hns[j][i] = hs[j][i] + cq[i];
    }
  }
  if constexpr (BITS == 2) {
    // The block's chunks cover NG consecutive groups: one coalesced store of
    // their minima into the mn section and one of their steps into the d
    // section (a scattered 4-byte store per group and section from the group's
    // own lanes measured 3 % slower on the whole kernel).
    constexpr int NG = NC * (kBlock / LANES);
    static_assert(2 * NG <= kBlock, "one lane per stored minimum and step");
    __syncthreads();
    const int64_t g0 = (int64_t)blockIdx.x * NG;
    if (threadIdx.x < 2 * NG) {
      const int t = threadIdx.x % NG;
      if (g0 + t < L.n / G) {
        float* dst = reinterpret_cast<float*>(threadIdx.x < NG ? meta : pk + L.sec_off[2]);
        dst[g0 + t] = q2_meta[threadIdx.x];
      }
    }
  }
  // every chunk's ahat, then every chunk's e: one array at a time reaches
  // memory in longer runs (2.5 % on this stream pattern, measured)
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kBlock + threadIdx.x;
    if (c < n4) store4(ahat + base + c * 4, hns[j]);
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kBlock + threadIdx.x;
    if (c < n4) store4(e + base + c * 4, evs[j]);
  }
}

template <int G, int BITS, int NC>
__global__ __launch_bounds__(kBlock) void q_decompress_kernel(PeerSet peers, Layout L) {
  constexpr int LANES = G / 4;
  const int b = blockIdx.y;
  const uint8_t* __restrict__ packed = peers.packed[blockIdx.z];
  float* __restrict__ ahat = peers.state[blockIdx.z];
  const int64_t n4 = L.n / 4;
  const int64_t base = (int64_t)b * L.n;
  const uint8_t* pk = packed + (int64_t)b * L.tstride;
  const uint8_t* meta = pk + L.sec_off[1];
  f32x4 hs[NC];
  uint32_t codes[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kBlock + threadIdx.x;
    const int64_t cc = c < n4 ? c : 0;
    hs[j] = load4<float>(ahat + base + cc * 4);
    codes[j] = BITS == 1 ? pk[cc >> 1] : pk[cc];
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t c = ((int64_t)blockIdx.x * NC + j) * kBlock + threadIdx.x;
    if (c >= n4) continue;
    f32x4 h = hs[j];
    if constexpr (BITS == 1) {
      const uint32_t nib = codes[j] >> (4 * (c & 1));
      const float scale = reinterpret_cast<const float*>(meta)[c / LANES];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = h[i] + (((nib >> i) & 1u) ? scale : -scale);
    } else {
      const float mn = reinterpret_cast<const float*>(meta)[c / LANES];
      const float d = reinterpret_cast<const float*>(pk + L.sec_off[2])[c / LANES];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = h[i] + fmaf((float)((codes[j] >> (2 * i)) & 3u), d, mn);
    }
    store4(ahat + base + c * 4, h);
  }
}

namespace {
constexpr int kChunks = 4;     // chunks per lane, sender
constexpr int kDecChunks = 2;  // chunks per lane, receiver

template <typename IN, int G, int BITS>
hipError_t q_compress_t(const void* a, float* ahat, float* e, uint8_t* packed, int batch,
                        const Layout& L, hipStream_t s) {
  const int64_t n4 = L.n / 4;
  const dim3 grid((unsigned)((n4 + kBlock * kChunks - 1) / (kBlock * kChunks)), (unsigned)batch);
  hipLaunchKernelGGL((q_compress_kernel<IN, G, BITS, kChunks>), grid, dim3(kBlock), 0, s,
                     static_cast<const IN*>(a), ahat, e, packed, L);
  return hipGetLastError();
}

template <int G, int BITS>
hipError_t q_decompress_t(const PeerSet& peers, int batch, const Layout& L, hipStream_t s) {
  const int64_t n4 = L.n / 4;
  const dim3 grid((unsigned)((n4 + kBlock * kDecChunks - 1) / (kBlock * kDecChunks)), (unsigned)batch,
                  (unsigned)peers.count);
  hipLaunchKernelGGL((q_decompress_kernel<G, BITS, kDecChunks>), grid, dim3(kBlock), 0, s, peers, L);
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
hipError_t q_decompress_g(int group, const PeerSet& peers, int batch, const Layout& L,
                          hipStream_t s) {
  switch (group) {
    case 32: return q_decompress_t<32, BITS>(peers, batch, L, s);
    case 64: return q_decompress_t<64, BITS>(peers, batch, L, s);
    case 128: return q_decompress_t<128, BITS>(peers, batch, L, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_q_compress(int bits, int group, bool bf16_input, const void* a, float* ahat,
                             float* e, uint8_t* packed, int batch, const Layout& L, hipStream_t s) {
  return bits == 1 ? q_compress_g<1>(group, bf16_input, a, ahat, e, packed, batch, L, s)
                   : q_compress_g<2>(group, bf16_input, a, ahat, e, packed, batch, L, s);
}

hipError_t launch_q_decompress(int bits, int group, const PeerSet& peers, int batch,
                               const Layout& L, hipStream_t s) {
  return bits == 1 ? q_decompress_g<1>(group, peers, batch, L, s)
                   : q_decompress_g<2>(group, peers, batch, L, s);
}

}  // namespace rc
