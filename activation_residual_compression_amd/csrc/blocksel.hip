// Otil-style block selection: send the few token blocks that changed most.
//
// Method: "Otil: Accelerating Diffusion Model Inference via
// Communication-Efficient Multi-GPU Parallelism", Key designs 1-3: the tokens
// of a share form a spatial grid cut into 8 x 8 square blocks; after each step
// every block is scored by the cosine dissimilarity between its values at this
// step and at the previous step, the top-k blocks among those not yet visited
// in the current round are sent, and the round restarts once every block has
// been visited. A sent block replaces the receiver's copy exactly, so in the
// residual framework of the CompactFusion notes (Overall framework, Error
// feedback) the sender keeps e = a_t - ahat on every block it did not send and
// e = 0 on the blocks it sent.
//
// The previous step's activation is kept by the plan (a copy of the last a_t,
// in the input dtype), written by the score pass as it reads the new one. On
// the first step after a reset there is no copy yet; there the sender's
// reconstruction is the previous activation (the warm-up sends a_0 in full),
// so the score pass compares with ahat. (Option: score against ahat, the
// receiver's copy, on every step; then no copy is kept.)
//
// Sender, per step (three launches):
//   bs_score_kernel  one workgroup per block row (8 tokens): streams a_t, ahat
//                    and the previous activation once (4 consecutive channels
//                    per lane), writes e = a_t - ahat everywhere and the new
//                    previous activation, and reduces <a, p>, |a|^2, |p|^2 in
//                    fp64 (exact fp32 products) for the row.
//   bs_select_kernel one workgroup per tensor: sums each block's 8 row
//                    partials, d = 1 - <a,p> / (|a| |p|) (both blocks
//                    zero -> 0, one zero -> 1), restarts the round if every
//                    block was visited, ranks every unvisited block by
//                    (d descending, index ascending), keeps ranks < k, marks
//                    them visited and writes the count and the ascending
//                    indices to the packed header.
//   bs_pack_kernel   one workgroup per sent slot and block row: copies a_t
//                    values into the packed stream and sets ahat = a_t,
//                    e = 0 there; unused slots are zero-filled.
// Receiver: bs_unpack_kernel writes every sent block into the receiver state.
#include "device_common.hpp"
#include "launch.hpp"

namespace rc {

constexpr int kBsThreads = 256;

// Tokens of block i: 8 rows of the grid, each 8 consecutive tokens; returns the
// first token of row dy of the block.
__device__ __forceinline__ int64_t bs_row_token(int i, int dy, int grid_w) {
  const int nbx = grid_w / 8;
  const int by = i / nbx, bx = i % nbx;
  return (int64_t)(by * 8 + dy) * grid_w + bx * 8;
}

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  // wave: butterfly over 64 lanes; then the 4 wave sums in wave order
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup per (block row, block, tensor): e = a - ahat over the row's 8
// tokens x m channels, and the row's fp64 partial sums <a, p>, |a|^2, |p|^2
// into part[tensor][block][row][3], where p is the previous step's activation
// (PREV: the plan's copy, or ahat while have_prev[b] is 0; it is replaced by a)
// or the receiver's copy ahat (!PREV).
template <typename IN, bool PREV>
__global__ __launch_bounds__(kBsThreads) void bs_score_kernel(const IN* __restrict__ a,
                                                              const float* __restrict__ ahat,
                                                              float* __restrict__ e,
                                                              IN* __restrict__ prev,
                                                              const uint8_t* __restrict__ have_prev,
                                                              double* __restrict__ part,
                                                              BlockSel S) {
  __shared__ double red[3][4];
  const int dy = blockIdx.x & 7, i = blockIdx.x >> 3, b = blockIdx.y;
  const int64_t m = S.cols;
  const int64_t seg = 8 * m;  // elements of one block row (8 tokens x m channels)
  const int64_t off0 = (int64_t)b * S.rows * m + bs_row_token(i, dy, S.grid_w) * m;
  const bool from_copy = PREV && have_prev[b] != 0;
  double dot = 0.0, na = 0.0, nb = 0.0;
  for (int64_t c = 4 * threadIdx.x; c < seg; c += 4 * kBsThreads) {
    const f32x4 x = load4<IN>(a + off0 + c);
    const f32x4 h = load4<float>(ahat + off0 + c);
    const f32x4 p = from_copy ? load4<IN>(prev + off0 + c) : h;
    f32x4 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      r[t] = x[t] - h[t];
      dot += (double)x[t] * (double)p[t];
      na += (double)x[t] * (double)x[t];
      nb += (double)p[t] * (double)p[t];
    }
    store4(e + off0 + c, r);
    if constexpr (PREV) {
      if constexpr (sizeof(IN) == 2)
        *reinterpret_cast<u32x2*>(prev + off0 + c) = *reinterpret_cast<const u32x2*>(a + off0 + c);
      else
        store4(reinterpret_cast<float*>(prev) + off0 + c, x);
    }
  }
  dot = block_sum_f64(dot, red[0]);
  na = block_sum_f64(na, red[1]);
  nb = block_sum_f64(nb, red[2]);
  if (threadIdx.x == 0) {
    double* o = part + (((int64_t)b * S.nblocks + i) * 8 + dy) * 3;
    o[0] = dot;
    o[1] = na;
    o[2] = nb;
  }
}

// One workgroup per tensor. part: row partial sums [batch][nblocks][8][3],
// combined per block as ((r0 + r1) + (r2 + r3)) + ((r4 + r5) + (r6 + r7));
// visited: [batch][nblocks]; the packed header of tensor b is u32 [1 + keep]:
// count, then block indices ascending.
__global__ __launch_bounds__(kBsThreads) void bs_select_kernel(const double* __restrict__ part,
                                                               uint8_t* __restrict__ visited,
                                                               uint8_t* __restrict__ have_prev,
                                                               uint8_t* __restrict__ packed,
                                                               BlockSel S) {
  __shared__ double sd[kBsMaxBlocks];
  __shared__ uint8_t sv[kBsMaxBlocks];
  __shared__ int sel_flag[kBsMaxBlocks];
  __shared__ int wave_cnt[4];
  __shared__ int all_visited;
  const int b = blockIdx.x, K = S.nblocks;
  uint8_t* vis = visited + (int64_t)b * K;
  uint32_t* head = reinterpret_cast<uint32_t*>(packed + (int64_t)b * S.L.tstride);
  if (threadIdx.x == 0) all_visited = 1;
  __syncthreads();
  for (int i = threadIdx.x; i < K; i += kBsThreads) {
    const double* p = part + ((int64_t)b * K + i) * 24;
    double v3[3];
#pragma unroll
    for (int q = 0; q < 3; ++q)
      v3[q] = ((p[0 * 3 + q] + p[1 * 3 + q]) + (p[2 * 3 + q] + p[3 * 3 + q])) +
              ((p[4 * 3 + q] + p[5 * 3 + q]) + (p[6 * 3 + q] + p[7 * 3 + q]));
    const double dot = v3[0], na = v3[1], nb = v3[2];
    double dv;
    if (na == 0.0 && nb == 0.0) dv = 0.0;
    else if (na == 0.0 || nb == 0.0) dv = 1.0;
    else dv = 1.0 - dot / sqrt(na * nb);
    sd[i] = dv;
    sv[i] = vis[i];
    if (!vis[i]) all_visited = 0;  // benign race: every writer stores 0
  }
  __syncthreads();
  if (all_visited)
    for (int i = threadIdx.x; i < K; i += kBsThreads) sv[i] = 0;
  __syncthreads();
  // rank of an unvisited block among the unvisited: (score descending, index ascending)
  for (int i = threadIdx.x; i < K; i += kBsThreads) {
    int sel = 0;
    if (!sv[i]) {
      const double di = sd[i];
      int rank = 0;
#pragma unroll 16
      for (int j = 0; j < K; ++j) {  // branch-free and unrolled, so the LDS reads overlap
        const double dj = sd[j];
        rank += (int)(sv[j] == 0) & ((int)(dj > di) | ((int)(dj == di) & (int)(j < i)));
      }
      sel = rank < S.keep;
    }
    sel_flag[i] = sel;
  }
  __syncthreads();
  // ascending slot of every selected block: exclusive prefix count in index order,
  // one chunk of indices per thread (chunks in thread order)
  const int per = (K + kBsThreads - 1) / kBsThreads;
  const int i0 = threadIdx.x * per, i1 = min(K, i0 + per);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += sel_flag[i];
  // inclusive scan of `mine` across the workgroup
  int v = mine;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wave_cnt[w] = v;
  __syncthreads();
  int before = 0;
  for (int q = 0; q < w; ++q) before += wave_cnt[q];
  int slot = before + v - mine;
  for (int i = i0; i < i1; ++i) {
    if (sel_flag[i]) {
      head[1 + slot] = (uint32_t)i;
      ++slot;
      vis[i] = 1;
    } else {
      vis[i] = sv[i];
    }
  }
  __syncthreads();
  const int count = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
  if (threadIdx.x == 0) {
    head[0] = (uint32_t)count;
    have_prev[b] = 1;  // the score pass has stored this step's activation
  }
  for (int s = count + threadIdx.x; s < S.keep; s += kBsThreads) head[1 + s] = 0u;
}

// One workgroup per (slot, block row, tensor): copy the row's values (8 tokens x
// m channels), update the sender state there.
template <typename IN>
__global__ __launch_bounds__(kBsThreads) void bs_pack_kernel(const IN* __restrict__ a,
                                                             float* __restrict__ ahat,
                                                             float* __restrict__ e,
                                                             uint8_t* __restrict__ packed,
                                                             BlockSel S) {
  const int s = blockIdx.x >> 3, dy = blockIdx.x & 7, b = blockIdx.y;
  const int64_t m = S.cols, seg = 8 * m;
  uint8_t* pk = packed + (int64_t)b * S.L.tstride;
  const uint32_t* head = reinterpret_cast<const uint32_t*>(pk);
  IN* vals = reinterpret_cast<IN*>(pk + S.L.sec_off[1]) + (int64_t)s * 64 * m + dy * seg;
  if (blockIdx.x == 0) {  // the tensor's section padding
    for (int q = 0; q < S.L.nsec; ++q) {
      const int64_t start = S.L.sec_off[q] + S.L.sec_len[q];
      const int64_t end = (q + 1 < S.L.nsec) ? S.L.sec_off[q + 1] : S.L.tstride;
      for (int64_t t = start + threadIdx.x; t < end; t += kBsThreads) pk[t] = 0;
    }
  }
  if (s >= (int)head[0]) {  // unused slot
    for (int64_t c = threadIdx.x; c < seg; c += kBsThreads) vals[c] = IN(0);
    return;
  }
  const int64_t off0 = (int64_t)b * S.rows * m + bs_row_token((int)head[1 + s], dy, S.grid_w) * m;
  for (int64_t c = 4 * threadIdx.x; c < seg; c += 4 * kBsThreads) {
    const f32x4 x = load4<IN>(a + off0 + c);
    store4(ahat + off0 + c, x);
    store4(e + off0 + c, f32x4{0.f, 0.f, 0.f, 0.f});
    if constexpr (sizeof(IN) == 2)
      *reinterpret_cast<u32x2*>(vals + c) = *reinterpret_cast<const u32x2*>(a + off0 + c);
    else
      *reinterpret_cast<f32x4*>(vals + c) = x;
  }
}

// Receiver: one workgroup per (slot, block row, tensor x peer).
template <typename IN>
__global__ __launch_bounds__(kBsThreads) void bs_unpack_kernel(PeerSet peers, BlockSel S, int batch) {
  const int s = blockIdx.x >> 3, dy = blockIdx.x & 7;
  const int peer = blockIdx.y / batch, b = blockIdx.y % batch;
  const int64_t m = S.cols, seg = 8 * m;
  const uint8_t* pk = peers.packed[peer] + (int64_t)b * S.L.tstride;
  const uint32_t* head = reinterpret_cast<const uint32_t*>(pk);
  if (s >= (int)head[0]) return;
  const IN* vals = reinterpret_cast<const IN*>(pk + S.L.sec_off[1]) + (int64_t)s * 64 * m + dy * seg;
  float* st = peers.state[peer] + (int64_t)b * S.rows * m + bs_row_token((int)head[1 + s], dy, S.grid_w) * m;
  for (int64_t c = 4 * threadIdx.x; c < seg; c += 4 * kBsThreads) {
    f32x4 v;
    if constexpr (sizeof(IN) == 2) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(vals + c);
      v = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    } else {
      v = *reinterpret_cast<const f32x4*>(vals + c);
    }
    store4(st + c, v);
  }
}

// Round-robin state of every tensor back to "nothing visited", and no previous
// activation (a fill kernel, so the call can sit in a captured graph).
__global__ __launch_bounds__(kBsThreads) void bs_clear_kernel(uint8_t* __restrict__ visited, int64_t n,
                                                              uint8_t* __restrict__ have_prev, int batch) {
  const int64_t i = (int64_t)blockIdx.x * kBsThreads + threadIdx.x;
  if (i < n) visited[i] = 0;
  if (i < batch) have_prev[i] = 0;
}

template <typename IN>
hipError_t bs_compress_t(const void* a, float* ahat, float* e, uint8_t* packed, int batch,
                         const BlockSel& S, const BsState& st, hipStream_t s) {
  const dim3 g_rows(S.nblocks * 8, batch), g_slots(S.keep * 8, batch);
  const IN* x = static_cast<const IN*>(a);
  IN* prev = static_cast<IN*>(st.prev);
  if (prev)
    hipLaunchKernelGGL((bs_score_kernel<IN, true>), g_rows, dim3(kBsThreads), 0, s, x, ahat, e, prev,
                       st.have_prev, st.part, S);
  else
    hipLaunchKernelGGL((bs_score_kernel<IN, false>), g_rows, dim3(kBsThreads), 0, s, x, ahat, e, prev,
                       st.have_prev, st.part, S);
  hipLaunchKernelGGL(bs_select_kernel, dim3(batch), dim3(kBsThreads), 0, s, st.part, st.visited,
                     st.have_prev, packed, S);
  hipLaunchKernelGGL((bs_pack_kernel<IN>), g_slots, dim3(kBsThreads), 0, s, x, ahat, e, packed, S);
  return hipGetLastError();
}

hipError_t launch_bs_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const BlockSel& S, const BsState& st,
                              hipStream_t s) {
  return bf16_input ? bs_compress_t<uint16_t>(a, ahat, e, packed, batch, S, st, s)
                    : bs_compress_t<float>(a, ahat, e, packed, batch, S, st, s);
}

hipError_t launch_bs_decompress(bool bf16_input, const PeerSet& peers, int batch, const BlockSel& S,
                                hipStream_t s) {
  const dim3 grid(S.keep * 8, batch * peers.count);
  if (bf16_input)
    hipLaunchKernelGGL((bs_unpack_kernel<uint16_t>), grid, dim3(kBsThreads), 0, s, peers, S, batch);
  else
    hipLaunchKernelGGL((bs_unpack_kernel<float>), grid, dim3(kBsThreads), 0, s, peers, S, batch);
  return hipGetLastError();
}

hipError_t launch_bs_reset(uint8_t* visited, int64_t n, uint8_t* have_prev, int batch, hipStream_t s) {
  hipLaunchKernelGGL(bs_clear_kernel, dim3((unsigned)((n + kBsThreads - 1) / kBsThreads)),
                     dim3(kBsThreads), 0, s, visited, n, have_prev, batch);
  return hipGetLastError();
}

}  // namespace rc
