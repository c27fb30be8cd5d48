// Internal interface between the C ABI (plan.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/librescomp.h"

namespace rc {

// Per-tensor packed layout: up to 4 sections, each at a multiple of 256 bytes
// inside the tensor's block; blocks of consecutive tensors are tstride apart.
struct Layout {
  int64_t rows = 0, cols = 0;
  int64_t n = 0;        // elements per tensor (rows * cols)
  int64_t tstride = 0;  // packed bytes per tensor (multiple of 256)
  int64_t sec_off[4] = {0, 0, 0, 0};
  int64_t sec_len[4] = {0, 0, 0, 0};
  int nsec = 0;
};

// Receivers decoded by one decompress launch: peer p applies packed[p] to
// state[p] (both [batch] tensors); the launch grid's z index is the peer.
constexpr int kMaxPeers = 8;
struct PeerSet {
  const uint8_t* packed[kMaxPeers];
  float* state[kMaxPeers];
  int count;
};

// Q1 (bits = 1) and Q2 (bits = 2) group quantisation, group in {32, 64, 128}.
hipError_t launch_q_compress(int bits, int group, bool bf16_input, const void* a, float* ahat,
                             float* e, uint8_t* packed, int batch, const Layout& L, hipStream_t s);
hipError_t launch_q_decompress(int bits, int group, const PeerSet& peers, int batch,
                               const Layout& L, hipStream_t s);

// 2:16 block sparsifier.
hipError_t launch_nm_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, hipStream_t s);
hipError_t launch_nm_decompress(const PeerSet& peers, int batch, const Layout& L, hipStream_t s);

// Low-rank workspace, carved out of one device allocation by the plan.
// ntiles = ceil(rows / 64); rows_pad = 64 * ntiles.
// rank is the width the iteration runs at (every piece below is sized by it);
// pay_rank (<= rank) is the rank the payload carries. Rank 8 runs at width 16
// with start-matrix columns 8 .. 15 zero: those columns stay exactly zero, are
// declared dead by every CholeskyQR pass and are not sent.
struct LowRankWork {
  int rank = 0, pay_rank = 0, iters = 0;
  bool bf16_factors = false;  // factors sent as bf16 instead of INT4 + scales
  int64_t ntiles = 0, rows_pad = 0;
  uint16_t* R = nullptr;     // bf16 residual: 64 x 128 tiles, column chunk, then tensor, then band (per launch)
  float* P = nullptr;        // fp32 panel [batch][rows][rank]
  uint16_t* Pbt = nullptr;   // bf16 orthonormal panel, transposed [batch][rank][rows_pad] in 32-row groups
  float* Qt = nullptr;       // fp32 Q^T [batch][rank][cols]
  uint16_t* Q0t = nullptr;   // bf16 start matrix, transposed [batch][rank][cols] in 32-column groups
  uint16_t* Qtb = nullptr;   // bf16 Q^T for the next product [batch][rank][cols] in 32-column groups
  float* gpart = nullptr;    // per-64-row-tile Gram partials [batch][ntiles][rank][rank]
  float* gsum = nullptr;     // summed Gram matrices [batch][rank][rank]
  float* linv = nullptr;     // inverse Cholesky factor, dead rows zeroed [batch][rank][rank]
  uint32_t* amax = nullptr;  // column absmax bits of U and V [batch][2][rank]
  uint32_t* dead = nullptr;  // optional: count of dead Cholesky pivots (sent columns)
};

// Reads of a low-rank plan's R in the pattern of its R*Q pass (0) or R^T*P
// pass (1), nothing else (diagnostics; sink is never written).
hipError_t launch_r_probe(int pattern, const uint16_t* R, int n, int m, int batch, int ntiles, int rows_pad,
                          uint32_t* sink, hipStream_t s);

// Start matrices: Q0t bf16 [batch][rank][cols] (rows kp .. rank-1 zero) from a
// device fp32 q0 [batch][cols][kp], or, when q0 is null, drawn from `seed`
// (SplitMix64 + Box-Muller, as the public header defines).
hipError_t launch_lr_q0(const float* q0, uint64_t seed, uint16_t* Q0t, int batch, int cols, int kp,
                        int rank, hipStream_t s);

// Host side (plan.cpp): request validation, packed layout, and the low-rank
// workspace pieces placed from `base` on (null: sizes only); returns the bytes.
rc_status_t validate(const rc_shape_t& sh, rc_dtype_t dtype, rc_scheme_t scheme, const rc_params_t* p);
rc_status_t make_layout(const rc_shape_t& sh, rc_dtype_t dtype, rc_scheme_t scheme, const rc_params_t& p,
                        Layout* L);
int64_t carve_lowrank(LowRankWork* w, const rc_shape_t& shape, const rc_params_t& p, void* base);

hipError_t launch_lr_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const Layout& L, const LowRankWork& w,
                              hipStream_t s);
// Receiver: every peer in one launch (the decode reads only the packed bytes).
hipError_t launch_lr_decompress(const PeerSet& peers, int batch, const Layout& L,
                                const LowRankWork& w, hipStream_t s);

// Debug checks: count[0] += number of non-finite values in a [n] (bf16 or
// fp32) and ahat [n] fp32; fill a u32 (kernels, so the calls can be captured).
hipError_t launch_count_nonfinite(const void* a, bool bf16, const float* ahat, int64_t n,
                                  uint32_t* count, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, hipStream_t s);

// Otil-style block selection: tokens on a grid of grid_w columns, 8 x 8-token
// blocks (nblocks per tensor, raster order), keep blocks sent per step.
constexpr int kBsMaxBlocks = 4096;
struct BlockSel {
  int64_t rows = 0, cols = 0;
  int grid_w = 0, nblocks = 0, keep = 0;
  Layout L;
};
// Per-tensor state of a launch (pointers already offset to its first tensor):
// part: fp64 [batch][nblocks][8][3] row partial sums (scratch); visited: u8
// [batch][nblocks] round state; prev: the previous step's activation
// [batch][rows][cols] in the input dtype, or null to score against ahat;
// have_prev: u8 [batch], 0 until the tensor's prev holds an activation.
struct BsState {
  double* part = nullptr;
  uint8_t* visited = nullptr;
  void* prev = nullptr;
  uint8_t* have_prev = nullptr;
};
hipError_t launch_bs_compress(bool bf16_input, const void* a, float* ahat, float* e,
                              uint8_t* packed, int batch, const BlockSel& S, const BsState& st,
                              hipStream_t s);
hipError_t launch_bs_decompress(bool bf16_input, const PeerSet& peers, int batch, const BlockSel& S,
                                hipStream_t s);
hipError_t launch_bs_reset(uint8_t* visited, int64_t n, uint8_t* have_prev, int batch, hipStream_t s);

}  // namespace rc
