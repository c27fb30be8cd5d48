// C ABI of librescomp: plan validation, packed-layout arithmetic, workspace,
// and dispatch to the kernels. Host code only; every step of the path runs in
// the HIP kernels launched from here.
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/librescomp.h"
#include "../../include/librescomp_diag.h"
#include "launch.hpp"

struct rc_plan {
  rc_shape_t shape;
  rc_dtype_t dtype;
  rc_scheme_t scheme;
  rc_params_t params;  // q0 cleared after the start matrices are set up
  rc::Layout layout;
  size_t packed_bytes = 0;
  int device = 0;
  // low rank
  void* ws = nullptr;
  size_t ws_bytes = 0;
  rc::LowRankWork lr;
  // low rank, batch >= 2: rc_compress runs the second half of the batch on a
  // stream of the plan's own, forked from and joined back to the caller's
  // stream with these events, so that one half's latency-bound factorisation
  // kernels overlap the other half's streaming kernels
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // block selection, in ws: fp64 row partial sums [B][K][8][3] (scratch), round
  // state [B][K], have-previous flags [B], previous activation [B][rows][cols]
  // (input dtype; absent with RC_BS_SCORE_LAST_SENT)
  rc::BlockSel bs;
  double* bs_score = nullptr;
  uint8_t* bs_visited = nullptr;
  uint8_t* bs_have_prev = nullptr;
  void* bs_prev = nullptr;
  // debug checks (RC_CHECK_FINITE, RC_LR_CHECK_NUMERIC): one u32 counter
  uint32_t* check = nullptr;
  // chunk-done events of rc_compress_send, created on first use on ev_device
  std::vector<hipEvent_t> events;
  int ev_device = 0;
};

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxElems = int64_t(1) << 40;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

rc_status_t rc::make_layout(const rc_shape_t& sh, rc_dtype_t dtype, rc_scheme_t scheme,
                            const rc_params_t& p, Layout* L) {
  L->rows = sh.rows;
  L->cols = sh.cols;
  L->n = (int64_t)sh.rows * sh.cols;
  const int64_t N = L->n;
  int64_t len[4] = {0, 0, 0, 0};
  int nsec = 0;
  switch (scheme) {
    case RC_Q1: len[0] = N / 8; len[1] = 4 * (N / p.group); nsec = 2; break;
    case RC_Q2: len[0] = N / 4; len[1] = 4 * (N / p.group); len[2] = 4 * (N / p.group); nsec = 3; break;
    case RC_NM: len[0] = 4 * (N / 16); len[1] = N / 16; nsec = 2; break;
    case RC_LOWRANK:
      if (p.flags & RC_LR_BF16_FACTORS) {
        len[0] = 2 * (int64_t)sh.rows * p.rank;
        len[1] = 2 * (int64_t)sh.cols * p.rank;
        nsec = 2;
        break;
      }
      len[0] = (int64_t)sh.rows * p.rank / 2;
      len[1] = (int64_t)sh.cols * p.rank / 2;
      len[2] = 4 * (int64_t)p.rank;
      len[3] = 4 * (int64_t)p.rank;
      nsec = 4;
      break;
    case RC_BLOCKSEL:
      len[0] = 4 * (1 + (int64_t)p.keep_blocks);
      len[1] = (int64_t)p.keep_blocks * 64 * sh.cols * (dtype == RC_BF16 ? 2 : 4);
      nsec = 2;
      break;
    default: return RC_ERR_INVALID_ARG;
  }
  int64_t off = 0;
  for (int s = 0; s < nsec; ++s) {
    L->sec_off[s] = off;
    L->sec_len[s] = len[s];
    off += align_up(len[s]);
  }
  L->nsec = nsec;
  L->tstride = off;
  return RC_OK;
}

rc_status_t rc::validate(const rc_shape_t& sh, rc_dtype_t dtype, rc_scheme_t scheme,
                         const rc_params_t* p) {
  if (!p) return RC_ERR_INVALID_ARG;
  if (sh.batch < 1 || sh.rows < 1 || sh.cols < 1) return RC_ERR_INVALID_ARG;
  if (sh.batch > 65535) return RC_ERR_UNSUPPORTED;  // one grid row per tensor
  if ((int64_t)sh.batch * sh.rows * sh.cols >= kMaxElems) return RC_ERR_UNSUPPORTED;
  if (dtype != RC_BF16 && dtype != RC_F32) return RC_ERR_INVALID_ARG;
  uint32_t allowed = RC_CHECK_FINITE;
  if (scheme == RC_LOWRANK) allowed |= RC_LR_BF16_FACTORS | RC_LR_ONE_STREAM | RC_LR_CHECK_NUMERIC;
  if (scheme == RC_BLOCKSEL) allowed |= RC_BS_SCORE_LAST_SENT;
  if (p->flags & ~allowed) return RC_ERR_INVALID_ARG;
  switch (scheme) {
    case RC_Q1:
    case RC_Q2:
      if (p->group != 32 && p->group != 64 && p->group != 128) {
        return (p->group > 0 && p->group % 8 == 0) ? RC_ERR_UNSUPPORTED : RC_ERR_INVALID_ARG;
      }
      if (sh.cols % p->group) return RC_ERR_INVALID_ARG;
      return RC_OK;
    case RC_NM:
      if (p->nm_keep < 1 || p->nm_block < 2 || p->nm_keep >= p->nm_block) return RC_ERR_INVALID_ARG;
      if (p->nm_keep != 2 || p->nm_block != 16) return RC_ERR_UNSUPPORTED;
      if (sh.cols % 16) return RC_ERR_INVALID_ARG;
      return RC_OK;
    case RC_LOWRANK:
      if (p->rank < 1 || p->iters < 1 || p->iters > 16) return RC_ERR_INVALID_ARG;
      if (p->q0 && ((uintptr_t)p->q0 & 3u)) return RC_ERR_ALIGNMENT;
      if (p->rank != 8 && (p->rank % 16 || p->rank > 64)) return RC_ERR_UNSUPPORTED;
      if (p->rank > sh.rows || p->rank > sh.cols) return RC_ERR_INVALID_ARG;
      if (sh.cols % 64) return RC_ERR_INVALID_ARG;
      if (sh.rows > 65535 * 32) return RC_ERR_UNSUPPORTED;  // reconstruct grid: 32-row chunks in y
      return RC_OK;
    case RC_BLOCKSEL: {
      if (p->grid_w < 8 || p->grid_w % 8 || sh.rows % p->grid_w || (sh.rows / p->grid_w) % 8)
        return RC_ERR_INVALID_ARG;
      if (sh.cols % 4) return RC_ERR_INVALID_ARG;
      const int64_t K = (int64_t)sh.rows / 64;
      if (K > rc::kBsMaxBlocks) return RC_ERR_UNSUPPORTED;
      if (p->keep_blocks < 1 || p->keep_blocks > K) return RC_ERR_INVALID_ARG;
      return RC_OK;
    }
  }
  return RC_ERR_INVALID_ARG;
}

// Low-rank workspace pieces for `shape` and `p`, each 256-byte aligned, placed
// from `base` on (or only sized, when base is null). Returns the bytes needed.
int64_t rc::carve_lowrank(LowRankWork* w, const rc_shape_t& shape, const rc_params_t& p, void* base) {
  const int64_t B = shape.batch, n = shape.rows, m = shape.cols;
  const int64_t kp = p.rank, k = kp < 16 ? 16 : kp;  // payload rank, iteration width
  struct Piece { void** dst; int64_t bytes; };
  w->rank = (int)k;
  w->pay_rank = (int)kp;
  w->iters = p.iters;
  w->bf16_factors = (p.flags & RC_LR_BF16_FACTORS) != 0;
  w->ntiles = (n + 63) / 64;
  w->rows_pad = 64 * w->ntiles;
  Piece pieces[] = {
      {(void**)&w->R, B * w->rows_pad * ((m + 127) / 128 * 128) * 2},
      {(void**)&w->P, B * n * k * 4},
      {(void**)&w->Pbt, B * k * w->rows_pad * 2},
      {(void**)&w->Qt, B * k * m * 4},
      {(void**)&w->Q0t, B * k * m * 2},
      {(void**)&w->Qtb, B * k * m * 2},
      {(void**)&w->gpart, B * w->ntiles * k * k * 4},
      {(void**)&w->gsum, B * k * k * 4},
      {(void**)&w->linv, B * k * k * 4},
      {(void**)&w->amax, B * 2 * k * 4},
  };
  int64_t off = 0;
  for (auto& pc : pieces) {
    *pc.dst = base ? static_cast<char*>(base) + off : nullptr;
    off += align_up(pc.bytes);
  }
  return off;
}

namespace {

rc_status_t setup_lowrank(rc_plan* pl, const float* q0) {
  const int64_t B = pl->shape.batch, m = pl->shape.cols;
  rc::LowRankWork& w = pl->lr;
  const int64_t total = rc::carve_lowrank(&w, pl->shape, pl->params, nullptr);
  hipError_t err = hipGetDevice(&pl->device);
  if (err != hipSuccess) return RC_ERR_HIP;
  err = hipMalloc(&pl->ws, (size_t)total);
  if (err != hipSuccess) { pl->ws = nullptr; return RC_ERR_HIP; }
  pl->ws_bytes = (size_t)total;
  rc::carve_lowrank(&w, pl->shape, pl->params, pl->ws);
  const int64_t kp = w.pay_rank, k = w.rank;
  // Q0 [B][m][kp] fp32 (device, or drawn from the seed) -> bf16 Q0^T [B][k][m],
  // once; rows kp .. k-1 of Q0^T are zero. The plan reads q0 before returning.
  err = rc::launch_lr_q0(q0, pl->params.seed, w.Q0t, (int)B, (int)m, (int)kp, (int)k, nullptr);
  if (err == hipSuccess) err = hipStreamSynchronize(nullptr);
  if (err != hipSuccess) return RC_ERR_HIP;
  if (B >= 2 && !(pl->params.flags & RC_LR_ONE_STREAM)) {
    if (hipStreamCreateWithFlags(&pl->side, hipStreamNonBlocking) != hipSuccess) {
      pl->side = nullptr;
      return RC_ERR_HIP;
    }
    if (hipEventCreateWithFlags(&pl->fork, hipEventDisableTiming) != hipSuccess) {
      pl->fork = nullptr;
      return RC_ERR_HIP;
    }
    if (hipEventCreateWithFlags(&pl->join, hipEventDisableTiming) != hipSuccess) {
      pl->join = nullptr;
      return RC_ERR_HIP;
    }
  }
  return RC_OK;
}

// Block selection: fp64 row partial sums, the round state and the previous
// activation, per tensor; the state starts cleared.
rc_status_t setup_blocksel(rc_plan* pl) {
  const int64_t B = pl->shape.batch, K = (int64_t)pl->shape.rows / 64;
  rc::BlockSel& S = pl->bs;
  S.rows = pl->shape.rows;
  S.cols = pl->shape.cols;
  S.grid_w = pl->params.grid_w;
  S.nblocks = (int)K;
  S.keep = pl->params.keep_blocks;
  S.L = pl->layout;
  const bool keep_prev = !(pl->params.flags & RC_BS_SCORE_LAST_SENT);
  const int64_t score_bytes = align_up(B * K * 8 * 3 * 8);  // fp64 row partial sums
  const int64_t state_bytes = align_up(B * K + B);          // visited, then have-previous
  const int64_t prev_bytes =
      keep_prev ? align_up(B * pl->layout.n * (pl->dtype == RC_BF16 ? 2 : 4)) : 0;
  const int64_t total = score_bytes + state_bytes + prev_bytes;
  if (hipGetDevice(&pl->device) != hipSuccess) return RC_ERR_HIP;
  if (hipMalloc(&pl->ws, (size_t)total) != hipSuccess) { pl->ws = nullptr; return RC_ERR_HIP; }
  pl->ws_bytes = (size_t)total;
  pl->bs_score = static_cast<double*>(pl->ws);
  pl->bs_visited = static_cast<uint8_t*>(pl->ws) + score_bytes;
  pl->bs_have_prev = pl->bs_visited + B * K;
  pl->bs_prev = keep_prev ? static_cast<uint8_t*>(pl->ws) + score_bytes + state_bytes : nullptr;
  if (hipMemset(pl->bs_visited, 0, (size_t)(B * K + B)) != hipSuccess) return RC_ERR_HIP;
  return RC_OK;
}

// The low-rank workspace seen from tensor b0 on (every piece is per tensor).
rc::LowRankWork lr_slice(const rc::LowRankWork& w, const rc::Layout& L, int64_t b0) {
  const int64_t n = L.rows, m = L.cols, k = w.rank;
  rc::LowRankWork s = w;
  s.R += b0 * w.rows_pad * ((m + 127) / 128 * 128);
  s.P += b0 * n * k;
  s.Pbt += b0 * k * w.rows_pad;
  s.Qt += b0 * k * m;
  s.Q0t += b0 * k * m;
  s.Qtb += b0 * k * m;
  s.gpart += b0 * w.ntiles * k * k;
  s.gsum += b0 * k * k;
  s.linv += b0 * k * k;
  s.amax += b0 * 2 * k;
  return s;
}

// Sender step on tensors [b0, b0 + nb) of the batch.
hipError_t compress_range(rc_plan* pl, hipStream_t stream, const void* a_t, const rc_state_t* st,
                          uint8_t* packed, int b0, int nb) {
  const int64_t N = pl->layout.n;
  const bool bf16 = pl->dtype == RC_BF16;
  const void* a = static_cast<const char*>(a_t) + (size_t)b0 * N * (bf16 ? 2 : 4);
  float* ahat = st->ahat + (size_t)b0 * N;
  float* e = st->e + (size_t)b0 * N;
  uint8_t* pk = packed + (size_t)b0 * pl->layout.tstride;
  switch (pl->scheme) {
    case RC_Q1:
    case RC_Q2:
      return rc::launch_q_compress(pl->scheme == RC_Q1 ? 1 : 2, pl->params.group, bf16, a, ahat, e,
                                   pk, nb, pl->layout, stream);
    case RC_NM:
      return rc::launch_nm_compress(bf16, a, ahat, e, pk, nb, pl->layout, stream);
    case RC_LOWRANK:
      return rc::launch_lr_compress(bf16, a, ahat, e, pk, nb, pl->layout,
                                    b0 ? lr_slice(pl->lr, pl->layout, b0) : pl->lr, stream);
    case RC_BLOCKSEL: {
      const int64_t K = pl->bs.nblocks;
      rc::BsState bst;
      bst.part = pl->bs_score + b0 * K * 24;
      bst.visited = pl->bs_visited + b0 * K;
      bst.have_prev = pl->bs_have_prev + b0;
      bst.prev = pl->bs_prev ? static_cast<char*>(pl->bs_prev) + (size_t)b0 * N * (bf16 ? 2 : 4) : nullptr;
      return rc::launch_bs_compress(bf16, a, ahat, e, pk, nb, pl->bs, bst, stream);
    }
  }
  return hipErrorInvalidValue;
}

// Receiver step for up to kMaxPeers states.
hipError_t decompress_peers(rc_plan* pl, hipStream_t stream, const uint8_t* const* packed,
                            float* const* states, int npeers) {
  rc::PeerSet ps{};
  ps.count = npeers;
  for (int p = 0; p < npeers; ++p) {
    ps.packed[p] = packed[p];
    ps.state[p] = states[p];
  }
  switch (pl->scheme) {
    case RC_Q1:
    case RC_Q2:
      return rc::launch_q_decompress(pl->scheme == RC_Q1 ? 1 : 2, pl->params.group, ps,
                                     pl->shape.batch, pl->layout, stream);
    case RC_NM:
      return rc::launch_nm_decompress(ps, pl->shape.batch, pl->layout, stream);
    case RC_LOWRANK:
      return rc::launch_lr_decompress(ps, pl->shape.batch, pl->layout, pl->lr, stream);
    case RC_BLOCKSEL:
      return rc::launch_bs_decompress(pl->dtype == RC_BF16, ps, pl->shape.batch, pl->bs, stream);
  }
  return hipErrorInvalidValue;
}

// Debug checks: launch `count` into the plan's counter (cleared first) on
// `stream`, wait for it, and return the count (or -1 on a HIP error).
template <typename F>
int64_t checked_count(rc_plan* pl, hipStream_t stream, F count) {
  uint32_t host = 0;
  if (rc::launch_fill_u32(pl->check, 0u, stream) != hipSuccess) return -1;
  if (count() != hipSuccess) return -1;
  if (hipStreamSynchronize(stream) != hipSuccess) return -1;
  if (hipMemcpy(&host, pl->check, sizeof host, hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return host;
}

// RC_CHECK_FINITE: non-finite values in a_t or the sender's ahat.
rc_status_t check_finite(rc_plan* pl, hipStream_t stream, const void* a_t, const float* ahat) {
  if (!(pl->params.flags & RC_CHECK_FINITE)) return RC_OK;
  const int64_t n = (int64_t)pl->shape.batch * pl->layout.n;
  const int64_t bad = checked_count(pl, stream, [&] {
    return rc::launch_count_nonfinite(a_t, pl->dtype == RC_BF16, ahat, n, pl->check, stream);
  });
  return bad < 0 ? RC_ERR_HIP : (bad ? RC_ERR_NONFINITE : RC_OK);
}

hipError_t compress_all(rc_plan* pl, hipStream_t stream, const void* a_t, const rc_state_t* state,
                        uint8_t* packed) {
  const int B = pl->shape.batch;
  if (!pl->side) return compress_range(pl, stream, a_t, state, packed, 0, B);
  // low rank: first half on the caller's stream, second half on the plan's
  // stream, which starts after everything already on `stream` and which
  // `stream` waits for before anything enqueued after this call
  const int h = (B + 1) / 2;
  if (hipEventRecord(pl->fork, stream) != hipSuccess) return hipErrorUnknown;
  if (hipStreamWaitEvent(pl->side, pl->fork, 0) != hipSuccess) return hipErrorUnknown;
  hipError_t err = compress_range(pl, stream, a_t, state, packed, 0, h);
  if (err == hipSuccess) err = compress_range(pl, pl->side, a_t, state, packed, h, B - h);
  if (hipEventRecord(pl->join, pl->side) != hipSuccess) return hipErrorUnknown;
  if (hipStreamWaitEvent(stream, pl->join, 0) != hipSuccess) return hipErrorUnknown;
  return err;
}

}  // namespace

extern "C" {

rc_status_t rc_plan_create(rc_shape_t shape, rc_dtype_t dtype, rc_scheme_t scheme,
                           const rc_params_t* params, rc_plan_t* out) {
  if (!out) return RC_ERR_INVALID_ARG;
  *out = nullptr;
  rc_status_t st = rc::validate(shape, dtype, scheme, params);
  if (st != RC_OK) return st;
  rc_plan* pl = new (std::nothrow) rc_plan();
  if (!pl) return RC_ERR_HIP;
  pl->shape = shape;
  pl->dtype = dtype;
  pl->scheme = scheme;
  pl->params = *params;
  pl->params.q0 = nullptr;
  st = rc::make_layout(shape, dtype, scheme, *params, &pl->layout);
  if (st != RC_OK) { delete pl; return st; }
  pl->packed_bytes = (size_t)(pl->layout.tstride * shape.batch);
  if (scheme == RC_LOWRANK) {
    st = setup_lowrank(pl, static_cast<const float*>(params->q0));
    if (st != RC_OK) { rc_plan_destroy(pl); return st; }
  }
  if (scheme == RC_BLOCKSEL) {
    st = setup_blocksel(pl);
    if (st != RC_OK) { rc_plan_destroy(pl); return st; }
  }
  if (params->flags & (RC_CHECK_FINITE | RC_LR_CHECK_NUMERIC)) {
    if (hipGetDevice(&pl->device) != hipSuccess ||
        hipMalloc((void**)&pl->check, sizeof(uint32_t)) != hipSuccess) {
      pl->check = nullptr;
      rc_plan_destroy(pl);
      return RC_ERR_HIP;
    }
  }
  *out = pl;
  return RC_OK;
}

rc_status_t rc_compress(rc_plan_t pl, hipStream_t stream, const void* a_t, const rc_state_t* state,
                        void* packed_out) {
  if (!pl || !a_t || !state || !state->ahat || !state->e || !packed_out) return RC_ERR_INVALID_ARG;
  if (!aligned16(a_t) || !aligned16(state->ahat) || !aligned16(state->e) || !aligned16(packed_out))
    return RC_ERR_ALIGNMENT;
  uint8_t* packed = static_cast<uint8_t*>(packed_out);
  rc_status_t st = check_finite(pl, stream, a_t, state->ahat);
  if (st != RC_OK) return st;
  if (pl->scheme == RC_LOWRANK && (pl->params.flags & RC_LR_CHECK_NUMERIC)) {
    // count the Cholesky pivots that fall under the dead-column threshold
    pl->lr.dead = pl->check;
    const int64_t dead = checked_count(pl, stream, [&] { return compress_all(pl, stream, a_t, state, packed); });
    return dead < 0 ? RC_ERR_HIP : (dead ? RC_ERR_NUMERIC : RC_OK);
  }
  return compress_all(pl, stream, a_t, state, packed) == hipSuccess ? RC_OK : RC_ERR_HIP;
}

rc_status_t rc_compress_send(rc_plan_t pl, hipStream_t stream, hipStream_t copy_stream,
                             const void* a_t, const rc_state_t* state, void* packed_out,
                             void* packed_dst, int chunk) {
  if (!pl || !a_t || !state || !state->ahat || !state->e || !packed_out || !packed_dst || chunk < 1)
    return RC_ERR_INVALID_ARG;
  if (!aligned16(a_t) || !aligned16(state->ahat) || !aligned16(state->e) || !aligned16(packed_out))
    return RC_ERR_ALIGNMENT;
  const rc_status_t st = check_finite(pl, stream, a_t, state->ahat);
  if (st != RC_OK) return st;
  const int B = pl->shape.batch;
  const int nchunks = (B + chunk - 1) / chunk;
  if (pl->events.empty() && hipGetDevice(&pl->ev_device) != hipSuccess) return RC_ERR_HIP;
  while ((int)pl->events.size() < nchunks) {
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return RC_ERR_HIP;
    pl->events.push_back(ev);
  }
  uint8_t* src = static_cast<uint8_t*>(packed_out);
  uint8_t* dst = static_cast<uint8_t*>(packed_dst);
  const size_t ts = (size_t)pl->layout.tstride;
  for (int c = 0; c < nchunks; ++c) {
    const int b0 = c * chunk, nb = (B - b0 < chunk) ? B - b0 : chunk;
    if (compress_range(pl, stream, a_t, state, src, b0, nb) != hipSuccess) return RC_ERR_HIP;
    if (hipEventRecord(pl->events[c], stream) != hipSuccess) return RC_ERR_HIP;
    if (hipStreamWaitEvent(copy_stream, pl->events[c], 0) != hipSuccess) return RC_ERR_HIP;
    if (hipMemcpyAsync(dst + b0 * ts, src + b0 * ts, nb * ts, hipMemcpyDefault, copy_stream) !=
        hipSuccess)
      return RC_ERR_HIP;
  }
  return RC_OK;
}

rc_status_t rc_decompress(rc_plan_t pl, hipStream_t stream, const void* packed_in,
                          float* recon_state) {
  if (!pl || !packed_in || !recon_state) return RC_ERR_INVALID_ARG;
  if (!aligned16(packed_in) || !aligned16(recon_state)) return RC_ERR_ALIGNMENT;
  const uint8_t* packed = static_cast<const uint8_t*>(packed_in);
  const hipError_t err = decompress_peers(pl, stream, &packed, &recon_state, 1);
  return err == hipSuccess ? RC_OK : RC_ERR_HIP;
}

rc_status_t rc_decompress_many(rc_plan_t pl, hipStream_t stream, const void* const* packed_in,
                               float* const* recon_states, int npeers) {
  if (!pl || !packed_in || !recon_states || npeers < 1 || npeers > RC_MAX_PEERS)
    return RC_ERR_INVALID_ARG;
  const uint8_t* packed[RC_MAX_PEERS];
  for (int p = 0; p < npeers; ++p) {
    if (!packed_in[p] || !recon_states[p]) return RC_ERR_INVALID_ARG;
    if (!aligned16(packed_in[p]) || !aligned16(recon_states[p])) return RC_ERR_ALIGNMENT;
    packed[p] = static_cast<const uint8_t*>(packed_in[p]);
  }
  const hipError_t err = decompress_peers(pl, stream, packed, recon_states, npeers);
  return err == hipSuccess ? RC_OK : RC_ERR_HIP;
}

rc_status_t rc_plan_reset_state(rc_plan_t pl, hipStream_t stream) {
  if (!pl) return RC_ERR_INVALID_ARG;
  if (pl->scheme != RC_BLOCKSEL) return RC_OK;
  const hipError_t err = rc::launch_bs_reset(pl->bs_visited, (int64_t)pl->shape.batch * pl->bs.nblocks,
                                             pl->bs_have_prev, pl->shape.batch, stream);
  return err == hipSuccess ? RC_OK : RC_ERR_HIP;
}

rc_status_t rc_plan_destroy(rc_plan_t pl) {
  if (!pl) return RC_OK;
  rc_status_t st = RC_OK;
  if (pl->ws || pl->check || !pl->events.empty()) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) st = RC_ERR_HIP;
    if (!pl->events.empty()) {
      if (cur != pl->ev_device && hipSetDevice(pl->ev_device) != hipSuccess) st = RC_ERR_HIP;
      for (hipEvent_t ev : pl->events)
        if (hipEventDestroy(ev) != hipSuccess) st = RC_ERR_HIP;
    }
    if (pl->ws || pl->check) {
      if (hipSetDevice(pl->device) != hipSuccess) st = RC_ERR_HIP;
      if (pl->check && hipFree(pl->check) != hipSuccess) st = RC_ERR_HIP;
      if (pl->ws && hipFree(pl->ws) != hipSuccess) st = RC_ERR_HIP;
      if (pl->side && hipStreamDestroy(pl->side) != hipSuccess) st = RC_ERR_HIP;
      if (pl->fork && hipEventDestroy(pl->fork) != hipSuccess) st = RC_ERR_HIP;
      if (pl->join && hipEventDestroy(pl->join) != hipSuccess) st = RC_ERR_HIP;
    }
    (void)hipSetDevice(cur);
  }
  delete pl;
  return st;
}

size_t rc_packed_bytes(rc_plan_t pl) { return pl ? pl->packed_bytes : 0; }

size_t rc_tensor_packed_bytes(rc_plan_t pl) { return pl ? (size_t)pl->layout.tstride : 0; }

size_t rc_workspace_bytes(rc_plan_t pl) { return pl ? pl->ws_bytes : 0; }

// Diagnostics (librescomp_diag.h): device pointers of the low-rank workspace
// pieces, in the order R, P, Pbt, Qt, Q0t, Qtb, gsum, linv.
int rcx_lowrank_workspace(rc_plan_t pl, void** ptrs, int count) {
  if (!pl || pl->scheme != RC_LOWRANK || !ptrs || count < 8) return -1;
  const rc::LowRankWork& w = pl->lr;
  void* v[8] = {w.R, w.P, w.Pbt, w.Qt, w.Q0t, w.Qtb, w.gsum, w.linv};
  for (int i = 0; i < 8; ++i) ptrs[i] = v[i];
  return (int)w.rows_pad;
}

int rcx_lowrank_r_probe(rc_plan_t pl, int pattern, hipStream_t stream) {
  if (!pl || pl->scheme != RC_LOWRANK) return -1;
  const rc::LowRankWork& w = pl->lr;
  // the sink is a piece of the workspace the probes never write (never = 0)
  return (int)rc::launch_r_probe(pattern, w.R, (int)pl->shape.rows, (int)pl->shape.cols, (int)pl->shape.batch,
                                 (int)w.ntiles, (int)w.rows_pad, reinterpret_cast<uint32_t*>(w.gsum), stream);
}

int rcx_device_to_host(void* dst, const void* src, size_t bytes) {
  if (!dst || !src) return (int)hipErrorInvalidValue;
  return (int)hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
}

const char* rc_status_string(rc_status_t s) {
  switch (s) {
    case RC_OK: return "RC_OK: success";
    case RC_ERR_INVALID_ARG: return "RC_ERR_INVALID_ARG: null pointer, bad shape or bad parameter";
    case RC_ERR_UNSUPPORTED: return "RC_ERR_UNSUPPORTED: valid request not implemented by librescomp";
    case RC_ERR_ALIGNMENT: return "RC_ERR_ALIGNMENT: tensor pointer not 16-byte aligned";
    case RC_ERR_HIP: return "RC_ERR_HIP: HIP runtime call or kernel launch failed";
    case RC_ERR_NUMERIC: return "RC_ERR_NUMERIC: a Cholesky pivot fell under the dead-column threshold";
    case RC_ERR_NONFINITE: return "RC_ERR_NONFINITE: the input holds NaN or Inf";
  }
  return "unknown rc_status_t";
}

}  // extern "C"
