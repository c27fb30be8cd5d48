/*
 * librescomp -- residual compression with error feedback for parallel
 * diffusion inference, as HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the paper-notes page "Accelerating
 * Parallel Diffusion Model Serving with Residual Compression" (CompactFusion):
 *   - Overall framework: instead of an activation a_t, a GPU sends C(r) for the
 *     residual r = a_t - ahat_{t-1} against the reconstruction ahat that the
 *     receiver holds; the receiver sets ahat_t = ahat_{t-1} + C(r).
 *   - Key designs / Error feedback: the part C dropped, e_t = r - C(r), stays on
 *     the sender. The sender keeps a bit-identical copy of the receiver's ahat,
 *     so a_t - ahat_t = e_t after every step and the next residual carries e_t.
 *   - Compressors C: 1-bit and 2-bit group quantisation (Main experiment table,
 *     16x / 8x), a 2:16 block sparsifier (Key designs / System co-design), and a
 *     rank-k factorisation by subspace iteration with INT4 factors (Key designs /
 *     Low-rank strategy for extreme compression).
 *   - Limitations: step 0 has no history and is sent in full. That warm-up is
 *     the caller's: send a_0, set sender ahat = receiver ahat = float(a_0) and
 *     e = 0 (plain device copies); every later step uses rc_compress on the
 *     sender and rc_decompress on each receiver.
 *
 * Conventions for every call:
 *   - Tensors are [batch][rows][cols], row-major, contiguous; groups and blocks
 *     run along cols. a_t is bf16 or fp32 (rc_dtype_t); ahat, e and the receiver
 *     state are fp32.
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned. The library never allocates or frees them.
 *   - Calls are asynchronous on the given HIP stream and never synchronise the
 *     host. Calls on one plan must be serialised on one stream (the low-rank
 *     and block-selection schemes keep per-plan device workspace and state).
 *     Separate plans share nothing and may run concurrently on separate streams.
 *   - A rejected request (RC_ERR_INVALID_ARG, RC_ERR_UNSUPPORTED,
 *     RC_ERR_ALIGNMENT, RC_ERR_NONFINITE) writes no buffer and launches
 *     nothing (RC_ERR_NONFINITE: nothing but the input scan that found it). RC_ERR_HIP reports a failed HIP call or kernel launch; the
 *     outputs of that call are then unspecified. RC_ERR_NUMERIC is a report
 *     after a completed call (see RC_LR_CHECK_NUMERIC).
 *   - Inputs holding NaN or Inf give unspecified (but memory-safe) results,
 *     unless RC_CHECK_FINITE asks for them to be rejected.
 */
#ifndef LIBRESCOMP_H
#define LIBRESCOMP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rc_plan* rc_plan_t; /* opaque; created and owned by the library */

/* The enumerations are int-sized in C and C++ alike. In C++ they are given int
 * as their fixed underlying type, so that any int a C caller passes for one
 * (an invalid value included, which the library rejects) is a value of the
 * type on the C++ side too. */
#ifdef __cplusplus
#define RC_ENUM enum : int
#else
#define RC_ENUM enum
#endif

typedef RC_ENUM {
  RC_OK = 0,
  RC_ERR_INVALID_ARG = 1, /* null pointer, bad shape, bad parameter value */
  RC_ERR_UNSUPPORTED = 2, /* valid request this library does not implement */
  RC_ERR_ALIGNMENT = 3,   /* a tensor pointer is not 16-byte aligned */
  RC_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  RC_ERR_NUMERIC = 5,     /* RC_LR_CHECK_NUMERIC: a Cholesky pivot broke down */
  RC_ERR_NONFINITE = 6,   /* RC_CHECK_FINITE: NaN or Inf in the input */
} rc_status_t;

typedef RC_ENUM { RC_BF16 = 0, RC_F32 = 1 } rc_dtype_t; /* dtype of a_t */

typedef RC_ENUM {
  RC_Q1 = 0,      /* 1-bit signs + per-group fp32 mean|r|                 */
  RC_Q2 = 1,      /* 2-bit uniform levels + per-group fp32 (min, step)   */
  RC_NM = 2,      /* keep 2 of every 16, bf16 values + 4-bit indices     */
  RC_LOWRANK = 3, /* rank-k subspace iteration, INT4 factors             */
  RC_BLOCKSEL = 4 /* Otil-style: the k most-changed 8x8-token blocks     */
} rc_scheme_t;

typedef struct {
  int32_t batch; /* tensors per call (e.g. 57 transformer blocks)  */
  int32_t rows;  /* tokens of this GPU's share                      */
  int32_t cols;  /* hidden size                                     */
} rc_shape_t;

/* Scheme parameters. The values the pages evaluate: 1-bit and 2-bit groups
 * (Main experiment table: 1-bit 16x, 2-bit 8x; group 64 and 128 in this
 * library's workloads), the 2:16 block sparsifier (Key designs / System
 * co-design: N:M instead of TopK), and rank / iterations / INT4 factors of the
 * subspace iteration (Key designs / Low-rank strategy for extreme compression;
 * Main experiment table: low rank at about 100x). Unused fields must be 0. */
typedef struct {
  int32_t group;    /* RC_Q1 / RC_Q2: group size along cols: 32, 64 or 128       */
  int32_t nm_keep;  /* RC_NM: kept per block, must be 2                           */
  int32_t nm_block; /* RC_NM: block size, must be 16                              */
  int32_t rank;     /* RC_LOWRANK: 8, 16, 32, 48 or 64, at most rows and cols     */
  int32_t iters;    /* RC_LOWRANK: subspace iterations, 1..16                     */
  uint64_t seed;    /* RC_LOWRANK with q0 == NULL: seed of the start matrices     */
  const void* q0;   /* RC_LOWRANK, optional: DEVICE fp32 [batch][cols][rank]      */
                    /*   start matrices (4-byte aligned), read by rc_plan_create  */
                    /*   before it returns and reused every step. NULL: drawn     */
                    /*   from `seed` (see RC_LOWRANK below).                      */
  uint32_t flags;   /* 0 or an OR of the RC_* flags below allowed for the scheme  */
  int32_t grid_w;      /* RC_BLOCKSEL: tokens per row of the spatial token grid     */
  int32_t keep_blocks; /* RC_BLOCKSEL: blocks sent per tensor and step (k)          */
} rc_params_t;

/* Seeded start matrices (RC_LOWRANK, q0 == NULL). Element (b, c, j) of the
 * [batch][cols][rank] start matrices is the (c * rank + j)-th value of the
 * standard normal sequence of stream K_b, rounded to fp32, where
 *   S(k, i) = i-th output of SplitMix64 seeded with k (Steele, Lea and Flood,
 *             OOPSLA 2014): mix(k + (i + 1) * 0x9E3779B97F4A7C15),
 *   K_b     = S(S(S(seed, 7), b), 0),
 *   u(i)    = ((S(K_b, i) >> 11) + 0.5) * 2^-53, uniform in (0, 1),
 *   normal element 2p / 2p + 1 = sqrt(-2 ln u(2p)) * cos / sin(2 pi u(2p + 1))
 *             (Box-Muller, 1958).
 * The start matrices are the subspace iteration's only random input. */

/* rc_params_t.flags for RC_LOWRANK: send the factors as bf16 (round to nearest
 * even) instead of INT4 with per-column scales -- the factor-precision side of
 * the low-rank trade-off (Key designs / Low-rank strategy for extreme
 * compression: at one payload, bf16 factors of rank k cost as much as INT4
 * factors of rank 4k). Packed layout per tensor: U bf16 [rows*rank] | V bf16
 * [cols*rank], row-major, each section 256-byte aligned. */
#define RC_LR_BF16_FACTORS 1u

/* rc_params_t.flags for RC_LOWRANK: keep every kernel of rc_compress on the
 * caller's stream. By default a plan with batch >= 2 owns a second stream and
 * runs half of the batch there (see rc_compress); the results are the same bit
 * for bit either way. For callers that want one stream, and for per-kernel
 * traces without overlapping kernels. */
#define RC_LR_ONE_STREAM 2u

/* rc_params_t.flags for RC_BLOCKSEL: score each block against the receiver's
 * copy (ahat, the block as last sent) instead of the previous step's
 * activation. An alternative to the page's rule; the plan then keeps no copy
 * of the previous activation. */
#define RC_BS_SCORE_LAST_SENT 4u

/* rc_params_t.flags, any scheme (debugging): rc_compress and rc_compress_send
 * first scan a_t and the sender's ahat and return RC_ERR_NONFINITE, launching
 * nothing else, if either holds NaN or Inf. The call then waits for the scan
 * (a host synchronisation on the stream; not for graph capture). */
#define RC_CHECK_FINITE 8u

/* rc_params_t.flags for RC_LOWRANK (debugging): rc_compress waits for its
 * kernels and returns RC_ERR_NUMERIC if any Cholesky pivot of the CholeskyQR2
 * passes fell under the dead-column threshold (a zero or rank-deficient
 * residual, or a breakdown). The results are those of the default path, which
 * zeroes such columns; the status only reports it. Not for graph capture. */
#define RC_LR_CHECK_NUMERIC 16u

typedef struct {
  float* ahat; /* sender's copy of the receiver reconstruction, fp32 [batch][rows][cols] */
  float* e;    /* error-feedback buffer, fp32 [batch][rows][cols] (written every step)  */
} rc_state_t;

/* RC_BLOCKSEL ("Otil: Accelerating Diffusion Model Inference via
 * Communication-Efficient Multi-GPU Parallelism", Key designs 1-3): the rows of
 * a tensor are tokens of a spatial grid with grid_w tokens per row (raster
 * order); the grid is cut into 8 x 8-token blocks (all channels), numbered in
 * raster order. Each step every block is scored by the cosine dissimilarity
 * 1 - <a_t, a_{t-1}> / (|a_t| |a_{t-1}|) between its values at this step and
 * at the previous step (Key design 2; both zero -> 0, one zero -> 1), and the
 * keep_blocks highest-scoring blocks among those not yet sent in the current
 * round (ties to the lower index) are sent; the round restarts once every block
 * has been sent, so every block is sent once per round (Key design 3). Sent
 * blocks carry the a_t values (input dtype) and replace the receiver's copy:
 * after the step ahat = a_t and e = 0 there, and e = a_t - ahat on the other
 * blocks. The plan keeps the round state and a copy of the previous a_t
 * (rc_workspace_bytes counts it); on the first step after creation or
 * rc_plan_reset_state it has none and compares with ahat, which the warm-up
 * set to a_{t-1}. RC_BS_SCORE_LAST_SENT scores against ahat on every step.
 * Requirements: rows % (8 grid_w) == 0, grid_w % 8 == 0, cols % 4 == 0,
 * 1 <= keep_blocks <= blocks <= 4096. */

/* Validate the request and build a plan. For RC_LOWRANK and RC_BLOCKSEL this
 * allocates the device workspace (rc_workspace_bytes) on the current device;
 * RC_LOWRANK also sets up the start matrices (from q0 or the seed) and waits
 * for that. Cols must be a multiple of the group (Q1/Q2), of 16 (NM) or of 64
 * (LR); LR rows at most 65535 * 32; rows*cols*batch must stay below 2^40.
 * Errors: RC_ERR_INVALID_ARG (null params or out, bad shape, bad value, a flag
 * the scheme does not take), RC_ERR_UNSUPPORTED (a valid value this library
 * does not implement), RC_ERR_ALIGNMENT (q0 not 4-byte aligned), RC_ERR_HIP
 * (allocation or launch failure; nothing is leaked). */
rc_status_t rc_plan_create(rc_shape_t shape, rc_dtype_t dtype, rc_scheme_t scheme,
                           const rc_params_t* params, rc_plan_t* out);

/* Sender step (Overall framework + Error feedback): for every tensor,
 *   r = a_t - ahat;  packed_out <- encode(C(r));  e = r - C(r);  ahat += C(r)
 * where C(r) is decoded from the packed bytes exactly as rc_decompress decodes
 * them, so a receiver that applies packed_out stays bit-identical to ahat.
 * a_t: [batch][rows][cols] of the plan's dtype. state->ahat is read and
 * updated in place, state->e is written. packed_out: rc_packed_bytes(plan)
 * bytes, written completely (padding included).
 * RC_LOWRANK with batch >= 2 runs the second half of the batch on a stream the
 * plan owns: it starts after the work already enqueued on `stream`, and
 * `stream` waits for it before the work enqueued after this call (events; this
 * also holds under stream capture). The results are those of one stream. */
rc_status_t rc_compress(rc_plan_t plan, hipStream_t stream, const void* a_t, const rc_state_t* state,
                        void* packed_out);

/* Sender step with the packed stream handed off chunk by chunk (Key designs /
 * System co-design: compression overlapped with communication). The batch is
 * compressed in chunks of `chunk` tensors on `stream`, with exactly the results
 * of rc_compress; as soon as a chunk's packed bytes are written, a copy of them
 * into the same place of `packed_dst` is queued on `copy_stream`
 * (hipMemcpyAsync, any destination the HIP runtime can copy to: a peer's
 * receive buffer, another device buffer, pinned host memory), so the copy of
 * chunk i runs while chunk i+1 is compressed. On return all copies are queued;
 * nothing waits for them. The caller must let copy_stream pass this call's
 * copies before packed_out is written again (e.g. alternate two packed_out
 * buffers, or make the next writer wait on an event recorded on copy_stream),
 * and before packed_dst is read. chunk >= 1 (chunk >= batch: one chunk).
 * The plan keeps one event per chunk, created on the first call on the
 * current device. */
rc_status_t rc_compress_send(rc_plan_t plan, hipStream_t stream, hipStream_t copy_stream,
                             const void* a_t, const rc_state_t* state, void* packed_out,
                             void* packed_dst, int chunk);

/* Receiver step (Overall framework): recon_state += decode(packed_in) for every
 * tensor. recon_state: fp32 [batch][rows][cols], updated in place. */
rc_status_t rc_decompress(rc_plan_t plan, hipStream_t stream, const void* packed_in,
                          float* recon_state);

/* Receiver step for several senders at once (a sequence-parallel receiver gets
 * one packed stream from each peer, Overall framework): recon_states[p] +=
 * decode(packed_in[p]) for p < npeers, 1 <= npeers <= RC_MAX_PEERS, each state
 * fp32 [batch][rows][cols] and each stream rc_packed_bytes(plan) bytes laid out
 * by this plan. The results equal npeers calls of rc_decompress; all peers are
 * decoded in one launch. The states must not overlap. */
#define RC_MAX_PEERS 8
rc_status_t rc_decompress_many(rc_plan_t plan, hipStream_t stream, const void* const* packed_in,
                               float* const* recon_states, int npeers);

/* Clear the state a plan keeps across steps (RC_BLOCKSEL: the round of sent
 * blocks and the previous activation), for a new sequence; asynchronous on
 * stream; no effect for the other schemes. */
rc_status_t rc_plan_reset_state(rc_plan_t plan, hipStream_t stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): the RC_LOWRANK sender
 * step of rc_compress without a plan. It validates shape, dtype and params as
 * rc_plan_create does (flags: 0 or RC_LR_BF16_FACTORS), sets up the start
 * matrices (from params->q0, a device pointer, or params->seed) and runs the
 * plan's kernels on `stream` alone; a_t, state and packed_out are as for
 * rc_compress (packed_out: the bytes rc_packed_bytes of such a plan reports),
 * and the results equal rc_compress's bit for bit. It allocates nothing: the
 * workspace is a fixed device array of RC_NOALLOC_SCRATCH_BYTES held by every
 * GPU the library runs on until the process ends, so shapes whose workspace
 * (rc_workspace_bytes of the equivalent plan) is larger are rejected with
 * RC_ERR_UNSUPPORTED before anything is launched. All calls on one GPU share
 * that array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller. A receiver decodes the
 * output with rc_decompress on a plan with the same parameters. */
#define RC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rc_status_t rc_compress_lowrank_noalloc(rc_shape_t shape, rc_dtype_t dtype, const rc_params_t* params,
                                        hipStream_t stream, const void* a_t, const rc_state_t* state,
                                        void* packed_out);

/* Free the plan and its workspace. Waits for nothing: the caller must make sure
 * no launched work still uses the plan. NULL is accepted. */
rc_status_t rc_plan_destroy(rc_plan_t plan);

/* Bytes of one call's packed stream (all batch tensors), and of one tensor's
 * slice of it. Layout, per tensor, each section starting at a multiple of 256
 * bytes, tensors back to back (N = rows*cols, G = group):
 *   Q1: sign bits [N/8] (element k = bit k%8 of byte k/8) | scale f32 [N/G]
 *   Q2: codes [N/4] (element k = bits 2(k%4)..+1 of byte k/4) | group minimum mn f32 [N/G]
 *       | group step d f32 [N/G]
 *   NM: {v_i0, v_i1} bf16 pairs [N/16] | index byte i0 | i1<<4 [N/16], i0 < i1
 *   LR: U nibbles [rows*rank/2] | V nibbles [cols*rank/2] | sU f32 [rank] | sV f32 [rank]
 *       (row-major INT4, element t in nibble t, even t low, two's complement);
 *       with RC_LR_BF16_FACTORS: U bf16 [rows*rank] | V bf16 [cols*rank]
 *   BLOCKSEL: u32 [1 + keep] (count, then the sent block indices ascending, unused
 *       slots 0) | values [keep][64 tokens][cols] in the dtype of a_t (tokens of a
 *       block in raster order; unused slots 0)
 * Returns 0 for a NULL plan. */
size_t rc_packed_bytes(rc_plan_t plan);
size_t rc_tensor_packed_bytes(rc_plan_t plan);

/* Device workspace owned by the plan (0 for Q1, Q2, NM; the debug flags add a
 * 4-byte counter not counted here). */
size_t rc_workspace_bytes(rc_plan_t plan);

/* Static description of a status code ("unknown rc_status_t" for a value that
 * is none). */
const char* rc_status_string(rc_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* LIBRESCOMP_H */
