/*
 * librescomp diagnostics: measurement helpers that are not part of the
 * compression path. The tests and the benchmark use them; applications do not
 * need them.
 */
#ifndef LIBRESCOMP_DIAG_H
#define LIBRESCOMP_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "librescomp.h"

#ifdef __cplusplus
extern "C" {
#endif

/* HBM reference kernels (roofline ceilings for the path's access patterns).
 * n = element count (multiple of 8). Device pointers, caller-owned:
 *   RCX_PROBE_COPY         b[0..n) = a[0..n)              fp32, 8 B/element
 *   RCX_PROBE_READ         reads a[0..n) fp32 (c: 1 float, written only in a
 *                          case that never occurs for finite data), 4 B/element
 *   RCX_PROBE_WRITE        writes b[0..n) fp32, 4 B/element
 *   RCX_PROBE_SENDER_MIX   reads bf16 a[0..n) and fp32 b, writes b and c,
 *                          14 B/element (the sender kernels' stream pattern)
 *   RCX_PROBE_RECEIVER_RMW reads and rewrites fp32 b in place, 8 B/element
 * Launches asynchronously on `stream`; returns a hipError_t value (0 = ok). */
enum {
  RCX_PROBE_COPY = 0,
  RCX_PROBE_READ = 1,
  RCX_PROBE_WRITE = 2,
  RCX_PROBE_SENDER_MIX = 3,
  RCX_PROBE_RECEIVER_RMW = 4,
};
int rcx_hbm_probe(int kind, const void* a, void* b, void* c, int64_t n, hipStream_t stream);

/* Device pointers of a low-rank plan's workspace pieces, in the order R, P,
 * Pbt, Qt, Q0t, Qtb, gsum, linv (count >= 8). Returns rows_pad, or -1 for a
 * NULL plan, another scheme, or count < 8. The pieces are as wide as the
 * iteration: max(rank, 16) (rank 8 runs 16 wide with columns 8 .. 15 zero).
 * The bf16 [width][cols] operands (Q0t, Qtb) and Pbt ([width][rows_pad]) are
 * stored in groups of 32 columns (rows): group g holds its width x 32 block
 * contiguously. */
int rcx_lowrank_workspace(rc_plan_t plan, void** ptrs, int count);

/* Reads the R workspace of a low-rank plan (bf16, batch x rows x cols) in the
 * access pattern of one of its products, with that product's grid, and does
 * nothing else: the measured ceiling of the passes that read R alone.
 *   RCX_R_PROBE_RQ   the R*Q pass (64-row bands walking 128-column chunks)
 *   RCX_R_PROBE_RTP  the R^T*P pass (128-column blocks walking 32-row steps)
 * Reads batch * rows * cols * 2 bytes; writes nothing. Launches asynchronously
 * on `stream`. Returns a hipError_t value, or -1 for a NULL plan or another
 * scheme. */
enum { RCX_R_PROBE_RQ = 0, RCX_R_PROBE_RTP = 1 };
int rcx_lowrank_r_probe(rc_plan_t plan, int pattern, hipStream_t stream);

/* Synchronous copy of `bytes` bytes from device address src to host memory dst
 * (for reading the workspace pieces above). Returns a hipError_t value. */
int rcx_device_to_host(void* dst, const void* src, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* LIBRESCOMP_DIAG_H */
