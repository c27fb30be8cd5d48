/* A plain C caller of librescomp: every scheme through rc_plan_create,
 * rc_compress, rc_decompress and rc_plan_destroy with device buffers from
 * hipMalloc, two steps each, no Python and no C++ involved.
 *
 * Checks, per scheme and step:
 *   - the receiver state equals the sender's ahat bit for bit;
 *   - e and the update of ahat add back up to the residual: with
 *     r = a_t - ahat_{t-1}, |e + (ahat_t - ahat_{t-1}) - r| stays within fp32
 *     rounding of the operands (the sender keeps e = r - c, ahat_t = ahat + c);
 *   - a NULL plan and a misaligned tensor pointer are rejected with the
 *     documented status codes, before anything is launched.
 * Exit status 0 when everything holds, 1 otherwise, 77 without a GPU. */
#include <librescomp.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CHECK_HIP(x)                                                       \
  do {                                                                     \
    hipError_t err_ = (x);                                                 \
    if (err_ != hipSuccess) {                                              \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(err_)); \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
static float uniform(void) { /* in [-1, 1) */
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((lcg_state >> 40) * (1.0 / 8388608.0)) - 1.0f;
}

static int run_scheme(const char* name, rc_scheme_t scheme, rc_shape_t shape, rc_params_t params) {
  const size_t count = (size_t)shape.batch * shape.rows * shape.cols;
  const size_t bytes = count * sizeof(float);
  float* h_a = (float*)malloc(bytes);
  float* h_prev = (float*)malloc(bytes);
  float* h_ahat = (float*)malloc(bytes);
  float* h_recon = (float*)malloc(bytes);
  float* h_e = (float*)malloc(bytes);
  int failures = 0;

  rc_plan_t plan = NULL;
  rc_status_t st = rc_plan_create(shape, RC_F32, scheme, &params, &plan);
  if (st != RC_OK) {
    fprintf(stderr, "%s: rc_plan_create: %s\n", name, rc_status_string(st));
    return 1;
  }
  float *d_a, *d_ahat, *d_e, *d_recon;
  void* d_packed;
  CHECK_HIP(hipMalloc((void**)&d_a, bytes));
  CHECK_HIP(hipMalloc((void**)&d_ahat, bytes));
  CHECK_HIP(hipMalloc((void**)&d_e, bytes));
  CHECK_HIP(hipMalloc((void**)&d_recon, bytes));
  CHECK_HIP(hipMalloc(&d_packed, rc_packed_bytes(plan)));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  /* step 0 is sent in full: both sides start from a_0 */
  for (size_t i = 0; i < count; ++i) h_prev[i] = uniform();
  CHECK_HIP(hipMemcpy(d_ahat, h_prev, bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_recon, h_prev, bytes, hipMemcpyHostToDevice));

  for (int step = 1; step <= 2; ++step) {
    for (size_t i = 0; i < count; ++i) h_a[i] = h_prev[i] + 0.25f * uniform();
    CHECK_HIP(hipMemcpy(d_a, h_a, bytes, hipMemcpyHostToDevice));
    rc_state_t state = {d_ahat, d_e};
    st = rc_compress(plan, stream, d_a, &state, d_packed);
    if (st == RC_OK) st = rc_decompress(plan, stream, d_packed, d_recon);
    if (st != RC_OK) {
      fprintf(stderr, "%s step %d: %s\n", name, step, rc_status_string(st));
      failures++;
      break;
    }
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(h_ahat, d_ahat, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_recon, d_recon, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_e, d_e, bytes, hipMemcpyDeviceToHost));
    if (memcmp(h_ahat, h_recon, bytes) != 0) {
      fprintf(stderr, "%s step %d: receiver differs from sender\n", name, step);
      failures++;
    }
    size_t bad = 0;
    for (size_t i = 0; i < count; ++i) {
      const double r = (double)(h_a[i] - h_prev[i]);
      const double back = (double)h_e[i] + ((double)h_ahat[i] - (double)h_prev[i]);
      const double scale = fabs((double)h_a[i]) + fabs((double)h_prev[i]) + fabs((double)h_ahat[i]);
      if (!isfinite(h_e[i]) || !isfinite(h_ahat[i]) || fabs(back - r) > 4.0 * 0x1p-24 * scale + 1e-30)
        bad++;
    }
    if (bad) {
      fprintf(stderr, "%s step %d: %zu elements where e + update != r\n", name, step, bad);
      failures++;
    }
    memcpy(h_prev, h_ahat, bytes);
  }

  /* rejected without launching */
  rc_state_t state = {d_ahat, d_e};
  if (rc_compress(NULL, stream, d_a, &state, d_packed) != RC_ERR_INVALID_ARG) {
    fprintf(stderr, "%s: NULL plan not rejected\n", name);
    failures++;
  }
  if (rc_compress(plan, stream, (const char*)d_a + 4, &state, d_packed) != RC_ERR_ALIGNMENT) {
    fprintf(stderr, "%s: misaligned a_t not rejected\n", name);
    failures++;
  }

  CHECK_HIP(hipStreamDestroy(stream));
  CHECK_HIP(hipFree(d_a));
  CHECK_HIP(hipFree(d_ahat));
  CHECK_HIP(hipFree(d_e));
  CHECK_HIP(hipFree(d_recon));
  CHECK_HIP(hipFree(d_packed));
  if (rc_plan_destroy(plan) != RC_OK) failures++;
  free(h_a);
  free(h_prev);
  free(h_ahat);
  free(h_recon);
  free(h_e);
  printf("%s: %s\n", name, failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    printf("no GPU\n");
    return 77;
  }
  const rc_shape_t shape = {2, 128, 256};
  int failures = 0;
  rc_params_t p;

  memset(&p, 0, sizeof p);
  p.group = 64;
  failures += run_scheme("q1", RC_Q1, shape, p);

  memset(&p, 0, sizeof p);
  p.group = 128;
  failures += run_scheme("q2", RC_Q2, shape, p);

  memset(&p, 0, sizeof p);
  p.nm_keep = 2;
  p.nm_block = 16;
  failures += run_scheme("nm", RC_NM, shape, p);

  /* start matrices given on the device, then drawn from a seed */
  const int rank = 16;
  const size_t q0_bytes = sizeof(float) * shape.batch * shape.cols * rank;
  float* q0 = (float*)malloc(q0_bytes);
  for (int i = 0; i < shape.batch * shape.cols * rank; ++i) q0[i] = uniform();
  void* d_q0;
  CHECK_HIP(hipMalloc(&d_q0, q0_bytes));
  CHECK_HIP(hipMemcpy(d_q0, q0, q0_bytes, hipMemcpyHostToDevice));
  memset(&p, 0, sizeof p);
  p.rank = rank;
  p.iters = 2;
  p.q0 = d_q0;
  failures += run_scheme("lowrank", RC_LOWRANK, shape, p);
  CHECK_HIP(hipFree(d_q0));
  free(q0);
  p.q0 = NULL;
  p.seed = 12345;
  failures += run_scheme("lowrank seeded", RC_LOWRANK, shape, p);

  memset(&p, 0, sizeof p);
  p.grid_w = 16; /* 128 tokens = 8 rows of 16: one row of two 8 x 8 blocks */
  p.keep_blocks = 1;
  failures += run_scheme("blocksel", RC_BLOCKSEL, shape, p);

  printf(failures ? "c_abi_roundtrip: FAILED\n" : "c_abi_roundtrip: all ok\n");
  return failures ? 1 : 0;
}
