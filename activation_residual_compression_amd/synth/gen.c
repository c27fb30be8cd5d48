/*
 * Seeded synthetic activation generators.
 *
 * This file holds no arithmetic of the compression method: it only makes the
 * inputs (activation sequences a_0..a_{T-1} and the random start matrix of the
 * subspace iteration) that both the GPU library and the CPU oracle consume.
 *
 * Random numbers come from one counter-based generator, so any element of any
 * stream can be produced independently and in parallel, and the result does
 * not depend on the thread count:
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): output i of the sequence seeded with key k is
 *     mix(k + (i+1)*gamma), gamma = 0x9E3779B97F4A7C15, with the 64-bit
 *     finaliser mix() given below.
 *   - uniform in (0,1): ((x >> 11) + 0.5) * 2^-53.
 *   - standard normal: Box-Muller (1958) on the uniform pair (2p, 2p+1);
 *     element 2p takes the cosine branch and element 2p+1 the sine branch.
 *
 * The workload shapes and statistics follow the pages' experimental setting
 * ("Accelerating Parallel Diffusion Model Serving with Residual Compression":
 * FLUX.1-dev sequence-parallel shares and CogVideoX-2b), rebuilt synthetically;
 * the exact recipes are documented beside each builder.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* i-th output of the SplitMix64 sequence whose seed is `key`. */
static inline uint64_t sm_at(uint64_t key, uint64_t i) {
  return sm_mix(key + (i + 1) * SM_GAMMA);
}

static inline double sm_uniform(uint64_t key, uint64_t i) {
  return ((double)(sm_at(key, i) >> 11) + 0.5) * 0x1p-53;
}

static inline double sm_normal(uint64_t key, uint64_t i) {
  const uint64_t p = i >> 1;
  const double u1 = sm_uniform(key, 2 * p);
  const double u2 = sm_uniform(key, 2 * p + 1);
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* Both normals of pair p (elements 2p and 2p+1) from one Box-Muller draw. */
static inline void sm_normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  const double u1 = sm_uniform(key, 2 * p);
  const double u2 = sm_uniform(key, 2 * p + 1);
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 6.283185307179586476925286766559 * u2;
  *z0 = rad * cos(ang);
  *z1 = rad * sin(ang);
}

/* Stream key for (seed, role, tensor, step). */
uint64_t sg_key(uint64_t seed, uint64_t role, uint64_t tensor, uint64_t step) {
  uint64_t k = sm_at(seed, role);
  k = sm_at(k, tensor);
  return sm_at(k, step);
}

uint64_t sg_u64(uint64_t key, uint64_t i) { return sm_at(key, i); }

void sg_uniform(uint64_t key, uint64_t first, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = sm_uniform(key, first + (uint64_t)i);
}

void sg_normal(uint64_t key, uint64_t first, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = sm_normal(key, first + (uint64_t)i);
}

void sg_normal_f32(uint64_t key, uint64_t first, int64_t count, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)sm_normal(key, first + (uint64_t)i);
}

/* fp32 -> bfloat16 bits, round to nearest, ties to even (input preparation). */
void sg_to_bf16(int64_t count, const float* x, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint32_t u;
    memcpy(&u, &x[i], 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
      out[i] = (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
      continue;
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[i] = (uint16_t)(u >> 16);
  }
}

enum {
  ROLE_SCALE = 1,
  ROLE_OUTLIER = 2,
  ROLE_A0 = 3,
  ROLE_STEP = 4,
  ROLE_DRIFT_A = 5,
  ROLE_DRIFT_B = 6,
  ROLE_Q0 = 7,
  ROLE_TEXT = 8,
};

/* ------------------------------------------------------------------------ */
/* Tiny fp32 random walk: s_c ~ LogNormal(0, sigma_s) per column,             */
/* a_0 = N(0,1) s_c, a_t = a_{t-1} + step_sigma N(0,1) s_c.                   */
/* ------------------------------------------------------------------------ */
void sg_walk_init(uint64_t seed, int tensor, int n, int m, double sigma_s, float* sc, float* a0) {
  const uint64_t ks = sg_key(seed, ROLE_SCALE, tensor, 0);
  for (int j = 0; j < m; ++j) sc[j] = (float)exp(sigma_s * sm_normal(ks, j));
  const uint64_t ka = sg_key(seed, ROLE_A0, tensor, 0);
#pragma omp parallel for schedule(static)
  for (int64_t idx = 0; idx < (int64_t)n * m; ++idx)
    a0[idx] = (float)(sm_normal(ka, idx) * (double)sc[idx % m]);
}

void sg_walk_step(uint64_t seed, int tensor, int t, int n, int m, double step_sigma, const float* sc,
                  float* a) {
  const uint64_t k = sg_key(seed, ROLE_STEP, tensor, t);
  const int64_t N = (int64_t)n * m;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (N + 1) / 2; ++p) {
    double z[2];
    sm_normal_pair(k, p, &z[0], &z[1]);
    for (int q = 0; q < 2; ++q) {
      const int64_t idx = 2 * p + q;
      if (idx < N) a[idx] = (float)((double)a[idx] + step_sigma * z[q] * (double)sc[idx % m]);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* FLUX-like share [n tokens x m hidden]:                                     */
/*   s_c ~ LogNormal(0,1); n_outlier channels (the ones with the smallest     */
/*   64-bit draw) get s_c * outlier_mult;                                     */
/*   drift D = A B^T / sqrt(rank_drift), A [n x rank_drift], B [m x           */
/*   rank_drift] ~ N(0,1), fixed for the whole sequence;                      */
/*   a_0 = N(0,1) s_c; a_t = a_{t-1} + (sigma/sqrt2) (N(0,1) + D) s_c, so the */
/*   step change has std sigma * s_c, split equally between noise and drift.  */
/* ------------------------------------------------------------------------ */
void sg_flux_init(uint64_t seed, int tensor, int n, int m, int n_outlier, double outlier_mult,
                  int rank_drift, float* sc, float* A, float* B, float* a0) {
  const uint64_t ks = sg_key(seed, ROLE_SCALE, tensor, 0);
  for (int j = 0; j < m; ++j) sc[j] = (float)exp(sm_normal(ks, j));
  /* outliers: n_outlier distinct channels with the smallest draws */
  const uint64_t ko = sg_key(seed, ROLE_OUTLIER, tensor, 0);
  unsigned char* taken = (unsigned char*)calloc((size_t)m, 1);
  for (int o = 0; o < n_outlier && o < m; ++o) {
    int best = -1;
    uint64_t bv = 0;
    for (int j = 0; j < m; ++j) {
      if (taken[j]) continue;
      const uint64_t v = sm_at(ko, j);
      if (best < 0 || v < bv) { best = j; bv = v; }
    }
    taken[best] = 1;
    sc[best] = (float)((double)sc[best] * outlier_mult);
  }
  free(taken);
  const uint64_t kA = sg_key(seed, ROLE_DRIFT_A, tensor, 0);
  const uint64_t kB = sg_key(seed, ROLE_DRIFT_B, tensor, 0);
  for (int64_t i = 0; i < (int64_t)n * rank_drift; ++i) A[i] = (float)sm_normal(kA, i);
  for (int64_t i = 0; i < (int64_t)m * rank_drift; ++i) B[i] = (float)sm_normal(kB, i);
  const uint64_t ka = sg_key(seed, ROLE_A0, tensor, 0);
#pragma omp parallel for schedule(static)
  for (int64_t idx = 0; idx < (int64_t)n * m; ++idx)
    a0[idx] = (float)(sm_normal(ka, idx) * (double)sc[idx % m]);
}

void sg_flux_step(uint64_t seed, int tensor, int t, int n, int m, double sigma, int rank_drift,
                  const float* sc, const float* A, const float* B, float* a) {
  const uint64_t k = sg_key(seed, ROLE_STEP, tensor, t);
  const double amp = sigma / sqrt(2.0);
  const double inv_sqrt_r = 1.0 / sqrt((double)rank_drift);
  const int64_t N = (int64_t)n * m;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (N + 1) / 2; ++p) {
    double z[2];
    sm_normal_pair(k, p, &z[0], &z[1]);
    for (int q = 0; q < 2; ++q) {
      const int64_t idx = 2 * p + q;
      if (idx >= N) break;
      const int64_t i = idx / m, j = idx % m;
      double d = 0.0;
      for (int r = 0; r < rank_drift; ++r) d += (double)A[i * rank_drift + r] * (double)B[j * rank_drift + r];
      d *= inv_sqrt_r;
      a[idx] = (float)((double)a[idx] + amp * (z[q] + d) * (double)sc[j]);
    }
  }
}

/* The FLUX-like step with the white and drift parts scaled separately:      */
/*   a += (amp_white z + amp_drift (A B^T)[i][j] / sqrt(r)) s_c               */
/* (the noise-schedule workload varies amp_white from step to step).         */
void sg_flux_step_mix(uint64_t seed, int tensor, int t, int n, int m, double amp_white,
                      double amp_drift, int rank_drift, const float* sc, const float* A,
                      const float* B, float* a) {
  const uint64_t k = sg_key(seed, ROLE_STEP, tensor, t);
  const double inv_sqrt_r = 1.0 / sqrt((double)rank_drift);
  const int64_t N = (int64_t)n * m;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (N + 1) / 2; ++p) {
    double z[2];
    sm_normal_pair(k, p, &z[0], &z[1]);
    for (int q = 0; q < 2; ++q) {
      const int64_t idx = 2 * p + q;
      if (idx >= N) break;
      const int64_t i = idx / m, j = idx % m;
      double d = 0.0;
      for (int r = 0; r < rank_drift; ++r) d += (double)A[i * rank_drift + r] * (double)B[j * rank_drift + r];
      d *= inv_sqrt_r;
      a[idx] = (float)((double)a[idx] + (amp_white * z[q] + amp_drift * d) * (double)sc[j]);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Video-like share (CogVideoX-2b-shaped): the token sequence is n_text text */
/* tokens followed by frames x height x width patch tokens; share s of       */
/* n_shares takes tokens [s*n, (s+1)*n). Per channel, the step noise xi_t is */
/* N(0,1) white noise blurred per frame by a 2-D Gaussian (std blur_sigma    */
/* tokens, radius ceil(3 sigma), mirror padding) and rescaled to unit        */
/* variance; text tokens take unblurred N(0,1).                              */
/*   a_0 = xi_0 s_c;  a_t = rho a_{t-1} + sqrt(1 - rho^2) xi_t s_c.          */
/* ------------------------------------------------------------------------ */
typedef struct {
  int n_text, frames, height, width, share, n; /* n = tokens in this share */
  double blur_sigma;
} sg_video_geom;

static int mirror(int i, int L) {
  while (i < 0 || i >= L) {
    if (i < 0) i = -i;
    if (i >= L) i = 2 * (L - 1) - i;
  }
  return i;
}

/* xi for tokens of the share; out [n][m] */
static void video_xi(uint64_t key_video, uint64_t key_text, const sg_video_geom* g, int m, float* out) {
  const int HW = g->height * g->width;
  const int64_t tok0 = (int64_t)g->share * g->n;
  const int64_t tok1 = tok0 + g->n;
  const int radius = (int)ceil(3.0 * g->blur_sigma);
  double w[64];
  double wsum = 0.0, w2 = 0.0;
  for (int k = -radius; k <= radius; ++k) {
    w[k + radius] = exp(-(double)k * k / (2.0 * g->blur_sigma * g->blur_sigma));
    wsum += w[k + radius];
  }
  for (int k = 0; k <= 2 * radius; ++k) { w[k] /= wsum; w2 += w[k] * w[k]; }
  const double renorm = 1.0 / w2; /* 1 / (sqrt(sum w^2))^2 for the separable 2-D kernel */

  /* text tokens */
  for (int64_t tok = tok0; tok < tok1 && tok < g->n_text; ++tok) {
    float* dst = out + (tok - tok0) * m;
    for (int j = 0; j < m; ++j) dst[j] = (float)sm_normal(key_text, (uint64_t)tok * m + j);
  }
  /* video frames overlapping the share */
  const int64_t v0 = tok0 > g->n_text ? tok0 - g->n_text : 0;
  const int64_t v1 = tok1 - g->n_text;
  if (v1 <= 0) return;
  const int f0 = (int)(v0 / HW), f1 = (int)((v1 - 1) / HW);
  for (int f = f0; f <= f1 && f < g->frames; ++f) {
#pragma omp parallel for schedule(static)
    for (int j = 0; j < m; ++j) {
      double* z = (double*)malloc(sizeof(double) * HW);
      double* tmp = (double*)malloc(sizeof(double) * HW);
      for (int p = 0; p < HW; ++p) z[p] = sm_normal(key_video, ((uint64_t)f * HW + p) * m + j);
      for (int h = 0; h < g->height; ++h)
        for (int x = 0; x < g->width; ++x) {
          double s = 0.0;
          for (int k = -radius; k <= radius; ++k) s += w[k + radius] * z[h * g->width + mirror(x + k, g->width)];
          tmp[h * g->width + x] = s;
        }
      for (int h = 0; h < g->height; ++h)
        for (int x = 0; x < g->width; ++x) {
          double s = 0.0;
          for (int k = -radius; k <= radius; ++k) s += w[k + radius] * tmp[mirror(h + k, g->height) * g->width + x];
          const int64_t vt = (int64_t)f * HW + h * g->width + x; /* video token index */
          const int64_t tok = vt + g->n_text;
          if (tok >= tok0 && tok < tok1) out[(tok - tok0) * m + j] = (float)(s * renorm);
        }
      free(z);
      free(tmp);
    }
  }
}

void sg_video_init(uint64_t seed, int tensor, const sg_video_geom* g, int m, float* sc, float* a0) {
  const uint64_t ks = sg_key(seed, ROLE_SCALE, tensor, 0);
  for (int j = 0; j < m; ++j) sc[j] = (float)exp(sm_normal(ks, j));
  video_xi(sg_key(seed, ROLE_STEP, tensor, 0), sg_key(seed, ROLE_TEXT, tensor, 0), g, m, a0);
#pragma omp parallel for schedule(static)
  for (int64_t idx = 0; idx < (int64_t)g->n * m; ++idx) a0[idx] = (float)((double)a0[idx] * sc[idx % m]);
}

void sg_video_step(uint64_t seed, int tensor, int t, const sg_video_geom* g, int m, double rho,
                   const float* sc, float* a, float* scratch /* [n][m] */) {
  video_xi(sg_key(seed, ROLE_STEP, tensor, t), sg_key(seed, ROLE_TEXT, tensor, t), g, m, scratch);
  const double b = sqrt(1.0 - rho * rho);
#pragma omp parallel for schedule(static)
  for (int64_t idx = 0; idx < (int64_t)g->n * m; ++idx)
    a[idx] = (float)(rho * (double)a[idx] + b * (double)scratch[idx] * (double)sc[idx % m]);
}

/* Start matrix of the subspace iteration: N(0,1) [m x rank] per tensor. */
void sg_q0(uint64_t seed, int tensor, int m, int rank, float* q0) {
  const uint64_t k = sg_key(seed, ROLE_Q0, tensor, 0);
  for (int64_t i = 0; i < (int64_t)m * rank; ++i) q0[i] = (float)sm_normal(k, i);
}

/* ------------------------------------------------------------------------ */
/* Latent-like share for block selection (the Otil page's setting: diffusion */
/* activations on a spatial token grid, where adjacent steps change mostly   */
/* in a few regions). Tokens form an H x W grid in raster order, C channels. */
/*   a_0 = N(0,1) s_c, s_c ~ LogNormal(0, 0.5) per channel;                  */
/*   a_t = a_{t-1} + sigma g_t(token) N(0,1) s_c, where the intensity field  */
/*   g_t = exp(gamma z / std(z)) / rms(...) comes from a per-step N(0,1)     */
/*   field z on the grid blurred by a 2-D Gaussian (std blur tokens, radius  */
/*   ceil(3 blur), mirror padding): smooth regions of strong and weak change */
/*   whose mean square is 1, so E[step^2] = sigma^2 s_c^2.                   */
/* ------------------------------------------------------------------------ */
enum { ROLE_FIELD = 9 };

void sg_latent_init(uint64_t seed, int tensor, int H, int W, int C, float* sc, float* a0) {
  const uint64_t ks = sg_key(seed, ROLE_SCALE, tensor, 0);
  for (int j = 0; j < C; ++j) sc[j] = (float)exp(0.5 * sm_normal(ks, j));
  const uint64_t ka = sg_key(seed, ROLE_A0, tensor, 0);
  const int64_t N = (int64_t)H * W * C;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) a0[i] = (float)(sm_normal(ka, i) * sc[i % C]);
}

void sg_latent_step(uint64_t seed, int tensor, int t, int H, int W, int C, double sigma,
                    double gamma, double blur, const float* sc, float* a, double* field /* [2][H*W] */) {
  const int HW = H * W;
  const uint64_t kf = sg_key(seed, ROLE_FIELD, tensor, t);
  double* z = field;
  double* tmp = field + HW;
  for (int p = 0; p < HW; ++p) z[p] = sm_normal(kf, p);
  const int radius = (int)ceil(3.0 * blur);
  double w[256];
  double wsum = 0.0;
  for (int k = -radius; k <= radius; ++k) {
    w[k + radius] = exp(-(double)k * k / (2.0 * blur * blur));
    wsum += w[k + radius];
  }
  for (int k = 0; k <= 2 * radius; ++k) w[k] /= wsum;
  for (int h = 0; h < H; ++h)
    for (int x = 0; x < W; ++x) {
      double s = 0.0;
      for (int k = -radius; k <= radius; ++k) s += w[k + radius] * z[h * W + mirror(x + k, W)];
      tmp[h * W + x] = s;
    }
  double m1 = 0.0, m2 = 0.0;
  for (int h = 0; h < H; ++h)
    for (int x = 0; x < W; ++x) {
      double s = 0.0;
      for (int k = -radius; k <= radius; ++k) s += w[k + radius] * tmp[mirror(h + k, H) * W + x];
      z[h * W + x] = s;
      m1 += s;
      m2 += s * s;
    }
  const double mean = m1 / HW, sd = sqrt(m2 / HW - mean * mean);
  double g2 = 0.0;
  for (int p = 0; p < HW; ++p) {
    z[p] = exp(gamma * (z[p] - mean) / sd);
    g2 += z[p] * z[p];
  }
  const double norm = 1.0 / sqrt(g2 / HW);
  const uint64_t kn = sg_key(seed, ROLE_STEP, tensor, t);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)HW * C; ++i) {
    const int64_t p = i / C;
    a[i] = (float)((double)a[i] + sigma * z[p] * norm * sm_normal(kn, i) * (double)sc[i % C]);
  }
}
