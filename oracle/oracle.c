/*
 * CPU ORACLE -- test infrastructure only.
 *
 * A plain, slow, single-threaded C implementation of what the residual
 * compression path computes. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the GPU library never does, and
 * the two share no code (not even headers or the packed-layout arithmetic).
 *
 * Source of the method: the paper-notes page "Accelerating Parallel Diffusion
 * Model Serving with Residual Compression" (CompactFusion), called "the
 * CompactFusion notes" below. Sections cited by their headings:
 *   - Method / Overall framework: send C(a_t - ahat_{t-1}); the receiver keeps
 *     ahat_t = ahat_{t-1} + C(.).
 *   - Key designs / Error feedback: the part of the residual that C drops,
 *     e_t = residual - C(residual), is kept locally and re-enters the next
 *     residual.
 *   - Key designs / Low-rank strategy for extreme compression: X ~ U V^T by
 *     subspace iteration (instead of an SVD), with INT4 factors.
 *   - Key designs / System co-design: N:M block sparsifier instead of TopK.
 *   - Main experiment table: 1-bit (16x) and 2-bit (8x) quantisation.
 * Where the pages leave a step open, the reading taken is stated at the
 * function; the full list of readings is kept with the design notes.
 *
 * Precision: the reconstruction ahat and the error-feedback buffer e are fp32
 * state, so every operation that produces them is one IEEE fp32 operation
 * (build with -ffp-contract=off, no fast-math). Decisions that turn floats into
 * integer codes (signs, 2-bit levels, N:M selection) are taken in fp32, the
 * precision the GPU kernels take them in. The low-rank factorisation is a
 * continuous computation and runs in fp64.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */
/* Round an fp32 value to the nearest bfloat16 (ties to even) and return its
 * 16-bit pattern: keep the top 16 bits after adding half of the dropped
 * range, plus one when the kept part is odd (textbook round-half-even on the
 * bit pattern; carries into the exponent give the correct overflow to inf). */
uint16_t orc_bf16_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x40u);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

float orc_bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

float orc_bf16_round(float x) { return orc_bf16_value(orc_bf16_bits(x)); }

void orc_bf16_round_array(int64_t count, const float* x, float* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = orc_bf16_round(x[i]);
}

/* ------------------------------------------------------------ recurrence */
/* Residual against the reconstruction the receiver holds (CompactFusion
 * notes, Overall framework): r = a_t - ahat_{t-1}, one fp32 subtraction.
 * Reading: this residual already carries the previous step's dropped error,
 * because a_{t-1} - ahat_{t-1} = e_{t-1} after every step (Error feedback);
 * no second e term is added. */
void orc_residual(int64_t count, const float* a, const float* ahat, float* r) {
  for (int64_t i = 0; i < count; ++i) r[i] = a[i] - ahat[i];
}

/* Error feedback and local reconstruction (Error feedback; Overall framework):
 *   e = r - C(r)          (what was not transmitted)
 *   ahat = ahat + C(r)    (the same update the receiver applies)          */
void orc_ef_update(int64_t count, const float* r, const float* c, float* e, float* ahat) {
  for (int64_t i = 0; i < count; ++i) {
    e[i] = r[i] - c[i];
    ahat[i] = ahat[i] + c[i];
  }
}

/* Receiver side (Overall framework): ahat_r = ahat_r + C(r). */
void orc_accumulate(int64_t count, const float* c, float* ahat) {
  for (int64_t i = 0; i < count; ++i) ahat[i] = ahat[i] + c[i];
}

/* Same two updates with a decoded value held in fp64 (low-rank path): the
 * fp32 state takes one rounding of the exact fp64 result. */
void orc_ef_update_f64(int64_t count, const float* r, const double* c, float* e, float* ahat) {
  for (int64_t i = 0; i < count; ++i) {
    e[i] = (float)((double)r[i] - c[i]);
    ahat[i] = (float)((double)ahat[i] + c[i]);
  }
}

void orc_accumulate_f64(int64_t count, const double* c, float* ahat) {
  for (int64_t i = 0; i < count; ++i) ahat[i] = (float)((double)ahat[i] + c[i]);
}

/* ------------------------------------------------------------ 1-bit (Q1) */
/* 1-bit binarisation of the residual (CompactFusion notes, Residual
 * compression; Main experiment table, "1bit (16x)"). Per group of `group`
 * contiguous elements: one sign bit per element and one fp32 magnitude.
 * Readings: the magnitude is the mean of |r| over the group (the value that
 * minimises the squared error for fixed signs), rounded once to fp32 (nearest,
 * ties to even): the exact mean, not the result of any particular order of
 * floating-point additions. The bit is 1 when r >= 0 (so -0 and +0 both give
 * 1). Bits are LSB-first: element k of the array is bit k%8 of byte k/8.
 *
 * Exact mean: every finite fp32 value is an integer multiple of 2^-149 below
 * 2^128, so the sum of at most 256 magnitudes is an integer S below 2^285 in
 * units of 2^-149. It is accumulated exactly in ten 32-bit limbs (a plain
 * multi-word integer), and the mean S * 2^-149 / group is rounded to fp32 bit
 * by bit from S. */
#define Q1_LIMBS 10

/* S += m * 2^pos (m < 2^24): schoolbook addition with carry. */
static void limbs_add(uint32_t* S, uint64_t m, int pos) {
  uint64_t carry = m << (pos % 32); /* at most 55 bits */
  for (int w = pos / 32; w < Q1_LIMBS && carry; ++w) {
    const uint64_t t = (uint64_t)S[w] + (carry & 0xFFFFFFFFu);
    S[w] = (uint32_t)t;
    carry = (carry >> 32) + (t >> 32);
  }
}

static int limbs_bit(const uint32_t* S, int i) { return (int)((S[i / 32] >> (i % 32)) & 1u); }

/* fp32 nearest to S * 2^(-149 - g), ties to even, for an integer S >= 0. */
static float limbs_round(const uint32_t* S, int g) {
  int top = -1; /* index of the highest set bit */
  for (int i = 32 * Q1_LIMBS - 1; i >= 0; --i)
    if (limbs_bit(S, i)) { top = i; break; }
  if (top < 0) return 0.0f;
  /* Bits below `drop` do not fit the result: 24 significant bits for a normal
   * result, or the subnormal grid 2^-149 = 2^g units of S. */
  int drop = top - 23;
  if (drop < g) drop = g;
  uint64_t q = 0; /* S >> drop (at most 24 bits) */
  for (int i = top; i >= drop; --i) q = (q << 1) | (uint64_t)limbs_bit(S, i);
  if (drop > 0) {
    const int half = limbs_bit(S, drop - 1);
    int below = 0;
    for (int i = 0; i < drop - 1; ++i) below |= limbs_bit(S, i);
    if (half && (below || (q & 1u))) q += 1; /* round to nearest, ties to even */
  }
  /* q * 2^(drop - 149 - g) is an fp32 value (q <= 2^24), so both conversions
   * below are exact. */
  return (float)ldexp((double)q, drop - 149 - g);
}

static float q1_mean_abs(const float* r, int group) {
  uint32_t S[Q1_LIMBS] = {0};
  int g = 0;
  while ((1 << g) < group) ++g; /* group is a power of two */
  for (int i = 0; i < group; ++i) {
    uint32_t u;
    memcpy(&u, &r[i], 4);
    const uint32_t ex = (u >> 23) & 0xFFu, frac = u & 0x7FFFFFu;
    if (ex == 0xFFu) continue; /* NaN / Inf: unspecified */
    /* |r| = mant * 2^(max(ex,1) - 150) = mant * 2^(max(ex,1) - 1) units of 2^-149 */
    const uint64_t mant = ex ? (frac | 0x800000u) : frac;
    limbs_add(S, mant, (ex ? (int)ex : 1) - 1);
  }
  return limbs_round(S, g);
}

void orc_q1_encode(int64_t count, int group, const float* r, uint8_t* bits, float* scale) {
  memset(bits, 0, (size_t)(count / 8));
  for (int64_t g = 0; g < count / group; ++g) scale[g] = q1_mean_abs(r + g * group, group);
  for (int64_t k = 0; k < count; ++k)
    if (r[k] >= 0.0f) bits[k / 8] |= (uint8_t)(1u << (k % 8));
}

void orc_q1_decode(int64_t count, int group, const uint8_t* bits, const float* scale, float* c) {
  for (int64_t k = 0; k < count; ++k) {
    const float s = scale[k / group];
    c[k] = ((bits[k / 8] >> (k % 8)) & 1u) ? s : -s;
  }
}

/* ------------------------------------------------------------ 2-bit (Q2) */
/* 2-bit uniform quantisation with group min/max (Main experiment table,
 * "2bit (8x)"; four levels mn + q*d, q = 0..3, d = (mx - mn)/3).
 * Readings (all fp32, one rounding per operation):
 *   mn  = group minimum, a zero stored as +0 (the page fixes no sign of zero;
 *         no decoded value depends on it)
 *   d   = (mx - mn) / 3, a zero stored as +0
 *   if d < FLT_MIN (constant or denormal-range group): q = 0 everywhere
 *   else inv = 1/d, t = (r - mn) * inv, q = min(3, round-half-even(t))
 *   decode c = fma(q, d, mn) (one rounding).
 * Codes are LSB-first: element k is bits 2(k%4)..2(k%4)+1 of byte k/4. */
void orc_q2_encode(int64_t count, int group, const float* r, uint8_t* codes, float* mn_out,
                   float* d_out) {
  memset(codes, 0, (size_t)(count / 4));
  for (int64_t g = 0; g < count / group; ++g) {
    const float* x = r + g * group;
    float mn = x[0], mx = x[0];
    for (int i = 1; i < group; ++i) {
      if (x[i] < mn) mn = x[i];
      if (x[i] > mx) mx = x[i];
    }
    /* a zero minimum or step is stored as +0 (x + 0 turns -0 into +0) */
    mn = mn + 0.0f;
    const float range = mx - mn;
    const float d = range / 3.0f + 0.0f;
    mn_out[g] = mn;
    d_out[g] = d;
    if (!(d >= FLT_MIN)) continue; /* all codes 0 */
    const float inv = 1.0f / d;
    for (int i = 0; i < group; ++i) {
      const float diff = x[i] - mn;
      const float t = diff * inv;
      int q = (int)rintf(t);
      if (q > 3) q = 3;
      if (q < 0) q = 0;
      const int64_t k = g * group + i;
      codes[k / 4] |= (uint8_t)(q << (2 * (k % 4)));
    }
  }
}

void orc_q2_decode(int64_t count, int group, const uint8_t* codes, const float* mn,
                   const float* d, float* c) {
  for (int64_t k = 0; k < count; ++k) {
    const int q = (codes[k / 4] >> (2 * (k % 4))) & 3;
    c[k] = fmaf((float)q, d[k / group], mn[k / group]);
  }
}

/* ------------------------------------------------------------ N:M (2:16) */
/* N:M block sparsifier (CompactFusion notes, System co-design): in every
 * block of 16 contiguous elements keep the 2 with the largest |r|, ties to the
 * lower index. Kept values travel as bf16 (round to nearest even); dropped
 * positions decode to 0, so their whole residual stays in e.
 * Storage per block: vals[2] = bf16 bits of the two kept values in ascending
 * index order, idx = i0 | (i1 << 4) with i0 < i1.
 * The selection is written as two plain arg-max scans (first maximum wins). */
void orc_nm_encode(int64_t count, const float* r, uint16_t* vals, uint8_t* idx) {
  for (int64_t b = 0; b < count / 16; ++b) {
    const float* x = r + b * 16;
    int best = 0;
    for (int i = 1; i < 16; ++i)
      if (fabsf(x[i]) > fabsf(x[best])) best = i;
    int second = (best == 0) ? 1 : 0;
    for (int i = 0; i < 16; ++i)
      if (i != best && fabsf(x[i]) > fabsf(x[second])) second = i;
    const int i0 = best < second ? best : second;
    const int i1 = best < second ? second : best;
    vals[2 * b] = orc_bf16_bits(x[i0]);
    vals[2 * b + 1] = orc_bf16_bits(x[i1]);
    idx[b] = (uint8_t)(i0 | (i1 << 4));
  }
}

void orc_nm_decode(int64_t count, const uint16_t* vals, const uint8_t* idx, float* c) {
  for (int64_t b = 0; b < count / 16; ++b) {
    for (int i = 0; i < 16; ++i) c[b * 16 + i] = 0.0f;
    const int i0 = idx[b] & 15, i1 = idx[b] >> 4;
    c[b * 16 + i0] = orc_bf16_value(vals[2 * b]);
    c[b * 16 + i1] = orc_bf16_value(vals[2 * b + 1]);
  }
}

/* ------------------------------------------------------- low rank (LR) */
/* Rank-k factorisation of the residual by subspace iteration, INT4 factors
 * (CompactFusion notes, Low-rank strategy for extreme compression).
 * Steps, for an n x m residual r (row-major) and a given start Q0 (m x k):
 *   R = bf16(r)
 *   Q = Q0
 *   repeat iters times:
 *     P = R * bf16(Q)                      (n x k)
 *     P = CQR(CQR(P))                      (CholeskyQR2: orthonormal columns)
 *     Q = R^T * bf16(P)                    (m x k)
 *   U = P, V = Q                           (so U V^T = P P^T R)
 *   INT4 per column of U and of V: s = absmax/7 (stored fp32),
 *   q = clamp(round-half-even(x / s), -7, 7), q = 0 when s = 0.
 * Readings: R is bf16 (the workload states it); the tall-skinny operands are
 * rounded to bf16 the same way since a bf16 product takes both operands in
 * bf16; everything else (products, Gram matrices, Cholesky, solves) is fp64.
 * CQR(P): G = P^T P, L = chol(G) (G = L L^T), P <- P L^{-T}. A column whose
 * Cholesky pivot is <= 2^-23 * max(trace(G), k*FLT_MIN) is declared dead: its
 * column of P is set to 0 (so a zero or rank-deficient residual gives zero
 * factor columns instead of NaN). */
static double bf16d(double x) { return (double)orc_bf16_round((float)x); }

/* G = L L^T by the Cholesky-Banachiewicz recurrence, with the dead-column
 * rule above. L is k x k lower triangular, dead[j] = 1 for dead columns. */
static void chol_dead(int k, const double* G, double* L, unsigned char* dead) {
  double trace = 0.0;
  for (int j = 0; j < k; ++j) trace += G[j * k + j];
  const double floor_ = (double)k * (double)FLT_MIN;
  const double tol = ldexp(trace > floor_ ? trace : floor_, -23);
  memset(L, 0, sizeof(double) * (size_t)k * k);
  for (int j = 0; j < k; ++j) {
    double d = G[j * k + j];
    for (int p = 0; p < j; ++p) d -= L[j * k + p] * L[j * k + p];
    if (d <= tol) {
      dead[j] = 1;
      for (int p = 0; p < j; ++p) L[j * k + p] = 0.0;
      L[j * k + j] = 1.0;
      continue; /* column j below the diagonal stays 0 */
    }
    dead[j] = 0;
    const double ljj = sqrt(d);
    L[j * k + j] = ljj;
    for (int i = j + 1; i < k; ++i) {
      double s = G[i * k + j];
      for (int p = 0; p < j; ++p) s -= L[i * k + p] * L[j * k + p];
      L[i * k + j] = s / ljj;
    }
  }
}

/* One CholeskyQR step on P (n x k, row-major, in place); returns the number
 * of dead columns. Each row p of P becomes x with x L^T = p, i.e. L x^T = p^T
 * (forward substitution). */
static int cqr(int n, int k, double* P) {
  double* G = (double*)calloc((size_t)k * k, sizeof(double));
  double* L = (double*)malloc(sizeof(double) * (size_t)k * k);
  unsigned char* dead = (unsigned char*)malloc((size_t)k);
  for (int a = 0; a < k; ++a)
    for (int b = 0; b < k; ++b) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += P[(size_t)i * k + a] * P[(size_t)i * k + b];
      G[a * k + b] = s;
    }
  chol_dead(k, G, L, dead);
  int ndead = 0;
  for (int j = 0; j < k; ++j) ndead += dead[j];
  for (int i = 0; i < n; ++i) {
    double* p = P + (size_t)i * k;
    for (int j = 0; j < k; ++j) {
      double s = p[j];
      for (int q = 0; q < j; ++q) s -= L[j * k + q] * p[q];
      p[j] = dead[j] ? 0.0 : s / L[j * k + j];
    }
  }
  free(G);
  free(L);
  free(dead);
  return ndead;
}

static void int4_columns(int rows, int k, const double* X, int8_t* q, float* s) {
  for (int j = 0; j < k; ++j) {
    double amax = 0.0;
    for (int i = 0; i < rows; ++i) {
      const double v = fabs(X[(size_t)i * k + j]);
      if (v > amax) amax = v;
    }
    s[j] = (float)(amax / 7.0);
    for (int i = 0; i < rows; ++i) {
      int v = 0;
      if (s[j] > 0.0f) {
        const double t = X[(size_t)i * k + j] / (double)s[j];
        v = (int)rint(t);
        if (v > 7) v = 7;
        if (v < -7) v = -7;
      }
      q[(size_t)i * k + j] = (int8_t)v;
    }
  }
}

/* Encode one n x m residual. Outputs: qu [n x k], qv [m x k] (INT4 values in
 * int8), su[k], sv[k]. Optional u_out [n x k], v_out [m x k]: the unquantised
 * fp64 factors. Returns the number of dead columns in the final CQR. */
int orc_lr_encode(int n, int m, int k, int iters, const float* r, const float* q0, int8_t* qu,
                  int8_t* qv, float* su, float* sv, double* u_out, double* v_out) {
  double* R = (double*)malloc(sizeof(double) * (size_t)n * m);
  double* Q = (double*)malloc(sizeof(double) * (size_t)m * k);
  double* P = (double*)malloc(sizeof(double) * (size_t)n * k);
  double* op = (double*)malloc(sizeof(double) * (size_t)(n > m ? n : m) * k);
  int ndead = 0;
  for (size_t i = 0; i < (size_t)n * m; ++i) R[i] = (double)orc_bf16_round(r[i]);
  for (size_t i = 0; i < (size_t)m * k; ++i) Q[i] = (double)q0[i];
  for (int it = 0; it < iters; ++it) {
    for (size_t i = 0; i < (size_t)m * k; ++i) op[i] = bf16d(Q[i]);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < k; ++j) {
        double s = 0.0;
        for (int c = 0; c < m; ++c) s += R[(size_t)i * m + c] * op[(size_t)c * k + j];
        P[(size_t)i * k + j] = s;
      }
    cqr(n, k, P);
    ndead = cqr(n, k, P);
    for (size_t i = 0; i < (size_t)n * k; ++i) op[i] = bf16d(P[i]);
    for (int c = 0; c < m; ++c)
      for (int j = 0; j < k; ++j) {
        double s = 0.0;
        for (int i = 0; i < n; ++i) s += R[(size_t)i * m + c] * op[(size_t)i * k + j];
        Q[(size_t)c * k + j] = s;
      }
  }
  int4_columns(n, k, P, qu, su);
  int4_columns(m, k, Q, qv, sv);
  if (u_out) memcpy(u_out, P, sizeof(double) * (size_t)n * k);
  if (v_out) memcpy(v_out, Q, sizeof(double) * (size_t)m * k);
  free(R);
  free(Q);
  free(P);
  free(op);
  return ndead;
}

/* c = Uq Vq^T with Uq = q_u * s_u and Vq = q_v * s_v per column (fp64). */
void orc_lr_decode(int n, int m, int k, const int8_t* qu, const int8_t* qv, const float* su,
                   const float* sv, double* c) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < m; ++j) {
      double s = 0.0;
      for (int p = 0; p < k; ++p)
        s += ((double)qu[(size_t)i * k + p] * su[p]) * ((double)qv[(size_t)j * k + p] * sv[p]);
      c[(size_t)i * m + j] = s;
    }
}

/* Unquantised subspace-iteration factors only (for the convergence checks):
 * same steps as orc_lr_encode without the INT4 stage. */
int orc_lr_factors(int n, int m, int k, int iters, const float* r, const float* q0, double* u,
                   double* v) {
  int8_t* qu = (int8_t*)malloc((size_t)n * k);
  int8_t* qv = (int8_t*)malloc((size_t)m * k);
  float* su = (float*)malloc(sizeof(float) * (size_t)k);
  float* sv = (float*)malloc(sizeof(float) * (size_t)k);
  const int nd = orc_lr_encode(n, m, k, iters, r, q0, qu, qv, su, sv, u, v);
  free(qu);
  free(qv);
  free(su);
  free(sv);
  return nd;
}

/* ------------------------------------------------------------ block selection */
/* Otil-style block selection ("Otil: Accelerating Diffusion Model Inference
 * via Communication-Efficient Multi-GPU Parallelism", Key designs 1 and 2).
 * Tokens form a grid of grid_w columns (raster order); a block is 8 x 8 tokens
 * with all m channels, blocks numbered in raster order. For block i the
 * dissimilarity is d = 1 - <A_i, B_i>_F / (|A_i|_F |B_i|_F) between two
 * activations A and B; the scheme passes the same block at two consecutive
 * denoising steps. Readings: both blocks zero -> d = 0; exactly one zero ->
 * d = 1. Sums in fp64 over the block's tokens in raster order, channels
 * innermost (products of two fp32 values are exact in fp64). */
void orc_bs_scores(int n, int m, int grid_w, const float* A, const float* B, double* d) {
  const int gh = n / grid_w, nbx = grid_w / 8, nby = gh / 8;
  for (int by = 0; by < nby; ++by)
    for (int bx = 0; bx < nbx; ++bx) {
      double dot = 0.0, na = 0.0, nb = 0.0;
      for (int dy = 0; dy < 8; ++dy)
        for (int dx = 0; dx < 8; ++dx) {
          const int64_t tok = (int64_t)(by * 8 + dy) * grid_w + bx * 8 + dx;
          for (int c = 0; c < m; ++c) {
            const double x = A[tok * m + c], y = B[tok * m + c];
            dot += x * y;
            na += x * x;
            nb += y * y;
          }
        }
      double v;
      if (na == 0.0 && nb == 0.0) v = 0.0;
      else if (na == 0.0 || nb == 0.0) v = 1.0;
      else v = 1.0 - dot / sqrt(na * nb);
      d[by * nbx + bx] = v;
    }
}
