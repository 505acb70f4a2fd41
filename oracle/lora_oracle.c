/*
 * Multi-LoRA shrink / expand / expand_slice oracle, with its segment metadata.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 CPU statement
 * of what the GPU path must compute.  Only the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg load it.  It shares no code, header, table
 * or constant with the HIP library, and includes nothing from it.
 *
 * Sources (the pages are the text of four web pages; citations name the page
 * and the passage on it):
 *  - vLLM PR "[misc] Add LoRA kernel micro benchmarks": the op set
 *    (bgmv/sgmv shrink, expand, expand_slice); one call computes a whole
 *    m x k x n product in which each token's rows use the one of num_loras
 *    weight matrices that its LoRA id selects; with add_inputs set, expand
 *    adds the product to the existing output instead of replacing it; the
 *    expand input is fp32 while weights and output are fp16 (the console
 *    table's dtype label); expand_slice equals separate expands issued back
 *    to back, one per output slice.
 *  - vLLM PR "[Hardware][TPU][V1] Multi-LoRA Optimisations for the V1 TPU
 *    backend", summary: shrink and expand as two separate ops; the adapters
 *    used by expand are pre-transposed once at load time.
 *  - punica issue "The smallest rank supported is 16?": segments of tokens
 *    that share an adapter (SGMV), BGMV as a strict subset of SGMV, and
 *    padding ranks up to a bin with zero columns.
 *
 * Conventions (readings where the pages are silent):
 *  - Adapter id -1 means "no adapter"; any id outside [-1, L) is treated as
 *    -1 and counted as bad.
 *  - A_l (H x r) is stored transposed, row-major [r][H]; B_l (r x n) is
 *    stored transposed, row-major [n][r].  Both keep the contraction index
 *    contiguous; the mathematics is unchanged.
 *  - Inputs arrive as raw 16-bit patterns (dtype 0 = IEEE binary16,
 *    dtype 1 = bfloat16) and are decoded exactly to fp64 here.
 *  - Sums run in ascending index order in fp64 and are never rounded; the
 *    result for a row does not depend on the thread count.
 *  - Rows of tokens without an adapter are never written by shrink and are
 *    returned unchanged (the decoded y0) by expand.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- exact decoding of the two 16-bit formats ------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zero and the subnormals (fraction * 2^-24); field 31
 * holds infinity (fraction 0) and NaN. */
double oracle_decode_f16(uint16_t bits) {
  int sign = bits >> 15;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0)
    mag = ldexp((double)frac, -24);
  else if (expo == 31)
    mag = frac ? NAN : INFINITY;
  else
    mag = ldexp((double)(frac + 1024), expo - 25);
  return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE 754 binary32 word. */
double oracle_decode_bf16(uint16_t bits) {
  uint32_t word = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

static double g_lut[2][65536];
static int g_lut_ready = 0;

static void build_luts(void) {
  if (g_lut_ready) return;
  for (int b = 0; b < 65536; ++b) {
    g_lut[0][b] = oracle_decode_f16((uint16_t)b);
    g_lut[1][b] = oracle_decode_bf16((uint16_t)b);
  }
  g_lut_ready = 1;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the loops below (n < 1 leaves the setting alone); returns the
 * previous count.  Every row's sum order is fixed, so results do not depend
 * on it: it only changes how long a call takes. */
int oracle_set_num_threads(int n) {
  int prev = oracle_num_threads();
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
  return prev;
}

static int active_id(int32_t id, int32_t L) { return id >= 0 && id < L; }

/* ---- segment metadata -------------------------------------------------
 * Tokens that share an adapter form one segment (the punica issue's
 * example is a batch of six tokens that uses only three adapters).  The order is the
 * stable sort by (adapter id, token index) for active tokens, followed by
 * the tokens without an adapter in ascending token order.
 *
 * Outputs (caller-allocated):
 *   sorted_token[T]  token indices in that order
 *   seg_lora[L]      adapter of segment s for s < S, then -1
 *   seg_start[L+1]   first position of segment s; entries S..L hold T_a
 *   counts[4]        {S, T_a, longest segment, number of bad ids}
 * Written as the plain double loop over adapters and tokens. */
int oracle_build_segments(const int32_t *ids, int32_t T, int32_t L,
                          int32_t *sorted_token, int32_t *seg_lora,
                          int32_t *seg_start, int32_t *counts) {
  if (T < 0 || L < 1) return -1;
  int32_t pos = 0, S = 0, longest = 0, bad = 0;
  for (int32_t a = 0; a < L; ++a) {
    int32_t start = pos;
    for (int32_t t = 0; t < T; ++t)
      if (ids[t] == a) sorted_token[pos++] = t;
    int32_t len = pos - start;
    if (len > 0) {
      seg_lora[S] = a;
      seg_start[S] = start;
      ++S;
      if (len > longest) longest = len;
    }
  }
  int32_t t_active = pos;
  for (int32_t t = 0; t < T; ++t) {
    if (!active_id(ids[t], L)) {
      sorted_token[pos++] = t;
      if (ids[t] != -1) ++bad;
    }
  }
  for (int32_t s = S; s < L; ++s) seg_lora[s] = -1;
  for (int32_t s = S; s <= L; ++s) seg_start[s] = t_active;
  counts[0] = S;
  counts[1] = t_active;
  counts[2] = longest;
  counts[3] = bad;
  return 0;
}

/* ---- shrink ------------------------------------------------------------
 * v[t][j] = sum_{h<H} x[t][h] * A[id(t)][j][h]   for j < r, active t only.
 * rows[0..nrows) lists the tokens to evaluate (NULL = all T in order);
 * out is [nrows][r] fp64.  A row whose token has no adapter is left as it
 * was in out (the caller decides what it holds). */
int oracle_shrink(int dtype, const uint16_t *x, int64_t ldx, const uint16_t *A,
                  int32_t H, int32_t r, const int32_t *ids, int32_t T,
                  int32_t L, const int32_t *rows, int32_t nrows, double *out) {
  if (dtype < 0 || dtype > 1 || H < 1 || r < 1 || T < 0 || L < 1 || ldx < H)
    return -1;
  build_luts();
  const double *dec = g_lut[dtype];
  if (!rows) nrows = T;
#pragma omp parallel for schedule(dynamic, 4)
  for (int32_t i = 0; i < nrows; ++i) {
    int32_t t = rows ? rows[i] : i;
    int32_t id = ids[t];
    if (!active_id(id, L)) continue;
    const uint16_t *xt = x + (int64_t)t * ldx;
    for (int32_t j = 0; j < r; ++j) {
      const uint16_t *aj = A + ((int64_t)id * r + j) * H;
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h) acc += dec[xt[h]] * dec[aj[h]];
      out[(int64_t)i * r + j] = acc;
    }
  }
  return 0;
}

/* ---- expand ------------------------------------------------------------
 * For one output slice of width n that starts at column col_off of y:
 *   y[t][col_off+c] = (add ? y0[t][col_off+c] : 0)
 *                     + sum_{j<r} v[t][j] * B[id(t)][c][j]      c < n
 * for active t; a token without an adapter keeps y0.  v is fp64 [T][ldv]
 * (either the oracle's own shrink, or the GPU's fp32 v widened exactly).
 * rows as for shrink; out is [nrows][n] fp64. */
int oracle_expand(int dtype, const double *v, int64_t ldv, const uint16_t *B,
                  int32_t r, int32_t n, const int32_t *ids, int32_t T,
                  int32_t L, const uint16_t *y0, int64_t ldy, int64_t col_off,
                  int add, const int32_t *rows, int32_t nrows, double *out) {
  if (dtype < 0 || dtype > 1 || r < 1 || n < 1 || T < 0 || L < 1 ||
      ldv < r || col_off < 0 || ldy < col_off + n)
    return -1;
  build_luts();
  const double *dec = g_lut[dtype];
  if (!rows) nrows = T;
#pragma omp parallel for schedule(dynamic, 4)
  for (int32_t i = 0; i < nrows; ++i) {
    int32_t t = rows ? rows[i] : i;
    int32_t id = ids[t];
    const uint16_t *yt = y0 + (int64_t)t * ldy + col_off;
    double *o = out + (int64_t)i * n;
    if (!active_id(id, L)) {
      for (int32_t c = 0; c < n; ++c) o[c] = dec[yt[c]];
      continue;
    }
    const double *vt = v + (int64_t)t * ldv;
    for (int32_t c = 0; c < n; ++c) {
      const uint16_t *bc = B + ((int64_t)id * n + c) * r;
      double acc = 0.0;
      for (int32_t j = 0; j < r; ++j) acc += vt[j] * dec[bc[j]];
      o[c] = (add ? dec[yt[c]] : 0.0) + acc;
    }
  }
  return 0;
}

/* ---- expand_slice ------------------------------------------------------
 * The same as issuing oracle_expand once per slice s, with that slice's
 * weights B_s, width n_s, column offset col_off_s and input
 * v_s = v + s * v_slice_stride.  out is [nrows][sum n_s], the slices'
 * columns placed one after another in slice order. */
int oracle_expand_slice(int dtype, const double *v, int64_t ldv,
                        int64_t v_slice_stride, const uint16_t *const *Bs,
                        const int32_t *n_s, const int64_t *col_off,
                        int32_t num_slices, int32_t r, const int32_t *ids,
                        int32_t T, int32_t L, const uint16_t *y0, int64_t ldy,
                        int add, const int32_t *rows, int32_t nrows,
                        double *out) {
  if (num_slices < 1) return -1;
  int64_t width = 0;
  for (int32_t s = 0; s < num_slices; ++s) width += n_s[s];
  if (!rows) nrows = T;
  int64_t done = 0;
  for (int32_t s = 0; s < num_slices; ++s) {
    double *part = (double *)malloc(sizeof(double) * (size_t)nrows * (size_t)n_s[s] + 1);
    if (!part) return -2;
    int rc = oracle_expand(dtype, v + s * v_slice_stride, ldv, Bs[s], r, n_s[s],
                           ids, T, L, y0, ldy, col_off[s], add, rows, nrows, part);
    if (rc) { free(part); return rc; }
    for (int32_t i = 0; i < nrows; ++i)
      memcpy(out + (int64_t)i * width + done, part + (int64_t)i * n_s[s],
             sizeof(double) * (size_t)n_s[s]);
    free(part);
    done += n_s[s];
  }
  return 0;
}

/* ---- rank bins -----------------------------------------------------------
 * The punica issue's mitigation for unsupported ranks: round r up to the
 * nearest supported bin, where the bins are 16 and the multiples of 32
 * (its examples: 12 -> 16, 17 -> 32, 45 -> 64). */
int32_t oracle_rank_bin(int32_t r) {
  if (r < 1) return -1;
  if (r <= 16) return 16;
  return ((r + 31) / 32) * 32;
}
