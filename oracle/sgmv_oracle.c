/*
 * sgmv_oracle.c -- plain, slow, obviously-correct fp64 reference for the
 * multi-LoRA delta path.  TEST INFRASTRUCTURE ONLY: nothing in the product
 * library links, loads or calls this file; only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark do.
 *
 * Source pages (cited by title and section):
 *   [LO0]  "Multi-LoRA serving: the single translator with a thousand
 *          glossaries" (blog.lo0.es) -- sections "The bare mechanism" (equations
 *          W' = W + BA and y = Wx + B(Ax); shapes A in R^{r x d_in},
 *          B in R^{d_out x r}) and "SGMV: the kernel that holds it all up"
 *          (equation y_t = W x_t + B_{a(t)} A_{a(t)} x_t; the shrink and expand
 *          phases; grouping of the batch's tokens by adapter).
 *   [CB]   "Multi-LoRA Inference Serving" (clusterbid.com), paragraph on the
 *          fixed-size adapter pool: only a request that names an adapter gets
 *          one, so a token may carry no adapter.
 *
 * Conventions (readings of the pages, listed with reasons in the design notes):
 *   - A_a is stored as r_a rows of length d_in ("A rows"); B_a is stored as its
 *     transpose, r_a rows of length d_out ("B^T rows").  B_a[i][j] = Bt_a[j][i].
 *   - The adapters of a batch are given densely: adapter a owns rows
 *     [row_off[a], row_off[a] + rank[a]) of a_rows (width d_in) and of bt_rows
 *     (width d_out).  Paging is a storage detail of the GPU side; the oracle
 *     never sees pages.
 *   - No alpha/r scale: the delta is exactly B(Ax).
 *   - Adapter id -1 means "no adapter": the token's output row equals its input.
 *   - Every bf16 or fp32 value is widened exactly to double before use and
 *     every sum runs in double, in plain sequential index order.
 *
 * Element types: 0 = fp32, 1 = bf16 (raw 16-bit patterns), 2 = fp64,
 * 3 = FP8 E4M3 (raw bytes), 4 = INT4 (packed nibbles).
 * Build: gcc -O2 -std=c11 -fopenmp -shared -fPIC (no -ffast-math, no BLAS, no
 * SIMD intrinsics; OpenMP only spreads independent tokens over threads).
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2
#define ORACLE_FP8_E4M3 3
#define ORACLE_INT4 4

/* bf16 is the upper half of an IEEE binary32: put the 16 bits on top of 16
 * zero bits and reinterpret.  Exact for every pattern, NaN and Inf included. */
static double widen_bf16(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* FP8 E4M3 in the OCP 8-bit floating-point format: 1 sign bit, 4 exponent bits
 * (bias 7), 3 fraction bits; exponent field 0 encodes subnormals f/8 * 2^-6;
 * no infinities, and S.1111.111 is NaN (largest finite magnitude 448).  Used
 * for low-precision adapter rows ("Multi-LoRA Inference Serving",
 * clusterbid.com, paragraph on the GPU memory budget: FP8 adapter storage
 * halves the memory). */
static double widen_fp8_e4m3(uint8_t b) {
  const int e = (b >> 3) & 15, f = b & 7;
  const double sign = (b & 0x80) ? -1.0 : 1.0;
  if (e == 15 && f == 7) return 0.0 / 0.0;
  if (e == 0) return sign * ((double)f / 8.0) * (1.0 / 64.0);
  double p = 1.0;
  for (int i = 0; i < e - 7; ++i) p *= 2.0;
  for (int i = 0; i < 7 - e; ++i) p /= 2.0;
  return sign * (1.0 + (double)f / 8.0) * p;
}

/* INT4: two's-complement 4-bit integers -8..7, two per byte, element 2i in the
 * low nibble of byte i ("Multi-LoRA Inference Serving", paragraph on adapter
 * weight quantization: INT4 adapters dequantised in the layer). */
static double widen_int4(const uint8_t *base, int64_t i) {
  const int nib = (base[i >> 1] >> ((i & 1) * 4)) & 15;
  return (double)(nib >= 8 ? nib - 16 : nib);
}

/* Element i of an array of the given element type, widened to double. */
static double elem(const void *base, int dtype, int64_t i) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[i];
    case ORACLE_BF16: return widen_bf16(((const uint16_t *)base)[i]);
    case ORACLE_FP8_E4M3: return widen_fp8_e4m3(((const uint8_t *)base)[i]);
    case ORACLE_INT4: return widen_int4((const uint8_t *)base, i);
    default: return ((const double *)base)[i];
  }
}

/* Dequantised rows: out[r][c] = code[r][c] * scale[r], exactly in double (a
 * code has at most 4 significant bits and a scale 24, so the product is
 * exact).  rows x width codes of type q_dtype (FP8_E4M3 or INT4). */
void oracle_dequant_rows(const void *q, int q_dtype, const float *scale, int64_t rows,
                         int64_t width, double *out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < width; ++c)
      out[r * width + c] = elem(q, q_dtype, r * width + c) * (double)scale[r];
}

/* Exact widening of n elements into dst (exposed so tests can pin it). */
void oracle_widen(const void *src, int dtype, int64_t n, double *dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, dtype, i);
}

/* ------------------------------------------------------------------------ */
/* Segment build: group the batch's tokens by adapter ([LO0] "SGMV" section:
 * the kernel groups tokens by adapter, i.e. segments them).  Written as a
 * comparison sort of (adapter, token) pairs followed by run-length encoding --
 * deliberately a different algorithm from a counting sort.
 *   in : ids[T]            adapter per token, -1 = none
 *   out: perm[T']          tokens with an adapter, by (adapter, original index)
 *        starts[S+1]       segment s covers perm[starts[s] .. starts[s+1])
 *        adapters[S]       adapter of segment s, strictly increasing
 * Returns 0, or -2 if some id is outside {-1} U [0, N). */
typedef struct { int32_t adapter, token; } pair_t;

static int cmp_pair(const void *pa, const void *pb) {
  const pair_t *a = (const pair_t *)pa, *b = (const pair_t *)pb;
  if (a->adapter != b->adapter) return a->adapter < b->adapter ? -1 : 1;
  if (a->token != b->token) return a->token < b->token ? -1 : 1;
  return 0;
}

int oracle_segments(const int32_t *ids, int32_t T, int32_t N, int32_t *perm,
                    int32_t *starts, int32_t *adapters, int32_t *num_segments) {
  pair_t *pairs = (pair_t *)malloc(sizeof(pair_t) * (size_t)(T > 0 ? T : 1));
  int32_t n = 0;
  for (int32_t t = 0; t < T; ++t) {
    if (ids[t] == -1) continue;
    if (ids[t] < 0 || ids[t] >= N) { free(pairs); return -2; }
    pairs[n].adapter = ids[t];
    pairs[n].token = t;
    ++n;
  }
  qsort(pairs, (size_t)n, sizeof(pair_t), cmp_pair);
  int32_t S = 0;
  for (int32_t i = 0; i < n; ++i) {
    perm[i] = pairs[i].token;
    if (i == 0 || pairs[i].adapter != pairs[i - 1].adapter) {
      starts[S] = i;
      adapters[S] = pairs[i].adapter;
      ++S;
    }
  }
  starts[S] = n;
  *num_segments = S;
  free(pairs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Shrink ([LO0] "SGMV" section, phase 1: d_in -> r through A_{a(t)}):
 *   v[t][j] = sum_{k < d_in} A_{a(t)}[j][k] * x[t][k]      for j < rank[a(t)]
 * v is [T, r_max] doubles; entries j >= rank and rows of tokens without an
 * adapter are set to 0. */
void oracle_shrink(int32_t T, int32_t d_in, int32_t r_max, const int32_t *ids,
                   const int32_t *rank, const int64_t *row_off, const void *x,
                   int x_dtype, const void *a_rows, int w_dtype, double *v) {
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < r_max; ++j) v[(int64_t)t * r_max + j] = 0.0;
    int32_t a = ids[t];
    if (a < 0) continue;
    for (int32_t j = 0; j < rank[a]; ++j) {
      double s = 0.0;
      int64_t arow = (row_off[a] + j) * (int64_t)d_in;
      for (int32_t k = 0; k < d_in; ++k)
        s += elem(a_rows, w_dtype, arow + k) * elem(x, x_dtype, (int64_t)t * d_in + k);
      v[(int64_t)t * r_max + j] = s;
    }
  }
}

/* Expand ([LO0] "SGMV" section, phase 2: r -> d_out through B_{a(t)}, added to
 * the output):
 *   y_out[t][i] = y_in[t][i] + sum_{j < rank} B_{a(t)}[i][j] * v[t][j]
 * with B[i][j] read from the B^T rows as bt[j][i].  v is given in doubles
 * ([T, r_max]); y_in in its element type; y_out is [T, d_out] doubles. */
void oracle_expand(int32_t T, int32_t d_out, int32_t r_max, const int32_t *ids,
                   const int32_t *rank, const int64_t *row_off, const double *v,
                   const void *bt_rows, int w_dtype, const void *y_in, int y_dtype,
                   double *y_out) {
  for (int32_t t = 0; t < T; ++t) {
    int32_t a = ids[t];
    for (int32_t i = 0; i < d_out; ++i) {
      double y = elem(y_in, y_dtype, (int64_t)t * d_out + i);
      if (a >= 0) {
        double s = 0.0;
        for (int32_t j = 0; j < rank[a]; ++j)
          s += elem(bt_rows, w_dtype, (row_off[a] + j) * (int64_t)d_out + i) *
               v[(int64_t)t * r_max + j];
        y += s;
      }
      y_out[(int64_t)t * d_out + i] = y;
    }
  }
}

/* The whole delta for one token t ([LO0] "The bare mechanism": y = Wx + B(Ax),
 * BA never formed; "SGMV" section: the per-token adapter a(t)).  y_in plays
 * the role of Wx.  v is caller scratch of at least rank[a(t)] doubles. */
static void apply_token(int32_t t, int32_t d_in, int32_t d_out, const int32_t *ids,
                        const int32_t *rank, const int64_t *row_off, const void *x,
                        int x_dtype, const void *a_rows, const void *bt_rows, int w_dtype,
                        const void *y_in, int y_dtype, double *y_out, double *v) {
  int32_t a = ids[t];
  int32_t r = a >= 0 ? rank[a] : 0;
  for (int32_t j = 0; j < r; ++j) {
    double s = 0.0;
    int64_t arow = (row_off[a] + j) * (int64_t)d_in;
    for (int32_t k = 0; k < d_in; ++k)
      s += elem(a_rows, w_dtype, arow + k) * elem(x, x_dtype, (int64_t)t * d_in + k);
    v[j] = s;
  }
  for (int32_t i = 0; i < d_out; ++i) {
    double y = elem(y_in, y_dtype, (int64_t)t * d_out + i);
    if (a >= 0) {
      double s = 0.0;
      for (int32_t j = 0; j < r; ++j)
        s += elem(bt_rows, w_dtype, (row_off[a] + j) * (int64_t)d_out + i) * v[j];
      y += s;
    }
    y_out[(int64_t)t * d_out + i] = y;
  }
}

static int32_t max_rank_used(int32_t T, const int32_t *ids, const int32_t *rank) {
  int32_t r_cap = 1;
  for (int32_t t = 0; t < T; ++t)
    if (ids[t] >= 0 && rank[ids[t]] > r_cap) r_cap = rank[ids[t]];
  return r_cap;
}

/* The whole delta, token by token, in token order.  Tokens are independent, so
 * one token's v lives only in a small buffer. */
void oracle_apply(int32_t T, int32_t d_in, int32_t d_out, const int32_t *ids,
                  const int32_t *rank, const int64_t *row_off, const void *x,
                  int x_dtype, const void *a_rows, const void *bt_rows, int w_dtype,
                  const void *y_in, int y_dtype, double *y_out) {
  double *v = (double *)malloc(sizeof(double) * (size_t)max_rank_used(T, ids, rank));
  for (int32_t t = 0; t < T; ++t)
    apply_token(t, d_in, d_out, ids, rank, row_off, x, x_dtype, a_rows, bt_rows, w_dtype, y_in,
                y_dtype, y_out, v);
  free(v);
}

/* oracle_apply with the tokens shared among `threads` OpenMP threads (each
 * token's arithmetic is apply_token's, so the output is bit-identical to
 * oracle_apply).  Returns the number of threads that ran. */
int oracle_apply_threads(int32_t T, int32_t d_in, int32_t d_out, const int32_t *ids,
                         const int32_t *rank, const int64_t *row_off, const void *x,
                         int x_dtype, const void *a_rows, const void *bt_rows, int w_dtype,
                         const void *y_in, int y_dtype, double *y_out, int threads) {
  const int32_t r_cap = max_rank_used(T, ids, rank);
  int used = 1;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
  {
    double *v = (double *)malloc(sizeof(double) * (size_t)r_cap);
#pragma omp single
    used = omp_get_num_threads();
#pragma omp for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t)
      apply_token(t, d_in, d_out, ids, rank, row_off, x, x_dtype, a_rows, bt_rows, w_dtype, y_in,
                  y_dtype, y_out, v);
    free(v);
  }
  return used;
}

/* The same delta, walked segment by segment over the output of
 * oracle_segments ([LO0] TL;DR: Y += sum_i X_i A_i B_i, one term per adapter
 * group).  Tokens outside every segment keep y_in.  Used to check that grouping
 * changes nothing. */
void oracle_apply_segmented(int32_t T, int32_t d_in, int32_t d_out,
                            const int32_t *perm, const int32_t *starts,
                            const int32_t *adapters, int32_t S, const int32_t *rank,
                            const int64_t *row_off, const void *x, int x_dtype,
                            const void *a_rows, const void *bt_rows, int w_dtype,
                            const void *y_in, int y_dtype, double *y_out) {
  for (int64_t i = 0; i < (int64_t)T * d_out; ++i) y_out[i] = elem(y_in, y_dtype, i);
  int32_t r_cap = 1;
  for (int32_t s = 0; s < S; ++s)
    if (rank[adapters[s]] > r_cap) r_cap = rank[adapters[s]];
  double *v = (double *)malloc(sizeof(double) * (size_t)r_cap);
  for (int32_t s = 0; s < S; ++s) {
    int32_t a = adapters[s], r = rank[a];
    for (int32_t p = starts[s]; p < starts[s + 1]; ++p) {
      int32_t t = perm[p];
      for (int32_t j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int32_t k = 0; k < d_in; ++k)
          acc += elem(a_rows, w_dtype, (row_off[a] + j) * (int64_t)d_in + k) *
                 elem(x, x_dtype, (int64_t)t * d_in + k);
        v[j] = acc;
      }
      for (int32_t i = 0; i < d_out; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < r; ++j)
          acc += elem(bt_rows, w_dtype, (row_off[a] + j) * (int64_t)d_out + i) * v[j];
        y_out[(int64_t)t * d_out + i] += acc;
      }
    }
  }
  free(v);
}

/* Base projection, sampled ([LO0] "The bare mechanism": the base term Wx with
 * W in R^{d_out x d_in}, stored row-major).  For each requested (token, column)
 * pair:  out[p] = sum_{k < d_in} W[col][k] * x[tok][k]. */
void oracle_base_sampled(int32_t d_in, const void *x, int x_dtype, const void *w,
                         int w_dtype, int32_t n_pairs, const int32_t *tok,
                         const int32_t *col, double *out) {
  for (int32_t p = 0; p < n_pairs; ++p) {
    double s = 0.0;
    for (int32_t k = 0; k < d_in; ++k)
      s += elem(w, w_dtype, (int64_t)col[p] * d_in + k) *
           elem(x, x_dtype, (int64_t)tok[p] * d_in + k);
    out[p] = s;
  }
}

/* Delta for a sample of (token, column) pairs, with the base value supplied
 * per pair (y_base[p]):  out[p] = y_base[p] + sum_j Bt[j][col] * (A x)[j].
 * Shares its definition with oracle_apply; lets full-size checks touch only
 * the sampled outputs. */
void oracle_apply_sampled(int32_t d_in, int32_t d_out, const int32_t *ids,
                          const int32_t *rank, const int64_t *row_off, const void *x,
                          int x_dtype, const void *a_rows, const void *bt_rows,
                          int w_dtype, int32_t n_pairs, const int32_t *tok,
                          const int32_t *col, const double *y_base, double *out) {
  for (int32_t p = 0; p < n_pairs; ++p) {
    int32_t t = tok[p], i = col[p], a = ids[t];
    double y = y_base[p];
    if (a >= 0) {
      double s = 0.0;
      for (int32_t j = 0; j < rank[a]; ++j) {
        double vj = 0.0;
        for (int32_t k = 0; k < d_in; ++k)
          vj += elem(a_rows, w_dtype, (row_off[a] + j) * (int64_t)d_in + k) *
                elem(x, x_dtype, (int64_t)t * d_in + k);
        s += elem(bt_rows, w_dtype, (row_off[a] + j) * (int64_t)d_out + i) * vj;
      }
      y += s;
    }
    out[p] = y;
  }
}
