/* Randomised driver of the fp64 oracle (test infrastructure), built with gcc
 * under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py: every entry point on random shapes, ids and
 * element types, the threaded leg against the one-thread leg. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_widen(const void *src, int dtype, int64_t n, double *dst);
void oracle_dequant_rows(const void *q, int q_dtype, const float *scale, int64_t rows, int64_t width,
                         double *out);
int oracle_segments(const int32_t *ids, int32_t T, int32_t N, int32_t *perm, int32_t *starts,
                    int32_t *adapters, int32_t *num_segments);
void oracle_shrink(int32_t T, int32_t d_in, int32_t r_max, const int32_t *ids, const int32_t *rank,
                   const int64_t *row_off, const void *x, int x_dtype, const void *a_rows, int w_dtype,
                   double *v);
void oracle_expand(int32_t T, int32_t d_out, int32_t r_max, const int32_t *ids, const int32_t *rank,
                   const int64_t *row_off, const double *v, const void *bt_rows, int w_dtype,
                   const void *y_in, int y_dtype, double *y_out);
void oracle_apply(int32_t T, int32_t d_in, int32_t d_out, const int32_t *ids, const int32_t *rank,
                  const int64_t *row_off, const void *x, int x_dtype, const void *a_rows,
                  const void *bt_rows, int w_dtype, const void *y_in, int y_dtype, double *y_out);
int oracle_apply_threads(int32_t T, int32_t d_in, int32_t d_out, const int32_t *ids, const int32_t *rank,
                         const int64_t *row_off, const void *x, int x_dtype, const void *a_rows,
                         const void *bt_rows, int w_dtype, const void *y_in, int y_dtype, double *y_out,
                         int threads);
void oracle_apply_segmented(int32_t T, int32_t d_in, int32_t d_out, const int32_t *perm,
                            const int32_t *starts, const int32_t *adapters, int32_t S,
                            const int32_t *rank, const int64_t *row_off, const void *x, int x_dtype,
                            const void *a_rows, const void *bt_rows, int w_dtype, const void *y_in,
                            int y_dtype, double *y_out);
void oracle_base_sampled(int32_t d_in, const void *x, int x_dtype, const void *w, int w_dtype,
                         int32_t n_pairs, const int32_t *tok, const int32_t *col, double *out);
void oracle_apply_sampled(int32_t d_in, int32_t d_out, const int32_t *ids, const int32_t *rank,
                          const int64_t *row_off, const void *x, int x_dtype, const void *a_rows,
                          const void *bt_rows, int w_dtype, int32_t n_pairs, const int32_t *tok,
                          const int32_t *col, const double *y_base, double *out);

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); exit(1); } } while (0)

static uint32_t st = 2463534242u;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 17; st ^= st << 5; return st; }

static void fill_f32(float *p, int64_t n) { for (int64_t i = 0; i < n; ++i) p[i] = (float)((int)(rnd() % 2001) - 1000) / 1000.f; }

int main(void) {
  for (int trial = 0; trial < 200; ++trial) {
    const int32_t T = (int32_t)(rnd() % 40), N = 1 + (int32_t)(rnd() % 6);
    const int32_t d_in = 1 + (int32_t)(rnd() % 50), d_out = 1 + (int32_t)(rnd() % 50);
    int32_t *rank = malloc(sizeof(int32_t) * N);
    int64_t *off = malloc(sizeof(int64_t) * N);
    int64_t rows = 0;
    int32_t r_max = 1;
    for (int a = 0; a < N; ++a) {
      rank[a] = 1 + (int32_t)(rnd() % 9);
      off[a] = rows;
      rows += rank[a];
      if (rank[a] > r_max) r_max = rank[a];
    }
    int32_t *ids = malloc(sizeof(int32_t) * (T + 1));
    for (int t = 0; t < T; ++t) ids[t] = (int32_t)(rnd() % (N + 1)) - 1;
    float *x = malloc(sizeof(float) * (T * d_in + 1)), *y = malloc(sizeof(float) * (T * d_out + 1));
    float *a = malloc(sizeof(float) * rows * d_in), *b = malloc(sizeof(float) * rows * d_out);
    fill_f32(x, T * d_in); fill_f32(y, T * d_out); fill_f32(a, rows * d_in); fill_f32(b, rows * d_out);
    double *out1 = malloc(sizeof(double) * (T * d_out + 1)), *out2 = malloc(sizeof(double) * (T * d_out + 1));
    double *v = malloc(sizeof(double) * (T * r_max + 1)), *out3 = malloc(sizeof(double) * (T * d_out + 1));
    oracle_apply(T, d_in, d_out, ids, rank, off, x, 0, a, b, 0, y, 0, out1);
    CHECK(oracle_apply_threads(T, d_in, d_out, ids, rank, off, x, 0, a, b, 0, y, 0, out2, 3) >= 1);
    CHECK(memcmp(out1, out2, sizeof(double) * T * d_out) == 0);
    oracle_shrink(T, d_in, r_max, ids, rank, off, x, 0, a, 0, v);
    oracle_expand(T, d_out, r_max, ids, rank, off, v, b, 0, y, 0, out3);
    int32_t *perm = malloc(sizeof(int32_t) * (T + 1)), *starts = malloc(sizeof(int32_t) * (T + 2));
    int32_t *ads = malloc(sizeof(int32_t) * (T + 1)), S = 0;
    CHECK(oracle_segments(ids, T, N, perm, starts, ads, &S) == 0);
    oracle_apply_segmented(T, d_in, d_out, perm, starts, ads, S, rank, off, x, 0, a, b, 0, y, 0, out2);
    if (T > 0) {
      int32_t tok[5], col[5];
      double base[5], o[5];
      for (int i = 0; i < 5; ++i) { tok[i] = (int32_t)(rnd() % T); col[i] = (int32_t)(rnd() % d_out); base[i] = 0.0; }
      float *w = malloc(sizeof(float) * d_out * d_in);
      fill_f32(w, d_out * d_in);
      oracle_base_sampled(d_in, x, 0, w, 0, 5, tok, col, o);
      oracle_apply_sampled(d_in, d_out, ids, rank, off, x, 0, a, b, 0, 5, tok, col, base, o);
      free(w);
    }
    uint16_t bits[64];
    uint8_t codes[32];
    double wide[64];
    float sc[4] = {1.f, 0.5f, 2.f, 0.25f};
    for (int i = 0; i < 64; ++i) bits[i] = (uint16_t)rnd();
    for (int i = 0; i < 32; ++i) codes[i] = (uint8_t)rnd();
    oracle_widen(bits, 1, 64, wide);
    oracle_widen(codes, 3, 32, wide);
    oracle_widen(codes, 4, 64, wide);
    oracle_dequant_rows(codes, 3, sc, 4, 8, wide);
    oracle_dequant_rows(codes, 4, sc, 4, 16, wide);
    free(rank); free(off); free(ids); free(x); free(y); free(a); free(b); free(out1); free(out2);
    free(out3); free(v); free(perm); free(starts); free(ads);
  }
  int32_t bad[3] = {0, 7, -2}, perm[3], starts[4], ads[3], S;
  CHECK(oracle_segments(bad, 3, 3, perm, starts, ads, &S) == -2);
  printf("oracle driver ok\n");
  return 0;
}
