/*
 * Sanitizer driver for the fp64 oracle (test infrastructure): every oracle
 * entry point on small seeded inputs, on row subsets, on empty inputs and
 * on rejected arguments, so that an AddressSanitizer / UndefinedBehavior-
 * Sanitizer build of wide_oracle.c sees every access pattern it has. Exits
 * non-zero on a wrong status; the sanitizers abort on a memory or UB error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_reorder(const uint8_t*, int64_t, int64_t, int64_t, int32_t*, int32_t*, int32_t*);
int oracle_ffn(const float*, const float*, const float*, const float*, const uint8_t*, int64_t,
               int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, double*);
int oracle_gemm_mn(const float*, const float*, const uint8_t*, int64_t, int64_t, int64_t, int64_t,
                   const int64_t*, int64_t, double*);
int oracle_gemm_k(const float*, const float*, const uint8_t*, int64_t, int64_t, int64_t, int64_t,
                  const int64_t*, int64_t, double*);
int oracle_router(const float*, const float*, const float*, int64_t, int64_t, int64_t, int64_t,
                  int, const int64_t*, int64_t, double*, uint8_t*);
int oracle_attention(const float*, const float*, const float*, const uint8_t*, int64_t, int64_t,
                     int64_t, int64_t, const int64_t*, int64_t, double*);
int oracle_num_threads(void);

static uint64_t state = 88172645463325252ull;
static double next01(void) { /* xorshift64: test data only */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / 9007199254740992.0;
}
static float* randf(int64_t n) {
  float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  for (int64_t i = 0; i < n; ++i) p[i] = (float)(2.0 * next01() - 1.0);
  return p;
}
static uint8_t* randm(int64_t n, double p) {
  uint8_t* m = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) m[i] = next01() < p ? (uint8_t)(1 + (i % 200)) : 0;
  return m;
}

static int fails = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static void ffn_case(int64_t T, int64_t d, int64_t d_ff, int64_t G, double p) {
  const int64_t ng = d_ff / G;
  float *X = randf(T * d), *Wg = randf(d_ff * d), *Wu = randf(d_ff * d), *Wd = randf(d * d_ff);
  uint8_t* m = randm(T * ng, p);
  const int64_t nr = T > 3 ? T : 3; /* output rows: every token, or the 3 sampled ones */
  double* H = (double*)malloc((size_t)nr * d_ff * sizeof(double));
  double* Y = (double*)malloc((size_t)nr * d * sizeof(double));
  EXPECT(oracle_ffn(X, Wg, Wu, Wd, m, T, d, d_ff, G, NULL, T, H, Y) == 0);
  if (T > 0) {
    int64_t rows[3] = {T - 1, 0, T / 2};
    EXPECT(oracle_ffn(X, Wg, Wu, Wd, m, T, d, d_ff, G, rows, 3, H, Y) == 0);
    int64_t bad[1] = {T};
    EXPECT(oracle_ffn(X, Wg, Wu, Wd, m, T, d, d_ff, G, bad, 1, H, Y) != 0);
  }
  int32_t* perm = (int32_t*)malloc((size_t)(T > 0 ? T : 1) * ng * sizeof(int32_t));
  int32_t* counts = (int32_t*)malloc((size_t)ng * sizeof(int32_t));
  int32_t* padded = (int32_t*)malloc((size_t)ng * sizeof(int32_t));
  EXPECT(oracle_reorder(m, T, ng, 7, perm, counts, padded) == 0);
  EXPECT(oracle_reorder(m, T, ng, 0, perm, counts, padded) != 0);
  /* masked GEMMs: N axis over d_ff outputs, K axis over d_ff inputs */
  double* C = (double*)malloc((size_t)(T > 0 ? T : 1) * (d_ff > d ? d_ff : d) * sizeof(double));
  EXPECT(oracle_gemm_mn(X, Wg, m, T, d_ff, d, G, NULL, T, C) == 0);
  float* A = randf(T * d_ff);
  EXPECT(oracle_gemm_k(A, Wd, m, T, d, d_ff, G, NULL, T, C) == 0);
  EXPECT(oracle_gemm_mn(X, Wg, m, T, d_ff, d, G + 1, NULL, T, C) != 0 || d_ff % (G + 1) == 0);
  EXPECT(oracle_ffn(X, Wg, Wu, Wd, m, T, d, d_ff, 0, NULL, T, H, Y) != 0);
  EXPECT(oracle_ffn(NULL, Wg, Wu, Wd, m, T, d, d_ff, G, NULL, T, H, Y) != 0);
  free(X); free(Wg); free(Wu); free(Wd); free(m); free(H); free(Y);
  free(perm); free(counts); free(padded); free(C); free(A);
}

int main(void) {
  ffn_case(5, 16, 64, 16, 0.5);
  ffn_case(1, 8, 24, 8, 1.0);
  ffn_case(9, 32, 96, 48, 0.3);
  ffn_case(0, 16, 32, 16, 0.5);
  ffn_case(3, 8, 32, 1, 0.5);
  /* router: three activations, rows subset, rejected r */
  {
    const int64_t T = 6, D = 32, r = 16, ng = 5;
    float *X = randf(T * D), *W1 = randf(r * D), *W2 = randf(2 * ng * r);
    double* lg = (double*)malloc((size_t)T * ng * 2 * sizeof(double));
    uint8_t* m = (uint8_t*)malloc((size_t)T * ng);
    for (int act = 0; act < 3; ++act) EXPECT(oracle_router(X, W1, W2, T, D, r, ng, act, NULL, T, lg, m) == 0);
    int64_t rows[2] = {5, 1};
    EXPECT(oracle_router(X, W1, W2, T, D, r, ng, 2, rows, 2, lg, m) == 0);
    EXPECT(oracle_router(X, W1, W2, T, D, 257, ng, 2, NULL, T, lg, m) != 0);
    EXPECT(oracle_router(X, W1, W2, T, D, r, ng, 3, NULL, T, lg, m) != 0);
    free(X); free(W1); free(W2); free(lg); free(m);
  }
  /* attention: GQA 4/2 heads, a skipped pair, rows subset */
  {
    const int64_t T = 7, Hq = 4, Hk = 2, dh = 16;
    float *Q = randf(T * Hq * dh), *K = randf(T * Hk * dh), *V = randf(T * Hk * dh);
    uint8_t* m = randm(T * Hk, 0.6);
    double* O = (double*)malloc((size_t)T * Hq * dh * sizeof(double));
    EXPECT(oracle_attention(Q, K, V, m, T, Hq, Hk, dh, NULL, T, O) == 0);
    int64_t rows[2] = {6, 0};
    EXPECT(oracle_attention(Q, K, V, m, T, Hq, Hk, dh, rows, 2, O) == 0);
    EXPECT(oracle_attention(Q, K, V, m, T, 3, Hk, dh, NULL, T, O) != 0);
    free(Q); free(K); free(V); free(m); free(O);
  }
  EXPECT(oracle_num_threads() >= 1);
  if (fails) return 1;
  printf("oracle sanitizer driver: ok\n");
  return 0;
}
