/*
 * fp64 CPU oracle for WIDE's token-wise group-sparse SwiGLU FFN.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or
 * loads this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header or table with the HIP path.
 *
 * What it computes is the plain definition, written out with no blocking,
 * fusion or reordering:
 *
 *   Groups: the FFN intermediate dimension d_ff is cut into contiguous groups
 *   of G channels; group g holds channels [g*G, (g+1)*G). One binary mask
 *   matrix M[T, ngroups] covers the whole FFN layer, and a token either keeps
 *   or skips each group.
 *     (WIDE, ai.info summary, "Methodology in Plain English" / "What gets
 *      pruned"; WIDE paper, Sec. 3.1 "Preliminaries")
 *
 *   Per token t and channel c in group g:
 *     H[t,c] = silu(X[t,:].Wg[c,:]) * (X[t,:].Wu[c,:])   if M[t,g] != 0
 *     H[t,c] = 0                                        otherwise (select)
 *   Y[t,n] = sum_c Wd[n,c] * H[t,c]
 *   with silu(a) = a / (1 + exp(-a)), no biases. Weights are stored [out, in]
 *   (C = A B^T, A [M,K], B [N,K]: WIDE paper Sec. 3.2 and App. B
 *   "Implementation of GEMM-MN"), and the pruned projections are gate/up on the
 *   N axis and down on the K axis (App. B, GEMM-MN and GEMM-K).
 *
 *   Mask reordering: for every group, the tokens are sorted so that active
 *   rows form a contiguous prefix (ai.info summary, "How the speedups are
 *   obtained"; WIDE paper Sec. 1, "tile-aligned prefixes"). The reading used
 *   here is a stable partition of [0, T): active tokens in ascending order,
 *   then inactive tokens in ascending order; counts[g] is the number of
 *   active tokens and padded[g] = ceil(counts[g] / tile) * tile.
 *
 * Inputs are float32 arrays whose values are exact (bf16 values are exactly
 * representable in float32); every product and sum is taken in double.
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* Stable partition of each mask column into active-then-inactive tokens. */
int oracle_reorder(const uint8_t* mask, int64_t T, int64_t ngroups, int64_t tile,
                   int32_t* perm, int32_t* counts, int32_t* padded) {
  if (!mask || !perm || !counts || !padded || T < 0 || ngroups <= 0 || tile <= 0)
    return ORACLE_BAD_ARG;
  for (int64_t g = 0; g < ngroups; ++g) {
    int64_t n = 0;
    for (int64_t t = 0; t < T; ++t)
      if (mask[t * ngroups + g] != 0) perm[g * T + n++] = (int32_t)t;
    int64_t count = n;
    for (int64_t t = 0; t < T; ++t)
      if (mask[t * ngroups + g] == 0) perm[g * T + n++] = (int32_t)t;
    counts[g] = (int32_t)count;
    padded[g] = (int32_t)(((count + tile - 1) / tile) * tile);
  }
  return ORACLE_OK;
}

static double silu(double a) { return a / (1.0 + exp(-a)); }

/*
 * Masked SwiGLU FFN for the tokens listed in rows[0..nrows) (rows == NULL
 * means tokens 0..nrows-1). Output row r of H ([nrows, d_ff]) and of Y
 * ([nrows, d]) belongs to token rows[r]. H is required: the function
 * allocates nothing and forms Y from the H row it has just written.
 */
int oracle_ffn(const float* X, const float* Wg, const float* Wu, const float* Wd,
               const uint8_t* mask, int64_t T, int64_t d, int64_t d_ff, int64_t G,
               const int64_t* rows, int64_t nrows, double* H, double* Y) {
  if (!X || !Wg || !Wu || !Wd || !mask || !H || !Y) return ORACLE_BAD_ARG;
  if (T < 0 || d <= 0 || d_ff <= 0 || G <= 0 || d_ff % G != 0 || nrows < 0)
    return ORACLE_BAD_ARG;
  const int64_t ng = d_ff / G;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t t = rows ? rows[r] : r;
    if (t < 0 || t >= T) return ORACLE_BAD_ARG;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t t = rows ? rows[r] : r;
    const float* x = X + t * d;
    double* h = H + r * d_ff;
    for (int64_t c = 0; c < d_ff; ++c) {
      const int64_t g = c / G;
      if (mask[t * ng + g] != 0) {
        double a = 0.0, b = 0.0;
        for (int64_t k = 0; k < d; ++k) {
          a += (double)x[k] * (double)Wg[c * d + k];
          b += (double)x[k] * (double)Wu[c * d + k];
        }
        h[c] = silu(a) * b;
      } else {
        h[c] = 0.0;
      }
    }
    double* y = Y + r * d;
    for (int64_t n = 0; n < d; ++n) {
      double s = 0.0;
      for (int64_t c = 0; c < d_ff; ++c) s += (double)Wd[n * d_ff + c] * h[c];
      y[n] = s;
    }
  }
  return ORACLE_OK;
}

/*
 * Group-masked GEMMs, the two kernel families of the method beyond the FFN
 * (WIDE paper App. B, "Implementation of GEMM-MN" and "Implementation of
 * GEMM-K"). C = A B^T with A [M, K], B [N, K] (WIDE paper Sec. 3.2).
 *
 *   N axis (GEMM-MN: W_q, W_up, W_gate; M-axis dynamic depth is the case of a
 *   single group, G == N): the columns of C are cut into groups of G and row m
 *   keeps or skips each group:
 *     C[m,n] = A[m,:].B[n,:]   if mask[m, n/G] != 0,   else 0 (select).
 *   mask is [M, N/G].
 *
 *   K axis (GEMM-K: W_o, W_down): the reduction axis is cut into groups of G
 *   and row m keeps or skips each group of its own input:
 *     C[m,n] = sum over k with mask[m, k/G] != 0 of A[m,k] * B[n,k].
 *   mask is [M, K/G].
 * Products and sums in double; rows m listed in rows[0..nrows) (NULL: 0..nrows-1).
 */
int oracle_gemm_mn(const float* A, const float* B, const uint8_t* mask, int64_t M, int64_t N,
                   int64_t K, int64_t G, const int64_t* rows, int64_t nrows, double* C) {
  if (!A || !B || !mask || !C || M < 0 || N <= 0 || K <= 0 || G <= 0 || N % G != 0 || nrows < 0)
    return ORACLE_BAD_ARG;
  const int64_t ng = N / G;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t m = rows ? rows[r] : r;
    if (m < 0 || m >= M) return ORACLE_BAD_ARG;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t m = rows ? rows[r] : r;
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      if (mask[m * ng + n / G] != 0)
        for (int64_t k = 0; k < K; ++k) acc += (double)A[m * K + k] * (double)B[n * K + k];
      C[r * N + n] = acc;
    }
  }
  return ORACLE_OK;
}

int oracle_gemm_k(const float* A, const float* B, const uint8_t* mask, int64_t M, int64_t N,
                  int64_t K, int64_t G, const int64_t* rows, int64_t nrows, double* C) {
  if (!A || !B || !mask || !C || M < 0 || N <= 0 || K <= 0 || G <= 0 || K % G != 0 || nrows < 0)
    return ORACLE_BAD_ARG;
  const int64_t ng = K / G;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t m = rows ? rows[r] : r;
    if (m < 0 || m >= M) return ORACLE_BAD_ARG;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t m = rows ? rows[r] : r;
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        if (mask[m * ng + k / G] != 0) acc += (double)A[m * K + k] * (double)B[n * K + k];
      C[r * N + n] = acc;
    }
  }
  return ORACLE_OK;
}

/*
 * Bottleneck router (ai.info summary, "How decisions are made": input
 * activations -> N_G two-way decisions per token through an inner dimension r
 * of 16 or 32; argmax at inference; class 0 = execute, class 1 = skip. The
 * paper's Sec. 3.1 "Routing Components" gives no formula.) Readings taken:
 * no biases, an activation between the two maps chosen by the caller, logits
 * laid out [T, N_G, 2] with the class fastest, and argmax taking the first
 * maximum, so a tie executes:
 *   z[t,j]       = act( sum_k X[t,k] * W1[j,k] )           j < r
 *   logit[t,g,c] = sum_j W2[2g + c, j] * z[t,j]             c in {0, 1}
 *   mask[t,g]    = 1 if logit[t,g,0] >= logit[t,g,1] else 0
 * act: 0 identity, 1 relu(a) = max(a, 0), 2 silu(a) = a / (1 + exp(-a)).
 * X [T, D], W1 [r, D], W2 [2*N_G, r]. Rows t listed in rows[0..nrows) (NULL:
 * 0..nrows-1); logits [nrows, N_G, 2] and mask [nrows, N_G] per listed row.
 */
static double router_act(double a, int act) {
  if (act == 1) return a > 0.0 ? a : 0.0;
  if (act == 2) return a / (1.0 + exp(-a));
  return a;
}

int oracle_router(const float* X, const float* W1, const float* W2, int64_t T, int64_t D,
                  int64_t r, int64_t ngroups, int act, const int64_t* rows, int64_t nrows,
                  double* logits, uint8_t* mask) {
  if (!X || !W1 || !W2 || !logits || !mask || T < 0 || D <= 0 || r <= 0 || r > 256 ||
      ngroups <= 0 || act < 0 || act > 2 || nrows < 0)
    return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t t = rows ? rows[i] : i;
    if (t < 0 || t >= T) return ORACLE_BAD_ARG;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t t = rows ? rows[i] : i;
    double zp[256];
    for (int64_t j = 0; j < r; ++j) {
      double s = 0.0;
      for (int64_t k = 0; k < D; ++k) s += (double)X[t * D + k] * (double)W1[j * D + k];
      zp[j] = router_act(s, act);
    }
    for (int64_t g = 0; g < ngroups; ++g) {
      double l[2];
      for (int c = 0; c < 2; ++c) {
        double s = 0.0;
        for (int64_t j = 0; j < r; ++j) s += (double)W2[(2 * g + c) * r + j] * zp[j];
        l[c] = s;
      }
      logits[(i * ngroups + g) * 2 + 0] = l[0];
      logits[(i * ngroups + g) * 2 + 1] = l[1];
      mask[i * ngroups + g] = l[0] >= l[1] ? 1 : 0;
    }
  }
  return ORACLE_OK;
}

/*
 * Head-group-pruned causal attention for prefill: the attention side of the
 * method (ai.info summary, "What gets pruned": the attention unit is a group
 * of H_q/H_k query heads aligned with GQA, and each token keeps or skips each
 * group; WIDE paper App. B "Implementation of Attention": a query tile of one
 * query head, the head fixing its KV head and routing group, the softmax
 * organised as in FlashAttention, the query side predicated and K/V dense).
 * Readings taken where the text is silent: causal self-attention over one
 * sequence (key j is valid for query t when j <= t), scale 1/sqrt(dh), group g
 * = KV head g = query heads [g*H_q/H_k, (g+1)*H_q/H_k), and a skipped
 * (token, group) pair has no output (+0.0 here):
 *   for t and query head h with mask[t, g] != 0, g = h / (H_q/H_k):
 *     s_j      = (Q[t,h,:] . K[j,g,:]) / sqrt(dh)          j = 0..t
 *     O[t,h,:] = sum_j exp(s_j) V[j,g,:] / sum_j exp(s_j)
 * (exp(s_j - max s) in both sums: the same ratio, without overflow).
 * Q [T, H_q*dh], K and V [T, H_k*dh], mask [T, H_k]; O [nrows, H_q*dh] for the
 * tokens listed in rows[0..nrows) (NULL: 0..nrows-1).
 */
int oracle_attention(const float* Q, const float* K, const float* V, const uint8_t* mask,
                     int64_t T, int64_t Hq, int64_t Hk, int64_t dh, const int64_t* rows,
                     int64_t nrows, double* O) {
  if (!Q || !K || !V || !mask || !O || T < 0 || Hq <= 0 || Hk <= 0 || Hq % Hk != 0 || dh <= 0 ||
      nrows < 0)
    return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t t = rows ? rows[i] : i;
    if (t < 0 || t >= T) return ORACLE_BAD_ARG;
  }
  const int64_t hpg = Hq / Hk;
  const double scale = 1.0 / sqrt((double)dh);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t t = rows ? rows[i] : i;
    double* s = (double*)malloc((size_t)(t + 1) * sizeof(double));
    if (!s) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / hpg;
      double* o = O + (i * Hq + h) * dh;
      if (!mask[t * Hk + g]) {
        for (int64_t e = 0; e < dh; ++e) o[e] = 0.0;
        continue;
      }
      const float* q = Q + (t * Hq + h) * dh;
      double mx = -INFINITY;
      for (int64_t j = 0; j <= t; ++j) {
        const float* k = K + (j * Hk + g) * dh;
        double d = 0.0;
        for (int64_t e = 0; e < dh; ++e) d += (double)q[e] * (double)k[e];
        s[j] = d * scale;
        if (s[j] > mx) mx = s[j];
      }
      double z = 0.0;
      for (int64_t e = 0; e < dh; ++e) o[e] = 0.0;
      for (int64_t j = 0; j <= t; ++j) {
        const double w = exp(s[j] - mx);
        z += w;
        const float* v = V + (j * Hk + g) * dh;
        for (int64_t e = 0; e < dh; ++e) o[e] += w * (double)v[e];
      }
      for (int64_t e = 0; e < dh; ++e) o[e] /= z;
    }
    free(s);
  }
  return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

/* Number of OpenMP threads the oracle runs with (1 when built without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
