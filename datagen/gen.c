/* Seeded synthetic inputs for the fused pattern's workloads.
 *
 * Input generation only: this file holds none of the pattern's arithmetic and
 * is shared by the tests, the smoke check and the benchmark (the oracle and the
 * GPU library each take the arrays it fills as plain inputs).
 *
 * Every random number is a pure function of (stream key, counter): the i-th
 * output of the SplitMix64 generator (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) started at the stream key,
 *     x_i = mix64(key + (i + 1) * 0x9e3779b97f4a7c15),
 * so results do not depend on the number of OpenMP threads.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (plain C11).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* independent sub-stream key for (key, index) */
uint64_t dg_substream(uint64_t key, uint64_t index) { return mix64(key ^ mix64(index + GOLDEN)); }

/* uniform double in [0, 1) with 53 random bits */
static inline double unif53(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

/* uniform float in [0, 1) with 24 random bits (exact in fp32) */
static inline float unif24(uint64_t x) { return (float)(x >> 40) * (1.0f / 16777216.0f); }

/* out[i] = lo + (hi - lo) * U_i, U_i uniform on [0, 1) with 24 bits; for (lo, hi) = (-1, 1)
 * every value is exactly representable. */
void dg_uniform(float* out, int64_t count, uint64_t key, float lo, float hi) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = lo + (hi - lo) * unif24(draw(key, (uint64_t)i));
}

/* out[i] = mean + std * N_i, N_i standard normal by the Box-Muller transform of two
 * 53-bit uniforms (counters 2i and 2i+1), evaluated in double and rounded to float. */
void dg_normal(float* out, int64_t count, uint64_t key, double mean, double std) {
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    double u1 = 1.0 - unif53(draw(key, 2 * (uint64_t)i));  /* (0, 1] */
    double u2 = unif53(draw(key, 2 * (uint64_t)i + 1));
    out[i] = (float)(mean + std * sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
  }
}

/* Bernoulli(p) sparsity over an m x n grid, one independent stream per row: the gaps
 * between nonzero columns of row i are geometric, G = floor(log(U) / log(1 - p)).
 * Pass 1 counts the nonzeros per row; pass 2 (same streams) writes the sorted columns. */
static int64_t bern_row(uint64_t key, int64_t i, int64_t n, double lq, int32_t* cols) {
  uint64_t rk = dg_substream(key, (uint64_t)i);
  int64_t c = -1, cnt = 0;
  for (uint64_t d = 0;; ++d) {
    double u = 1.0 - unif53(draw(rk, d)); /* (0, 1] */
    double g = floor(log(u) / lq);
    if (g >= (double)n) break;
    c += 1 + (int64_t)g;
    if (c >= n) break;
    if (cols) cols[cnt] = (int32_t)c;
    ++cnt;
  }
  return cnt;
}

int dg_bernoulli_count(int64_t m, int64_t n, double p, uint64_t key, int32_t* row_len) {
  if (!(p > 0.0 && p < 1.0) || m < 0 || n <= 0) return 1;
  const double lq = log1p(-p);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) row_len[i] = (int32_t)bern_row(key, i, n, lq, NULL);
  return 0;
}

int dg_bernoulli_fill(int64_t m, int64_t n, double p, uint64_t key, const int64_t* row_ptr,
                      int32_t* col_idx) {
  if (!(p > 0.0 && p < 1.0) || m < 0 || n <= 0) return 1;
  const double lq = log1p(-p);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) bern_row(key, i, n, lq, col_idx + row_ptr[i]);
  return 0;
}

/* cumulative distribution of the Zipf law truncated to 1..K: P(k) proportional to k^-s */
static double* zipf_cdf(double s, int64_t K) {
  double* cdf = (double*)malloc(sizeof(double) * (size_t)K);
  if (!cdf) return NULL;
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    acc += pow((double)(k + 1), -s);
    cdf[k] = acc;
  }
  for (int64_t k = 0; k < K; ++k) cdf[k] /= acc;
  cdf[K - 1] = 1.0;
  return cdf;
}

/* smallest k with cdf[k] > u, i.e. the sampled value is k + 1 */
static inline int64_t inv_cdf(const double* cdf, int64_t K, double u) {
  int64_t lo = 0, hi = K - 1;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (cdf[mid] > u) hi = mid; else lo = mid + 1;
  }
  return lo;
}

/* row_len[i] ~ Zipf(s) truncated to 1..K (inverse-CDF sampling) */
int dg_zipf_lengths(int64_t m, double s, int64_t K, uint64_t key, int32_t* row_len) {
  if (K < 1 || K > 2147483647LL || m < 0) return 1;
  double* cdf = zipf_cdf(s, K);
  if (!cdf) return 2;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) row_len[i] = (int32_t)(inv_cdf(cdf, K, unif53(draw(key, (uint64_t)i))) + 1);
  free(cdf);
  return 0;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Columns of row i: the first L_i distinct values of an i.i.d. stream of ranks
 * r ~ Zipf(s) truncated to 1..n (column = perm[r - 1], or r - 1 when perm is NULL),
 * then sorted ascending. Returns 3 if a row needs more than max(64 L_i, 10^6) draws. */
int dg_zipf_columns(int64_t m, int64_t n, double s, uint64_t key, const int64_t* row_ptr,
                    const int32_t* perm, int32_t* col_idx) {
  if (n < 1 || n > 2147483647LL || m < 0) return 1;
  for (int64_t i = 0; i < m; ++i)
    if (row_ptr[i + 1] - row_ptr[i] > n) return 1;
  double* cdf = zipf_cdf(s, n);
  if (!cdf) return 2;
  int failed = 0;
#pragma omp parallel
  {
    int64_t* stamp = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!stamp) {
#pragma omp atomic write
      failed = 2;
    } else {
      for (int64_t j = 0; j < n; ++j) stamp[j] = -1;
#pragma omp for schedule(dynamic, 256)
      for (int64_t i = 0; i < m; ++i) {
        const int64_t L = row_ptr[i + 1] - row_ptr[i];
        int32_t* out = col_idx + row_ptr[i];
        const uint64_t rk = dg_substream(key, (uint64_t)i);
        const uint64_t cap = (uint64_t)(64 * L > 1000000 ? 64 * L : 1000000);
        int64_t got = 0;
        for (uint64_t d = 0; got < L; ++d) {
          if (d >= cap) {
#pragma omp atomic write
            failed = 3;
            break;
          }
          int64_t r = inv_cdf(cdf, n, unif53(draw(rk, d)));
          int32_t c = perm ? perm[r] : (int32_t)r;
          if (stamp[c] != i) {
            stamp[c] = i;
            out[got++] = c;
          }
        }
        qsort(out, (size_t)got, sizeof(int32_t), cmp_i32);
      }
      free(stamp);
    }
  }
  free(cdf);
  return failed;
}

/* Logistic-regression curvature weights for a CSR design matrix X and coefficients w:
 * v_i = p_i (1 - p_i) with p_i = 1 / (1 + exp(-(X w)_i)), evaluated in double. */
int dg_logistic_weights(int64_t m, const int64_t* row_ptr, const int32_t* col_idx,
                        const float* values, const float* w, float* v) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    double eta = 0.0;
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) eta += (double)values[p] * (double)w[col_idx[p]];
    double pr = 1.0 / (1.0 + exp(-eta));
    v[i] = (float)(pr * (1.0 - pr));
  }
  return 0;
}

/* Labels of the same planted logistic model: c_i = 1 when U_i < sigmoid(x_i . w), else 0,
 * with U_i a 53-bit uniform from stream `key` (counter i). */
int dg_logistic_labels(int64_t m, const int64_t* row_ptr, const int32_t* col_idx, const float* values,
                       const float* w, uint64_t key, float* labels) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    double eta = 0.0;
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) eta += (double)values[p] * (double)w[col_idx[p]];
    double pr = 1.0 / (1.0 + exp(-eta));
    labels[i] = unif53(draw(key, (uint64_t)i)) < pr ? 1.0f : 0.0f;
  }
  return 0;
}
