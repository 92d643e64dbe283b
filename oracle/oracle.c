/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the activation-sparse FFN decode path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or loads this
 * file; only the test-suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (sources are the pages' prose; no page prints code for any of it):
 *  - predict:   a low-rank predictor scores every FFN neuron; only neurons predicted
 *               active are computed ("Predictores de espacialidad adaptativa" on the
 *               unite.ai PowerInfer overview; section 自適應稀疏預測器 of the novita.ai
 *               activation-sparsity article, which describes the predictor as an MLP with
 *               input, hidden and output layers whose hidden size is tuned).
 *               Reading taken: linear two-stage form s = P2 (P1 x) + c, no hidden
 *               nonlinearity.
 *  - threshold: neuron i is active iff s_i > tau (strict; NaN is inactive).
 *  - compact:   ascending list of active neurons plus, for a batch, the per-token
 *               membership bits; the union decides which rows are read.
 *  - forward:   only the rows/columns of the active neurons are touched ("Operador
 *               consciente de neuronas" on the unite.ai overview; section 單層計算優化 of
 *               the novita.ai article: neurons 3,4,5 predicted active are computed and the
 *               rest skipped). ReLU sits between up and down (section 激活稀疏性的可行性:
 *               rows whose ReLU output is zero contribute zero to the down projection);
 *               the gated form puts the ReLU on the gate (section 第一階段).
 *  - dense:     the same FFN over every neuron with no mask (the definition the sparse
 *               output must reduce to when the mask covers every true activation).
 *  - dense_f16act: dense with x rounded to binary16 before the up products and h before
 *               the down product (the library's optional fp16-activation prefill; the
 *               pages run prefill dense and fix no precision for it: PowerInfer-2
 *               article, section 4.1.1 NPU-Centric Prefill).
 *  - profile, permutation, pack: offline activation counts, hot neurons first, and a
 *               neuron table back to the original positions ("Fase fuera de línea" and
 *               "Colocación y gestión de neuronas" on the unite.ai overview).
 *
 * Arithmetic: every stored value (fp16, fp32) is widened exactly to double; sums run in
 * plain ascending order in double; nothing is rounded in between. Build with
 * -ffp-contract=off and without -ffast-math so each line is evaluated as written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_F64 = 2 };
enum { ORC_OK = 0, ORC_ERR = -1 };

/* IEEE 754 binary16 -> double, from the format definition: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits; exponent 0 is subnormal (fraction * 2^-24), 31 is inf/NaN. */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 31;
  int frac = h & 1023;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25);
  }
  return sign ? -v : v;
}

static double elem(const void* base, int dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_F16) return oracle_half_to_double(((const uint16_t*)base)[i]);
  return ((const double*)base)[i];
}

static int dtype_ok(int dtype) { return dtype == ORC_F32 || dtype == ORC_F16 || dtype == ORC_F64; }

/* Predictor, both stages, per token b:
 *   q[b][j] = sum_t P1[j][t] * x[b][t]          (P1 is r x d, row-major)
 *   s[b][i] = sum_j P2[i][j] * q[b][j] + c[i]     (P2 is n x r, row-major; c may be NULL = 0)
 * Q (B x r) may be NULL. */
int oracle_predict(int32_t d, int32_t n, int32_t r, int32_t B, const float* X,
                   const void* P1, const void* P2, int32_t p_dtype, const float* c,
                   double* S, double* Q) {
  if (d <= 0 || n <= 0 || r <= 0 || B <= 0 || !X || !P1 || !P2 || !S || !dtype_ok(p_dtype))
    return ORC_ERR;
  double* q = (double*)malloc(sizeof(double) * (size_t)r);
  if (!q) return ORC_ERR;
  for (int32_t b = 0; b < B; ++b) {
    const float* x = X + (size_t)b * d;
#pragma omp parallel for schedule(static)
    for (int32_t j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int32_t t = 0; t < d; ++t) acc += elem(P1, p_dtype, (size_t)j * d + t) * (double)x[t];
      q[j] = acc;
      if (Q) Q[(size_t)b * r + j] = acc;
    }
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int32_t j = 0; j < r; ++j) acc += elem(P2, p_dtype, (size_t)i * r + j) * q[j];
      S[(size_t)b * n + i] = acc + (c ? (double)c[i] : 0.0);
    }
  }
  free(q);
  return ORC_OK;
}

/* Threshold: M[b][i] = 1 iff S[b][i] > tau. A NaN score compares false, so it is inactive. */
int oracle_threshold(int32_t B, int32_t n, const double* S, double tau, uint8_t* M) {
  if (B <= 0 || n <= 0 || !S || !M) return ORC_ERR;
  for (size_t k = 0; k < (size_t)B * n; ++k) M[k] = (S[k] > tau) ? 1 : 0;
  return ORC_OK;
}

/* Compaction: idx = ascending list of neurons active for at least one token; count = its
 * length; tokmask[k] bit b = 1 iff token b has neuron idx[k] active. tokmask may be NULL.
 * B is at most 64 (one bit per token in a 64-bit word). */
int oracle_compact(int32_t B, int32_t n, const uint8_t* M, int32_t* idx, int32_t* count,
                   uint64_t* tokmask) {
  if (B <= 0 || B > 64 || n <= 0 || !M || !idx || !count) return ORC_ERR;
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    uint64_t bits = 0;
    for (int32_t b = 0; b < B; ++b)
      if (M[(size_t)b * n + i]) bits |= (uint64_t)1 << b;
    if (bits) {
      idx[k] = i;
      if (tokmask) tokmask[k] = bits;
      ++k;
    }
  }
  *count = k;
  return ORC_OK;
}

/* Forward over a given active list, per token b, k ascending:
 *   i = idx[k]; skip if tokmask given and bit b of tokmask[k] is 0
 *   a = sum_t Wa[i][t] x[b][t] + b_a[i]
 *   plain: h = relu(a);  gated: h = relu(a) * (sum_t Wu[i][t] x[b][t])
 *   y[b][j] += h * Wo[i][j]   for every j
 * then y[b][j] += b_o[j]. Wa, Wu and Wo (= W_down transposed) are n x d row-major.
 * relu(a) = a if a > 0 else +0.0. b_a and b_o may be NULL (= 0).
 * Written as two loops per token: every listed neuron's h first (each depends on its own
 * row only), then the output elements, each starting at 0 and adding its h * Wo terms in
 * ascending k, then b_o. Each output element sees exactly the operations of the one-loop
 * form above, in the same order, so the result is the same bit for bit; an OpenMP build
 * may run either loop's iterations on several threads without changing any sum. */
int oracle_forward(int32_t d, int32_t n, int32_t B, int32_t gated, const float* X,
                   const void* Wa, const void* Wu, const void* Wo, int32_t w_dtype,
                   const float* b_a, const float* b_o, const int32_t* idx, int32_t count,
                   const uint64_t* tokmask, double* Y) {
  if (d <= 0 || n <= 0 || B <= 0 || B > 64 || count < 0 || count > n || !X || !Wa || !Wo ||
      !Y || !dtype_ok(w_dtype) || (gated && !Wu) || (count > 0 && !idx))
    return ORC_ERR;
  for (int32_t k = 0; k < count; ++k)
    if (idx[k] < 0 || idx[k] >= n) return ORC_ERR;
  double* hk = (double*)malloc(sizeof(double) * (size_t)(count > 0 ? count : 1));
  uint8_t* use = (uint8_t*)malloc((size_t)(count > 0 ? count : 1));
  if (!hk || !use) { free(hk); free(use); return ORC_ERR; }
  for (int32_t b = 0; b < B; ++b) {
    const float* x = X + (size_t)b * d;
    double* y = Y + (size_t)b * d;
#pragma omp parallel for schedule(dynamic, 16)
    for (int32_t k = 0; k < count; ++k) {
      use[k] = 0;
      if (tokmask && !((tokmask[k] >> b) & 1)) continue;
      int32_t i = idx[k];
      double a = 0.0;
      for (int32_t t = 0; t < d; ++t) a += elem(Wa, w_dtype, (size_t)i * d + t) * (double)x[t];
      a += b_a ? (double)b_a[i] : 0.0;
      double h = (a > 0.0) ? a : 0.0;
      if (gated) {
        double u = 0.0;
        for (int32_t t = 0; t < d; ++t) u += elem(Wu, w_dtype, (size_t)i * d + t) * (double)x[t];
        h = h * u;
      }
      hk[k] = h;
      use[k] = 1;
    }
#pragma omp parallel for schedule(static)
    for (int32_t jb = 0; jb < d; jb += 64) {
      const int32_t je = jb + 64 < d ? jb + 64 : d;
      for (int32_t j = jb; j < je; ++j) y[j] = 0.0;
      for (int32_t k = 0; k < count; ++k) {
        if (!use[k]) continue;
        const int32_t i = idx[k];
        const double h = hk[k];
        for (int32_t j = jb; j < je; ++j) y[j] += h * elem(Wo, w_dtype, (size_t)i * d + j);
      }
      if (b_o)
        for (int32_t j = jb; j < je; ++j) y[j] += (double)b_o[j];
    }
  }
  free(hk);
  free(use);
  return ORC_OK;
}

/* Threads the oracle's loops run on: 1 in the plain build, OpenMP's count in an OpenMP
 * build (timing reports only). */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Dense FFN: the forward above with every neuron 0..n-1, ascending, and no mask. */
int oracle_dense(int32_t d, int32_t n, int32_t B, int32_t gated, const float* X,
                 const void* Wa, const void* Wu, const void* Wo, int32_t w_dtype,
                 const float* b_a, const float* b_o, double* Y) {
  if (d <= 0 || n <= 0 || B <= 0 || !X || !Wa || !Wo || !Y || !dtype_ok(w_dtype) ||
      (gated && !Wu))
    return ORC_ERR;
  for (int32_t b = 0; b < B; ++b) {
    const float* x = X + (size_t)b * d;
    double* y = Y + (size_t)b * d;
    for (int32_t j = 0; j < d; ++j) y[j] = 0.0;
    for (int32_t i = 0; i < n; ++i) {
      double a = 0.0;
      for (int32_t t = 0; t < d; ++t) a += elem(Wa, w_dtype, (size_t)i * d + t) * (double)x[t];
      a += b_a ? (double)b_a[i] : 0.0;
      double h = (a > 0.0) ? a : 0.0;
      if (gated) {
        double u = 0.0;
        for (int32_t t = 0; t < d; ++t) u += elem(Wu, w_dtype, (size_t)i * d + t) * (double)x[t];
        h = h * u;
      }
      for (int32_t j = 0; j < d; ++j) y[j] += h * elem(Wo, w_dtype, (size_t)i * d + j);
    }
    if (b_o)
      for (int32_t j = 0; j < d; ++j) y[j] += (double)b_o[j];
  }
  return ORC_OK;
}

/* A double rounded to the nearest IEEE 754 binary16 value, ties to even. The format has
 * normal numbers from 2^-14 up, spaced 2^(e-10) in the binade [2^e, 2^(e+1)); below 2^-14
 * the subnormals keep the spacing 2^-24; the largest finite value is 65504 = (2 - 2^-10)
 * 2^15, and magnitudes from the midpoint 65520 on round to infinity. Zeros, infinities and
 * NaN pass through. */
double oracle_round_half(double v) {
  if (v != v || v == 0.0) return v;
  const double a = fabs(v);
  if (a >= 65520.0) return copysign(INFINITY, v);
  int ex;
  (void)frexp(a, &ex); /* a = m 2^ex, m in [0.5, 1): a lies in [2^(ex-1), 2^ex) */
  int e = ex - 1;
  if (e < -14) e = -14; /* subnormals: the smallest binade's spacing */
  const double q = ldexp(1.0, e - 10);
  /* a / q is exact (q is a power of two); nearbyint rounds to nearest, ties to even, in
   * the default rounding mode */
  return copysign(nearbyint(a / q) * q, v);
}

int oracle_round_half_array(int64_t count, const double* in, double* out) {
  if (count < 0 || (count > 0 && (!in || !out))) return ORC_ERR;
  for (int64_t k = 0; k < count; ++k) out[k] = oracle_round_half(in[k]);
  return ORC_OK;
}

/* dense with fp16 activations: x rounded to binary16 before the up (and gate) products, h
 * rounded before the down product; every other step as in oracle_dense, in double. */
int oracle_dense_f16act(int32_t d, int32_t n, int32_t B, int32_t gated, const float* X,
                        const void* Wa, const void* Wu, const void* Wo, int32_t w_dtype,
                        const float* b_a, const float* b_o, double* Y) {
  if (d <= 0 || n <= 0 || B <= 0 || !X || !Wa || !Wo || !Y || !dtype_ok(w_dtype) ||
      (gated && !Wu))
    return ORC_ERR;
  double* xr = (double*)malloc((size_t)d * sizeof(double));
  if (!xr) return ORC_ERR;
  for (int32_t b = 0; b < B; ++b) {
    const float* x = X + (size_t)b * d;
    double* y = Y + (size_t)b * d;
    for (int32_t t = 0; t < d; ++t) xr[t] = oracle_round_half((double)x[t]);
    for (int32_t j = 0; j < d; ++j) y[j] = 0.0;
    for (int32_t i = 0; i < n; ++i) {
      double a = 0.0;
      for (int32_t t = 0; t < d; ++t) a += elem(Wa, w_dtype, (size_t)i * d + t) * xr[t];
      a += b_a ? (double)b_a[i] : 0.0;
      double h = (a > 0.0) ? a : 0.0;
      if (gated) {
        double u = 0.0;
        for (int32_t t = 0; t < d; ++t) u += elem(Wu, w_dtype, (size_t)i * d + t) * xr[t];
        h = h * u;
      }
      h = oracle_round_half(h);
      for (int32_t j = 0; j < d; ++j) y[j] += h * elem(Wo, w_dtype, (size_t)i * d + j);
    }
    if (b_o)
      for (int32_t j = 0; j < d; ++j) y[j] += (double)b_o[j];
  }
  free(xr);
  return ORC_OK;
}

/* Pre-activations A[b][i] = sum_t Wa[i][t] x[b][t] + b_a[i] (the true ReLU input; for the
 * gated form, the gate). Used for the true-sign mask T(x) = {i : A[i] > 0}. */
int oracle_preact(int32_t d, int32_t n, int32_t B, const float* X, const void* Wa,
                  int32_t w_dtype, const float* b_a, double* A) {
  if (d <= 0 || n <= 0 || B <= 0 || !X || !Wa || !A || !dtype_ok(w_dtype)) return ORC_ERR;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t i = 0; i < n; ++i) {
      double a = 0.0;
      for (int32_t t = 0; t < d; ++t)
        a += elem(Wa, w_dtype, (size_t)i * d + t) * (double)X[(size_t)b * d + t];
      A[(size_t)b * n + i] = a + (b_a ? (double)b_a[i] : 0.0);
    }
  return ORC_OK;
}

/* Offline profile ("Fase fuera de línea", unite.ai overview: the profiler records which
 * neurons activate over a set of requests): counts[i] = number of the N profiling tokens
 * whose pre-activation A[i] is > 0. */
int oracle_profile_counts(int32_t d, int32_t n, int32_t N, const float* X, const void* Wa,
                          int32_t w_dtype, const float* b_a, int64_t* counts) {
  if (d <= 0 || n <= 0 || N <= 0 || !X || !Wa || !counts || !dtype_ok(w_dtype)) return ORC_ERR;
  for (int32_t i = 0; i < n; ++i) {
    int64_t cnt = 0;
    for (int32_t b = 0; b < N; ++b) {
      double a = 0.0;
      for (int32_t t = 0; t < d; ++t)
        a += elem(Wa, w_dtype, (size_t)i * d + t) * (double)X[(size_t)b * d + t];
      a += b_a ? (double)b_a[i] : 0.0;
      if (a > 0.0) ++cnt;
    }
    counts[i] = cnt;
  }
  return ORC_OK;
}

/* Hot-first permutation. The n_hot neurons with the largest counts (ties: smaller original
 * index first) come first, in that order; every other neuron follows in ascending original
 * index. perm[new] = old: the neuron table back to original positions ("Colocación y
 * gestión de neuronas", unite.ai overview). */
static const int64_t* g_counts; /* qsort comparator context (single-threaded use only) */
static int cmp_hot(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  if (g_counts[a] != g_counts[b]) return g_counts[a] > g_counts[b] ? -1 : 1;
  return a < b ? -1 : (a > b ? 1 : 0);
}
int oracle_permutation(const int64_t* counts, int32_t n, int32_t n_hot, int32_t* perm) {
  if (!counts || !perm || n <= 0 || n_hot < 0 || n_hot > n) return ORC_ERR;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  uint8_t* is_hot = (uint8_t*)calloc((size_t)n, 1);
  if (!order || !is_hot) { free(order); free(is_hot); return ORC_ERR; }
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  g_counts = counts;
  qsort(order, (size_t)n, sizeof(int32_t), cmp_hot);
  g_counts = NULL;
  int32_t k = 0;
  for (; k < n_hot; ++k) { perm[k] = order[k]; is_hot[order[k]] = 1; }
  for (int32_t i = 0; i < n; ++i)
    if (!is_hot[i]) perm[k++] = i;
  free(order);
  free(is_hot);
  return ORC_OK;
}

/* Pack: destination row i is source row perm[i] (a byte copy of row_bytes per row). */
int oracle_pack_rows(const void* src, const int32_t* perm, void* dst, int32_t rows,
                     int64_t row_bytes) {
  if (!src || !perm || !dst || rows <= 0 || row_bytes <= 0) return ORC_ERR;
  for (int32_t i = 0; i < rows; ++i) {
    if (perm[i] < 0 || perm[i] >= rows) return ORC_ERR;
    memcpy((char*)dst + (size_t)i * row_bytes, (const char*)src + (size_t)perm[i] * row_bytes,
           (size_t)row_bytes);
  }
  return ORC_OK;
}
