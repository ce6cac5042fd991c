/*
 * Plain C fp64 oracle of ExTernD's greedy sequential decomposition.
 *
 * Test infrastructure: only tests, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no code with the GPU library
 * and includes none of its headers.
 *
 * Source: "ExTernD: Expanded-Rank Ternary Decomposition Ternary LLM PTQ with
 * Accuracy Approaching Any Quantization Level":
 *   §2.1  A ~ B diag(D) C with ternary B (m x k), C (k x n); energy
 *         E = 1 - ||A - B diag(D) C||^2 / ||A||^2.
 *   §2.2  T_tau: sign(x_i) where |x_i| > tau * mean|x|, else 0; if nothing
 *         is kept, the largest entry alone.
 *   §2.3  per component: alternate v = T_tau(R^T u), u = T_tau(R v) for a
 *         fixed number of iterations, take d = u^T R v / (||u||^2 ||v||^2),
 *         subtract d u v^T from R.
 *
 * Readings the pages leave open (the same ones the numpy oracle takes):
 *   - the mean is over the vector's own length N, in an exact fixed point:
 *     M = max|x|, e the frexp exponent of M, L = ceil(log2 N),
 *     s = 52 - e - L, q_j = floor(|x_j| 2^s) (integers below 2^(52-L)),
 *     S = (sum q_j) 2^-s, threshold = (tau S) / N in fp64, tau being the
 *     fp32 value widened; strict comparison; sign(0) = 0;
 *   - fallback: the smallest index attaining M keeps its sign; x = 0 gives
 *     +1 at index 0;
 *   - u0 of component i: +-1 per row r from the SplitMix64 output function
 *     (Steele, Lea & Flood 2014) used as a hash,
 *     h = mix(mix(mix(seed) + i) + r), -1 when the top bit of h is set,
 *     mix(x) = fin(x + 0x9E3779B97F4A7C15), fin as published;
 *   - one iteration is the v update then the u update; no early stop;
 *   - k = mu * min(m, n) rounded half away from zero (the caller passes k);
 *   - trace[i] = ||R||^2 after component i, recomputed from R.
 *
 * Everything is plain loops in fp64 in index order; nothing is blocked,
 * fused or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static uint64_t splitmix64_mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* u0[r] for component i (values -1 or +1). */
void orc_start_vector(uint64_t seed, int64_t i, int64_t m, double* u) {
  const uint64_t base = splitmix64_mix(splitmix64_mix(seed) + (uint64_t)i);
  for (int64_t r = 0; r < m; ++r) u[r] = (splitmix64_mix(base + (uint64_t)r) >> 63) ? -1.0 : 1.0;
}

uint64_t orc_splitmix64_mix(uint64_t x) { return splitmix64_mix(x); }

static int ceil_log2(int64_t n) {
  int l = 0;
  while (((int64_t)1 << l) < n) ++l;
  return l;
}

/* The fixed-point threshold of T_tau; *maxabs receives M.  Returns 0.0 when
 * M == 0. */
double orc_threshold(const double* x, int64_t n, float tau, double* maxabs) {
  double big = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double a = fabs(x[j]);
    if (a > big) big = a;
  }
  if (maxabs) *maxabs = big;
  if (big == 0.0) return 0.0;
  int e;
  (void)frexp(big, &e);
  const int s = 52 - e - ceil_log2(n);
  uint64_t total = 0;
  for (int64_t j = 0; j < n; ++j) total += (uint64_t)floor(ldexp(fabs(x[j]), s));
  const double S = ldexp((double)total, -s);   /* total < 2^52: exact */
  return ((double)tau * S) / (double)n;
}

/* T_tau(x) into t (values -1, 0, +1).  Returns the number of nonzeros. */
int64_t orc_ternarize(const double* x, int64_t n, float tau, int8_t* t) {
  double big;
  const double thr = orc_threshold(x, n, tau, &big);
  memset(t, 0, (size_t)n);
  if (big == 0.0) {
    t[0] = 1;
    return 1;
  }
  int64_t cnt = 0;
  for (int64_t j = 0; j < n; ++j) {
    if (fabs(x[j]) > thr) {
      t[j] = x[j] > 0.0 ? 1 : -1;
      ++cnt;
    }
  }
  if (cnt > 0) return cnt;
  for (int64_t j = 0; j < n; ++j) {
    if (fabs(x[j]) == big) {
      t[j] = x[j] > 0.0 ? 1 : -1;
      return 1;
    }
  }
  return 0;   /* not reached for finite x */
}

/*
 * Greedy sequential decomposition of A (m x n, fp32 row-major) with k
 * components.  Outputs: B (k x m, component-major, int8), C (k x n, int8),
 * D (k, fp64), trace (k, fp64, may be NULL), *energy.  Returns 0, or -1 when
 * memory runs out.
 */
int orc_decompose_seq(const float* A, int64_t m, int64_t n, int64_t k, float tau, int iters, uint64_t seed,
                      int8_t* B, int8_t* C, double* D, double* trace, double* energy) {
  double* R = (double*)malloc(sizeof(double) * (size_t)(m * n));
  double* u = (double*)malloc(sizeof(double) * (size_t)m);
  double* x = (double*)malloc(sizeof(double) * (size_t)m);
  double* v = (double*)malloc(sizeof(double) * (size_t)n);
  double* y = (double*)malloc(sizeof(double) * (size_t)n);
  int8_t* tu = (int8_t*)malloc((size_t)m);
  int8_t* tv = (int8_t*)malloc((size_t)n);
  if (!R || !u || !x || !v || !y || !tu || !tv) {
    free(R); free(u); free(x); free(v); free(y); free(tu); free(tv);
    return -1;
  }
  double norm_a2 = 0.0;
  for (int64_t p = 0; p < m * n; ++p) {
    R[p] = (double)A[p];
    norm_a2 += R[p] * R[p];
  }
  double r2 = norm_a2;
  for (int64_t i = 0; i < k; ++i) {
    orc_start_vector(seed, i, m, u);
    int64_t nu = 0, nv = 0;
    for (int it = 0; it < iters; ++it) {
      /* y = R^T u */
      for (int64_t c = 0; c < n; ++c) y[c] = 0.0;
      for (int64_t r = 0; r < m; ++r)
        if (u[r] != 0.0)
          for (int64_t c = 0; c < n; ++c) y[c] += u[r] * R[r * n + c];
      nv = orc_ternarize(y, n, tau, tv);
      for (int64_t c = 0; c < n; ++c) v[c] = (double)tv[c];
      /* x = R v */
      for (int64_t r = 0; r < m; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < n; ++c) acc += R[r * n + c] * v[c];
        x[r] = acc;
      }
      nu = orc_ternarize(x, m, tau, tu);
      for (int64_t r = 0; r < m; ++r) u[r] = (double)tu[r];
    }
    double cuv = 0.0;   /* u^T R v = u . x with x from the last iteration */
    for (int64_t r = 0; r < m; ++r) cuv += u[r] * x[r];
    const double d = cuv / ((double)nu * (double)nv);
    r2 = 0.0;
    for (int64_t r = 0; r < m; ++r)
      for (int64_t c = 0; c < n; ++c) {
        R[r * n + c] -= d * u[r] * v[c];
        r2 += R[r * n + c] * R[r * n + c];
      }
    memcpy(B + i * m, tu, (size_t)m);
    memcpy(C + i * n, tv, (size_t)n);
    D[i] = d;
    if (trace) trace[i] = r2;
  }
  *energy = norm_a2 > 0.0 ? 1.0 - r2 / norm_a2 : 1.0;
  free(R); free(u); free(x); free(v); free(y); free(tu); free(tv);
  return 0;
}
