/*
 * Plain C fp64 oracle of ExTernD's greedy sequential decomposition and its
 * batched block ALS.
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
 *   §2.4  per block of b components: decorrelated targets through the
 *         ridge-regularised inverse Grams, T_tau by columns, the joint
 *         scale solve, the rank-b deflation (orc_decompose_block).
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
 *   - trace[i] = ||R||^2 after component i, recomputed from R;
 *   - block mode: the ridge eps = 1e-6 trace(G) / b of each Gram G; the
 *     joint solve by Cholesky, retried once with that kind of ridge when a
 *     pivot is not positive; the starting vectors of a block are those of
 *     its components' global indices.
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

/*
 * Batched block ALS (§2.4), plain: for each block of b components (the last
 * block takes what is left), U0 is the start vectors of the block's
 * components; each of `iters` iterations takes
 *   V = T_tau by columns of [(U^T U + eps I)^-1 U^T R]^T,
 *   U = T_tau by columns of R V (V^T V + eps I)^-1,
 * with eps = 1e-6 trace(G) / b for each Gram G; then the b scales solve
 * [(U^T U) o (V^T V)] d = diag(U^T R V) by Cholesky (retried once with the
 * same kind of ridge when a pivot is not positive), and R <- R - U diag(d)
 * V^T.  trace[blk] = ||R||^2 after each block.  Outputs as for
 * orc_decompose_seq; *retries counts the ridge retries.  Returns 0, or -1
 * when memory runs out.
 */

/* Cholesky factor of the symmetric matrix a (n x n, row-major) in place
 * (lower triangle); 0 when a pivot is not positive. */
static int cholesky(double* a, int n) {
  for (int j = 0; j < n; ++j) {
    double s = a[j * n + j];
    for (int k = 0; k < j; ++k) s -= a[j * n + k] * a[j * n + k];
    if (!(s > 0.0)) return 0;
    const double ljj = sqrt(s);
    a[j * n + j] = ljj;
    for (int i = j + 1; i < n; ++i) {
      double t = a[i * n + j];
      for (int k = 0; k < j; ++k) t -= a[i * n + k] * a[j * n + k];
      a[i * n + j] = t / ljj;
    }
  }
  return 1;
}

/* x <- (L L^T)^-1 x for the vector x of length n held with stride `st`. */
static void cholesky_solve(const double* L, int n, double* x, int64_t st) {
  for (int i = 0; i < n; ++i) {
    double t = x[i * st];
    for (int k = 0; k < i; ++k) t -= L[i * n + k] * x[k * st];
    x[i * st] = t / L[i * n + i];
  }
  for (int i = n - 1; i >= 0; --i) {
    double t = x[i * st];
    for (int k = i + 1; k < n; ++k) t -= L[k * n + i] * x[k * st];
    x[i * st] = t / L[i * n + i];
  }
}

/* G + eps I with eps = 1e-6 trace(G) / n, then its Cholesky factor. */
static int ridge_factor(double* g, int n) {
  double tr = 0.0;
  for (int i = 0; i < n; ++i) tr += g[i * n + i];
  const double eps = 1e-6 * tr / (double)n;
  for (int i = 0; i < n; ++i) g[i * n + i] += eps;
  return cholesky(g, n);
}

int orc_decompose_block(const float* A, int64_t m, int64_t n, int64_t k, int b, float tau, int iters,
                        uint64_t seed, int8_t* B, int8_t* C, double* D, double* trace, double* energy,
                        int64_t* retries) {
  if (b < 1) return -1;
  double* R = (double*)malloc(sizeof(double) * (size_t)(m * n));
  double* U = (double*)malloc(sizeof(double) * (size_t)(m * b));    /* m x b */
  double* V = (double*)malloc(sizeof(double) * (size_t)(n * b));    /* n x b */
  double* Tv = (double*)malloc(sizeof(double) * (size_t)(b * n));   /* b x n: V target, row per component */
  double* Tu = (double*)malloc(sizeof(double) * (size_t)(b * m));   /* b x m: U target */
  double* Q = (double*)malloc(sizeof(double) * (size_t)(m * b));    /* R V */
  double* G = (double*)malloc(sizeof(double) * (size_t)(b * b));
  double* G2 = (double*)malloc(sizeof(double) * (size_t)(b * b));
  double* rhs = (double*)malloc(sizeof(double) * (size_t)b);
  int8_t* t8 = (int8_t*)malloc((size_t)(m > n ? m : n));
  double* col = (double*)malloc(sizeof(double) * (size_t)(m > n ? m : n));
  if (!R || !U || !V || !Tv || !Tu || !Q || !G || !G2 || !rhs || !t8 || !col) {
    free(R); free(U); free(V); free(Tv); free(Tu); free(Q); free(G); free(G2); free(rhs); free(t8); free(col);
    return -1;
  }
  double norm_a2 = 0.0;
  for (int64_t p = 0; p < m * n; ++p) {
    R[p] = (double)A[p];
    norm_a2 += R[p] * R[p];
  }
  double r2 = norm_a2;
  int64_t nretry = 0;
  const int64_t nblocks = (k + b - 1) / b;
  for (int64_t blk = 0; blk < nblocks; ++blk) {
    const int64_t c0 = blk * b;
    const int bb = (int)(k - c0 < b ? k - c0 : b);
    for (int j = 0; j < bb; ++j) {
      orc_start_vector(seed, c0 + j, m, col);
      for (int64_t r = 0; r < m; ++r) U[r * bb + j] = col[r];
    }
    for (int it = 0; it < iters; ++it) {
      /* G = U^T U, the V target rows Tv = (G + eps I)^-1 U^T R */
      for (int i = 0; i < bb; ++i)
        for (int j = 0; j < bb; ++j) {
          double s = 0.0;
          for (int64_t r = 0; r < m; ++r) s += U[r * bb + i] * U[r * bb + j];
          G[i * bb + j] = s;
        }
      for (int i = 0; i < bb; ++i)
        for (int64_t c = 0; c < n; ++c) Tv[i * n + c] = 0.0;
      for (int64_t r = 0; r < m; ++r)
        for (int i = 0; i < bb; ++i) {
          const double ur = U[r * bb + i];
          if (ur != 0.0)
            for (int64_t c = 0; c < n; ++c) Tv[i * n + c] += ur * R[r * n + c];
        }
      if (!ridge_factor(G, bb)) goto fail;
      for (int64_t c = 0; c < n; ++c) cholesky_solve(G, bb, Tv + c, n);
      for (int i = 0; i < bb; ++i) {
        orc_ternarize(Tv + (int64_t)i * n, n, tau, t8);
        for (int64_t c = 0; c < n; ++c) V[c * bb + i] = (double)t8[c];
      }
      /* Q = R V, G = V^T V, the U target rows Tu = (G + eps I)^-1 Q^T */
      for (int64_t r = 0; r < m; ++r)
        for (int j = 0; j < bb; ++j) {
          double s = 0.0;
          for (int64_t c = 0; c < n; ++c) s += R[r * n + c] * V[c * bb + j];
          Q[r * bb + j] = s;
        }
      for (int i = 0; i < bb; ++i)
        for (int j = 0; j < bb; ++j) {
          double s = 0.0;
          for (int64_t c = 0; c < n; ++c) s += V[c * bb + i] * V[c * bb + j];
          G[i * bb + j] = s;
        }
      for (int i = 0; i < bb; ++i)
        for (int64_t r = 0; r < m; ++r) Tu[i * m + r] = Q[r * bb + i];
      if (!ridge_factor(G, bb)) goto fail;
      for (int64_t r = 0; r < m; ++r) cholesky_solve(G, bb, Tu + r, m);
      for (int i = 0; i < bb; ++i) {
        orc_ternarize(Tu + (int64_t)i * m, m, tau, t8);
        for (int64_t r = 0; r < m; ++r) U[r * bb + i] = (double)t8[r];
      }
    }
    /* the joint scales: [(U^T U) o (V^T V)] d = diag(U^T R V), read off Q */
    for (int j = 0; j < bb; ++j) {
      double s = 0.0;
      for (int64_t r = 0; r < m; ++r) s += U[r * bb + j] * Q[r * bb + j];
      rhs[j] = s;
    }
    for (int i = 0; i < bb; ++i)
      for (int j = 0; j < bb; ++j) {
        double gu = 0.0, gv = 0.0;
        for (int64_t r = 0; r < m; ++r) gu += U[r * bb + i] * U[r * bb + j];
        for (int64_t c = 0; c < n; ++c) gv += V[c * bb + i] * V[c * bb + j];
        G[i * bb + j] = gu * gv;
      }
    memcpy(G2, G, sizeof(double) * (size_t)(bb * bb));
    if (!cholesky(G2, bb)) {
      ++nretry;
      memcpy(G2, G, sizeof(double) * (size_t)(bb * bb));
      if (!ridge_factor(G2, bb)) goto fail;
    }
    for (int j = 0; j < bb; ++j) col[j] = rhs[j];
    cholesky_solve(G2, bb, col, 1);
    r2 = 0.0;
    for (int64_t r = 0; r < m; ++r)
      for (int64_t c = 0; c < n; ++c) {
        double s = 0.0;
        for (int j = 0; j < bb; ++j) s += U[r * bb + j] * col[j] * V[c * bb + j];
        R[r * n + c] -= s;
        r2 += R[r * n + c] * R[r * n + c];
      }
    for (int j = 0; j < bb; ++j) {
      for (int64_t r = 0; r < m; ++r) B[(c0 + j) * m + r] = (int8_t)U[r * bb + j];
      for (int64_t c = 0; c < n; ++c) C[(c0 + j) * n + c] = (int8_t)V[c * bb + j];
      D[c0 + j] = col[j];
    }
    if (trace) trace[blk] = r2;
  }
  *energy = norm_a2 > 0.0 ? 1.0 - r2 / norm_a2 : 1.0;
  if (retries) *retries = nretry;
  free(R); free(U); free(V); free(Tv); free(Tu); free(Q); free(G); free(G2); free(rhs); free(t8); free(col);
  return 0;
fail:
  free(R); free(U); free(V); free(Tv); free(Tu); free(Q); free(G); free(G2); free(rhs); free(t8); free(col);
  return -2;
}
