// Optimal ternary projection (ExTernD §2.2) by one workgroup: the t in
// {-1,0,1}^N and alpha minimising ||x - alpha t|| keep the s largest |x_j|
// with their signs, s maximising (sum of the s largest |x|) / sqrt(s).  The
// prefix score is not unimodal, so every prefix is scored:
//
//   1. keys (|x_j| bits << 32 | ~j) go to LDS and are sorted descending by a
//      bitonic network (equal magnitudes in index order; the keys are unique);
//   2. each thread takes a contiguous chunk of the sorted order and sums the
//      fixed-point magnitudes q_j = floor(|x_j| 2^s) of the mean threshold
//      (exact integers, all partial sums below 2^52, hence exact in fp64 in
//      any order); a block scan gives every prefix sum Q_p exactly;
//   3. prefixes are compared exactly, Q_p^2 r against Q_r^2 p in 128-bit
//      integers, the shorter prefix winning a tie; an argmax over the block;
//   4. entry j is kept iff its key is >= the key at the chosen prefix end.
//
// N <= P <= PMAX with P a power of two; the caller handles max|x| = 0.
#pragma once
#include "device_common.hpp"
#include "kernels.hpp"

namespace externd {

__device__ inline uint64_t proj_key(float v, int j) {
  return ((uint64_t)(__float_as_uint(v) & 0x7fffffffu) << 32) | (uint32_t)(~(uint32_t)j);
}

// Is prefix (q1, s1) better than (q2, s2)?  s = 0 marks "no candidate".
__device__ inline bool proj_better(double q1, int s1, double q2, int s2) {
  if (s1 == 0) return false;
  if (s2 == 0) return true;
  const unsigned long long a = (unsigned long long)q1, b = (unsigned long long)q2;
  const unsigned __int128 l = (unsigned __int128)a * a * (unsigned)s2;
  const unsigned __int128 r = (unsigned __int128)b * b * (unsigned)s1;
  return l > r || (l == r && s1 < s2);
}

struct ProjScratch {
  double q[1024];   // per-thread chunk sums, then the scan, then argmax values
  int s[1024];
  uint64_t kstar;
};

// Returns the key threshold K*: entry j is kept iff proj_key(x_j, j) >= K*.
// M = max |x| > 0.  keys must hold P entries.
template <int T>
__device__ uint64_t projection_threshold(const float* __restrict__ x, int N, float M, uint64_t* keys,
                                         ProjScratch& sc) {
  static_assert(T <= 1024, "scratch holds 1024 threads");
  const int t = threadIdx.x;
  int P = 1;
  while (P < N) P <<= 1;
  for (int j = t; j < P; j += T) keys[j] = j < N ? proj_key(x[j], j) : 0ull;
  __syncthreads();
  // 1. bitonic sort, descending
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < P / 2; i += T) {
        const int lo = 2 * jj * (i / jj) + (i % jj), hi = lo + jj;
        const uint64_t a = keys[lo], b = keys[hi];
        const bool desc = (lo & k) == 0;
        if ((a < b) == desc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  // 2. chunk sums and an exact block scan (Hillis-Steele over T values)
  const int s = fixed_point_shift(M, N);
  const int C = (P + T - 1) / T;
  const int p0 = t * C, p1 = min(p0 + C, N);
  double part = 0.0;
  for (int p = p0; p < p1; ++p) part += fixed_point_q(__uint_as_float((uint32_t)(keys[p] >> 32)), s);
  sc.q[t] = part;
  __syncthreads();
  for (int off = 1; off < T; off <<= 1) {
    const double add = t >= off ? sc.q[t - off] : 0.0;
    __syncthreads();
    sc.q[t] += add;
    __syncthreads();
  }
  double run = sc.q[t] - part;   // exclusive prefix: all exact integers
  // 3. this thread's best prefix, then the block's
  double bq = 0.0;
  int bs = 0;
  for (int p = p0; p < p1; ++p) {
    run += fixed_point_q(__uint_as_float((uint32_t)(keys[p] >> 32)), s);
    if (proj_better(run, p + 1, bq, bs)) {
      bq = run;
      bs = p + 1;
    }
  }
  __syncthreads();
  sc.q[t] = bq;
  sc.s[t] = bs;
  __syncthreads();
  for (int off = T / 2; off > 0; off >>= 1) {
    if (t < off && proj_better(sc.q[t + off], sc.s[t + off], sc.q[t], sc.s[t])) {
      sc.q[t] = sc.q[t + off];
      sc.s[t] = sc.s[t + off];
    }
    __syncthreads();
  }
  // 4. the key at the end of the chosen prefix
  // (the top entry alone is always a candidate: its q is at least 2^37)
  if (t == 0) sc.kstar = keys[max(sc.s[0], 1) - 1];
  __syncthreads();
  return sc.kstar;
}

}  // namespace externd
