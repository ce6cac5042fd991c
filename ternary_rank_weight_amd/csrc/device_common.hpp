// Device helpers shared by the ExTernD kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace externd {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Starting vectors.  The pages leave u's initial value open (ExTernD §2.3); this
// library fixes it as a dense +-1 vector drawn from SplitMix64's output
// function (Steele, Lea & Flood 2014) used as a stateless hash:
//   mix(x) = fin(x + 0x9E3779B97F4A7C15), fin(z) = z^(z>>30), *0xBF58476D1CE4E5B9,
//            z^(z>>27), *0x94D049BB133111EB, z^(z>>31)
//   h = mix(mix(mix(seed) + i) + r), u0[r] = (h >> 63) ? -1 : +1
// for global component index i and row r.
// ---------------------------------------------------------------------------
__host__ __device__ inline uint64_t sm64_mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__host__ __device__ inline uint64_t start_base(uint64_t seed, uint64_t comp) {
  return sm64_mix(sm64_mix(seed) + comp);
}
__host__ __device__ inline float start_sign(uint64_t base, uint64_t row) {
  return (sm64_mix(base + row) >> 63) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// Fixed-point mean used by T_tau (§2.2).  For a vector of length N with
// maximum magnitude M > 0: e = frexp exponent of M, s = 62 - e - ceil(log2 N),
// q_j = floor(|x_j| * 2^s) (exact int64), S = double(sum q) * 2^-s and
// thr = (tau * S) / N.  Integer sums make the result independent of the
// reduction order and of the grid shape.
// ---------------------------------------------------------------------------
__host__ __device__ inline int ceil_log2_i64(int64_t n) {
  int l = 0;
  while ((int64_t(1) << l) < n) ++l;
  return l;
}
__device__ inline int fixed_point_shift(float maxabs, int64_t N) {
  int e;
  (void)frexp((double)maxabs, &e);
  return 62 - e - ceil_log2_i64(N);
}
__device__ inline int64_t fixed_point_q(float v, int s) {
  return (int64_t)floor(ldexp((double)fabsf(v), s));
}
__device__ inline double fixed_point_threshold(int64_t qsum, int s, float tau, int64_t N) {
  double S = ldexp((double)qsum, -s);
  return ((double)tau * S) / (double)N;
}

// ---------------------------------------------------------------------------
// Block-wide reductions for a block of T threads (T a multiple of 64).  The
// combination order is fixed (xor butterfly inside a wave, waves in index
// order), so repeated runs give identical results.  `scratch` must hold
// T/64 elements of 8 bytes; every thread of the block must call.
// ---------------------------------------------------------------------------
template <typename V>
__device__ inline V wave_sum(V v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ inline int wave_min_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, kWave));
  return v;
}

template <int T, typename V>
__device__ inline V block_sum(V v, V* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  V r = scratch[0];
#pragma unroll
  for (int i = 1; i < T / kWave; ++i) r += scratch[i];
  return r;
}
template <int T>
__device__ inline float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < T / kWave; ++i) r = fmaxf(r, scratch[i]);
  return r;
}
template <int T>
__device__ inline int block_min_i(int v, int* scratch) {
  v = wave_min_i(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int i = 1; i < T / kWave; ++i) r = min(r, scratch[i]);
  return r;
}

// 2-bit code of a ternary value: 0 -> 00, +1 -> 01, -1 -> 11.
__host__ __device__ inline uint32_t code_of(float t) {
  return t > 0.f ? 1u : (t < 0.f ? 3u : 0u);
}
__host__ __device__ inline float value_of_code(uint32_t c) {
  return c == 1u ? 1.0f : (c == 3u ? -1.0f : 0.0f);
}
__device__ inline float code_at(const uint32_t* codes, int64_t j) {
  return value_of_code((codes[j >> 4] >> (2 * (j & 15))) & 3u);
}

}  // namespace externd
