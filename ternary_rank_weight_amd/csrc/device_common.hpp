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
// maximum magnitude M > 0: e = frexp exponent of M, s = 52 - e - ceil(log2 N),
// q_j = floor(|x_j| * 2^s) (exact integers, each < 2^(52 - ceil(log2 N))),
// S = (sum q) * 2^-s (the sum is < 2^52, so exact in fp64 in any order) and
// thr = (tau * S) / N.  The result does not depend on the reduction order
// or on the grid shape.
// ---------------------------------------------------------------------------
__device__ inline int ceil_log2_i32(int n) { return n <= 1 ? 0 : 32 - __clz(n - 1); }
__device__ inline int fixed_point_shift(float maxabs, int N) {
  int e;
  (void)frexp((double)maxabs, &e);
  return 52 - e - ceil_log2_i32(N);
}
// q = floor(|x| * 2^s), an exact integer held in an fp64 (|x| * 2^s is exact
// and below 2^52).
__device__ inline double fixed_point_q(float absval, int s) {
  return floor(ldexp((double)absval, s));
}
__device__ inline double fixed_point_threshold(double qsum, int s, float tau, int64_t N) {
  const double S = ldexp(qsum, -s);
  return ((double)tau * S) / (double)N;
}
// Bits of the largest fp32 value <= thr (thr >= 0).  For a finite fp32
// magnitude a, a > thr exactly when bits(a) > the returned bits.
__device__ inline uint32_t threshold_bits(double thr) {
  const float f = (float)thr;
  uint32_t b = __float_as_uint(f);
  if ((double)f > thr) b -= 1u;
  return b;
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

// Max of a non-negative fp64 value over the wave, stored by lane 0 into
// part[wave index of the whole launch] (blockIdx.y-major, then blockIdx.x,
// then the wave within the workgroup): one plain store per wave and no
// atomics, the consumer taking the max of the launch's partials.  Every
// lane of the wave must call.
__device__ inline void wave_max_nonneg_part(double v, double* part) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) {
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    part[wg * (blockDim.x / kWave) + threadIdx.x / kWave] = v;
  }
}
// Waves of a launch of grid x workgroups of `threads`: partials it leaves.
inline int64_t wave_partials(int64_t workgroups, int threads) { return workgroups * (threads / kWave); }

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
__device__ inline double block_max_f64(double v, double* scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < T / kWave; ++i) r = fmax(r, scratch[i]);
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

// ---------------------------------------------------------------------------
// Wave64 reductions with DPP row operations (fixed combination order):
// xor-1 and xor-2 inside quads, half-row and row mirrors, then the two row
// broadcasts; lane 63 ends up holding the full result.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK>
__device__ inline int dpp_i32(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
__device__ inline float dpp_f32(float identity, float v) {
  return __int_as_float(dpp_i32<CTRL, ROWMASK>(__float_as_int(identity), __float_as_int(v)));
}
template <int CTRL, int ROWMASK>
__device__ inline double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL, ROWMASK>(0, (int)(b & 0xffffffffll));
  const int hi = dpp_i32<CTRL, ROWMASK>(0, (int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
// Sum over the wave; the result is valid in lane 63.
__device__ inline float wave_sum_to63(float v) {
  v += dpp_f32<0xB1, 0xF>(0.f, v);
  v += dpp_f32<0x4E, 0xF>(0.f, v);
  v += dpp_f32<0x141, 0xF>(0.f, v);
  v += dpp_f32<0x140, 0xF>(0.f, v);
  v += dpp_f32<0x142, 0xA>(0.f, v);
  v += dpp_f32<0x143, 0xC>(0.f, v);
  return v;
}
__device__ inline double wave_sum_to63(double v) {
  v += dpp_f64<0xB1, 0xF>(v);
  v += dpp_f64<0x4E, 0xF>(v);
  v += dpp_f64<0x141, 0xF>(v);
  v += dpp_f64<0x140, 0xF>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  return v;
}
// Maximum over the wave of non-negative values; valid in lane 63.
__device__ inline float wave_max_to63(float v) {
  v = fmaxf(v, dpp_f32<0xB1, 0xF>(0.f, v));
  v = fmaxf(v, dpp_f32<0x4E, 0xF>(0.f, v));
  v = fmaxf(v, dpp_f32<0x141, 0xF>(0.f, v));
  v = fmaxf(v, dpp_f32<0x140, 0xF>(0.f, v));
  v = fmaxf(v, dpp_f32<0x142, 0xA>(0.f, v));
  v = fmaxf(v, dpp_f32<0x143, 0xC>(0.f, v));
  return v;
}
// Maximum over the wave of unsigned values; valid in lane 63.
__device__ inline uint32_t wave_umax_to63(uint32_t v) {
  v = max(v, (uint32_t)dpp_i32<0xB1, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i32<0x4E, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i32<0x141, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i32<0x140, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i32<0x142, 0xA>(0, (int)v));
  v = max(v, (uint32_t)dpp_i32<0x143, 0xC>(0, (int)v));
  return v;
}
__device__ inline float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline double lane63(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
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
