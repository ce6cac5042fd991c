// Streaming sequential path: R lives in device memory and every ALS half-step
// is one or two kernels.  Also provides the single-step entry points.
//
// ExTernD §2.3: for each component, alternate v = T_tau(R^T u), u = T_tau(R v)
// for `iters` iterations, take d = u^T R v / (|u|^2 |v|^2) and deflate
// R <- R - d u v^T.  T_tau is the mean-threshold ternarizer of §2.2.
#include "device_common.hpp"
#include "kernels.hpp"
#include "projection.hpp"

namespace externd {

// ---------------------------------------------------------------------------
// T_tau on one vector by a single workgroup (§2.2).  Writes 2-bit codes of
// all ceil(N/16) words, the nonzero count, and bumps *fallbacks when the
// single-largest-entry rule fires.
// ---------------------------------------------------------------------------
constexpr int kTernT = 1024;

__global__ __launch_bounds__(kTernT) void k_ternarize(const float* __restrict__ x, int64_t N,
                                                      float tau, uint32_t* __restrict__ codes,
                                                      int32_t* __restrict__ nnz_out,
                                                      long long* __restrict__ fallbacks,
                                                      const float* __restrict__ wt,
                                                      double* __restrict__ wsum,
                                                      long long* __restrict__ nnz_sum) {
  // wsum (with wt): sum of wt over the kept entries, i.e. v^T diag(wt) v (§2.5);
  // nnz_sum (optional) accumulates the nonzero count (one workgroup, stream order)
  __shared__ double scratch[kTernT / kWave];
  float* fs = reinterpret_cast<float*>(scratch);
  int* is = reinterpret_cast<int*>(scratch);
  const int tid = threadIdx.x;
  float mx = 0.f;
  for (int64_t j = tid; j < N; j += kTernT) mx = fmaxf(mx, fabsf(x[j]));
  const float M = block_max<kTernT>(mx, fs);
  const int64_t words = (N + 15) / 16;
  if (M == 0.f) {
    for (int64_t w = tid; w < words; w += kTernT) codes[w] = (w == 0) ? 1u : 0u;
    if (tid == 0) {
      if (nnz_out) *nnz_out = 1;
      if (nnz_sum) *nnz_sum += 1;
      if (wsum) *wsum = (double)wt[0];
      if (fallbacks) atomicAdd(reinterpret_cast<unsigned long long*>(fallbacks), 1ull);
    }
    return;
  }
  const int s = fixed_point_shift(M, (int)N);
  double q = 0.0;  // integer-valued partial sums below 2^52: exact in any order
  for (int64_t j = tid; j < N; j += kTernT) q += fixed_point_q(fabsf(x[j]), s);
  const double Q = block_sum<kTernT>(q, scratch);
  const double thr = fixed_point_threshold(Q, s, tau, N);
  int cnt = 0;
  double ws = 0.0;
  for (int64_t w = tid; w < words; w += kTernT) {
    uint32_t word = 0;
    for (int e = 0; e < 16; ++e) {
      const int64_t j = w * 16 + e;
      if (j < N) {
        const float v = x[j];
        if ((double)fabsf(v) > thr) {
          word |= code_of(v) << (2 * e);
          ++cnt;
          if (wsum) ws += (double)wt[j];
        }
      }
    }
    codes[w] = word;
  }
  if ((double)M > thr) {
    const int total = block_sum<kTernT>(cnt, is);
    if (wsum) {
      const double wt_total = block_sum<kTernT>(ws, scratch);
      if (tid == 0) *wsum = wt_total;
    }
    if (tid == 0 && nnz_out) *nnz_out = total;
  if (tid == 0 && nnz_sum) *nnz_sum += total;
    return;
  }
  // Nothing passed: keep the smallest index holding the largest magnitude.
  int first = INT32_MAX;
  for (int64_t j = tid; j < N; j += kTernT)
    if (fabsf(x[j]) == M) { first = (int)j; break; }
  const int idx = block_min_i<kTernT>(first, is);
  __syncthreads();  // codes words written above are visible block-wide below
  if (tid == 0) {
    codes[idx >> 4] = code_of(x[idx]) << (2 * (idx & 15));
    if (nnz_out) *nnz_out = 1;
      if (nnz_sum) *nnz_sum += 1;
    if (wsum) *wsum = (double)wt[idx];
    if (fallbacks) atomicAdd(reinterpret_cast<unsigned long long*>(fallbacks), 1ull);
  }
}

// The same rule for N <= 256 K with the vector held in registers: one read of
// x, and the codes packed from wave ballots (wave w of pass j covers entries
// 256 j + 64 w .. + 63, i.e. code words 16 j + 4 w .. + 3).  Outputs as
// k_ternarize.
__device__ inline uint32_t spread_bits16(uint32_t v) {   // bit e -> bit 2e
  v &= 0xffffu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  v = (v | (v << 4)) & 0x0F0F0F0Fu;
  v = (v | (v << 2)) & 0x33333333u;
  v = (v | (v << 1)) & 0x55555555u;
  return v;
}

template <int K>
__global__ __launch_bounds__(256) void k_ternarize_reg(const float* __restrict__ x, int64_t N, float tau,
                                                       uint32_t* __restrict__ codes, int32_t* __restrict__ nnz_out,
                                                       long long* __restrict__ fallbacks,
                                                       const float* __restrict__ wt, double* __restrict__ wsum,
                                                       long long* __restrict__ nnz_sum) {
  constexpr int T = 256, W = T / kWave;
  __shared__ int scratch[W];
  __shared__ int wcnt[W];
  __shared__ double wws[W];
  __shared__ unsigned s_max;   // bits of the largest |x| (LDS atomic max)
  __shared__ double s_sum;     // the fixed-point sum (LDS atomic add of exact integers)
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  if (tid == 0) {
    s_max = 0u;
    s_sum = 0.0;
  }
  float v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t idx = tid + (int64_t)T * j;
    const float a = x[idx < N ? idx : 0];
    v[j] = idx < N ? a : 0.f;
  }
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) mx = fmaxf(mx, fabsf(v[j]));
  // DPP inside the wave, one LDS atomic per wave; a wave whose entries are
  // all NaN adds nothing, as a NaN operand of fmaxf adds nothing
  const float wm = wave_max_to63(mx);
  if (lane == kWave - 1) atomicMax(&s_max, wm == wm ? __float_as_uint(wm) : 0u);
  __syncthreads();
  const float M = __uint_as_float(s_max);
  const int64_t words = (N + 15) / 16;
  if (M == 0.f) {
    for (int64_t q = tid; q < words; q += T) codes[q] = (q == 0) ? 1u : 0u;
    if (tid == 0) {
      if (nnz_out) *nnz_out = 1;
      if (nnz_sum) *nnz_sum += 1;
      if (wsum) *wsum = (double)wt[0];
      if (fallbacks) atomicAdd(reinterpret_cast<unsigned long long*>(fallbacks), 1ull);
    }
    return;
  }
  const int s = fixed_point_shift(M, (int)N);
  double q = 0.0;   // integer-valued partial sums below 2^52: exact in any order
#pragma unroll
  for (int j = 0; j < K; ++j) q += fixed_point_q(fabsf(v[j]), s);
  const double qw = wave_sum_to63(q);
  if (lane == kWave - 1) atomicAdd(&s_sum, qw);
  __syncthreads();
  const double thr = fixed_point_threshold(s_sum, s, tau, N);
  int cnt = 0;       // this wave's kept entries (wave-uniform, from the ballots)
  double ws = 0.0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t idx = tid + (int64_t)T * j;
    const bool keep = idx < N && (double)fabsf(v[j]) > thr;
    const unsigned long long nz = __ballot(keep);
    const unsigned long long ng = __ballot(keep && v[j] < 0.f);
    cnt += __popcll(nz);
    if (wsum && keep) ws += (double)wt[idx];
    if (lane < 4) {
      const int64_t wd = (int64_t)16 * j + 4 * w + lane;
      if (wd < words)
        codes[wd] = spread_bits16((uint32_t)(nz >> (16 * lane))) | (spread_bits16((uint32_t)(ng >> (16 * lane))) << 1);
    }
  }
  if ((double)M > thr) {
    // per-wave parts in fixed order: DPP inside the wave, waves in index order
    const double wsw = wsum ? wave_sum_to63(ws) : 0.0;
    if (lane == kWave - 1) {
      wcnt[w] = cnt;
      wws[w] = wsw;
    }
    __syncthreads();
    if (tid == 0) {
      int total = 0;
      double wt_total = 0.0;
#pragma unroll
      for (int u = 0; u < W; ++u) {
        total += wcnt[u];
        wt_total += wws[u];
      }
      if (wsum) *wsum = wt_total;
      if (nnz_out) *nnz_out = total;
      if (nnz_sum) *nnz_sum += total;
    }
    return;
  }
  // Nothing passed: keep the smallest index holding the largest magnitude.
  int first = INT32_MAX;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t idx = tid + (int64_t)T * j;
    if (idx < N && fabsf(v[j]) == M) first = min(first, (int)idx);
  }
  const int pick = block_min_i<T>(first, scratch);
  __syncthreads();  // the zero code words written above are visible block-wide below
  if (tid == 0) {
    codes[pick >> 4] = code_of(x[pick]) << (2 * (pick & 15));
    if (nnz_out) *nnz_out = 1;
    if (nnz_sum) *nnz_sum += 1;
    if (wsum) *wsum = (double)wt[pick];
    if (fallbacks) atomicAdd(reinterpret_cast<unsigned long long*>(fallbacks), 1ull);
  }
}

// ---------------------------------------------------------------------------
// The optimal ternary projection of one vector (§2.2) by a single workgroup,
// the alternative to T_tau: same outputs (codes, nnz, fallback count for an
// all-zero vector, weighted support sum).  PMAX >= the padded length.
// ---------------------------------------------------------------------------
template <int PMAX>
__global__ __launch_bounds__(kTernT) void k_project(const float* __restrict__ x, int64_t N,
                                                    uint32_t* __restrict__ codes, int32_t* __restrict__ nnz_out,
                                                    long long* __restrict__ fallbacks,
                                                    const float* __restrict__ wt, double* __restrict__ wsum,
                                                    long long* __restrict__ nnz_sum) {
  __shared__ uint64_t keys[PMAX];
  __shared__ ProjScratch sc;
  __shared__ double scratch[kTernT / kWave];
  const int tid = threadIdx.x;
  float mx = 0.f;
  for (int64_t j = tid; j < N; j += kTernT) mx = fmaxf(mx, fabsf(x[j]));
  const float M = block_max<kTernT>(mx, reinterpret_cast<float*>(scratch));
  const int64_t words = (N + 15) / 16;
  if (M == 0.f) {
    for (int64_t w = tid; w < words; w += kTernT) codes[w] = (w == 0) ? 1u : 0u;
    if (tid == 0) {
      if (nnz_out) *nnz_out = 1;
      if (nnz_sum) *nnz_sum += 1;
      if (wsum) *wsum = (double)wt[0];
      if (fallbacks) atomicAdd(reinterpret_cast<unsigned long long*>(fallbacks), 1ull);
    }
    return;
  }
  const uint64_t K = projection_threshold<kTernT>(x, (int)N, M, keys, sc);
  int cnt = 0;
  double ws = 0.0;
  for (int64_t w = tid; w < words; w += kTernT) {
    uint32_t word = 0;
    for (int e = 0; e < 16; ++e) {
      const int64_t j = w * 16 + e;
      if (j < N) {
        const float v = x[j];
        if (proj_key(v, (int)j) >= K) {
          word |= code_of(v) << (2 * e);
          ++cnt;
          if (wsum) ws += (double)wt[j];
        }
      }
    }
    codes[w] = word;
  }
  const int total = block_sum<kTernT>(cnt, reinterpret_cast<int*>(scratch));
  if (wsum) {
    const double wt_total = block_sum<kTernT>(ws, scratch);
    if (tid == 0) *wsum = wt_total;
  }
  if (tid == 0 && nnz_out) *nnz_out = total;
  if (tid == 0 && nnz_sum) *nnz_sum += total;
}

// ---------------------------------------------------------------------------
// y = R^T u, in two deterministic stages: per row-chunk partial sums, then a
// fixed-order sum over chunks.  Rows with u_r = 0 are skipped (never read).
// When `dprev` is non-null the previous component is first deflated out of
// every row the chunk touches (§2.3 step 3 fused into the next step 1):
// R_rc <- fl32(R_rc - d u'_r v'_c), written back.
// ---------------------------------------------------------------------------
constexpr int kGtT = 256;     // columns per workgroup
constexpr int kGtRows = 128;  // rows per chunk

// mpart (optional, with a dense u): per-wave partial maxima of w_c R_rc^2
// over the rows read, after the fused deflation (the single-entry bound of
// appendix §7), one per wave of the launch.
__global__ __launch_bounds__(kGtT) void k_gemv_t_partial(
    float* __restrict__ R, int64_t m, int64_t n, const uint32_t* __restrict__ u_codes,
    float* __restrict__ partial, const float* __restrict__ dprev,
    const uint32_t* __restrict__ uprev, const uint32_t* __restrict__ vprev,
    double* __restrict__ mpart, const float* __restrict__ wt) {
  const int64_t c = (int64_t)blockIdx.x * kGtT + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kGtRows;
  const int64_t r1 = min(m, r0 + kGtRows);
  float acc = 0.f;
  uint32_t mb = 0u;   // largest |R_rc| read (bits)
  const bool incol = c < n;
  if (dprev) {
    const float d = *dprev;
    const float vc = incol ? code_at(vprev, c) : 0.f;
    for (int64_t r = r0; r < r1; ++r) {
      const float ur = code_at(u_codes, r);
      const float up = code_at(uprev, r);
      if (up != 0.f && incol) {
        float val = R[r * n + c];
        if (vc != 0.f) {
          val = fmaf(-d, up * vc, val);
          R[r * n + c] = val;
        }
        acc = fmaf(ur, val, acc);
        mb = max(mb, __float_as_uint(val) & 0x7fffffffu);
      } else if (ur != 0.f && incol) {
        const float val = R[r * n + c];
        acc = fmaf(ur, val, acc);
        mb = max(mb, __float_as_uint(val) & 0x7fffffffu);
      }
    }
  } else {
    for (int64_t r = r0; r < r1; ++r) {
      const float ur = code_at(u_codes, r);
      if (ur != 0.f && incol) {
        const float val = R[r * n + c];
        acc = fmaf(ur, val, acc);
        mb = max(mb, __float_as_uint(val) & 0x7fffffffu);
      }
    }
  }
  if (incol) partial[(int64_t)blockIdx.y * n + c] = acc;
  if (mpart) {
    const double x = (double)__uint_as_float(mb);
    wave_max_nonneg_part(incol ? x * x * (wt ? (double)wt[c] : 1.0) : 0.0, mpart);
  }
}

// The same partial products for n % 4 == 0, built for bandwidth: a
// workgroup takes 256 columns (one float4 per lane) and the chunk's 128 rows,
// wave w the rows r0 + w + 4i.  The chunk's code words are read first; then
// every row load of the wave is issued before any is used, unconditionally
// (a row the wave does not need reads row 0's entries and is multiplied by
// u_r = 0), so no load waits on a branch.  The four waves' sums are combined
// in LDS in wave order.
constexpr int kGtWave = kGtRows / 4;   // rows per wave

__global__ __launch_bounds__(256) void k_gemv_t_vec(
    float* __restrict__ R, int64_t m, int64_t n, const uint32_t* __restrict__ u_codes,
    float* __restrict__ partial, const float* __restrict__ dprev,
    const uint32_t* __restrict__ uprev, const uint32_t* __restrict__ vprev,
    double* __restrict__ mpart, const float* __restrict__ wt) {
  static_assert(kGtRows == 128, "eight code words per chunk");
  __shared__ float4 red[3][kWave];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t n4 = n >> 2;
  const int64_t c4 = (int64_t)blockIdx.x * kWave + lane;   // float4 column
  const bool incol = c4 < n4;
  const int64_t c4s = incol ? c4 : 0;
  const int64_t r0 = (int64_t)blockIdx.y * kGtRows;
  const int64_t wm = (m + 15) >> 4;
  float4* R4 = reinterpret_cast<float4*>(R);
  // the chunk's code words: rows r0 .. r0 + 127
  uint32_t uw[8], pw[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t wi = (r0 >> 4) + q;
    const uint32_t a = u_codes[wi < wm ? wi : 0];
    const uint32_t b = dprev ? uprev[wi < wm ? wi : 0] : 0u;
    uw[q] = wi < wm ? a : 0u;
    pw[q] = wi < wm ? b : 0u;
  }
  const float d = dprev ? *dprev : 0.f;
  float vp[4] = {0.f, 0.f, 0.f, 0.f};
  bool vany = false;
  if (dprev && incol) {
    const uint32_t word = vprev[c4 >> 2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vp[e] = value_of_code((word >> (8 * (c4 & 3) + 2 * e)) & 3u);
      vany = vany || vp[e] != 0.f;
    }
  }
  float4 v[kGtWave];
  float ur[kGtWave], up[kGtWave];
#pragma unroll
  for (int k = 0; k < kGtWave; ++k) {
    // row r0 + w + 4k: word k / 4 of the chunk, entry w + 4 (k % 4)
    const int sh = 2 * (w + 4 * (k & 3));
    ur[k] = value_of_code((uw[k >> 2] >> sh) & 3u);
    up[k] = value_of_code((pw[k >> 2] >> sh) & 3u);
    const int64_t r = r0 + w + 4 * k;
    const bool need = r < m && (ur[k] != 0.f || up[k] != 0.f);
    v[k] = R4[need ? r * n4 + c4s : c4s];
  }
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  uint32_t mb[4] = {0u, 0u, 0u, 0u};   // largest |R| per column over the rows read (bits)
#pragma unroll
  for (int k = 0; k < kGtWave; ++k) {
    float4 val = v[k];
    if (up[k] != 0.f && vany) {
      val.x = vp[0] != 0.f ? fmaf(-d, up[k] * vp[0], val.x) : val.x;
      val.y = vp[1] != 0.f ? fmaf(-d, up[k] * vp[1], val.y) : val.y;
      val.z = vp[2] != 0.f ? fmaf(-d, up[k] * vp[2], val.z) : val.z;
      val.w = vp[3] != 0.f ? fmaf(-d, up[k] * vp[3], val.w) : val.w;
      R4[(r0 + w + 4 * k) * n4 + c4] = val;
    }
    acc.x = fmaf(ur[k], val.x, acc.x);
    acc.y = fmaf(ur[k], val.y, acc.y);
    acc.z = fmaf(ur[k], val.z, acc.z);
    acc.w = fmaf(ur[k], val.w, acc.w);
    if (mpart && r0 + w + 4 * k < m) {
      mb[0] = max(mb[0], __float_as_uint(val.x) & 0x7fffffffu);
      mb[1] = max(mb[1], __float_as_uint(val.y) & 0x7fffffffu);
      mb[2] = max(mb[2], __float_as_uint(val.z) & 0x7fffffffu);
      mb[3] = max(mb[3], __float_as_uint(val.w) & 0x7fffffffu);
    }
  }
  if (mpart) {
    double mx = 0.0;
    if (incol) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double x = (double)__uint_as_float(mb[e]);
        mx = fmax(mx, x * x * (wt ? (double)wt[4 * c4 + e] : 1.0));
      }
    }
    wave_max_nonneg_part(mx, mpart);
  }
  if (w > 0) red[w - 1][lane] = acc;
  __syncthreads();
  if (w == 0 && incol) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const float4 o = red[q][lane];
      acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
    }
    reinterpret_cast<float4*>(partial)[(int64_t)blockIdx.y * n4 + c4] = acc;
  }
}

__global__ void k_sum_chunks(const float* __restrict__ partial, int64_t chunks, int64_t n,
                             float* __restrict__ y) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  // chunk order; 32 loads in flight
  float acc = 0.f;
  for (int64_t q0 = 0; q0 < chunks; q0 += 32) {
    float v[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const bool ok = q0 + k < chunks;
      const float x = partial[ok ? (q0 + k) * n + c : c];
      v[k] = ok ? x : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) acc += v[k];
  }
  y[c] = acc;
}

// x = R v: one wave per row, lanes stride the row; masked add/sub as FMA with
// v in {-1, 0, 1} (exact products).  With column weights wt the target is
// x = R diag(wt) v (§2.5): each product uses wt_c v_c (exact sign change).
constexpr int kGnT = 256;

__global__ __launch_bounds__(kGnT) void k_gemv_n(const float* __restrict__ R, int64_t m,
                                                 int64_t n, const uint32_t* __restrict__ v_codes,
                                                 float* __restrict__ x, const float* __restrict__ wt) {
  const int64_t row = (int64_t)blockIdx.x * (kGnT / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= m) return;
  const float* rp = R + row * n;
  float acc = 0.f;
  if (wt) {
    for (int64_t c = lane; c < n; c += kWave) acc = fmaf(code_at(v_codes, c) * wt[c], rp[c], acc);
  } else {
    for (int64_t c = lane; c < n; c += kWave) acc = fmaf(code_at(v_codes, c), rp[c], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) x[row] = acc;
}

// The same for n % 4 == 0, built for bandwidth: lane l reads float4 column
// l + 64 i of the row, 8 loads (and their code words) issued before any is
// used; the four partial lanes of the float4 are added at the end.
constexpr int kGnBatch = 8;

template <bool W>
__global__ __launch_bounds__(kGnT) void k_gemv_n_vec(const float* __restrict__ R, int64_t m,
                                                     int64_t n, const uint32_t* __restrict__ v_codes,
                                                     float* __restrict__ x, const float* __restrict__ wt) {
  const int64_t row = (int64_t)blockIdx.x * (kGnT / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= m) return;
  const int64_t n4 = n >> 2;
  const float4* rp = reinterpret_cast<const float4*>(R + row * n);
  const float4* w4 = reinterpret_cast<const float4*>(wt);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i0 = 0; i0 < n4; i0 += (int64_t)kWave * kGnBatch) {
    float4 v[kGnBatch], ww[kGnBatch];
    uint32_t cw[kGnBatch];
#pragma unroll
    for (int k = 0; k < kGnBatch; ++k) {
      const int64_t i = i0 + lane + (int64_t)kWave * k;
      const bool ok = i < n4;
      const float4 a = rp[ok ? i : 0];
      const uint32_t c = v_codes[ok ? i >> 2 : 0];
      v[k] = ok ? a : float4{0.f, 0.f, 0.f, 0.f};
      cw[k] = ok ? (c >> (8 * (i & 3))) & 0xFFu : 0u;
      if constexpr (W) {
        const float4 b = w4[ok ? i : 0];
        ww[k] = b;
      }
    }
#pragma unroll
    for (int k = 0; k < kGnBatch; ++k) {
      float t0 = value_of_code(cw[k] & 3u), t1 = value_of_code((cw[k] >> 2) & 3u);
      float t2 = value_of_code((cw[k] >> 4) & 3u), t3 = value_of_code((cw[k] >> 6) & 3u);
      if constexpr (W) {
        t0 *= ww[k].x; t1 *= ww[k].y; t2 *= ww[k].z; t3 *= ww[k].w;
      }
      acc.x = fmaf(t0, v[k].x, acc.x);
      acc.y = fmaf(t1, v[k].y, acc.y);
      acc.z = fmaf(t2, v[k].z, acc.z);
      acc.w = fmaf(t3, v[k].w, acc.w);
    }
  }
  float sum = (acc.x + acc.y) + (acc.z + acc.w);
  sum = wave_sum(sum);
  if (lane == 0) x[row] = sum;
}

// R <- R - d u v^T (one rounding per entry), d read from device memory.
__global__ void k_deflate(float* __restrict__ R, int64_t m, int64_t n,
                          const uint32_t* __restrict__ u_codes,
                          const uint32_t* __restrict__ v_codes, const float* __restrict__ dptr) {
  const int64_t r = blockIdx.y;
  const float ur = code_at(u_codes, r);
  if (ur == 0.f) return;
  const float d = *dptr;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (int64_t)gridDim.x * blockDim.x) {
    const float vc = code_at(v_codes, c);
    if (vc != 0.f) R[r * n + c] = fmaf(-d, ur * vc, R[r * n + c]);
  }
}

// u0 of component `comp` as 2-bit codes.
__global__ void k_start_codes(uint64_t seed, int64_t comp, int64_t m, uint32_t* __restrict__ codes) {
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w * 16 >= m) return;
  const uint64_t base = start_base(seed, (uint64_t)comp);
  uint32_t word = 0;
  for (int e = 0; e < 16; ++e) {
    const int64_t r = w * 16 + e;
    if (r < m) word |= code_of(start_sign(base, (uint64_t)r)) << (2 * e);
  }
  codes[w] = word;
}

// d = (u . x) / (nnz_u nnz_v) in fp64, stored as fp32 in D[i]; trace update.
// With column weights, x = R diag(wt) v and the v factor of the denominator
// is v^T diag(wt) v (*sv); d = 0 when that is zero (every weight on supp(v)
// is zero, so u . x = 0 too and any d fits equally).
__global__ __launch_bounds__(kTernT) void k_scale(const float* __restrict__ x, int64_t m,
                                                  const uint32_t* __restrict__ u_codes,
                                                  const int32_t* __restrict__ nnz_u,
                                                  const int32_t* __restrict__ nnz_v,
                                                  float* __restrict__ D, int64_t i,
                                                  double* __restrict__ trace_state,
                                                  double* __restrict__ trace,
                                                  long long* __restrict__ stats,
                                                  const double* __restrict__ sv,
                                                  const double* __restrict__ mpart, int64_t nmpart,
                                                  double* __restrict__ sg_state) {
  __shared__ double scratch[kTernT / kWave];
  double acc = 0.0;
  for (int64_t r = threadIdx.x; r < m; r += kTernT) acc += (double)code_at(u_codes, r) * (double)x[r];
  const double c = block_sum<kTernT>(acc, scratch);
  // the single-entry bound of R before this component, from the first pass's partials
  double bmx = 0.0;
  for (int64_t q = threadIdx.x; q < nmpart; q += kTernT) bmx = fmax(bmx, mpart[q]);
  const double bound = block_max_f64<kTernT>(bmx, scratch);
  if (threadIdx.x == 0) {
    const double den = (double)(*nnz_u) * (sv ? *sv : (double)(*nnz_v));
    const double d = den > 0.0 ? c / den : 0.0;
    D[i] = (float)d;
    const double dec = den > 0.0 ? c * c / den : 0.0;
    const double t = trace_state[0] - dec;
    trace_state[0] = t;
    if (trace) trace[i] = t;
    if (stats) {
      stats[EXTERND_STAT_NNZ_B] += *nnz_u;
      stats[EXTERND_STAT_NNZ_C] += *nnz_v;
    }
    // Single-entry safeguard check (appendix §7) against the bound the
    // component's first pass measured.  With sg_state (the safeguard
    // applied), the decision, the fit's decrease and the bound are left for
    // k_safeguard_argmax / k_safeguard_apply.
    const bool would = dec < bound;
    if (would && stats) stats[EXTERND_STAT_SAFEGUARD] += 1;
    if (sg_state) {
      sg_state[0] = would ? 1.0 : 0.0;
      sg_state[1] = dec;
      reinterpret_cast<unsigned long long*>(sg_state)[2] = ~0ull;   // argmin index
      sg_state[3] = bound;
    }
  }
}

// The safeguard's replacement (appendix §7), when k_scale flagged it: the
// position of the single-entry bound, the smallest row-major index r n + c
// whose w_c R_rc^2 equals it (the same fp64 expression the bound was taken
// over), found over R before component i's deflation.
__global__ void k_safeguard_argmax(const float* __restrict__ R, int64_t m, int64_t n, const float* __restrict__ wt,
                                   double* __restrict__ sg_state) {
  if (sg_state[0] == 0.0) return;
  const double bound = sg_state[3];
  const int64_t total = m * n;
  unsigned long long best = ~0ull;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const double x = (double)R[e];
    const double v = x * x * (wt ? (double)wt[e % n] : 1.0);
    if (v == bound && (unsigned long long)e < best) best = (unsigned long long)e;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(best, off, kWave);
    best = o < best ? o : best;
  }
  if ((threadIdx.x & (kWave - 1)) == 0 && best != ~0ull)
    atomicMin(reinterpret_cast<unsigned long long*>(sg_state) + 2, best);
}

// Replace component i by the single entry e_r e_c^T with d = R_rc: codes,
// scale, predicted trace and nonzero counts.
__global__ void k_safeguard_apply(const float* __restrict__ R, int64_t m, int64_t n, const float* __restrict__ wt,
                                  uint32_t* __restrict__ ub, int64_t wm, uint32_t* __restrict__ vc, int64_t wn,
                                  float* __restrict__ D, int64_t i, double* __restrict__ trace_state,
                                  double* __restrict__ trace, long long* __restrict__ stats,
                                  const int32_t* __restrict__ nnz_u, const int32_t* __restrict__ nnz_v,
                                  double* __restrict__ sg_state) {
  const bool take = sg_state[0] != 0.0;
  const unsigned long long idx = reinterpret_cast<const unsigned long long*>(sg_state)[2];
  const bool ok = take && idx < (unsigned long long)(m * n);
  if (ok) {
    const int64_t r = (int64_t)(idx / (unsigned long long)n), c = (int64_t)(idx % (unsigned long long)n);
    for (int64_t q = threadIdx.x; q < wm; q += blockDim.x) ub[q] = (q == r / 16) ? (1u << (2 * (r % 16))) : 0u;
    for (int64_t q = threadIdx.x; q < wn; q += blockDim.x) vc[q] = (q == c / 16) ? (1u << (2 * (c % 16))) : 0u;
    if (threadIdx.x == 0) {
      const float rv = R[idx];
      D[i] = rv;
      const double x = (double)rv;
      const double t = trace_state[0] + sg_state[1] - x * x * (wt ? (double)wt[c] : 1.0);
      trace_state[0] = t;
      if (trace) trace[i] = t;
      stats[EXTERND_STAT_NNZ_B] += 1 - *nnz_u;
      stats[EXTERND_STAT_NNZ_C] += 1 - *nnz_v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) sg_state[0] = 0.0;
}


// ---------------------------------------------------------------------------
// Squared Frobenius norm with a fixed reduction order, plus a count of
// non-finite entries.  Stage 1 writes one fp64 partial per workgroup.
// ---------------------------------------------------------------------------
constexpr int kNormT = 256;

__global__ __launch_bounds__(kNormT) void k_norm2_partial(const float* __restrict__ A, int64_t total,
                                                          int64_t per_block,
                                                          double* __restrict__ partial,
                                                          long long* __restrict__ nonfinite,
                                                          const float* __restrict__ wt, int64_t ncols,
                                                          double* __restrict__ mpart) {
  // with column weights wt (ncols columns): sum_j wt_j A_ij^2 (§2.5); mpart
  // (optional) receives per-wave maxima of wt_j A_ij^2 (the single-entry bound)
  __shared__ double scratch[kNormT / kWave];
  const int64_t b0 = (int64_t)blockIdx.x * per_block;
  const int64_t b1 = min(total, b0 + per_block);
  double acc = 0.0, mx = 0.0;
  long long bad = 0;
  if (wt) {
    for (int64_t j = b0 + threadIdx.x; j < b1; j += kNormT) {
      const float v = A[j];
      if (!isfinite(v)) ++bad;
      const double e = (double)v * (double)v * (double)wt[j % ncols];
      acc += e;
      mx = fmax(mx, e);
    }
  } else {
    for (int64_t j = b0 + threadIdx.x; j < b1; j += kNormT) {
      const float v = A[j];
      if (!isfinite(v)) ++bad;
      const double e = (double)v * (double)v;
      acc += e;
      mx = fmax(mx, e);
    }
  }
  if (mpart) wave_max_nonneg_part(mx, mpart);
  const double s = block_sum<kNormT>(acc, scratch);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
  if (nonfinite) {
    const long long b = block_sum<kNormT>(bad, reinterpret_cast<long long*>(scratch));
    if (threadIdx.x == 0 && b) atomicAdd(reinterpret_cast<unsigned long long*>(nonfinite), (unsigned long long)b);
  }
}

// Column weights from per-input-channel second moments (§2.5): one workgroup
// takes M = max(h), then wt_j = fl32(h_j / M) + lambda (wt = lambda if M = 0).
// Negative or non-finite entries of h are counted into *nonfinite.
__global__ __launch_bounds__(kTernT) void k_importance_weights(const float* __restrict__ h, int64_t n,
                                                               float lambda, float* __restrict__ wt,
                                                               long long* __restrict__ nonfinite) {
  __shared__ double scratch[kTernT / kWave];
  float mx = 0.f;
  long long bad = 0;
  for (int64_t j = threadIdx.x; j < n; j += kTernT) {
    const float v = h[j];
    if (!isfinite(v) || v < 0.f) ++bad;
    else mx = fmaxf(mx, v);
  }
  const float M = block_max<kTernT>(mx, reinterpret_cast<float*>(scratch));
  for (int64_t j = threadIdx.x; j < n; j += kTernT) wt[j] = (M > 0.f ? h[j] / M : 0.f) + lambda;
  const long long b = block_sum<kTernT>(bad, reinterpret_cast<long long*>(scratch));
  if (threadIdx.x == 0 && b) atomicAdd(reinterpret_cast<unsigned long long*>(nonfinite), (unsigned long long)b);
}

__global__ void k_sum_partials(const double* __restrict__ partial, int64_t count,
                               double* __restrict__ out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double s = 0.0;
  for (int64_t i = 0; i < count; ++i) s += partial[i];
  *out = s;
}

// energy = 1 - r2 / a2 (1 when a2 = 0, NaN when A had non-finite entries).
__global__ void k_energy_finish(const double* __restrict__ a2, const double* __restrict__ r2,
                                const long long* __restrict__ nonfinite, double* __restrict__ energy,
                                double* __restrict__ trace_state) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double e;
  if (nonfinite && *nonfinite > 0) e = __longlong_as_double(0x7ff8000000000000ll);
  else if (*a2 == 0.0) e = 1.0;
  else e = 1.0 - *r2 / *a2;
  *energy = e;
  (void)trace_state;
}

__global__ void k_fill_u32(uint32_t* p, int64_t count, uint32_t v) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = v;
}
__global__ void k_fill_f32(float* p, int64_t count, float v) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = v;
}
__global__ void k_fill_i64(long long* p, int64_t count, long long v) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = v;
}
__global__ void k_copy_f32(const float* __restrict__ a, float* __restrict__ b, int64_t count) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    b[j] = a[j];
}
__global__ void k_copy_i64(const long long* __restrict__ a, long long* __restrict__ b, int64_t count) {
  for (int64_t j = threadIdx.x; j < count; j += blockDim.x) b[j] = a[j];
}
__global__ void k_set_f64(double* p, const double* src) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = *src;
}
__global__ void k_codes_to_i8(const uint32_t* __restrict__ codes, int64_t N, int8_t* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < N) out[j] = (int8_t)code_at(codes, j);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static inline unsigned grid1(int64_t count, int threads, int64_t cap = 4096) {
  int64_t g = (count + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid1(count, 256)), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}
hipError_t launch_fill_f32(float* p, int64_t count, float v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid1(count, 256)), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}
hipError_t launch_fill_i64(long long* p, int64_t count, long long v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i64, dim3(grid1(count, 256)), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}

hipError_t launch_ternarize(const float* x, int64_t N, float tau, uint32_t* codes, int32_t* nnz,
                            long long* fallbacks, hipStream_t s, const float* wt, double* wsum,
                            long long* nnz_sum) {
  if (N <= 1024)
    hipLaunchKernelGGL(k_ternarize_reg<4>, dim3(1), dim3(256), 0, s, x, N, tau, codes, nnz, fallbacks, wt, wsum, nnz_sum);
  else if (N <= 4096)
    hipLaunchKernelGGL(k_ternarize_reg<16>, dim3(1), dim3(256), 0, s, x, N, tau, codes, nnz, fallbacks, wt, wsum, nnz_sum);
  else
    hipLaunchKernelGGL(k_ternarize, dim3(1), dim3(kTernT), 0, s, x, N, tau, codes, nnz, fallbacks, wt, wsum, nnz_sum);
  return hipGetLastError();
}

hipError_t launch_project(const float* x, int64_t N, uint32_t* codes, int32_t* nnz, long long* fallbacks,
                          hipStream_t s, const float* wt, double* wsum, long long* nnz_sum) {
  if (N < 1 || N > kProjMaxN) return hipErrorInvalidValue;
  if (N <= 4096)
    hipLaunchKernelGGL(k_project<4096>, dim3(1), dim3(kTernT), 0, s, x, N, codes, nnz, fallbacks, wt, wsum, nnz_sum);
  else
    hipLaunchKernelGGL(k_project<kProjMaxN>, dim3(1), dim3(kTernT), 0, s, x, N, codes, nnz, fallbacks, wt, wsum, nnz_sum);
  return hipGetLastError();
}

hipError_t launch_importance_weights(const float* h, int64_t n, float lambda, float* wt,
                                     long long* nonfinite, hipStream_t s) {
  hipLaunchKernelGGL(k_importance_weights, dim3(1), dim3(kTernT), 0, s, h, n, lambda, wt, nonfinite);
  return hipGetLastError();
}

int64_t gemv_t_chunks(int64_t m) { return (m + kGtRows - 1) / kGtRows; }

int64_t gemv_t_max_partials(int64_t m, int64_t n) {
  const int64_t chunks = gemv_t_chunks(m);
  const int64_t wgs = (n & 3) == 0 ? (n / 4 + kWave - 1) / kWave * chunks : (n + kGtT - 1) / kGtT * chunks;
  return wave_partials(wgs, 256);
}

hipError_t launch_gemv_t(float* R, int64_t m, int64_t n, const uint32_t* u_codes, float* partial,
                         float* y, const float* dprev, const uint32_t* uprev,
                         const uint32_t* vprev, hipStream_t s, double* mpart, const float* wt) {
  const int64_t chunks = gemv_t_chunks(m);
  if ((n & 3) == 0) {
    dim3 grid((unsigned)((n / 4 + kWave - 1) / kWave), (unsigned)chunks);
    hipLaunchKernelGGL(k_gemv_t_vec, grid, dim3(256), 0, s, R, m, n, u_codes, partial, dprev, uprev, vprev,
                       mpart, wt);
  } else {
    dim3 grid((unsigned)((n + kGtT - 1) / kGtT), (unsigned)chunks);
    hipLaunchKernelGGL(k_gemv_t_partial, grid, dim3(kGtT), 0, s, R, m, n, u_codes, partial, dprev,
                       uprev, vprev, mpart, wt);
  }
  hipLaunchKernelGGL(k_sum_chunks, dim3(grid1(n, 256, 1 << 30)), dim3(256), 0, s, partial, chunks,
                     n, y);
  return hipGetLastError();
}

hipError_t launch_gemv_n(const float* R, int64_t m, int64_t n, const uint32_t* v_codes, float* x,
                         hipStream_t s, const float* wt) {
  const unsigned rows_per_block = kGnT / kWave;
  dim3 grid((unsigned)((m + rows_per_block - 1) / rows_per_block));
  if ((n & 3) == 0 && wt)
    hipLaunchKernelGGL(k_gemv_n_vec<true>, grid, dim3(kGnT), 0, s, R, m, n, v_codes, x, wt);
  else if ((n & 3) == 0)
    hipLaunchKernelGGL(k_gemv_n_vec<false>, grid, dim3(kGnT), 0, s, R, m, n, v_codes, x, wt);
  else
    hipLaunchKernelGGL(k_gemv_n, grid, dim3(kGnT), 0, s, R, m, n, v_codes, x, wt);
  return hipGetLastError();
}

hipError_t launch_deflate(float* R, int64_t m, int64_t n, const uint32_t* u_codes,
                          const uint32_t* v_codes, const float* dptr, hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 64), (unsigned)m);
  hipLaunchKernelGGL(k_deflate, grid, dim3(256), 0, s, R, m, n, u_codes, v_codes, dptr);
  return hipGetLastError();
}

hipError_t launch_norm2(const float* A, int64_t total, double* partial, int64_t partial_cap,
                        double* out, long long* nonfinite, hipStream_t s, const float* wt,
                        int64_t ncols, double* mpart, int64_t* nmpart) {
  int64_t blocks = std::min<int64_t>(partial_cap, std::max<int64_t>(1, (total + 65535) / 65536));
  const int64_t per_block = (total + blocks - 1) / blocks;
  if (total == 0) blocks = 1;
  if (wt && ncols < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_norm2_partial, dim3((unsigned)blocks), dim3(kNormT), 0, s, A, total,
                     std::max<int64_t>(per_block, 1), partial, nonfinite, wt, ncols, mpart);
  if (nmpart) *nmpart = wave_partials(blocks, kNormT);
  hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(64), 0, s, partial, blocks, out);
  return hipGetLastError();
}

__global__ void k_copy_f64(const double* __restrict__ src, double* __restrict__ dst, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
hipError_t launch_copy_f64(const double* src, double* dst, int64_t count, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_f64, dim3(1), dim3(64), 0, s, src, dst, count);
  return hipGetLastError();
}

hipError_t launch_energy_finish(const double* a2, const double* r2, const long long* nonfinite,
                                double* energy, hipStream_t s) {
  hipLaunchKernelGGL(k_energy_finish, dim3(1), dim3(64), 0, s, a2, r2, nonfinite, energy, nullptr);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* a, float* b, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_f32, dim3(grid1(count, 256)), dim3(256), 0, s, a, b, count);
  return hipGetLastError();
}

// Whole streaming decomposition (sequential mode).  ws must hold
// stream_workspace_bytes(m, n) bytes.
size_t stream_workspace_bytes(int64_t m, int64_t n) {
  const int64_t chunks = gemv_t_chunks(m);
  size_t b = 0;
  b += sizeof(float) * (size_t)(m * n);          // R
  b += sizeof(float) * (size_t)(chunks * n);     // partials
  b += sizeof(float) * (size_t)(m + n);          // x, y
  b += sizeof(double) * 4096;                    // norm partials
  b += sizeof(double) * 8;                       // a2, r2, trace state
  b += sizeof(int32_t) * 8;                      // nnz counters
  b += sizeof(long long) * EXTERND_STATS_LEN;    // local stats
  b += sizeof(float) * (size_t)n + sizeof(double) * 8;   // column weights, v^T diag(wt) v
  b += sizeof(double) * 8;                       // safeguard state
  b += sizeof(double) * (size_t)gemv_t_max_partials(m, n);   // single-entry bound partials
  b += 256 * 12;                                 // alignment slack
  return b;
}

static inline char* align_up(char* p, size_t a) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + a - 1) & ~(uintptr_t)(a - 1));
}

hipError_t run_stream_seq(const SeqArgs& a, void* ws, hipStream_t s) {
  const int64_t m = a.m, n = a.n, k = a.k;
  const int64_t wm = (m + 15) / 16, wn = (n + 15) / 16;
  const int64_t chunks = gemv_t_chunks(m);
  char* p = align_up(static_cast<char*>(ws), 256);
  float* R = reinterpret_cast<float*>(p); p = align_up(p + sizeof(float) * m * n, 256);
  float* partial = reinterpret_cast<float*>(p); p = align_up(p + sizeof(float) * chunks * n, 256);
  float* x = reinterpret_cast<float*>(p); p = align_up(p + sizeof(float) * m, 256);
  float* y = reinterpret_cast<float*>(p); p = align_up(p + sizeof(float) * n, 256);
  double* npart = reinterpret_cast<double*>(p); p = align_up(p + sizeof(double) * 4096, 256);
  double* a2 = reinterpret_cast<double*>(p);
  double* r2 = a2 + 1;
  double* tstate = a2 + 2;
  p = align_up(p + sizeof(double) * 8, 256);
  int32_t* nnz_u = reinterpret_cast<int32_t*>(p);
  int32_t* nnz_v = nnz_u + 1;
  p = align_up(p + sizeof(int32_t) * 8, 256);
  long long* st = reinterpret_cast<long long*>(p);
  p = align_up(p + sizeof(long long) * EXTERND_STATS_LEN, 256);
  float* wt = a.importance ? reinterpret_cast<float*>(p) : nullptr;   // column weights (§2.5)
  p = align_up(p + sizeof(float) * n, 256);
  double* sv = a.importance ? reinterpret_cast<double*>(p) : nullptr;  // v^T diag(wt) v
  p = align_up(p + sizeof(double) * 8, 256);
  // the safeguard's state: flag, the fit's decrease, the argmax index, the
  // bound; then the per-wave partial maxima of the single-entry bound
  // (appendix §7) left by each component's first pass
  double* sg_state = reinterpret_cast<double*>(p);
  p = align_up(p + sizeof(double) * 8, 256);
  double* mpart = reinterpret_cast<double*>(p);
  const int64_t nmpart = gemv_t_max_partials(m, n);

  hipError_t e;
  if ((e = launch_fill_i64(reinterpret_cast<long long*>(sg_state), 4, 0, s)) != hipSuccess) return e;
  if ((e = launch_fill_i64(st, EXTERND_STATS_LEN, 0, s)) != hipSuccess) return e;
  if (wt && (e = launch_importance_weights(a.importance, n, a.lambda, wt, st + EXTERND_STAT_NONFINITE, s)) != hipSuccess)
    return e;
  if ((e = launch_norm2(a.A, m * n, npart, 4096, a2, st + EXTERND_STAT_NONFINITE, s, wt, n)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_set_f64, dim3(1), dim3(1), 0, s, tstate, a2);
  if ((e = launch_copy_f32(a.A, R, m * n, s)) != hipSuccess) return e;

  // The deflation of component i-1 is normally fused into component i's first
  // R^T u step; `pending` says whether it still has to be applied.
  bool pending = false;
  for (int64_t i = 0; i < k; ++i) {
    uint32_t* ub = a.B2 + i * wm;
    uint32_t* vc = a.C2 + i * wn;
    const uint32_t* ub_prev = i > 0 ? a.B2 + (i - 1) * wm : nullptr;
    const uint32_t* vc_prev = i > 0 ? a.C2 + (i - 1) * wn : nullptr;
    hipLaunchKernelGGL(k_start_codes, dim3(grid1(wm, 256, 1 << 30)), dim3(256), 0, s, a.seed, i, m, ub);
    const bool cap = (i == a.capture_component);
    if (cap && (a.capture_R || a.capture_Rcol)) {
      if (pending) {
        if ((e = launch_deflate(R, m, n, ub_prev, vc_prev, a.D + i - 1, s)) != hipSuccess) return e;
        pending = false;
      }
      if (a.capture_R && (e = launch_copy_f32(R, a.capture_R, m * n, s)) != hipSuccess) return e;
      if (a.capture_Rcol && (e = launch_copy_f32(R, a.capture_Rcol, m * n, s)) != hipSuccess) return e;
    }
    for (int t = 0; t < a.iters; ++t) {
      const bool fuse = (t == 0 && pending);
      // the first pass (dense u0, every row read) also measures the bound
      e = launch_gemv_t(R, m, n, ub, partial, y, fuse ? a.D + i - 1 : nullptr,
                        fuse ? ub_prev : nullptr, fuse ? vc_prev : nullptr, s, t == 0 ? mpart : nullptr, wt);
      if (e != hipSuccess) return e;
      pending = false;
      e = a.projection ? launch_project(y, n, vc, nnz_v, st + EXTERND_STAT_FALLBACKS, s, wt, sv,
                                        st + EXTERND_STAT_SUM_NNZ_V)
                       : launch_ternarize(y, n, a.tau, vc, nnz_v, st + EXTERND_STAT_FALLBACKS, s, wt, sv,
                                          st + EXTERND_STAT_SUM_NNZ_V);
      if (e != hipSuccess) return e;
      if ((e = launch_gemv_n(R, m, n, vc, x, s, wt)) != hipSuccess) return e;
      e = a.projection ? launch_project(x, m, ub, nnz_u, st + EXTERND_STAT_FALLBACKS, s, nullptr, nullptr,
                                        st + EXTERND_STAT_SUM_NNZ_U)
                       : launch_ternarize(x, m, a.tau, ub, nnz_u, st + EXTERND_STAT_FALLBACKS, s, nullptr, nullptr,
                                          st + EXTERND_STAT_SUM_NNZ_U);
      if (e != hipSuccess) return e;
      if (cap) {
        if (a.capture_y && (e = launch_copy_f32(y, a.capture_y + (int64_t)t * n, n, s)) != hipSuccess) return e;
        if (a.capture_x && (e = launch_copy_f32(x, a.capture_x + (int64_t)t * m, m, s)) != hipSuccess) return e;
        if (a.capture_v) hipLaunchKernelGGL(k_codes_to_i8, dim3(grid1(n, 256, 1 << 30)), dim3(256), 0, s, vc, n, a.capture_v + (int64_t)t * n);
        if (a.capture_u) hipLaunchKernelGGL(k_codes_to_i8, dim3(grid1(m, 256, 1 << 30)), dim3(256), 0, s, ub, m, a.capture_u + (int64_t)t * m);
      }
    }
    hipLaunchKernelGGL(k_scale, dim3(1), dim3(kTernT), 0, s, x, m, ub, nnz_u, nnz_v, a.D, i, tstate,
                       a.trace, st, (const double*)sv, (const double*)mpart, nmpart,
                       a.safeguard ? sg_state : (double*)nullptr);
    if (a.safeguard) {
      hipLaunchKernelGGL(k_safeguard_argmax, dim3(grid1(m * n, 256, 1024)), dim3(256), 0, s, R, m, n,
                         (const float*)wt, sg_state);
      hipLaunchKernelGGL(k_safeguard_apply, dim3(1), dim3(256), 0, s, R, m, n, (const float*)wt, ub, wm, vc, wn,
                         a.D, i, tstate, a.trace, st, nnz_u, nnz_v, sg_state);
    }
    pending = true;
    if (cap && a.capture_d && (e = launch_copy_f32(a.D + i, a.capture_d, 1, s)) != hipSuccess) return e;
    if (cap && a.capture_R_next) {
      if ((e = launch_deflate(R, m, n, ub, vc, a.D + i, s)) != hipSuccess) return e;
      pending = false;
      if ((e = launch_copy_f32(R, a.capture_R_next, m * n, s)) != hipSuccess) return e;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // Deflate the last component and measure the final residual.
  if (pending) {
    if ((e = launch_deflate(R, m, n, a.B2 + (k - 1) * wm, a.C2 + (k - 1) * wn, a.D + k - 1, s)) != hipSuccess) return e;
  }
  if ((e = launch_norm2(R, m * n, npart, 4096, r2, nullptr, s, wt, n)) != hipSuccess) return e;
  if ((e = launch_energy_finish(a2, r2, st + EXTERND_STAT_NONFINITE, a.energy, s)) != hipSuccess) return e;
  if (a.norm_a2 && (e = launch_copy_f64(a2, a.norm_a2, 1, s)) != hipSuccess) return e;
  if (a.stats) {
    // the streaming path runs every iteration of every component
    if ((e = launch_fill_i64(st + EXTERND_STAT_ITERATIONS, 1, (long long)(k * a.iters), s)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_copy_i64, dim3(1), dim3(64), 0, s, st, a.stats, (int64_t)EXTERND_STATS_LEN);
  }
  return hipGetLastError();
}

}  // namespace externd
