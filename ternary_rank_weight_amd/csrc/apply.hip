// Inference with the 2-bit factors (ExTernD §2.6): y = B (diag(D) (C x)).
// C x and B w are multiplication-free: each is a sum of signed copies of x
// (or of the scaled components w), so the kernels only read the packed codes
// once and add or subtract.  k multiplies (w = D * C x) remain.  All sums are
// fp32 in a fixed order, so repeated calls give identical bits.
//
// Step 1 (k_apply_cx): w[i] = D[i] * sum_j C[i][j] x[j].  Each wave takes
//   16 code rows (4 when k is small, for more workgroups); per step lane l reads word q0 + l of every row (coalesced)
//   and the 16 x values of that word once, for all 16 rows; a DPP reduction
//   combines the lanes.  Each element costs a 2-bit sign extension, a
//   conversion and an FMA by -1, 0 or +1, which is exact.
// Step 2 (k_apply_bw): partial sums of y over chunks of components (sized
//   for about 1024 workgroups).  A workgroup takes 64 code words (component-major B2: row i,
//   word q holds rows 16q .. 16q+15 of column i of B) of one chunk; four
//   threads share each word, each summing a quarter of the chunk into 16 row
//   accumulators, and the quarters are combined in order through LDS.
// Step 3 (k_apply_sum): y[r] = sum over chunks, in chunk order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace externd {

namespace {

constexpr int kApplyT = 256;
constexpr int kApplyMaxChunk = 4096;   // components per partial sum of y, at most
constexpr int kApplyMinChunk = 256;    // and at least (bounds the number of partial sums)
constexpr int kApplySub = 4;       // threads sharing one code word, each a quarter of the chunk
constexpr int kApplyBigK = 16384;   // from this many components on, 16 code rows per wave (else 4)

inline unsigned grid1d(int64_t count, int threads, int64_t cap = 8192) {
  const int64_t g = (count + threads - 1) / threads;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

// Ternary value of code c (2 bits at bit offset sh): a signed 2-bit field
// extract maps 00 -> 0, 01 -> +1, 11 -> -1.
__device__ inline float tval(uint32_t word, int sh) {
  return (float)((int)(word << (30 - sh)) >> 30);
}

template <int kApplyRowsPerWave>
__global__ __launch_bounds__(kApplyT) void k_apply_cx(const uint32_t* __restrict__ C2,
                                                      const float* __restrict__ D, int64_t n, int64_t k,
                                                      const float* __restrict__ x, float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wn = (n + 15) / 16;
  const int64_t row0 = ((int64_t)blockIdx.x * (kApplyT / kWave) + threadIdx.x / kWave) * kApplyRowsPerWave;
  float acc[kApplyRowsPerWave];
#pragma unroll
  for (int r = 0; r < kApplyRowsPerWave; ++r) acc[r] = 0.f;
  for (int64_t q0 = 0; q0 < wn; q0 += kWave) {
    const int64_t q = q0 + lane;            // this lane's code word: columns 16q .. 16q+15
    float xv[16];
    if (q < wn && 16 * q + 16 <= n) {
      const float4* xp = reinterpret_cast<const float4*>(x + 16 * q);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 f = xp[v];
        xv[4 * v] = f.x; xv[4 * v + 1] = f.y; xv[4 * v + 2] = f.z; xv[4 * v + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) xv[e] = (q < wn && 16 * q + e < n) ? x[16 * q + e] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kApplyRowsPerWave; ++r) {
      const int64_t i = row0 + r;
      const uint32_t word = (q < wn && i < k) ? C2[i * wn + q] : 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r] = fmaf(tval(word, 2 * e), xv[e], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kApplyRowsPerWave; ++r) {
    const float sum = wave_sum_to63(acc[r]);
    const int64_t i = row0 + r;
    if (lane == kWave - 1 && i < k) w[i] = sum * D[i];
  }
}

__global__ __launch_bounds__(kApplyT) void k_apply_bw(const uint32_t* __restrict__ B2,
                                                      const float* __restrict__ w, int64_t m, int64_t k,
                                                      int chunk_len, float* __restrict__ ypart) {
  constexpr int kCols = kApplyT / kApplySub;           // code words per workgroup
  extern __shared__ float ws[];                         // chunk_len scales
  __shared__ float red[kApplySub - 1][kCols * 16];
  const int64_t wm = (m + 15) / 16;
  const int64_t chunk = blockIdx.y;
  const int64_t i0 = chunk * chunk_len;
  const int64_t nc = min<int64_t>(chunk_len, k - i0);
  for (int e = threadIdx.x; e < chunk_len; e += kApplyT) ws[e] = e < nc ? w[i0 + e] : 0.f;
  __syncthreads();
  const int per_sub = chunk_len / kApplySub;
  const int col = threadIdx.x % kCols, sub = threadIdx.x / kCols;
  const int64_t q = (int64_t)blockIdx.x * kCols + col;   // code word (16 rows)
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  if (q < wm) {
    const int64_t ib = (int64_t)sub * per_sub, ie = min<int64_t>(nc, ib + per_sub);
    const uint32_t* colp = B2 + (i0 + ib) * wm + q;
    int64_t i = ib;
    for (; i + 8 <= ie; i += 8, colp += 8 * wm) {   // eight code loads in flight
      uint32_t words[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) words[u] = colp[u * wm];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wi = ws[i + u];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = fmaf(tval(words[u], 2 * e), wi, acc[e]);
      }
    }
    for (; i < ie; ++i, colp += wm) {
      const uint32_t word = *colp;
      const float wi = ws[i];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = fmaf(tval(word, 2 * e), wi, acc[e]);
    }
  }
  // combine the sub-chunks in order 0, 1, 2, 3
  if (sub > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[sub - 1][col * 16 + e] = acc[e];
  }
  __syncthreads();
  if (sub == 0 && q < wm) {
    float* out = ypart + chunk * (wm * 16) + q * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float sum = acc[e];
#pragma unroll
      for (int u = 0; u < kApplySub - 1; ++u) sum += red[u][col * 16 + e];
      out[e] = sum;
    }
  }
}

__global__ void k_apply_sum(const float* __restrict__ ypart, int64_t m, int64_t nchunks, float* __restrict__ y) {
  const int64_t stride = ((m + 15) / 16) * 16;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < m; r += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int64_t c = 0; c < nchunks; ++c) s += ypart[c * stride + r];
    y[r] = s;
  }
}

}  // namespace

// Components per partial sum of y: enough chunks for about 1024 workgroups
// in step 2, a multiple of kApplySub, between kApplyMinChunk and
// kApplyMaxChunk.
static int apply_chunk(int64_t m, int64_t k) {
  const int64_t wm = (m + 15) / 16;
  const int64_t xwg = (wm + kApplyT / kApplySub - 1) / (kApplyT / kApplySub);
  const int64_t target = std::max<int64_t>(1, 1024 / xwg);
  int64_t c = (k + target - 1) / target;
  c = (c + kApplySub - 1) / kApplySub * kApplySub;
  return (int)std::max<int64_t>(kApplyMinChunk, std::min<int64_t>(kApplyMaxChunk, c));
}

size_t apply_workspace_bytes(int64_t m, int64_t k) {
  const int64_t nchunks = k > 0 ? (k + apply_chunk(m, k) - 1) / apply_chunk(m, k) : 0;
  return sizeof(float) * (size_t)k + 256 + sizeof(float) * (size_t)nchunks * (size_t)(((m + 15) / 16) * 16) + 256;
}

hipError_t run_apply(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m, int64_t n, int64_t k,
                     const float* x, float* y, void* ws, hipStream_t s) {
  if (k == 0) {
    hipLaunchKernelGGL(k_apply_sum, dim3(grid1d(m, 256)), dim3(256), 0, s, (const float*)nullptr, m, (int64_t)0, y);
    return hipGetLastError();
  }
  char* p = static_cast<char*>(ws);
  float* w = reinterpret_cast<float*>(p);
  p += ((sizeof(float) * (size_t)k + 255) / 256) * 256;
  float* ypart = reinterpret_cast<float*>(p);
  const int64_t wm = (m + 15) / 16;
  const int chunk = apply_chunk(m, k);
  const int64_t nchunks = (k + chunk - 1) / chunk;
  constexpr int kCols = kApplyT / kApplySub;
  if (k >= kApplyBigK) {
    constexpr int rows = 16 * (kApplyT / kWave);
    hipLaunchKernelGGL(k_apply_cx<16>, dim3((unsigned)((k + rows - 1) / rows)), dim3(kApplyT), 0, s, C2, D, n, k, x, w);
  } else {
    constexpr int rows = 4 * (kApplyT / kWave);
    hipLaunchKernelGGL(k_apply_cx<4>, dim3((unsigned)((k + rows - 1) / rows)), dim3(kApplyT), 0, s, C2, D, n, k, x, w);
  }
  hipLaunchKernelGGL(k_apply_bw, dim3((unsigned)((wm + kCols - 1) / kCols), (unsigned)nchunks), dim3(kApplyT),
                     sizeof(float) * (size_t)chunk, s, B2, w, m, k, chunk, ypart);
  hipLaunchKernelGGL(k_apply_sum, dim3(grid1d(m, 256)), dim3(256), 0, s, ypart, m, nchunks, y);
  return hipGetLastError();
}

}  // namespace externd
