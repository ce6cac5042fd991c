// Reconstruction A_hat = B diag(D) C and the energy metric from 2-bit factors
// (ExTernD §2.1: E = 1 - ||A - A_hat||_F^2 / ||A||_F^2).  Each entry of A_hat
// is accumulated in fp64 over all k components.
#include "device_common.hpp"
#include "kernels.hpp"

namespace externd {

namespace {

constexpr int kTile = 64;     // output tile edge
constexpr int kRT = 256;      // threads per tile: 16 x 16, each 4 x 4 entries
constexpr int kChunk = 64;    // components staged in LDS at a time

// Accumulate a 64 x 64 tile of B diag(D) C in fp64.  acc[a][b] is entry
// (r0 + 4*ty + a, c0 + 4*tx + b).
__device__ inline void tile_accumulate(const uint32_t* __restrict__ B2, const uint32_t* __restrict__ C2,
                                       const float* __restrict__ D, int64_t m, int64_t n, int64_t k,
                                       int64_t r0, int64_t c0, double (&acc)[4][4],
                                       uint32_t (*bw)[4], uint32_t (*cw)[4], double* dv) {
  const int t = threadIdx.x;
  const int ty = t / 16, tx = t % 16;
  const int64_t wm = (m + 15) / 16, wn = (n + 15) / 16;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t i0 = 0; i0 < k; i0 += kChunk) {
    __syncthreads();
    {
      // 64 components x 4 words each for B (rows) and C (columns)
      const int ci = t / 4, q = t % 4;
      const int64_t i = i0 + ci;
      const int64_t wb = r0 / 16 + q, wc = c0 / 16 + q;
      bw[ci][q] = (i < k && wb < wm) ? B2[i * wm + wb] : 0u;
      cw[ci][q] = (i < k && wc < wn) ? C2[i * wn + wc] : 0u;
      if (q == 0) dv[ci] = i < k ? (double)D[i] : 0.0;
    }
    __syncthreads();
    const int rsh = 2 * ((4 * ty) % 16), csh = 2 * ((4 * tx) % 16);
    const int rq = (4 * ty) / 16, cq = (4 * tx) / 16;
    const int64_t cnt = min<int64_t>(kChunk, k - i0);
    for (int ci = 0; ci < cnt; ++ci) {
      const uint32_t bbits = bw[ci][rq] >> rsh;
      const uint32_t cbits = cw[ci][cq] >> csh;
      if ((bbits & 0xffu) == 0u || (cbits & 0xffu) == 0u) continue;
      const double d = dv[ci];
      double bv[4], cv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) bv[a] = d * (double)value_of_code((bbits >> (2 * a)) & 3u);
#pragma unroll
      for (int b = 0; b < 4; ++b) cv[b] = (double)value_of_code((cbits >> (2 * b)) & 3u);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(bv[a], cv[b], acc[a][b]);
    }
  }
}

__global__ __launch_bounds__(kRT) void k_reconstruct(const uint32_t* __restrict__ B2,
                                                     const uint32_t* __restrict__ C2,
                                                     const float* __restrict__ D, int64_t m,
                                                     int64_t n, int64_t k, float* __restrict__ out) {
  __shared__ uint32_t bw[kChunk][4];
  __shared__ uint32_t cw[kChunk][4];
  __shared__ double dv[kChunk];
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  double acc[4][4];
  tile_accumulate(B2, C2, D, m, n, k, r0, c0, acc, bw, cw, dv);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t r = r0 + 4 * ty + a, c = c0 + 4 * tx + b;
      if (r < m && c < n) out[r * n + c] = (float)acc[a][b];
    }
}

__global__ __launch_bounds__(kRT) void k_energy_tiles(const float* __restrict__ A,
                                                      const uint32_t* __restrict__ B2,
                                                      const uint32_t* __restrict__ C2,
                                                      const float* __restrict__ D, int64_t m,
                                                      int64_t n, int64_t k,
                                                      double* __restrict__ partial) {
  __shared__ uint32_t bw[kChunk][4];
  __shared__ uint32_t cw[kChunk][4];
  __shared__ double dv[kChunk];
  __shared__ double scratch[kRT / kWave];
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  double acc[4][4];
  tile_accumulate(B2, C2, D, m, n, k, r0, c0, acc, bw, cw, dv);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  double s = 0.0;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t r = r0 + 4 * ty + a, c = c0 + 4 * tx + b;
      if (r < m && c < n) {
        const double e = (double)A[r * n + c] - acc[a][b];
        s += e * e;
      }
    }
  s = block_sum<kRT>(s, scratch);
  if (threadIdx.x == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = s;
}

__global__ void k_energy_final(const double* __restrict__ partial, int64_t count,
                               const double* __restrict__ a2, double* __restrict__ energy) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double s = 0.0;
  for (int64_t i = 0; i < count; ++i) s += partial[i];
  *energy = (*a2 == 0.0) ? 1.0 : 1.0 - s / *a2;
}

}  // namespace

size_t energy_workspace_bytes(int64_t m, int64_t n) {
  const int64_t tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  return sizeof(double) * (size_t)(tiles + 4096 + 8) + 512;
}

hipError_t run_energy(const float* A, int64_t m, int64_t n, const uint32_t* B2, const uint32_t* C2,
                      const float* D, int64_t k, double* energy, void* ws, hipStream_t s) {
  char* p = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  const int64_t tx = (n + kTile - 1) / kTile, ty = (m + kTile - 1) / kTile;
  double* partial = reinterpret_cast<double*>(p);
  double* npart = partial + tx * ty;
  double* a2 = npart + 4096;
  hipError_t e = launch_norm2(A, m * n, npart, 4096, a2, nullptr, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_energy_tiles, dim3((unsigned)tx, (unsigned)ty), dim3(kRT), 0, s, A, B2, C2, D,
                     m, n, k, partial);
  hipLaunchKernelGGL(k_energy_final, dim3(1), dim3(64), 0, s, partial, tx * ty, a2, energy);
  return hipGetLastError();
}

hipError_t run_reconstruct(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m,
                           int64_t n, int64_t k, float* out, hipStream_t s) {
  const int64_t tx = (n + kTile - 1) / kTile, ty = (m + kTile - 1) / kTile;
  hipLaunchKernelGGL(k_reconstruct, dim3((unsigned)tx, (unsigned)ty), dim3(kRT), 0, s, B2, C2, D, m,
                     n, k, out);
  return hipGetLastError();
}

}  // namespace externd
