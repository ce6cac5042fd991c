// Grid-wide exchange and distributed T_tau, shared by the persistent
// sequential kernels (resident and streaming).
//
// A vector of length N is distributed over a workgroup of T threads as
// val[j] = x[t + T j].  After a half-step every workgroup publishes the
// entries it finished as 32-bit words whose lowest bit is replaced by the
// parity of the round (agent-scope relaxed atomic stores), each word in kRep
// replicas; every workgroup then gathers all N words of its replica, polling
// until each carries the current parity, and applies T_tau (§2.2)
// redundantly and identically.  A word is never overwritten with the next
// round of the same parity before every workgroup has read it, because
// nobody publishes round r+1 before it has gathered all of round r.
#pragma once
#include "device_common.hpp"

namespace externd {
namespace xchg {

constexpr unsigned kSpinLimit = 1u << 21;
constexpr int kRep = 4;   // replicas of every exchange word
// words between replicas of a length-len slot array: a whole number of 4 KB
__host__ __device__ inline int rep_stride(int len) { return (len + 1023) / 1024 * 1024; }
// the replica workgroup g reads: one per pair of XCDs (round-robin dispatch)
__device__ inline int rep_of(int g) { return (g & 7) >> 1; }

// The thread index through an empty asm statement: index arithmetic built
// from it inside a loop body stays there instead of being hoisted out of the
// loop and kept live (or spilled to scratch) across the whole loop.
__device__ inline int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Exchange word: the value with its lowest bit replaced by the round parity.
__device__ inline unsigned xw_pack(unsigned round, float v) {
  return (__float_as_uint(v) & ~1u) | (round & 1u);
}
__device__ inline float xw_value(unsigned w) { return __uint_as_float(w & ~1u); }

// Sum acc[l] over the T threads for l < L (DPP inside each wave, then the
// waves in index order) and publish output l < nvalid as slot[base + l] in
// each of the kRep replicas, rstride words apart.
template <int T, int L>
__device__ inline void reduce_publish(const float (&acc)[L], float* red, int nvalid,
                                      unsigned* slot, int base, unsigned round, int rstride) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
  float sums[L];
#pragma unroll
  for (int l = 0; l < L; ++l) sums[l] = wave_sum_to63(acc[l]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int l = 0; l < L; ++l) red[w * L + l] = sums[l];
  }
  __syncthreads();
  if (t < nvalid) {
    float s = red[t];
#pragma unroll
    for (int q = 1; q < T / kWave; ++q) s += red[q * L + t];
    const unsigned word = xw_pack(round, s);
#pragma unroll
    for (int r = 0; r < kRep; ++r)
      __hip_atomic_store(slot + r * rstride + base + t, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Block reductions with one barrier each.  buf is double[T/64][4]; two
// consecutive reductions must use different buffers.
template <int T, int NV>
__device__ inline void block_sum_f64(double (&v)[NV], double (*buf)[4]) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const double s = wave_sum_to63(v[i]);
    if (lane == kWave - 1) buf[w][i] = s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    double r = buf[0][i];
#pragma unroll
    for (int q = 1; q < T / kWave; ++q) r += buf[q][i];
    v[i] = r;
  }
}
template <int T>
__device__ inline int block_min_idx(int v, double (*buf)[4]) {
  const int t = threadIdx.x;
  const int w = t / kWave;
  v = wave_min_i(v);
  if ((t & (kWave - 1)) == 0) buf[w][0] = (double)v;
  __syncthreads();
  int r = INT32_MAX;
#pragma unroll
  for (int q = 0; q < T / kWave; ++q) r = min(r, (int)buf[q][0]);
  return r;
}

// Morton spread of 16 bits: bit e -> bit 2e.
__device__ inline uint32_t spread16(uint32_t x) {
  x &= 0xffffu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  x = (x | (x << 1)) & 0x55555555u;
  return x;
}

// Write the 2-bit codes of a distributed ternary vector val[j] = t[tid + T*j]
// (length N) into dst[0 .. ceil(N/16)); workgroup g of G writes the words
// w with w % G == g.  Uses wave ballots, no LDS and no barrier.
template <int T, int K>
__device__ inline void store_codes(const float (&val)[K], int N, uint32_t* dst, int g, int G, int tid = -1) {
  const int t = tid >= 0 ? tid : (int)threadIdx.x;
  const int lane = t & (kWave - 1);
  const int words = (N + 15) / 16;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const unsigned long long nz = __ballot(val[j] != 0.f);
    const unsigned long long ng = __ballot(val[j] < 0.f);
    const int row_base = (t & ~(kWave - 1)) + T * j;
    if (lane < 4) {
      const int w = (row_base >> 4) + lane;
      if (w < words && w % G == g) {
        const uint32_t a = (uint32_t)(nz >> (16 * lane)) & 0xffffu;
        const uint32_t b = (uint32_t)(ng >> (16 * lane)) & 0xffffu;
        dst[w] = spread16(a) | (spread16(b) << 1);
      }
    }
  }
}

// Read the n (or m) published words of the current round into val[j] for
// index t + T*j.  Returns false if a wait ran out.  tid: the thread index,
// when the caller has one of its own (opaque_tid).
template <int T, int K>
__device__ inline bool gather(const unsigned* slot, int N, unsigned round, float (&val)[K],
                              const unsigned* err, int tid = -1) {
  const int t = tid >= 0 ? tid : (int)threadIdx.x;
  const unsigned par = round & 1u;
  unsigned w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const unsigned idx = (unsigned)(t + T * j);
    w[j] = idx < (unsigned)N ? __hip_atomic_load(slot + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : par;
  }
  unsigned spins = 0;
  bool ok = true;
  while (true) {
    bool all = true;
#pragma unroll
    for (int j = 0; j < K; ++j) all = all && (w[j] & 1u) == par;
    if (all) break;
    if (++spins > kSpinLimit) { ok = false; break; }
    if ((spins & 255u) == 0 &&
        __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
      ok = false;
      break;
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const unsigned idx = (unsigned)(t + T * j);
      if ((w[j] & 1u) != par)
        w[j] = __hip_atomic_load(slot + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) val[j] = ok ? xw_value(w[j]) : 0.f;
  return ok;
}

// T_tau (§2.2) of a vector distributed as val[j] = x[t + T*j] (zeros beyond
// N), identical in every workgroup.  `bad` folds a failed gather into the
// first reduction: if any thread of the block has it set, returns false and
// the caller leaves.  Writes T_tau(x) to out in the same layout; cnt gets
// this thread's nonzeros, fallback whether the largest-entry rule applied.
// The block reductions are LDS atomics, one per wave after its DPP
// reduction: the maximum magnitude's bits (a failed gather adds
// 0xffffffff, above every finite magnitude) and the fixed-point sum, whose
// terms are integers with a total below 2^52, so the order of the adds
// cannot change it.  The sum is formed before the first barrier, at the
// shift of a guessed exponent eg of max|x| (block-uniform; the caller
// keeps one guess per kind of vector).  When the true exponent equals eg the
// sum is the one the plain rule forms (the same shift, the same integers) and
// one barrier serves both reductions; otherwise the sum is formed again at
// the true shift after a second barrier.  eg is replaced by the true
// exponent.  Slots (LDS, clear at the caller's first barrier): slot[0..1]
// the guessed-shift sums and the low words of slot[2..3] the maxima, both
// taken by the parity of the call count `par` (the caller's count of calls,
// +1 per call); slot[4] the second sum.  On entry thread 0 clears the other
// parity's slots and slot[4]: every thread read them before the barrier
// that separates two calls, which the caller keeps.  bufs[0] serves the
// fallback's argmin.
template <int T, int K>
__device__ inline bool ternarize_dist_guess(const float (&val)[K], bool bad, int N, float tau,
                                            float (&out)[K], double (*bufs)[T / kWave][4], double* slot,
                                            unsigned par, int& eg, int& cnt, int& fallback, int tid = -1) {
  const int t = tid >= 0 ? tid : (int)threadIdx.x;
  const int lane = t & (kWave - 1);
  const unsigned p = par & 1u;
  double* const gsum = slot + p;
  unsigned* const mslot = reinterpret_cast<unsigned*>(slot + 2 + p);
  if (t == 0) {
    slot[p ^ 1u] = 0.0;
    *reinterpret_cast<unsigned*>(slot + 2 + (p ^ 1u)) = 0u;
    slot[4] = 0.0;
  }
  const int L = ceil_log2_i32(N);
  const int sg = 52 - eg - L;
  uint32_t ab[K];
  uint32_t mx = 0u;
  double qs = 0.0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    ab[j] = __float_as_uint(val[j]) & 0x7fffffffu;
    mx = max(mx, ab[j]);
    qs += fixed_point_q(__uint_as_float(ab[j]), sg);
  }
  if (bad) mx = 0xffffffffu;
  const uint32_t mw = wave_umax_to63(mx);
  const double qw = wave_sum_to63(qs);
  if (lane == kWave - 1) {
    atomicMax(mslot, mw);
    atomicAdd(gsum, qw);
  }
  __syncthreads();
  const uint32_t Mb = *mslot;
  if (Mb == 0xffffffffu) return false;
  cnt = 0;
  if (Mb == 0u) {
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = (t + T * j == 0) ? 1.f : 0.f;
    fallback = 1;
    cnt = t == 0 ? 1 : 0;
    return true;
  }
  int e;
  (void)frexp((double)__uint_as_float(Mb), &e);
  e = __builtin_amdgcn_readfirstlane(e);
  const int s = 52 - e - L;
  double S;
  if (e == eg) {
    S = *gsum;
  } else {
    double q2 = 0.0;
#pragma unroll
    for (int j = 0; j < K; ++j) q2 += fixed_point_q(__uint_as_float(ab[j]), s);
    const double q2w = wave_sum_to63(q2);
    if (lane == kWave - 1) atomicAdd(slot + 4, q2w);
    __syncthreads();
    S = slot[4];
  }
  eg = e;
  const double thr = fixed_point_threshold(S, s, tau, N);
  const uint32_t tb = threshold_bits(thr);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const bool keep = ab[j] > tb;
    out[j] = keep ? (val[j] > 0.f ? 1.f : -1.f) : 0.f;
    cnt += keep ? 1 : 0;
  }
  fallback = 0;
  if (Mb > tb) return true;
  int first = INT32_MAX;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int idx = t + T * j;
    if (idx < N && ab[j] == Mb) first = min(first, idx);
  }
  const int pick = block_min_idx<T>(first, bufs[0]);
  cnt = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (t + T * j == pick) {
      out[j] = val[j] > 0.f ? 1.f : -1.f;
      cnt = 1;
    }
  }
  fallback = 1;
  return true;
}

}  // namespace xchg
}  // namespace externd
