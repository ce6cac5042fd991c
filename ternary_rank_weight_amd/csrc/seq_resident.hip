// Resident sequential path: one cooperative kernel runs every component and
// every alternating iteration of the greedy ALS (ExTernD §2.3) with the
// residual R held on chip for the whole decomposition.
//
// Layout.  Workgroup g of G owns
//   * the row block  rows [g*RB, g*RB+RB) x all n columns, kept in LDS, used
//     for x = R v (each workgroup finishes its rows' dot products locally);
//   * the column block  all m rows x columns [g*CB, g*CB+CB), kept in VGPRs,
//     used for y = R^T u (each workgroup finishes its columns locally).
// Both copies receive the same fp32 deflation R <- fl32(R - d u v^T), so they
// stay bit-identical.  Thread t holds entries of index t + T*j of every
// length-m or length-n vector, which is exactly the set of rows (column copy)
// and columns (row copy) it multiplies, so the vectors never move through LDS.
//
// Exchange.  After a half-step every workgroup publishes its finished outputs
// (RB values of x or CB values of y) as 32-bit words whose lowest bit is
// replaced by the parity of the round (the value keeps 31 bits: at most one
// unit in the last place, always toward zero once the reader clears the bit),
// written with agent-scope atomic stores.  It then reads all m (or n) words
// with agent-scope atomic loads until each carries the current parity.  A
// word cannot be overwritten with the next round of the same parity before
// every workgroup has read it, because nobody publishes round r+1 before it
// has gathered all of round r; coherence of the single word then rules out
// reading a value two rounds old.  Value and tag share one atomic word, so no
// fence or grid barrier is needed: one exchange per half-step, two per ALS
// iteration.  Every workgroup then holds the whole vector (the same bits in
// every workgroup) and applies T_tau (§2.2) redundantly and identically.
//
// Termination.  Every wait is bounded: a workgroup that waits too long sets a
// device error flag and the whole grid returns; the host reports EHIP.
#include "device_common.hpp"
#include "kernels.hpp"

namespace externd {

namespace {

constexpr unsigned kSpinLimit = 1u << 21;

struct ResArgs {
  const float* A;
  int m, n, k;
  float tau;
  int iters;
  uint64_t seed;
  int G, RB, CB;
  uint32_t* B2;
  uint32_t* C2;
  float* D;
  double* trace;
  long long* stats;            // EXTERND_STATS_LEN, written by workgroup 0
  const double* a2;            // ||A||^2 (weighted when wt is set)
  const float* wt;             // optional column weights (§2.5), n floats
  const long long* nonfinite;  // count of non-finite entries of A
  unsigned* yslot;             // n words
  unsigned* xslot;             // m words
  unsigned* err;
  double* r2_partial;          // G fp64
  int64_t cap_i;
  float* cap_R;
  float* cap_Rcol;
  float* cap_R_next;
  float* cap_y;
  float* cap_x;
  int8_t* cap_v;
  int8_t* cap_u;
  float* cap_d;
};

// Exchange word: the value with its lowest bit replaced by the round parity.
__device__ inline unsigned xw_pack(unsigned round, float v) {
  return (__float_as_uint(v) & ~1u) | (round & 1u);
}
__device__ inline float xw_value(unsigned w) { return __uint_as_float(w & ~1u); }

// Sum acc[l] over the T threads for l < L (DPP inside each wave, then the
// waves in index order) and publish output l < nvalid as slot[base + l].
template <int T, int L>
__device__ inline void reduce_publish(const float (&acc)[L], float* red, int nvalid,
                                      unsigned* slot, int base, unsigned round) {
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
    __hip_atomic_store(slot + base + t, xw_pack(round, s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Block reductions with one barrier each.  buf is double[T/64][4]; two
// consecutive reductions must use different buffers.
template <int T>
__device__ inline uint32_t block_umax_flag(uint32_t v, bool bad, double (*buf)[4], bool& any_bad) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
  const uint32_t mw = wave_umax_to63(v);
  const bool bw = __any(bad);
  if (lane == kWave - 1) {
    buf[w][0] = (double)mw;
    buf[w][1] = bw ? 1.0 : 0.0;
  }
  __syncthreads();
  uint32_t r = 0u;
  bool b = false;
#pragma unroll
  for (int q = 0; q < T / kWave; ++q) {
    r = max(r, (uint32_t)buf[q][0]);
    b = b || buf[q][1] != 0.0;
  }
  any_bad = b;
  return r;
}
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
__device__ inline void store_codes(const float (&val)[K], int N, uint32_t* dst, int g, int G) {
  const int t = threadIdx.x;
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
// index t + T*j.  Returns false if a wait ran out.
template <int T, int K>
__device__ inline bool gather(const unsigned* slot, int N, unsigned round, float (&val)[K],
                              const unsigned* err) {
  const int t = threadIdx.x;
  const unsigned par = round & 1u;
  unsigned w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int idx = t + T * j;
    w[j] = idx < N ? __hip_atomic_load(slot + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : par;
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
      const int idx = t + T * j;
      if ((w[j] & 1u) != par)
        w[j] = __hip_atomic_load(slot + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) val[j] = ok ? xw_value(w[j]) : 0.f;
  return ok;
}

// T_tau (§2.2) of a vector distributed as val[j] = x[t + T*j] (zeros beyond N),
// identical in every workgroup.  `bad` folds a failed gather into the first
// reduction: if any thread of the block has it set, returns false and the
// caller leaves.  bufs[0..1] are used alternately (see block_umax_flag).
// Writes T_tau(x) to out in the same layout; cnt gets this thread's nonzeros.
template <int T, int K>
__device__ inline bool ternarize_dist(const float (&val)[K], bool bad, int N, float tau,
                                      float (&out)[K], double (*bufs)[T / kWave][4], int& cnt,
                                      int& fallback) {
  const int t = threadIdx.x;
  uint32_t ab[K];
  uint32_t mx = 0u;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    ab[j] = __float_as_uint(val[j]) & 0x7fffffffu;
    mx = max(mx, ab[j]);
  }
  bool any_bad;
  const uint32_t Mb = block_umax_flag<T>(mx, bad, bufs[0], any_bad);
  if (any_bad) return false;
  cnt = 0;
  if (Mb == 0u) {
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = (t + T * j == 0) ? 1.f : 0.f;
    fallback = 1;
    cnt = t == 0 ? 1 : 0;
    return true;
  }
  const int s = fixed_point_shift(__uint_as_float(Mb), N);
  // Every partial sum is an integer below 2^52, so the fp64 sums are exact.
  double qs[1] = {0.0};
#pragma unroll
  for (int j = 0; j < K; ++j) qs[0] += fixed_point_q(__uint_as_float(ab[j]), s);
  block_sum_f64<T, 1>(qs, bufs[1]);
  const double thr = fixed_point_threshold(qs[0], s, tau, N);
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

// Copy this workgroup's rows of the row-resident residual to dst (m x n).
template <int T, int KR, int LR>
__device__ void dump_rows(const float* rrow, const ResArgs& a, int row0, float* dst) {
  const int t = threadIdx.x;
  for (int l = 0; l < LR; ++l)
    for (int j = 0; j < KR; ++j) {
      const int row = row0 + l, col = t + T * j;
      if (l < a.RB && row < a.m && col < a.n) dst[(int64_t)row * a.n + col] = rrow[(l * KR + j) * T + t];
    }
}

// CAP selects the test-capture instantiation: the same arithmetic plus stores
// of one component's intermediate vectors and residuals.
template <int T, int KR, int LR, int KC, int LC, bool CAP>
__global__ __launch_bounds__(T) void k_seq_resident(ResArgs a) {
  constexpr int W = T / kWave;
  constexpr int LMAX = LR > LC ? LR : LC;
  __shared__ float rrow[LR * KR * T];
  __shared__ float red[W * LMAX];
  __shared__ float u_own[LR];
  __shared__ float v_own[LC];
  __shared__ double bufs[3][W][4];

  const int t = threadIdx.x;
  const int g = blockIdx.x;
  const int m = a.m, n = a.n;
  const int row0 = g * a.RB, col0 = g * a.CB;
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;

  if (*a.nonfinite > 0) {
    // Nothing sensible can be computed: zero this workgroup's share of the outputs.
    for (int64_t w = (int64_t)g * T + t; w < (int64_t)a.k * wm; w += (int64_t)a.G * T) a.B2[w] = 0u;
    for (int64_t w = (int64_t)g * T + t; w < (int64_t)a.k * wn; w += (int64_t)a.G * T) a.C2[w] = 0u;
    for (int64_t w = (int64_t)g * T + t; w < a.k; w += (int64_t)a.G * T) a.D[w] = 0.f;
    if (t == 0) a.r2_partial[g] = 0.0;
    return;
  }

  // R <- A into both copies.
#pragma unroll
  for (int l = 0; l < LR; ++l) {
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int row = row0 + l, col = t + T * j;
      rrow[(l * KR + j) * T + t] =
          (l < a.RB && row < m && col < n) ? a.A[(int64_t)row * n + col] : 0.f;
    }
  }
  float rc[LC][KC];
#pragma unroll
  for (int l = 0; l < LC; ++l) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int col = col0 + l, row = t + T * j;
      rc[l][j] = (l < a.CB && col < n && row < m) ? a.A[(int64_t)row * n + col] : 0.f;
    }
  }
  __syncthreads();

  float u[KC], v[KR];
#pragma unroll
  for (int j = 0; j < KC; ++j) u[j] = 0.f;
#pragma unroll
  for (int j = 0; j < KR; ++j) v[j] = 0.f;
  // column weights of this thread's columns (§2.5); exactly 1 when unweighted,
  // which leaves every product and sum below unchanged
  float wv[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    const int col = t + T * j;
    wv[j] = (a.wt && col < n) ? a.wt[col] : 1.f;
  }
  float d32 = 0.f;
  unsigned ry = 0, rx = 0;
  long long st_nnz_u = 0, st_nnz_v = 0, st_fb = 0, st_b = 0, st_c = 0;
  double trace_state = *a.a2;
  const bool capturer = (g == 0);

  for (int i = 0; i <= a.k; ++i) {
    // ---- deflate component i-1 out of both copies (§2.3 step 3) ----
    if (i > 0) {
#pragma unroll
      for (int l = 0; l < LR; ++l) {
        const float ul = (l < a.RB && row0 + l < m) ? u_own[l] : 0.f;
        if (ul != 0.f) {
          float* rp = rrow + l * KR * T + t;
#pragma unroll
          for (int j = 0; j < KR; ++j) rp[j * T] = fmaf(-d32, ul * v[j], rp[j * T]);
        }
      }
#pragma unroll
      for (int l = 0; l < LC; ++l) {
        const float vl = (l < a.CB && col0 + l < n) ? v_own[l] : 0.f;
        if (vl != 0.f) {
#pragma unroll
          for (int j = 0; j < KC; ++j) rc[l][j] = fmaf(-d32, u[j] * vl, rc[l][j]);
        }
      }
      if constexpr (CAP) {
        if (i - 1 == a.cap_i && a.cap_R_next) dump_rows<T, KR, LR>(rrow, a, row0, a.cap_R_next);
      }
    }
    if (i == a.k) break;
    if (CAP && i == a.cap_i) {
      if (a.cap_R) dump_rows<T, KR, LR>(rrow, a, row0, a.cap_R);
      if (a.cap_Rcol) {
        for (int l = 0; l < LC; ++l)
#pragma unroll
          for (int j = 0; j < KC; ++j) {
            const int col = col0 + l, row = t + T * j;
            if (l < a.CB && col < n && row < m) a.cap_Rcol[(int64_t)row * n + col] = rc[l][j];
          }
      }
    }

    // ---- starting vector u0 of component i ----
    {
      const uint64_t base = start_base(a.seed, (uint64_t)i);
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int row = t + T * j;
        u[j] = row < m ? start_sign(base, (uint64_t)row) : 0.f;
      }
    }

    double cpart = 0.0;  // u . x of the last iteration, this thread's share
    for (int it = 0; it < a.iters; ++it) {
      const bool cap = CAP && (i == a.cap_i) && capturer;
      int cnt, fb;
      // ---- y = R^T u on the column copy; v = T_tau(y) ----
      {
        float acc[LC];
#pragma unroll
        for (int l = 0; l < LC; ++l) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < KC; ++j) s = fmaf(u[j], rc[l][j], s);
          acc[l] = s;
        }
        ++ry;
        reduce_publish<T, LC>(acc, red, min(a.CB, n - col0), a.yslot, col0, ry);
        float y[KR];
        const bool bad = !gather<T, KR>(a.yslot, n, ry, y, a.err);
        if (!ternarize_dist<T, KR>(y, bad, n, a.tau, v, bufs, cnt, fb)) {
          if (t == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        st_nnz_v += cnt;
        st_fb += fb;
        if (cap) {
          for (int j = 0; j < KR; ++j) {
            const int col = t + T * j;
            if (col < n) {
              if (a.cap_y) a.cap_y[(int64_t)it * n + col] = y[j];
              if (a.cap_v) a.cap_v[(int64_t)it * n + col] = (int8_t)v[j];
            }
          }
        }
      }
      // ---- x = R diag(w) v on the row copy; u = T_tau(x) ----
      {
        float vw[KR];
#pragma unroll
        for (int j = 0; j < KR; ++j) vw[j] = v[j] * wv[j];
        float acc[LR];
#pragma unroll
        for (int l = 0; l < LR; ++l) {
          const float* rp = rrow + l * KR * T + t;
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < KR; ++j) s = fmaf(vw[j], rp[j * T], s);
          acc[l] = s;
        }
        ++rx;
        reduce_publish<T, LR>(acc, red, min(a.RB, m - row0), a.xslot, row0, rx);
        float x[KC];
        const bool bad = !gather<T, KC>(a.xslot, m, rx, x, a.err);
        if (!ternarize_dist<T, KC>(x, bad, m, a.tau, u, bufs, cnt, fb)) {
          if (t == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        st_nnz_u += cnt;
        st_fb += fb;
        if (it == a.iters - 1) {
#pragma unroll
          for (int j = 0; j < KC; ++j) cpart += (double)u[j] * (double)x[j];
        }
        if (cap) {
          for (int j = 0; j < KC; ++j) {
            const int row = t + T * j;
            if (row < m) {
              if (a.cap_x) a.cap_x[(int64_t)it * m + row] = x[j];
              if (a.cap_u) a.cap_u[(int64_t)it * m + row] = (int8_t)u[j];
            }
          }
        }
      }
    }

    // ---- own-row u and own-column v for the next deflation ----
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int row = t + T * j;
      if (row >= row0 && row < row0 + a.RB && row < m) u_own[row - row0] = u[j];
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int col = t + T * j;
      if (col >= col0 && col < col0 + a.CB && col < n) v_own[col - col0] = v[j];
    }

    // ---- scale d = u.x / (nnz_u v^T diag(w) v) (§2.3 step 2, §2.5); one barrier ----
    {
      double sums[4] = {cpart, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < KC; ++j) sums[1] += (u[j] != 0.f) ? 1.0 : 0.0;
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        sums[2] += (v[j] != 0.f) ? 1.0 : 0.0;
        sums[3] += (v[j] != 0.f) ? (double)wv[j] : 0.0;
      }
      block_sum_f64<T, 4>(sums, bufs[2]);
      const double c = sums[0], nu = sums[1], nv = sums[2];
      const double den = nu * sums[3];
      d32 = den > 0.0 ? (float)(c / den) : 0.f;
      trace_state -= den > 0.0 ? c * c / den : 0.0;
      st_b += (long long)nu;
      st_c += (long long)nv;
      if (g == 0 && t == 0) {
        a.D[i] = d32;
        if (a.trace) a.trace[i] = trace_state;
        if (CAP && i == a.cap_i && a.cap_d) *a.cap_d = d32;
      }
    }

    // ---- 2-bit codes of u and v into B2 / C2 row i (ballots, no barrier) ----
    store_codes<T, KC>(u, m, a.B2 + (int64_t)i * wm, g, a.G);
    store_codes<T, KR>(v, n, a.C2 + (int64_t)i * wn, g, a.G);
  }

  // ---- ||R||^2 of the final residual over this workgroup's rows ----
  __syncthreads();
  double r2[1] = {0.0};
#pragma unroll
  for (int l = 0; l < LR; ++l)
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const double r = (double)rrow[(l * KR + j) * T + t];
      r2[0] += r * r * (double)wv[j];
    }
  block_sum_f64<T, 1>(r2, bufs[0]);
  if (t == 0) a.r2_partial[g] = r2[0];

  if (g == 0 && a.stats) {
    double cnts[2] = {(double)st_nnz_u, (double)st_nnz_v};
    block_sum_f64<T, 2>(cnts, bufs[1]);
    if (t == 0) {
      a.stats[EXTERND_STAT_SUM_NNZ_U] = (long long)cnts[0];
      a.stats[EXTERND_STAT_SUM_NNZ_V] = (long long)cnts[1];
      a.stats[EXTERND_STAT_NNZ_B] = st_b;
      a.stats[EXTERND_STAT_NNZ_C] = st_c;
      a.stats[EXTERND_STAT_FALLBACKS] = st_fb;
      a.stats[EXTERND_STAT_MODE] = EXTERND_MODE_RESIDENT;
      a.stats[EXTERND_STAT_GRID] = a.G;
      a.stats[EXTERND_STAT_ITERATIONS] = (long long)a.k * a.iters;
    }
  }
}

__global__ void k_fill_u64(unsigned long long* p, int64_t count) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = 0ull;
}
__global__ void k_resident_finish(const double* __restrict__ r2_partial, int G,
                                  const double* __restrict__ a2, const long long* __restrict__ nonfinite,
                                  const unsigned* __restrict__ err, double* __restrict__ energy,
                                  long long* __restrict__ stats) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double r2 = 0.0;
  for (int g = 0; g < G; ++g) r2 += r2_partial[g];
  double e;
  if (*nonfinite > 0 || *err != 0u) e = __longlong_as_double(0x7ff8000000000000ll);
  else if (*a2 == 0.0) e = 1.0;
  else e = 1.0 - r2 / *a2;
  *energy = e;
  if (stats) {
    stats[EXTERND_STAT_NONFINITE] = *nonfinite;
    stats[EXTERND_STAT_TIMEOUTS] = *err;
  }
}

// Tile instantiations: (threads, columns per thread KR, rows per workgroup LR,
// rows per thread KC, columns per workgroup LC).
struct Tile {
  int KR, LR, KC, LC;
};
constexpr int kResT = 512;
constexpr Tile kTiles[] = {{1, 32, 1, 32}, {2, 16, 2, 16}, {5, 10, 5, 10}};

inline int tile_grid(const Tile& tl, int64_t m, int64_t n) {
  const int64_t g1 = (m + tl.LR - 1) / tl.LR, g2 = (n + tl.LC - 1) / tl.LC;
  return (int)std::max<int64_t>(1, std::max(g1, g2));
}
inline bool tile_fits(const Tile& tl, int64_t m, int64_t n, int num_cus) {
  if (m < 1 || n < 1) return false;
  if ((m + kResT - 1) / kResT > tl.KC || (n + kResT - 1) / kResT > tl.KR) return false;
  return tile_grid(tl, m, n) <= std::min(256, num_cus);
}
inline int pick_tile(int64_t m, int64_t n, int num_cus) {
  for (int i = 0; i < (int)(sizeof(kTiles) / sizeof(kTiles[0])); ++i)
    if (tile_fits(kTiles[i], m, n, num_cus)) return i;
  return -1;
}

template <int KR, int LR, int KC, int LC>
hipError_t launch_tile(ResArgs& ra, hipStream_t s) {
  void* args[] = {&ra};
  void* fn = ra.cap_i >= 0 ? reinterpret_cast<void*>(&k_seq_resident<kResT, KR, LR, KC, LC, true>)
                           : reinterpret_cast<void*>(&k_seq_resident<kResT, KR, LR, KC, LC, false>);
  return hipLaunchCooperativeKernel(fn, dim3(ra.G), dim3(kResT), args, 0, s);
}

}  // namespace

bool resident_fits(int64_t m, int64_t n, int num_cus) {
  if (m > (1 << 30) || n > (1 << 30)) return false;
  return pick_tile(m, n, num_cus) >= 0;
}

size_t resident_workspace_bytes(int64_t m, int64_t n) {
  return sizeof(unsigned long long) * (size_t)(m + n) + sizeof(double) * (256 + 4096 + 8) +
         sizeof(long long) * 8 + sizeof(unsigned) * 64 + sizeof(float) * (size_t)n + 256 * 9;
}

static inline char* align256(char* p) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 255) & ~(uintptr_t)255);
}

hipError_t run_resident_seq(const SeqArgs& a, void* ws, int num_cus, hipStream_t s, int* grid_out) {
  const int ti = pick_tile(a.m, a.n, num_cus);
  if (ti < 0) return hipErrorInvalidValue;
  const Tile tl = kTiles[ti];
  char* p = align256(static_cast<char*>(ws));
  unsigned long long* yslot = reinterpret_cast<unsigned long long*>(p);
  p = align256(p + sizeof(unsigned long long) * a.n);
  unsigned long long* xslot = reinterpret_cast<unsigned long long*>(p);
  p = align256(p + sizeof(unsigned long long) * a.m);
  double* r2p = reinterpret_cast<double*>(p);
  p = align256(p + sizeof(double) * 256);
  double* npart = reinterpret_cast<double*>(p);
  p = align256(p + sizeof(double) * 4096);
  double* a2 = reinterpret_cast<double*>(p);
  p = align256(p + sizeof(double) * 8);
  long long* nonfinite = reinterpret_cast<long long*>(p);
  p = align256(p + sizeof(long long) * 8);
  unsigned* err = reinterpret_cast<unsigned*>(p);
  p = align256(p + sizeof(unsigned) * 64);
  float* wt = a.importance ? reinterpret_cast<float*>(p) : nullptr;   // column weights (§2.5)

  hipError_t e;
  hipLaunchKernelGGL(k_fill_u64, dim3(64), dim3(256), 0, s, yslot, (int64_t)a.n);
  hipLaunchKernelGGL(k_fill_u64, dim3(64), dim3(256), 0, s, xslot, (int64_t)a.m);
  if ((e = launch_fill_i64(nonfinite, 1, 0, s)) != hipSuccess) return e;
  if ((e = launch_fill_u32(err, 1, 0u, s)) != hipSuccess) return e;
  if (wt && (e = launch_importance_weights(a.importance, a.n, a.lambda, wt, nonfinite, s)) != hipSuccess) return e;
  if ((e = launch_norm2(a.A, a.m * a.n, npart, 4096, a2, nonfinite, s, wt, a.n)) != hipSuccess) return e;
  if (a.stats && (e = launch_fill_i64(a.stats, EXTERND_STATS_LEN, 0, s)) != hipSuccess) return e;

  ResArgs ra{};
  ra.A = a.A;
  ra.m = (int)a.m;
  ra.n = (int)a.n;
  ra.k = (int)a.k;
  ra.tau = a.tau;
  ra.iters = a.iters;
  ra.seed = a.seed;
  ra.G = tile_grid(tl, a.m, a.n);
  ra.RB = (int)((a.m + ra.G - 1) / ra.G);
  ra.CB = (int)((a.n + ra.G - 1) / ra.G);
  ra.B2 = a.B2;
  ra.C2 = a.C2;
  ra.D = a.D;
  ra.trace = a.trace;
  ra.stats = a.stats;
  ra.a2 = a2;
  ra.wt = wt;
  ra.nonfinite = nonfinite;
  ra.yslot = reinterpret_cast<unsigned*>(yslot);   // 32-bit words; zero = parity 0
  ra.xslot = reinterpret_cast<unsigned*>(xslot);
  ra.err = err;
  ra.r2_partial = r2p;
  ra.cap_i = a.capture_component;
  ra.cap_R = a.capture_R;
  ra.cap_Rcol = a.capture_Rcol;
  ra.cap_R_next = a.capture_R_next;
  ra.cap_y = a.capture_y;
  ra.cap_x = a.capture_x;
  ra.cap_v = a.capture_v;
  ra.cap_u = a.capture_u;
  ra.cap_d = a.capture_d;
  if (grid_out) *grid_out = ra.G;

  switch (ti) {
    case 0: e = launch_tile<1, 32, 1, 32>(ra, s); break;
    case 1: e = launch_tile<2, 16, 2, 16>(ra, s); break;
    default: e = launch_tile<5, 10, 5, 10>(ra, s); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_resident_finish, dim3(1), dim3(64), 0, s, r2p, ra.G, a2, nonfinite, err,
                     a.energy, a.stats);
  if (a.norm_a2 && (e = launch_copy_f64(a2, a.norm_a2, 1, s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace externd
