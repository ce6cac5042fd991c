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
// iteration.  Each word is published in kRep = 4 replicas, 4 KB-aligned
// apart, and workgroup g gathers replica (g mod 8) / 2: with workgroups
// dispatched round-robin over the 8 XCDs, each pair of XCDs reads its own
// copy, so the misses of a replica's 64 readers meet in their XCDs' L2s and
// no single set of lines serves the whole device (measured: 4 replicas read
// by XCD pairs 612 ms at 2560 x 2560, k = 5120; one copy 678 ms; 8 copies,
// one per XCD, 637 ms; copies that mix XCDs, or strides that are not 4 KB
// multiples, were slower still).  The mapping only places the reads;
// correctness does not depend on where a workgroup runs.  Every workgroup then holds the whole vector (the same bits in
// every workgroup) and applies T_tau (§2.2) redundantly and identically.
//
// Termination.  Every wait is bounded: a workgroup that waits too long sets a
// device error flag and the whole grid returns; the energy is then NaN and
// stats[EXTERND_STAT_TIMEOUTS] is set (the call itself still returns OK).
//
// Safeguard check (appendix §7).  Every thread keeps the largest w_j R_ij^2
// of the column-copy entries it holds (each residual entry is held by exactly
// one thread of one workgroup), so the single-entry bound max_ij w_j R_ij^2
// is exceeded by the component's decrease everywhere or not: a wave with a
// thread whose own maximum beats the decrease sets the component's bit in
// the workgroup's LDS window of 1024 components (an idempotent OR, so no
// reduction or barrier is needed), every full window is ORed into the
// global bitmap, and the bits are counted at the end.
#include "device_common.hpp"
#include "kernels.hpp"
#include "exchange.hpp"

namespace externd {

namespace {

using namespace xchg;

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
  unsigned* yslot;             // kRep replicas of n words, rep_stride(n) apart (placement 0)
  unsigned* xslot;             // kRep replicas of m words, rep_stride(m) apart (placement 0)
  const int* place;            // the placement of the word arrays to use (see k_place_probe)
  int64_t place_words;         // words between consecutive placements
  unsigned* err;
  double* r2_partial;          // G fp64
  unsigned* sg_bits;           // ceil(k/32) words, zeroed: components failing the single-entry bound
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
  __shared__ unsigned sg_win[32];   // safeguard bits of the current window of 1024 components
  __shared__ double tslot[6];        // T_tau's reduction slots (ternarize_dist_guess)

  const int t = threadIdx.x;
  const int g = blockIdx.x;
  const int m = a.m, n = a.n;
  const int row0 = g * a.RB, col0 = g * a.CB;
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  const int64_t poff = (int64_t)__builtin_amdgcn_readfirstlane(*a.place) * a.place_words;
  unsigned* const yslot = a.yslot + poff;
  unsigned* const xslot = a.xslot + poff;

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
  // weights of the column copy's columns (the same for every thread: scalar registers)
  float wcol[LC];
#pragma unroll
  for (int l = 0; l < LC; ++l)
    wcol[l] = __int_as_float(__builtin_amdgcn_readfirstlane(
        __float_as_int((a.wt && l < a.CB && col0 + l < n) ? a.wt[col0 + l] : 1.f)));
  if (t < 32) sg_win[t] = 0u;   // published by the first barrier below
  if (t < 6) tslot[t] = 0.0;
  float d32 = 0.f;
  unsigned ry = 0, rx = 0;
  long long st_nnz_u = 0, st_nnz_v = 0, st_fb = 0, st_b = 0, st_c = 0;
  double trace_state = *a.a2;
  const bool capturer = (g == 0);

  const int sg_words = (a.k + 31) / 32;
  // guesses of the exponent of max|y| and max|x| for T_tau (block-uniform),
  // kept apart for the first, the second and the later iterations
  int egy0 = 0, egy1 = 0, egy2 = 0, egx0 = 0, egx1 = 0, egx2 = 0;
  for (int i = 0; i <= a.k; ++i) {
    // ---- a finished window of safeguard bits (or the last one) to the global bitmap ----
    if (i > 0 && ((i & 1023) == 0 || i == a.k)) {
      __syncthreads();
      if (t < 32) {
        const int word = ((i - 1) >> 10) * 32 + t;
        const unsigned b = sg_win[t];
        if (b != 0u && word < sg_words) atomicOr(a.sg_bits + word, b);
        sg_win[t] = 0u;
      }
    }
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
    // this thread's share of the single-entry bound max_ij w_j R_ij^2 of the
    // residual before component i (exact: w (|x|)^2 with x^2 exact in fp64)
    double rmax2 = 0.0;
#pragma unroll
    for (int l = 0; l < LC; ++l) {
      uint32_t mb = 0u;
#pragma unroll
      for (int j = 0; j < KC; ++j) mb = max(mb, __float_as_uint(rc[l][j]) & 0x7fffffffu);
      const double x = (double)__uint_as_float(mb);
      float wl = wcol[l];
      asm volatile("" : "+s"(wl));   // converted here, not hoisted out of the loop as fp64
      rmax2 = fmax(rmax2, x * x * (double)wl);
    }
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
        reduce_publish<T, LC>(acc, red, min(a.CB, n - col0), yslot, col0, ry, rep_stride(n));
        float y[KR];
        const bool bad = !gather<T, KR>(yslot + rep_of(g) * rep_stride(n), n, ry, y, a.err);
        int eg = it == 0 ? egy0 : (it == 1 ? egy1 : egy2);
        if (!ternarize_dist_guess<T, KR>(y, bad, n, a.tau, v, bufs, tslot, ry + rx, eg, cnt, fb)) {
          if (t == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        if (it == 0) egy0 = eg; else if (it == 1) egy1 = eg; else egy2 = eg;
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
        reduce_publish<T, LR>(acc, red, min(a.RB, m - row0), xslot, row0, rx, rep_stride(m));
        float x[KC];
        const bool bad = !gather<T, KC>(xslot + rep_of(g) * rep_stride(m), m, rx, x, a.err);
        int eg = it == 0 ? egx0 : (it == 1 ? egx1 : egx2);
        if (!ternarize_dist_guess<T, KC>(x, bad, m, a.tau, u, bufs, tslot, ry + rx, eg, cnt, fb)) {
          if (t == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        if (it == 0) egx0 = eg; else if (it == 1) egx1 = eg; else egx2 = eg;
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
      const double dec = den > 0.0 ? c * c / den : 0.0;
      trace_state -= dec;
      if (__any(dec < rmax2) && (t & (kWave - 1)) == 0) atomicOr(&sg_win[(i & 1023) >> 5], 1u << (i & 31));
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

// Placement probe.  Where the exchange words sit in device memory changes
// the time of the whole decomposition by up to 6 % (2560 x 2560: 512
// components take 60.0 to 63.7 ms depending on the 2 KB step of the word
// arrays' start within 16 KB, and which step is fastest differs from one
// allocation to the next), so it cannot be fixed in advance.  The exchange
// alone predicts it (correlation 0.92 over 32 placements): this kernel runs
// `rounds` exchanges of y and x, exactly as k_seq_resident publishes and
// gathers them but with no arithmetic between, on each candidate placement
// in turn (disjoint copies of the word arrays, place_words apart, each
// starting 2 KB later within 16 KB than the one before), and workgroup 0
// stores the index of the fastest in *place.  The values exchanged are
// never used, so the choice cannot change any result.  Waits are bounded;
// if one runs out, placement 0 is kept.
struct ProbeArgs {
  int m, n, G, RB, CB;
  unsigned* yslot;
  unsigned* xslot;
  int64_t place_words;
  int cands, rounds;
  unsigned* err;   // the probe's own flag
  int* place;
};

template <int T, int KR, int LR, int KC, int LC>
__global__ __launch_bounds__(T) void k_place_probe(ProbeArgs a) {
  constexpr int W = T / kWave;
  constexpr int LMAX = LR > LC ? LR : LC;
  __shared__ float red[W * LMAX];
  const int g = blockIdx.x;
  const int m = a.m, n = a.n;
  const int row0 = g * a.RB, col0 = g * a.CB;
  float accy[LC], accx[LR];
#pragma unroll
  for (int l = 0; l < LC; ++l) accy[l] = 0.f;
#pragma unroll
  for (int l = 0; l < LR; ++l) accx[l] = 0.f;
  bool ok = true;
  unsigned long long best = ~0ull;
  int best_c = 0;
  for (int c = 0; c < a.cands && ok; ++c) {
    unsigned* const ys = a.yslot + (int64_t)c * a.place_words;
    unsigned* const xs = a.xslot + (int64_t)c * a.place_words;
    __syncthreads();
    const unsigned long long t0 = wall_clock64();
    for (unsigned r = 1; r <= (unsigned)a.rounds && ok; ++r) {   // every placement starts at parity 0
      reduce_publish<T, LC>(accy, red, min(a.CB, n - col0), ys, col0, r, rep_stride(n));
      float y[KR];
      ok = gather<T, KR>(ys + rep_of(g) * rep_stride(n), n, r, y, a.err);
      ok = __syncthreads_and(ok);
      reduce_publish<T, LR>(accx, red, min(a.RB, m - row0), xs, row0, r, rep_stride(m));
      float x[KC];
      if (ok) ok = gather<T, KC>(xs + rep_of(g) * rep_stride(m), m, r, x, a.err);
      ok = __syncthreads_and(ok);
    }
    const unsigned long long dt = wall_clock64() - t0;
    if (dt < best) {
      best = dt;
      best_c = c;
    }
  }
  if (!ok && threadIdx.x == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (g == 0 && threadIdx.x == 0) *a.place = ok ? best_c : 0;
}

__global__ void k_fill_u64(unsigned long long* p, int64_t count) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = 0ull;
}
__global__ void k_resident_finish(const double* __restrict__ r2_partial, int G,
                                  const double* __restrict__ a2, const long long* __restrict__ nonfinite,
                                  const unsigned* __restrict__ err, double* __restrict__ energy,
                                  long long* __restrict__ stats, const unsigned* __restrict__ sg_bits,
                                  int64_t sg_words) {
  if (stats && blockIdx.x == 0) {
    long long c = 0;
    for (int64_t q = threadIdx.x; q < sg_words; q += blockDim.x) c += __popc(sg_bits[q]);
    c = wave_sum(c);
    if (threadIdx.x == 0) stats[EXTERND_STAT_SAFEGUARD] = c;
  }
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
hipError_t launch_probe(ProbeArgs& pa, hipStream_t s) {
  void* args[] = {&pa};
  return hipLaunchCooperativeKernel(reinterpret_cast<void*>(&k_place_probe<kResT, KR, LR, KC, LC>), dim3(pa.G),
                                    dim3(kResT), args, 0, s);
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

// Placements of the exchange words tried by k_place_probe: disjoint copies
// of the y and x word arrays, each starting 2 KB later within 16 KB.
constexpr int kPlaceCands = 8;
constexpr int kProbeRounds = 48;
static int64_t place_words(int64_t m, int64_t n) {
  const int64_t w = (int64_t)kRep * (rep_stride((int)m) + rep_stride((int)n));
  return (w + 4095) / 4096 * 4096 + 512;   // a multiple of 16 KB, plus 2 KB
}

int resident_place_candidates(int64_t m, int64_t n, int64_t k) {
  // the probe costs about 0.25 ms per candidate: worth it for long runs only
  return (k >= 1024 && m * n >= (int64_t(1) << 20)) ? kPlaceCands : 1;
}

size_t resident_workspace_bytes(int64_t m, int64_t n, int64_t k, int cands) {
  return sizeof(unsigned) * (size_t)(place_words(m, n) * cands) + sizeof(double) * (256 + 4096 + 8) +
         sizeof(long long) * 8 + sizeof(unsigned) * 64 * 2 + sizeof(float) * (size_t)n +
         sizeof(unsigned) * (size_t)((k + 31) / 32) + sizeof(int) * 64 + 256 * 12;
}

static inline char* align256(char* p) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 255) & ~(uintptr_t)255);
}

hipError_t run_resident_seq(const SeqArgs& a, void* ws, int cands, int num_cus, hipStream_t s, int* grid_out) {
  const int ti = pick_tile(a.m, a.n, num_cus);
  if (ti < 0 || cands < 1) return hipErrorInvalidValue;
  const Tile tl = kTiles[ti];
  const int64_t pw = place_words(a.m, a.n);
  char* p = align256(static_cast<char*>(ws));
  unsigned* yslot = reinterpret_cast<unsigned*>(p);   // placement c at yslot + c * pw
  unsigned* xslot = yslot + (int64_t)kRep * rep_stride((int)a.n);
  p = align256(p + sizeof(unsigned) * (size_t)(pw * cands));
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
  unsigned* probe_err = reinterpret_cast<unsigned*>(p);
  p = align256(p + sizeof(unsigned) * 64);
  int* place = reinterpret_cast<int*>(p);
  p = align256(p + sizeof(int) * 64);
  float* wt = a.importance ? reinterpret_cast<float*>(p) : nullptr;   // column weights (§2.5)
  p = align256(p + sizeof(float) * a.n);
  unsigned* sg_bits = reinterpret_cast<unsigned*>(p);
  const int64_t sg_words = (a.k + 31) / 32;

  hipError_t e;
  if ((e = launch_fill_u32(sg_bits, sg_words, 0u, s)) != hipSuccess) return e;
  // every replica word of every placement starts at parity 0 (pw is even: whole 8-byte fills)
  hipLaunchKernelGGL(k_fill_u64, dim3(64), dim3(256), 0, s, reinterpret_cast<unsigned long long*>(yslot),
                     pw * cands / 2);
  if ((e = launch_fill_u32(reinterpret_cast<uint32_t*>(place), 1, 0u, s)) != hipSuccess) return e;
  const int G = tile_grid(tl, a.m, a.n);
  if (cands > 1) {
    if ((e = launch_fill_u32(probe_err, 1, 0u, s)) != hipSuccess) return e;
    ProbeArgs pa{};
    pa.m = (int)a.m;
    pa.n = (int)a.n;
    pa.G = G;
    pa.RB = (int)((a.m + G - 1) / G);
    pa.CB = (int)((a.n + G - 1) / G);
    pa.yslot = yslot;
    pa.xslot = xslot;
    pa.place_words = pw;
    pa.cands = cands;
    pa.rounds = kProbeRounds;
    pa.err = probe_err;
    pa.place = place;
    switch (ti) {
      case 0: e = launch_probe<1, 32, 1, 32>(pa, s); break;
      case 1: e = launch_probe<2, 16, 2, 16>(pa, s); break;
      default: e = launch_probe<5, 10, 5, 10>(pa, s); break;
    }
    if (e != hipSuccess) return e;
    // the probe left every placement at some parity: back to 0
    hipLaunchKernelGGL(k_fill_u64, dim3(64), dim3(256), 0, s, reinterpret_cast<unsigned long long*>(yslot),
                       pw * cands / 2);
  }
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
  ra.G = G;
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
  ra.yslot = yslot;   // 32-bit words; zero = parity 0
  ra.xslot = xslot;
  ra.place = place;
  ra.place_words = pw;
  ra.err = err;
  ra.r2_partial = r2p;
  ra.sg_bits = sg_bits;
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
                     a.energy, a.stats, sg_bits, sg_words);
  if (a.norm_a2 && (e = launch_copy_f64(a2, a.norm_a2, 1, s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace externd
