// Persistent streaming sequential path: one cooperative kernel runs every
// component and every alternating iteration of the greedy ALS (ExTernD §2.3)
// with the residual R in device memory, for shapes too large to keep on chip.
//
// Layout.  Workgroup g of G (one per CU) owns the row slab
// [g RB, g RB + RB) of R and is the only one to read or write it, so the
// fused deflation needs no synchronisation.  The first L rows of the slab
// (as many as the LDS left over by the vectors holds) live in LDS for the
// whole decomposition, the others in device memory; each row has exactly one
// home.  Vectors are distributed as in the resident kernel (thread t holds
// entries t + T j).
//
// y = R^T u (§2.3 step 1) in three phases:
//   1. every workgroup lists its slab rows with u_r != 0 (device-memory rows
//      first), sums u_r R_r over them (reading only those rows; the previous
//      component's deflation is applied to the rows of supp(u_prev) on the
//      way, one rounding per entry, and written back), stages the n sums in
//      LDS and publishes them, one word per column, into each column block's
//      contiguous G x CB area of the partial array (word (h, c mod CB) of
//      block c / CB for workgroup h);
//   2. workgroup g owns the column block [g CB, g CB + CB), CB a power of two
//      from 16 to 64: lane t reads the words (h, t mod CB) for
//      h = t / CB + LPC q with LPC = T / CB (one contiguous run of the area
//      per q), and the lanes of a column are added by a fixed butterfly
//      inside the wave, then the waves in order, before y_c is published;
//   3. every workgroup gathers all n words of y and applies T_tau.
// x = R diag(w) v: each wave takes whole rows of the slab (device-memory rows
// dealt out first, then the LDS rows, so the waves' loads stay even), sums
// across its lanes and publishes x_r itself; then every workgroup gathers
// all m words and applies T_tau.  u, v and their codes live only inside the
// step that makes them: the slab's u and v diag(w) stay in LDS.
//
// Exchange words carry the round parity in their lowest bit (exchange.hpp);
// the partial array is one replica, read by its column block's owner only.
// Its round r+1 is published only after the publisher has gathered y of
// round r, which every owner published after reading all of its partials of
// round r, so no partial word is overwritten while it may still be read.
//
// Every R entry is read by exactly one thread in a component's first pass
// (dense u0: every row is read), so the single-entry safeguard check
// (appendix §7) is the resident kernel's: a thread keeps the largest
// w_c R_rc^2 it saw in that pass and flags the component when the decrease
// falls below it.
#include "device_common.hpp"
#include "exchange.hpp"
#include "kernels.hpp"

namespace externd {

namespace {

using namespace xchg;

constexpr int kPerT = 512;     // threads per workgroup
constexpr int kRBMax = 64;     // slab rows per workgroup, at most (one wave lists them)
constexpr int kQMax = 32;      // partials each phase-2 lane gathers, at most
constexpr int kLdsBytes = 160 * 1024;

// LDS of one workgroup: the vectors first, the row cache takes the rest.
template <int T, int KR>
struct PerLds {
  static constexpr int W = T / kWave;
  static constexpr int kVec = KR * T * 4 + KR * T + kRBMax * 4 * 3 + T * 4 + 3 * W * 4 * 8 + 32 * 4 + 64;
  static constexpr int kCache = (kLdsBytes - kVec - 1024) / 16 * 4;   // floats, a multiple of 4
};

struct PerArgs {
  float* R;                    // m x n residual (a copy of A), row-major
  int m, n, k;
  float tau;
  int iters;
  uint64_t seed;
  int G, RB, CB, LPC;          // workgroups, slab rows, y column block, lanes per column in phase 2
  int lgCB;                    // CB = 2^lgCB
  uint32_t* B2;
  uint32_t* C2;
  float* D;
  double* trace;
  long long* stats;
  const double* a2;
  const float* wt;             // optional column weights (§2.5)
  const long long* nonfinite;
  unsigned* pslot;             // ceil(n / CB) column blocks of G x CB partial words
  unsigned* yslot;             // kRep replicas of n words
  unsigned* xslot;             // kRep replicas of m words
  unsigned* err;
  double* r2_partial;          // G
  unsigned* sg_bits;
  int64_t cap_i;
  float* cap_R;
  float* cap_R_next;
  float* cap_y;
  float* cap_x;
  int8_t* cap_v;
  int8_t* cap_u;
  float* cap_d;
};

// A value the whole wave holds (read from LDS or computed identically),
// moved to a scalar register so that addresses built from it stay scalar.
__device__ inline float uniform_f(float x) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x))); }
__device__ inline int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Poll one exchange word until it carries the round's parity (bounded).
__device__ inline bool poll_word(const unsigned* p, unsigned par, unsigned& w, const unsigned* err) {
  unsigned spins = 0;
  while ((w & 1u) != par) {
    if (++spins > kSpinLimit) return false;
    if ((spins & 255u) == 0 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
      return false;
    w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// Dot product of one row (float4 view, n4 entries) with vsh, across a wave;
// every lane returns its share, the caller sums the wave.
template <int F4, typename P>
__device__ inline float4 row_dot(P r4, const float4* vs4, int n4, int lane) {
  constexpr int FB = F4 < 10 ? F4 : 10;   // loads in flight per batch
  float4 acc4 = {0.f, 0.f, 0.f, 0.f};
  for (int f0 = 0; f0 < F4; f0 += FB) {
    float4 rv[FB];
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int c4 = lane + kWave * (f0 + f);
      if (c4 < n4) rv[f] = r4[c4];
    }
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int c4 = lane + kWave * (f0 + f);
      if (c4 < n4) {
        const float4 vv = vs4[c4];
        acc4.x = fmaf(vv.x, rv[f].x, acc4.x);
        acc4.y = fmaf(vv.y, rv[f].y, acc4.y);
        acc4.z = fmaf(vv.z, rv[f].z, acc4.z);
        acc4.w = fmaf(vv.w, rv[f].w, acc4.w);
      }
    }
  }
  return acc4;
}

// KR: entries of an n-vector per thread (n <= T KR), KC: of an m-vector (m <= T KC).
template <int T, int KR, int KC, bool CAP>
__global__ __launch_bounds__(T) void k_seq_persist(PerArgs a) {
  constexpr int W = T / kWave;
  constexpr int NF4 = (KR * T / 4 + T - 1) / T;          // phase-1 float4 per row per thread, at most
  constexpr int NB = NF4 <= 2 ? 8 : (NF4 <= 5 ? 4 : 2);  // phase-1 rows per batch of loads
  constexpr int F4 = (KR * T / 4 + kWave - 1) / kWave;   // x-pass float4 per row per lane, at most
  constexpr int kCache = PerLds<T, KR>::kCache;
  __shared__ __align__(16) float4 rcache[kCache / 4];    // slab rows [0, L)
  __shared__ __align__(16) float vsh[KR * T];            // v diag(w) for the x pass
  __shared__ __align__(16) signed char vpl[KR * T];      // v itself (the deflation in the next component's first pass)
  __shared__ float u_own[kRBMax];                        // u of the slab rows
  __shared__ float up_own[kRBMax];                       // u of the previous component on the slab rows
  __shared__ int rl[kRBMax];                             // phase-1 row list
  __shared__ float red[W * kWave];                       // phase-2 wave sums
  __shared__ double bufs[3][W][4];
  __shared__ unsigned sg_win[32];
  __shared__ int nlist[2];
  __shared__ double tslot[6];   // T_tau's reduction slots (ternarize_dist_guess)

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wv_id = t / kWave;
  const int g = blockIdx.x;
  const int m = a.m, n = a.n;
  const int row0 = g * a.RB;
  const int rows = max(0, min(a.RB, m - row0));
  const int wm = (m + 15) / 16, wn = (n + 15) / 16;
  const int n4 = n >> 2;
  const int L = min(rows, kCache / n);   // slab rows kept in LDS
  const int H = rows - L;                // slab rows in device memory
  float* R = a.R;
  const float4* vs4 = reinterpret_cast<const float4*>(vsh);
  const char4* vp4 = reinterpret_cast<const char4*>(vpl);

  if (*a.nonfinite > 0) {
    for (int64_t w = (int64_t)g * T + t; w < (int64_t)a.k * wm; w += (int64_t)a.G * T) a.B2[w] = 0u;
    for (int64_t w = (int64_t)g * T + t; w < (int64_t)a.k * wn; w += (int64_t)a.G * T) a.C2[w] = 0u;
    for (int64_t w = (int64_t)g * T + t; w < a.k; w += (int64_t)a.G * T) a.D[w] = 0.f;
    if (t == 0) a.r2_partial[g] = 0.0;
    return;
  }

  {
    const float4* src = reinterpret_cast<const float4*>(R + (int64_t)row0 * n);
    for (int q = t; q < L * n4; q += T) rcache[q] = src[q];
  }
  if (t < 32) sg_win[t] = 0u;
  if (t < 6) tslot[t] = 0.0;
  if (t < kRBMax) up_own[t] = 0.f;
  for (int c = t; c < KR * T; c += T) vpl[c] = 0;
  float d32 = 0.f;
  unsigned rp = 0, ry = 0, rx = 0;
  long long st_nnz_u = 0, st_nnz_v = 0, st_fb = 0, st_b = 0, st_c = 0;
  double trace_state = *a.a2;
  const bool capturer = (g == 0);
  const int sg_words = (a.k + 31) / 32;
  // guesses of the exponent of max|y| and max|x| for T_tau (block-uniform),
  // kept apart for the first, the second and the later iterations
  int egy0 = 0, egy1 = 0, egy2 = 0, egx0 = 0, egx1 = 0, egx2 = 0;

  for (int i = 0; i <= a.k; ++i) {
    if (i > 0 && ((i & 1023) == 0 || i == a.k)) {
      __syncthreads();
      if (t < 32) {
        const int word = ((i - 1) >> 10) * 32 + t;
        const unsigned b = sg_win[t];
        if (b != 0u && word < sg_words) atomicOr(a.sg_bits + word, b);
        sg_win[t] = 0u;
      }
    }
    if (i == a.k) break;

    // ---- starting vector u0 of component i, on the slab rows ----
    if (t < rows) u_own[t] = start_sign(start_base(a.seed, (uint64_t)i), (uint64_t)(row0 + t));
    const float dprev = d32;
    double rmax2 = 0.0;   // this thread's share of the single-entry bound of R before component i
    double sums[4] = {0.0, 0.0, 0.0, 0.0};   // u.x, nnz(u), nnz(v), sum of w over supp(v): last iteration
    for (int it = 0; it < a.iters; ++it) {
      const bool cap = CAP && (i == a.cap_i) && capturer;
      const bool first = (it == 0);
      const bool last = (it == a.iters - 1);
      int cnt, fb;
      __syncthreads();   // u_own, up_own and vsh of the previous steps are visible
      // ---- y phase 1: row list ----
      if (wv_id == 0) {
        const bool need = lane < rows && (first || u_own[lane] != 0.f);
        const unsigned long long mh = __ballot(need && lane >= L), ml = __ballot(need && lane < L);
        const unsigned long long lt = (1ull << lane) - 1ull;
        const int nh = __popcll(mh);
        if (need) rl[lane >= L ? __popcll(mh & lt) : nh + __popcll(ml & lt)] = lane;
        if (lane == 0) {
          nlist[0] = nh;
          nlist[1] = nh + __popcll(ml);
        }
      }
      __syncthreads();
      // ---- y phase 1: partial sums over the listed rows (with the fused deflation) ----
      // thread t takes the float4 columns c4 = t + T f of every row it reads
      {
        const int to = opaque_tid();
        const int nh = nlist[0], nall = nlist[1];
        float4 acc[NF4];
#pragma unroll
        for (int f = 0; f < NF4; ++f) acc[f] = float4{0.f, 0.f, 0.f, 0.f};
        const bool dump_R = CAP && first && i == a.cap_i && a.cap_R;
        const bool dump_next = CAP && first && i - 1 == a.cap_i && a.cap_R_next;
        // one row's values: deflate (written back to the row's home), accumulate, check
        auto consume = [&](float4 (&val)[NF4], float ur, float up, int l, auto home) {
          if (up != 0.f) {
#pragma unroll
            for (int f = 0; f < NF4; ++f) {
              const int c4 = to + T * f;
              if (c4 < n4) {
                const char4 vc = vp4[c4];
                if (vc.x != 0 || vc.y != 0 || vc.z != 0 || vc.w != 0) {
                  float4 x = val[f];
                  x.x = vc.x != 0 ? fmaf(-dprev, up * (float)vc.x, x.x) : x.x;
                  x.y = vc.y != 0 ? fmaf(-dprev, up * (float)vc.y, x.y) : x.y;
                  x.z = vc.z != 0 ? fmaf(-dprev, up * (float)vc.z, x.z) : x.z;
                  x.w = vc.w != 0 ? fmaf(-dprev, up * (float)vc.w, x.w) : x.w;
                  val[f] = x;
                  home[c4] = x;
                }
              }
            }
          }
#pragma unroll
          for (int f = 0; f < NF4; ++f) {
            acc[f].x = fmaf(ur, val[f].x, acc[f].x);
            acc[f].y = fmaf(ur, val[f].y, acc[f].y);
            acc[f].z = fmaf(ur, val[f].z, acc[f].z);
            acc[f].w = fmaf(ur, val[f].w, acc[f].w);
          }
          if (first) {
            // this thread's share of the single-entry bound (exact: x^2 is exact in fp64)
#pragma unroll
            for (int f = 0; f < NF4; ++f) {
              const int c4 = to + T * f;
              if (c4 < n4) {
                const float xs[4] = {val[f].x, val[f].y, val[f].z, val[f].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const double x = (double)xs[e];
                  rmax2 = fmax(rmax2, x * x * (a.wt ? (double)a.wt[4 * c4 + e] : 1.0));
                }
              }
            }
          }
          if (dump_R || dump_next) {
#pragma unroll
            for (int f = 0; f < NF4; ++f) {
              const int c4 = to + T * f;
              if (c4 < n4) {
                if (dump_R) reinterpret_cast<float4*>(a.cap_R + (int64_t)(row0 + l) * n)[c4] = val[f];
                if (dump_next) reinterpret_cast<float4*>(a.cap_R_next + (int64_t)(row0 + l) * n)[c4] = val[f];
              }
            }
          }
        };
        // device-memory rows: NB rows of loads in flight
        for (int q0 = 0; q0 < nh; q0 += NB) {
          float4 val[NB][NF4];
          int lr[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            lr[b] = uniform_i(q0 + b < nh ? rl[q0 + b] : 0);
            const float4* r4 = reinterpret_cast<const float4*>(R + (int64_t)(row0 + lr[b]) * n);
#pragma unroll
            for (int f = 0; f < NF4; ++f) {
              const int c4 = to + T * f;
              val[b][f] = float4{0.f, 0.f, 0.f, 0.f};
              if (q0 + b < nh && c4 < n4) val[b][f] = r4[c4];
            }
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if (q0 + b >= nh) break;   // uniform
            const int l = lr[b];
            consume(val[b], uniform_f(u_own[l]), first ? uniform_f(up_own[l]) : 0.f, l,
                    reinterpret_cast<float4*>(R + (int64_t)(row0 + l) * n));
          }
        }
        // LDS rows
        for (int q = nh; q < nall; ++q) {
          const int l = uniform_i(rl[q]);
          float4* r4 = rcache + l * n4;
          float4 val[NF4];
#pragma unroll
          for (int f = 0; f < NF4; ++f) {
            const int c4 = to + T * f;
            val[f] = c4 < n4 ? r4[c4] : float4{0.f, 0.f, 0.f, 0.f};
          }
          consume(val, uniform_f(u_own[l]), first ? uniform_f(up_own[l]) : 0.f, l, r4);
        }
        ++rp;
        // publish: the sums are staged in vsh (free until v is made), then column
        // c goes to word (c / CB, g, c % CB) of the partial array, so that each
        // wave writes whole runs of CB words
        float4* st4 = reinterpret_cast<float4*>(vsh);
#pragma unroll
        for (int f = 0; f < NF4; ++f) {
          const int c4 = to + T * f;
          if (c4 < n4) st4[c4] = acc[f];
        }
        __syncthreads();
        const int lg = a.lgCB;
#pragma unroll
        for (int j = 0; j < KR; ++j) {
          const int c = to + T * j;
          if (c < n)
            __hip_atomic_store(a.pslot + ((((int64_t)(c >> lg) * a.G + g)) << lg) + (c & ((1 << lg) - 1)),
                               xw_pack(rp, vsh[c]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // ---- y phase 2: the column block's sums over the G partials ----
      ++ry;
      {
        const int to = opaque_tid();
        const int lg = a.lgCB, cb = 1 << lg;
        const int cbn = min(cb, n - g * cb);   // columns of this block (none past the end)
        const int sub = to >> lg, cl = to & (cb - 1);
        const bool act = cl < cbn;
        const unsigned par = rp & 1u;
        const unsigned* area = a.pslot + (int64_t)g * a.G * cb;
        float s = 0.f;
        bool ok = true;
        if (act) {
          constexpr int QB = 8;   // partial words in flight per lane
          for (int q0 = 0; q0 < kQMax && sub + a.LPC * q0 < a.G; q0 += QB) {
            unsigned w[QB];
#pragma unroll
            for (int q = 0; q < QB; ++q) {
              const int h = sub + a.LPC * (q0 + q);
              w[q] = h < a.G ? __hip_atomic_load(area + h * cb + cl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : par;
            }
#pragma unroll
            for (int q = 0; q < QB; ++q) {
              const int h = sub + a.LPC * (q0 + q);
              if (h < a.G) {
                ok = ok && poll_word(area + h * cb + cl, par, w[q], a.err);
                s += xw_value(w[q]);
              }
            }
          }
        }
        if (!ok) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the wave's lanes of one column (lane mod CB) by a fixed butterfly, then the waves in order
        for (int o = cb; o < kWave; o <<= 1) s += __shfl_xor(s, o, kWave);
        if ((to & (kWave - 1)) < cb) red[(to >> 6) * cb + (to & (kWave - 1))] = s;
        __syncthreads();
        if (to < cbn) {
          float y = 0.f;
#pragma unroll
          for (int q = 0; q < W; ++q) y += red[q * cb + to];
          const unsigned word = xw_pack(ry, y);
#pragma unroll
          for (int r = 0; r < kRep; ++r)
            __hip_atomic_store(a.yslot + r * rep_stride(n) + g * cb + to, word, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // ---- y phase 3: gather y, v = T_tau(y) ----
      {
        const int to = opaque_tid();
        float y[KR], v[KR];
        const bool bad = !gather<T, KR>(a.yslot + rep_of(g) * rep_stride(n), n, ry, y, a.err, to);
        int eg = it == 0 ? egy0 : (it == 1 ? egy1 : egy2);
        if (!ternarize_dist_guess<T, KR>(y, bad, n, a.tau, v, bufs, tslot, ry + rx, eg, cnt, fb, to)) {
          if (to == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        if (it == 0) egy0 = eg; else if (it == 1) egy1 = eg; else egy2 = eg;
        st_nnz_v += cnt;
        st_fb += fb;
#pragma unroll
        for (int j = 0; j < KR; ++j) {
          const int col = to + T * j;
          const float wv = (a.wt && col < n) ? a.wt[col] : 1.f;
          vsh[col] = col < n ? v[j] * wv : 0.f;
          vpl[col] = col < n ? (signed char)v[j] : (signed char)0;
          if (last && v[j] != 0.f) {
            sums[2] += 1.0;
            sums[3] += (double)wv;
          }
        }
        if (last) store_codes<T, KR>(v, n, a.C2 + (int64_t)i * wn, g, a.G, to);
        if (cap) {
          for (int j = 0; j < KR; ++j) {
            const int col = to + T * j;
            if (col < n) {
              if (a.cap_y) a.cap_y[(int64_t)it * n + col] = y[j];
              if (a.cap_v) a.cap_v[(int64_t)it * n + col] = (int8_t)v[j];
            }
          }
        }
      }
      __syncthreads();   // vsh complete
      // ---- x = R diag(w) v: whole rows per wave, published by the wave ----
      ++rx;
      const int xlane = opaque_tid() & (kWave - 1);
      for (int sq = uniform_i(wv_id); sq < rows; sq += W) {
        const int l = sq < H ? L + sq : sq - H;
        const float4 acc4 = sq < H
            ? row_dot<F4>(reinterpret_cast<const float4*>(R + (int64_t)(row0 + l) * n), vs4, n4, xlane)
            : row_dot<F4>(static_cast<const float4*>(rcache + l * n4), vs4, n4, xlane);
        const float sum = wave_sum_to63((acc4.x + acc4.y) + (acc4.z + acc4.w));
        if (xlane == kWave - 1) {
          const unsigned word = xw_pack(rx, sum);
#pragma unroll
          for (int r = 0; r < kRep; ++r)
            __hip_atomic_store(a.xslot + r * rep_stride(m) + row0 + l, word, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // ---- gather x, u = T_tau(x) ----
      {
        const int to = opaque_tid();
        float x[KC], u[KC];
        const bool bad = !gather<T, KC>(a.xslot + rep_of(g) * rep_stride(m), m, rx, x, a.err, to);
        int eg = it == 0 ? egx0 : (it == 1 ? egx1 : egx2);
        if (!ternarize_dist_guess<T, KC>(x, bad, m, a.tau, u, bufs, tslot, ry + rx, eg, cnt, fb, to)) {
          if (to == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        if (it == 0) egx0 = eg; else if (it == 1) egx1 = eg; else egx2 = eg;
        st_nnz_u += cnt;
        st_fb += fb;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          const int row = to + T * j;
          if (row >= row0 && row < row0 + rows) u_own[row - row0] = u[j];
          if (last) {
            sums[0] += (double)u[j] * (double)x[j];
            sums[1] += (u[j] != 0.f) ? 1.0 : 0.0;
          }
        }
        if (last) store_codes<T, KC>(u, m, a.B2 + (int64_t)i * wm, g, a.G, to);
        if (cap) {
          for (int j = 0; j < KC; ++j) {
            const int row = to + T * j;
            if (row < m) {
              if (a.cap_x) a.cap_x[(int64_t)it * m + row] = x[j];
              if (a.cap_u) a.cap_u[(int64_t)it * m + row] = (int8_t)u[j];
            }
          }
        }
      }
    }
    __syncthreads();   // u_own final
    if (t < rows) up_own[t] = u_own[t];

    // ---- scale d = u.x / (nnz_u v^T diag(w) v) (§2.3 step 2, §2.5) ----
    {
      block_sum_f64<T, 4>(sums, bufs[2]);
      const double c = sums[0], nu = sums[1], nv = sums[2];
      const double den = nu * sums[3];
      d32 = den > 0.0 ? (float)(c / den) : 0.f;
      const double dec = den > 0.0 ? c * c / den : 0.0;
      trace_state -= dec;
      if (__any(dec < rmax2) && lane == 0) atomicOr(&sg_win[(i & 1023) >> 5], 1u << (i & 31));
      st_b += (long long)nu;
      st_c += (long long)nv;
      if (g == 0 && t == 0) {
        a.D[i] = d32;
        if (a.trace) a.trace[i] = trace_state;
        if (CAP && i == a.cap_i && a.cap_d) *a.cap_d = d32;
      }
    }
  }

  // ---- deflate the last component; ||R||^2 of the slab ----
  __syncthreads();
  double r2[1] = {0.0};
  const bool dump_next = CAP && a.k > 0 && a.cap_i == a.k - 1 && a.cap_R_next;
  float* rc = reinterpret_cast<float*>(rcache);
  for (int l = 0; l < rows; ++l) {
    const float upl = a.k > 0 ? up_own[l] : 0.f;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int col = t + T * j;
      if (col < n) {
        float* home = l < L ? rc + l * n + col : R + (int64_t)(row0 + l) * n + col;
        float x = *home;
        const float vj = (float)vpl[col];
        if (upl != 0.f && vj != 0.f) {
          x = fmaf(-d32, upl * vj, x);
          *home = x;
        }
        if (dump_next) a.cap_R_next[(int64_t)(row0 + l) * n + col] = x;
        r2[0] += (double)x * (double)x * (a.wt ? (double)a.wt[col] : 1.0);
      }
    }
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
      a.stats[EXTERND_STAT_MODE] = 3;   // persistent streaming
      a.stats[EXTERND_STAT_GRID] = a.G;
      a.stats[EXTERND_STAT_ITERATIONS] = (long long)a.k * a.iters;
    }
  }
}

__global__ void k_persist_finish(const double* __restrict__ r2_partial, int G, const double* __restrict__ a2,
                                 const long long* __restrict__ nonfinite, const unsigned* __restrict__ err,
                                 double* __restrict__ energy, long long* __restrict__ stats,
                                 const unsigned* __restrict__ sg_bits, int64_t sg_words) {
  if (stats) {
    long long c = 0;
    for (int64_t q = threadIdx.x; q < sg_words; q += blockDim.x) c += __popc(sg_bits[q]);
    c = wave_sum(c);
    if (threadIdx.x == 0) stats[EXTERND_STAT_SAFEGUARD] = c;
  }
  if (threadIdx.x != 0) return;
  double r2 = 0.0;
  for (int q = 0; q < G; ++q) r2 += r2_partial[q];
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

struct PerShape {
  int KR, KC;
};
// instantiations: (KR, KC) with n <= 512 KR, m <= 512 KC
constexpr PerShape kPerShapes[] = {{5, 5}, {5, 10}, {10, 5}, {8, 8}, {5, 20}, {20, 5}, {20, 20}};

int pick_persist(int64_t m, int64_t n) {
  for (int i = 0; i < (int)(sizeof(kPerShapes) / sizeof(kPerShapes[0])); ++i)
    if (m <= (int64_t)kPerT * kPerShapes[i].KC && n <= (int64_t)kPerT * kPerShapes[i].KR) return i;
  return -1;
}

struct PerLayout {
  int G, RB, CB, LPC, lgCB;
  int64_t pwords;
  size_t bytes;
};

PerLayout persist_layout(int64_t m, int64_t n, int64_t k, int num_cus) {
  PerLayout L{};
  L.G = std::min(256, std::max(1, num_cus));
  L.RB = (int)((m + L.G - 1) / L.G);
  // column blocks of 16, 32 or 64 words: whole runs for the writers, a wave
  // butterfly for the owner
  L.lgCB = 4;
  while (L.lgCB < 6 && ((int64_t)L.G << L.lgCB) < n) ++L.lgCB;
  L.CB = 1 << L.lgCB;
  L.LPC = kPerT / L.CB;
  L.pwords = (int64_t)((n + L.CB - 1) / L.CB) * L.G * L.CB;
  size_t b = 0;
  b += sizeof(float) * (size_t)(m * n);                                  // R
  b += sizeof(unsigned) * (size_t)L.pwords;                              // partial words
  b += sizeof(unsigned) * (size_t)kRep * (rep_stride((int)n) + rep_stride((int)m));   // y, x words
  b += sizeof(double) * (256 + 4096 + 8) + sizeof(long long) * 8 + sizeof(unsigned) * 64;
  b += sizeof(float) * (size_t)n + sizeof(unsigned) * (size_t)((k + 31) / 32);
  b += 256 * 12;
  L.bytes = b;
  return L;
}

inline char* align256p(char* p) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 255) & ~(uintptr_t)255);
}

template <int KR, int KC>
hipError_t launch_persist(PerArgs& pa, hipStream_t s) {
  void* args[] = {&pa};
  void* fn = pa.cap_i >= 0 ? reinterpret_cast<void*>(&k_seq_persist<kPerT, KR, KC, true>)
                           : reinterpret_cast<void*>(&k_seq_persist<kPerT, KR, KC, false>);
  return hipLaunchCooperativeKernel(fn, dim3(pa.G), dim3(kPerT), args, 0, s);
}

}  // namespace

bool persist_fits(int64_t m, int64_t n, int num_cus) {
  if (m < 1 || n < 1 || (n & 3) != 0) return false;
  if (pick_persist(m, n) < 0) return false;
  const PerLayout L = persist_layout(m, n, 1, num_cus);
  return L.RB <= kRBMax && (int64_t)L.G * L.RB >= m && ((int64_t)L.G << L.lgCB) >= n &&
         (int64_t)L.LPC * kQMax >= L.G;
}

size_t persist_workspace_bytes(int64_t m, int64_t n, int64_t k, int num_cus) {
  return persist_layout(m, n, k, num_cus).bytes;
}

hipError_t run_persist_seq(const SeqArgs& a, void* ws, int num_cus, hipStream_t s) {
  const int si = pick_persist(a.m, a.n);
  if (si < 0 || !persist_fits(a.m, a.n, num_cus)) return hipErrorInvalidValue;
  const PerLayout L = persist_layout(a.m, a.n, a.k, num_cus);
  char* p = align256p(static_cast<char*>(ws));
  float* R = reinterpret_cast<float*>(p);
  p = align256p(p + sizeof(float) * a.m * a.n);
  unsigned* pslot = reinterpret_cast<unsigned*>(p);
  p = align256p(p + sizeof(unsigned) * (size_t)L.pwords);
  unsigned* yslot = reinterpret_cast<unsigned*>(p);
  p = align256p(p + sizeof(unsigned) * kRep * rep_stride((int)a.n));
  unsigned* xslot = reinterpret_cast<unsigned*>(p);
  p = align256p(p + sizeof(unsigned) * kRep * rep_stride((int)a.m));
  double* r2p = reinterpret_cast<double*>(p);
  p = align256p(p + sizeof(double) * 256);
  double* npart = reinterpret_cast<double*>(p);
  p = align256p(p + sizeof(double) * 4096);
  double* a2 = reinterpret_cast<double*>(p);
  p = align256p(p + sizeof(double) * 8);
  long long* nonfinite = reinterpret_cast<long long*>(p);
  p = align256p(p + sizeof(long long) * 8);
  unsigned* err = reinterpret_cast<unsigned*>(p);
  p = align256p(p + sizeof(unsigned) * 64);
  float* wt = a.importance ? reinterpret_cast<float*>(p) : nullptr;
  p = align256p(p + sizeof(float) * a.n);
  unsigned* sg_bits = reinterpret_cast<unsigned*>(p);
  const int64_t sg_words = (a.k + 31) / 32;

  hipError_t e;
  // partial, y and x words start at parity 0 (round 1 is odd)
  if ((e = launch_fill_u32(pslot, L.pwords, 0u, s)) != hipSuccess) return e;
  if ((e = launch_fill_u32(yslot, (int64_t)kRep * rep_stride((int)a.n), 0u, s)) != hipSuccess) return e;
  if ((e = launch_fill_u32(xslot, (int64_t)kRep * rep_stride((int)a.m), 0u, s)) != hipSuccess) return e;
  if ((e = launch_fill_u32(sg_bits, sg_words, 0u, s)) != hipSuccess) return e;
  if ((e = launch_fill_i64(nonfinite, 1, 0, s)) != hipSuccess) return e;
  if ((e = launch_fill_u32(err, 1, 0u, s)) != hipSuccess) return e;
  if (wt && (e = launch_importance_weights(a.importance, a.n, a.lambda, wt, nonfinite, s)) != hipSuccess) return e;
  if ((e = launch_norm2(a.A, a.m * a.n, npart, 4096, a2, nonfinite, s, wt, a.n)) != hipSuccess) return e;
  if (a.stats && (e = launch_fill_i64(a.stats, EXTERND_STATS_LEN, 0, s)) != hipSuccess) return e;
  if ((e = launch_copy_f32(a.A, R, a.m * a.n, s)) != hipSuccess) return e;

  PerArgs pa{};
  pa.R = R;
  pa.m = (int)a.m;
  pa.n = (int)a.n;
  pa.k = (int)a.k;
  pa.tau = a.tau;
  pa.iters = a.iters;
  pa.seed = a.seed;
  pa.G = L.G;
  pa.RB = L.RB;
  pa.CB = L.CB;
  pa.LPC = L.LPC;
  pa.lgCB = L.lgCB;
  pa.B2 = a.B2;
  pa.C2 = a.C2;
  pa.D = a.D;
  pa.trace = a.trace;
  pa.stats = a.stats;
  pa.a2 = a2;
  pa.wt = wt;
  pa.nonfinite = nonfinite;
  pa.pslot = pslot;
  pa.yslot = yslot;
  pa.xslot = xslot;
  pa.err = err;
  pa.r2_partial = r2p;
  pa.sg_bits = sg_bits;
  pa.cap_i = a.capture_component;
  pa.cap_R = a.capture_R ? a.capture_R : a.capture_Rcol;
  pa.cap_R_next = a.capture_R_next;
  pa.cap_y = a.capture_y;
  pa.cap_x = a.capture_x;
  pa.cap_v = a.capture_v;
  pa.cap_u = a.capture_u;
  pa.cap_d = a.capture_d;

  switch (si) {
    case 0: e = launch_persist<5, 5>(pa, s); break;
    case 1: e = launch_persist<5, 10>(pa, s); break;
    case 2: e = launch_persist<10, 5>(pa, s); break;
    case 3: e = launch_persist<8, 8>(pa, s); break;
    case 4: e = launch_persist<5, 20>(pa, s); break;
    case 5: e = launch_persist<20, 5>(pa, s); break;
    default: e = launch_persist<20, 20>(pa, s); break;
  }
  if (e != hipSuccess) return e;
  if (a.capture_component >= 0 && a.capture_R && a.capture_Rcol &&
      (e = launch_copy_f32(a.capture_R, a.capture_Rcol, a.m * a.n, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_persist_finish, dim3(1), dim3(64), 0, s, r2p, L.G, a2, nonfinite, err, a.energy, a.stats,
                     sg_bits, sg_words);
  if (a.norm_a2 && (e = launch_copy_f64(a2, a.norm_a2, 1, s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace externd
