// Block ALS path (ExTernD §2.4): b components are fitted together.
//
// Per block, with U (m x b) and V (n x b) ternary and R the residual:
//   repeat `iters` times:
//     P  = R^T U                     (MFMA contraction over m)
//     V  = T_col( P (U^T U + eps I)^-1 )
//     Q  = R V                       (MFMA contraction over n)
//     U  = T_col( Q (V^T V + eps I)^-1 )
//   solve [(U^T U) o (V^T V)] d = diag(U^T R V)   (diag read off the last Q)
//   R <- R - U diag(d) V^T           (MFMA rank-b update)
// The Gram matrices of ternary factors are exact integers (popcounts of the
// 2-bit codes, or int8 MFMA on the unpacked codes).  The regularised Gram
// inverse is exact fp64 for b > 64; below, Newton-Schulz whose residuals are
// exact (int8 MFMA on base-256 digits) is run to ||I - G'X||_F of about
// 1e-6 (bf16 MFMA updates, split operands); the joint scale solve is fp64.  The
// contractions and the deflation are fp32-accurate (exact products, fp32
// sums) on bf16 MFMA.  T_col applies the mean-threshold ternarizer T_tau
// (§2.2) to each column.  U and V live as 2-bit codes directly in their
// B2 / C2 output rows.
#include "device_common.hpp"
#include "exchange.hpp"
#include "kernels.hpp"
#include "projection.hpp"

namespace externd {

namespace {

constexpr int kMaxB = 128;  // widest block the kernels handle

using f4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;

__device__ inline f4 mfma16x16x4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Ternary value of element e of a row of 2-bit codes.
__device__ inline float tern(const uint32_t* row, int e) {
  return value_of_code((row[e >> 4] >> (2 * (e & 15))) & 3u);
}

// ---------------------------------------------------------------------------
// Starting block U0 (same rule as the sequential path, global component index).
// ---------------------------------------------------------------------------
__global__ void k_block_start(uint64_t seed, int64_t c0, int bb, int64_t m, uint32_t* __restrict__ B2,
                              int* __restrict__ warm_flags) {
  const int64_t wm = (m + 15) / 16;
  if (blockIdx.x == 0 && threadIdx.x < 2) warm_flags[threadIdx.x] = 0;
  const int64_t total = (int64_t)bb * wm;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t comp = idx / wm, w = idx % wm;
    const uint64_t base = start_base(seed, (uint64_t)(c0 + comp));
    uint32_t word = 0;
    for (int e = 0; e < 16; ++e) {
      const int64_t r = w * 16 + e;
      if (r < m) word |= code_of(start_sign(base, (uint64_t)r)) << (2 * e);
    }
    B2[(c0 + comp) * wm + w] = word;
  }
}

// ---------------------------------------------------------------------------
// Exact Gram matrix G = X^T X of a ternary block held as 2-bit code rows
// (X's column i = code row i, wl words).  Workgroup (tile, split) owns the
// 16 x 16 tile (I, J), I >= J, of G over the words [split * words, ...):
// it stages the 32 code rows of the tile in LDS with coalesced loads, thread
// (r, c) takes the pair (16I + r, 16J + c), and the integer partial sums go to
// G with atomics (exact, so order-free).  Per word pair, the product sum is
// popcount(both nonzero) - 2 popcount(both nonzero, signs differ).  G must be
// zeroed beforehand.
// ---------------------------------------------------------------------------
constexpr int kGramChunk = 64;    // words per LDS stage
// words per Gram workgroup: 32 for b <= 64, 64 above (measured best at
// 2560 x 2560, b = 64 and 9728 x 2560, b = 128)
inline int gram_words(int b) { return b <= 64 ? 32 : 64; }
constexpr int kGramSplit = 16;    // words per workgroup of the weighted Gram (one LDS stage)

__device__ __forceinline__ void gram_tile_body(const uint32_t* __restrict__ codes, int64_t wl, int bb,
                                               int* __restrict__ G, int tile, int split, int words,
                                               uint32_t (*rows)[kGramChunk + 1]) {
  const int t = threadIdx.x;
  // triangular tile index -> (I, J), J <= I
  int I = 0;
  while ((I + 1) * (I + 2) / 2 <= tile) ++I;
  const int J = tile - I * (I + 1) / 2;
  const int r = t >> 4, c = t & 15;
  const int i = 16 * I + r, j = 16 * J + c;
  const int64_t w_begin = (int64_t)split * words;
  const int64_t w_end = min(wl, w_begin + words);
  unsigned pos = 0u, neg = 0u;
  for (int64_t w0 = w_begin; w0 < w_end; w0 += kGramChunk) {
    const int cw = (int)min<int64_t>(kGramChunk, w_end - w0);
    __syncthreads();
    for (int e = t; e < 32 * kGramChunk; e += 256) {
      const int row = e / kGramChunk, w = e % kGramChunk;
      const int comp = row < 16 ? 16 * I + row : 16 * J + row - 16;
      rows[row][w] = (w < cw && comp < bb) ? codes[(int64_t)comp * wl + w0 + w] : 0u;
    }
    __syncthreads();
    for (int w = 0; w < cw; ++w) {
      const uint32_t x = rows[r][w], y = rows[16 + c][w];
      const uint32_t both = x & y & 0x55555555u;
      pos += __popc(both);
      neg += __popc(((x ^ y) >> 1) & both);
    }
  }
  const int acc = (int)pos - 2 * (int)neg;
  if (i < bb && j < bb && acc != 0) {
    atomicAdd(G + i * bb + j, acc);
    if (I != J) atomicAdd(G + j * bb + i, acc);
  }
}

__global__ __launch_bounds__(256) void k_gram(const uint32_t* __restrict__ codes, int64_t wl, int bb,
                                              int* __restrict__ G, int words) {
  __shared__ uint32_t rows[32][kGramChunk + 1];
  gram_tile_body(codes, wl, bb, G, (int)blockIdx.x, (int)blockIdx.y, words, rows);
}

// ---------------------------------------------------------------------------
// Weighted Gram matrix G = X^T diag(wt) X (§2.5) of a ternary block held as
// 2-bit code rows over L columns.  Workgroup (tile, split) stages the 32 code
// rows of its 16 x 16 tile and the weights of its kGramSplit words in LDS;
// thread (r, c) adds +-wt over the columns where both codes are nonzero, in
// fp64 and in column order, and writes the split's partial for (i, j) (and
// (j, i)) to Gpart[split].  Every split writes every entry below bb, so no
// zeroing is needed; k_gram_w_reduce then sums the splits in order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gram_w_partial(const uint32_t* __restrict__ codes, int64_t wl, int bb,
                                                        const float* __restrict__ wt, int64_t L,
                                                        double* __restrict__ Gpart) {
  __shared__ uint32_t rows[32][kGramSplit + 1];
  __shared__ float ws[kGramSplit * 16];
  const int t = threadIdx.x;
  int I = 0;
  while ((I + 1) * (I + 2) / 2 <= (int)blockIdx.x) ++I;
  const int J = (int)blockIdx.x - I * (I + 1) / 2;
  const int r = t >> 4, c = t & 15;
  const int i = 16 * I + r, j = 16 * J + c;
  const int64_t w0 = (int64_t)blockIdx.y * kGramSplit;
  const int cw = (int)min<int64_t>(kGramSplit, wl - w0);
  for (int e = t; e < 32 * kGramSplit; e += 256) {
    const int row = e / kGramSplit, w = e % kGramSplit;
    const int comp = row < 16 ? 16 * I + row : 16 * J + row - 16;
    rows[row][w] = (w < cw && comp < bb) ? codes[(int64_t)comp * wl + w0 + w] : 0u;
  }
  for (int e = t; e < kGramSplit * 16; e += 256) {
    const int64_t col = w0 * 16 + e;
    ws[e] = col < L ? wt[col] : 0.f;
  }
  __syncthreads();
  double acc = 0.0;
  for (int w = 0; w < cw; ++w) {
    const uint32_t x = rows[r][w], y = rows[16 + c][w];
    const uint32_t both = x & y & 0x55555555u;
    const uint32_t neg = ((x ^ y) >> 1) & both;
    // every element in column order, the ones not in both adding zero: the
    // same additions as skipping them, without divergent loops
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double wv = (double)ws[w * 16 + e];
      const double sv = ((neg >> (2 * e)) & 1u) ? -wv : wv;
      acc += ((both >> (2 * e)) & 1u) ? sv : 0.0;
    }
  }
  if (i < bb && j < bb) {
    double* Gs = Gpart + (int64_t)blockIdx.y * bb * bb;
    Gs[i * bb + j] = acc;
    if (I != J) Gs[j * bb + i] = acc;
  }
}

__global__ void k_gram_w_reduce(const double* __restrict__ Gpart, int splits, int bb, double* __restrict__ G) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= bb * bb) return;
  double s = 0.0;
  for (int q = 0; q < splits; ++q) s += Gpart[(int64_t)q * bb * bb + e];
  G[e] = s;
}

// ---------------------------------------------------------------------------
// Small dense fp64 linear algebra on one workgroup: the inverse of a
// symmetric positive definite matrix, used to decorrelate the ALS targets
// and to solve for the joint scales.
// ---------------------------------------------------------------------------
constexpr int kCholT = 256;

// Inverse of a symmetric positive definite matrix (b <= 16 T) on one
// workgroup of 4 waves, by the block sweep operator in fp64 with 16 x 16
// pivot blocks and fp64 MFMA (16x16x4) updates.  One step on the pivot
// block K (R the rest) maps
//   A_KK -> -P,  P = A_KK^-1,   A_KR -> P A_KR,   A_RK -> A_RK P,
//   A_RR -> A_RR - (A_RK P) A_KR,
// which keeps the matrix symmetric; after every block has been swept it
// holds -A^-1, negated at the end.  No pivoting is needed: every pivot block
// of the Schur complements of an SPD matrix is SPD.
//
// Layout: the matrix is a T x T grid of 16 x 16 tiles in the fp64 MFMA
// accumulator layout (lane j + 16 g, register v holds row g + 4 v, column j
// of the tile); wave w keeps the tile rows w, w + 4 (acc[r][J] is tile
// (w + 4 r, J)).  Entries from b up to 16 T must hold the identity.  Per
// step the owner of tile row K publishes it in LDS; every wave inverts A_KK
// itself (sweep16), and by the symmetry of P and of the matrix the MFMA
// operands come straight from P's registers and the published row:
//   W^T = P A_KI  (its registers are the A operand of the update),
//   W = A_IK P    (the new tile A_IK),
//   A_IJ -= W A_KJ for J != K,  and for the pivot row itself
//   A_KJ -= (I - P) A_KJ, i.e. A_KJ -> P A_KJ.
// ok is cleared (uniformly) when a pivot is not positive, i.e. when the
// matrix is not positive definite.
// ---------------------------------------------------------------------------
typedef double d4 __attribute__((ext_vector_type(4)));

template <int T>
struct SweepShared {
  double prow[16][16 * T + 2];   // the published tile row (rows of the pivot block)
};

__device__ inline d4 mfma16x16x4f64(double a, double b, d4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ inline double bpermute_f64(int src_lane, double v) {
  const int a = src_lane << 2;
  const int lo = __builtin_amdgcn_ds_bpermute(a, __double2loint(v));
  const int hi = __builtin_amdgcn_ds_bpermute(a, __double2hiint(v));
  return __hiloint2double(hi, lo);
}
__device__ inline double readlane_f64(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}

// Sweep of a 16 x 16 SPD tile inside one wave, pivot by pivot (reciprocals
// by rcp and two Newton steps; the pivot row comes from the lane group that
// holds it, the pivot column from the same row by symmetry).  Leaves -A^-1.
__device__ inline void sweep16(d4& p, bool& ok) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int pp = 0; pp < 16; ++pp) {
    const int gp = pp & 3, vp = pp >> 2;
    const double app = readlane_f64(p[vp], pp + 16 * gp);
    ok = ok && (app > 0.0);
    double inv = __builtin_amdgcn_rcp(app);
    double e = fma(-app, inv, 1.0);
    inv = fma(inv, e, inv);
    e = fma(-app, inv, 1.0);
    inv = fma(inv, e, inv);
    const double rj = bpermute_f64(j + 16 * gp, p[vp]);   // A[pp][j]
    double ci[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) ci[v] = bpermute_f64(g + 4 * v + 16 * gp, p[vp]);   // A[pp][g + 4v]
    const double rjs = rj * inv;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = g + 4 * v;
      const double sc = ci[v] * inv;
      double nv = fma(-sc, rj, p[v]);
      nv = (j == pp) ? sc : nv;
      nv = (i == pp) ? rjs : nv;
      nv = (i == pp && j == pp) ? -inv : nv;
      p[v] = nv;
    }
  }
}

template <int T>
__device__ bool sweep_inverse(d4 (&acc)[(T + 3) / 4][T], int bb, SweepShared<T>& sh) {
  constexpr int TR = (T + 3) / 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  bool ok = true;
  const int nK = (bb + 15) / 16;
  for (int K = 0; K < nK; ++K) {
    if (w == (K & 3)) {
#pragma unroll
      for (int r = 0; r < TR; ++r)
        if (r == (K >> 2)) {
#pragma unroll
          for (int J = 0; J < T; ++J)
#pragma unroll
            for (int v = 0; v < 4; ++v) sh.prow[g + 4 * v][16 * J + j] = acc[r][J][v];
        }
    }
    __syncthreads();
    d4 p;
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = sh.prow[g + 4 * v][16 * K + j];
    sweep16(p, ok);
    p = -p;   // P = A_KK^-1; by symmetry lane i + 16 k, register s also holds P[i][4 s + k]
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int I = w + 4 * r;
      if (I >= T) continue;
      if (I == K) {
        double wa[4];   // -(I - P) as the A operand
#pragma unroll
        for (int q = 0; q < 4; ++q) wa[q] = p[q] - (j == 4 * q + g ? 1.0 : 0.0);
#pragma unroll
        for (int J = 0; J < T; ++J) {
          if (J == K) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[r][J] = mfma16x16x4f64(wa[q], sh.prow[4 * q + g][16 * J + j], acc[r][J]);
        }
#pragma unroll
        for (int J = 0; J < T; ++J)
          if (J == K) acc[r][J] = -p;
      } else {
        d4 wt = {0.0, 0.0, 0.0, 0.0}, wi = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double ak = sh.prow[4 * q + g][16 * I + j];
          wt = mfma16x16x4f64(p[q], ak, wt);   // W^T = P A_KI
          wi = mfma16x16x4f64(ak, p[q], wi);   // W = A_IK P
        }
#pragma unroll
        for (int J = 0; J < T; ++J) {
          if (J == K) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[r][J] = mfma16x16x4f64(-wt[q], sh.prow[4 * q + g][16 * J + j], acc[r][J]);
        }
#pragma unroll
        for (int J = 0; J < T; ++J)
          if (J == K) acc[r][J] = wi;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < TR; ++r)
#pragma unroll
    for (int J = 0; J < T; ++J) acc[r][J] = -acc[r][J];
  return ok;
}

// Row and column of entry v of tile (w + 4 r, J) held by this lane.
__device__ inline int sweep_row(int r, int v) { return 16 * ((threadIdx.x >> 6) + 4 * r) + ((threadIdx.x >> 4) & 3) + 4 * v; }
__device__ inline int sweep_col(int J) { return 16 * J + (threadIdx.x & 15); }

// Ginv = (G + eps I)^-1 with eps = 1e-6 trace(G)/b (fp64, written as fp32).
// G is an exact integer Gram (int, zeroed after being read so the next
// accumulation starts from zero) or a weighted one (double, left as is).
// `fail` is set if G + eps I is not positive definite.  One workgroup.
template <typename GT>
__device__ inline void consume_gram(GT* G, int e) {
  if constexpr (sizeof(GT) == sizeof(int)) G[e] = 0;
}

template <int T, typename GT>  // bb <= 16 T
__device__ __forceinline__ void spd_inverse_body(GT* __restrict__ G, int bb, float* __restrict__ Ginv,
                                 int* __restrict__ fail) {
  constexpr int TR = (T + 3) / 4;
  __shared__ SweepShared<T> sh;
  __shared__ double red[kCholT / kWave];
  const int t = threadIdx.x, w = t >> 6;
  d4 acc[TR][T];
  double diag = 0.0;   // this lane's diagonal entries (integer valued when G is: any order is exact)
#pragma unroll
  for (int r = 0; r < TR; ++r)
#pragma unroll
    for (int J = 0; J < T; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = sweep_row(r, v), j = sweep_col(J);
        const bool in = w + 4 * r < T && i < bb && j < bb;
        acc[r][J][v] = in ? (double)G[i * bb + j] : (i == j ? 1.0 : 0.0);
        if (in) consume_gram(G, i * bb + j);
        if (in && i == j) diag += acc[r][J][v];
      }
  const double eps = 1e-6 * block_sum<kCholT>(diag, red) / bb;
#pragma unroll
  for (int r = 0; r < TR; ++r)
#pragma unroll
    for (int J = 0; J < T; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (sweep_row(r, v) == sweep_col(J) && sweep_col(J) < bb) acc[r][J][v] += eps;
  const bool ok = sweep_inverse<T>(acc, bb, sh);
  if (!ok && t == 0) *fail = 1;
#pragma unroll
  for (int r = 0; r < TR; ++r)
#pragma unroll
    for (int J = 0; J < T; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = sweep_row(r, v), j = sweep_col(J);
        if (w + 4 * r < T && i < bb && j < bb) Ginv[i * bb + j] = (float)acc[r][J][v];
      }
}


// ---------------------------------------------------------------------------
// The two contractions, on bf16 MFMA (16x16x32) with exact fp32 inputs.  A
// residual entry x is split as x = h + mid + lo, three bf16 numbers whose sum
// is exact (each part keeps 8 significant bits of the 24: h is x with the
// low 16 bits cleared, mid the same of x - h, lo what remains), and the
// ternary factor is exact in bf16, so every product is exact and each of the
// three MFMA passes accumulates in fp32, like an fp32 contraction.
//
// A workgroup (4 waves) takes 64 outputs (columns of R for P = U^T R, rows of
// R for Q = R V) and one split of the contracted dimension, walked in chunks
// of 64.  Per chunk the block's codes are decoded once into bf16 rows in LDS
// (double buffered, one barrier per chunk), each wave loads its R values,
// splits them, and runs 3 x NSUB MFMAs per 32-long slab, the ternary operand
// read from LDS.  Loads read clamped addresses and select 0 outside the
// matrix (no branches).  Components from bb up to 16 NSUB have zero codes.
// ---------------------------------------------------------------------------
constexpr int kCT = 256;
constexpr int kChunk = 256;    // splits of the contracted dimension are whole multiples of this when long enough
constexpr int kAC = 64;        // rows (or columns) per staged chunk
constexpr int kAS = kAC + 8;   // bf16 per staged component row (16 bytes of padding: conflict-free reads)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline f4 mfma16x16x32bf16(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Decoded ternary rows of the chunk: a[buf][component][row in chunk].
template <int NSUB>
struct TernStage {
  unsigned short a[2][16 * NSUB][kAS];
};

// The 16 2-bit codes of a word as 16 bf16 (two per dword).  For a code c in
// {0, 1, 3}, c * 0x3F80 + (c & 2) * 0x80 is 0, 0x3F80 (+1) or 0xBF80 (-1);
// the pair (c0, c1) is first spread to bits 0 and 16 by one multiply.
__device__ inline void decode16(uint32_t w, uint32_t (&o)[8]) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t y = (w >> (4 * p)) & 0xFu;
    const uint32_t z = (y * 0x4001u) & 0x30003u;
    o[p] = z * 0x3F80u + (z & 0x20002u) * 0x80u;
  }
}

// Decode the code words [w0, w0 + 4) of components 0 .. 16 NSUB - 1.
template <int NSUB>
__device__ inline void stage_decode(TernStage<NSUB>& st, int buf, const uint32_t* __restrict__ codes, int64_t wl,
                                    int bb, int64_t w0) {
  constexpr int kWords = 16 * NSUB * (kAC / 16);
  for (int e = threadIdx.x; e < kWords; e += kCT) {
    const int comp = e / (kAC / 16), wi = e % (kAC / 16);
    const bool ok = comp < bb && w0 + wi < wl;
    const uint32_t x = codes[ok ? (int64_t)comp * wl + w0 + wi : 0];
    uint32_t o[8];
    decode16(ok ? x : 0u, o);
    u32x4* dst = reinterpret_cast<u32x4*>(&st.a[buf][comp][wi * 16]);
    dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4{o[4], o[5], o[6], o[7]};
  }
}

// x = h + mid + lo exactly, as three bf16x8 operands.
__device__ inline void split3(const float (&x)[8], bf16x8& h, bf16x8& mid, bf16x8& lo) {
  uint32_t hw[4], mw[4], lw[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u0 = __float_as_uint(x[2 * p]), u1 = __float_as_uint(x[2 * p + 1]);
    const float r0 = x[2 * p] - __uint_as_float(u0 & 0xFFFF0000u);
    const float r1 = x[2 * p + 1] - __uint_as_float(u1 & 0xFFFF0000u);
    const uint32_t v0 = __float_as_uint(r0), v1 = __float_as_uint(r1);
    const float l0 = r0 - __uint_as_float(v0 & 0xFFFF0000u);
    const float l1 = r1 - __uint_as_float(v1 & 0xFFFF0000u);
    hw[p] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // the high halves of u0, u1
    mw[p] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
    lw[p] = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
  }
  h = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
  mid = __builtin_bit_cast(bf16x8, u32x4{mw[0], mw[1], mw[2], mw[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
}

// The 3 NSUB MFMAs of one 32-long slab: the ternary operand of lane
// (i + 16 g) is component 16 sub + i at positions 8 g .. 8 g + 7 of the slab.
template <int NSUB>
__device__ inline void slab_mfma(const TernStage<NSUB>& st, int buf, int slab, int i, int g, const float (&x)[8],
                                 f4 (&acc)[NSUB]) {
  bf16x8 h, mid, lo;
  split3(x, h, mid, lo);
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&st.a[buf][16 * sub + i][32 * slab + 8 * g]);
    acc[sub] = mfma16x16x32bf16(a, h, acc[sub]);
    acc[sub] = mfma16x16x32bf16(a, mid, acc[sub]);
    acc[sub] = mfma16x16x32bf16(a, lo, acc[sub]);
  }
}

// Pt_part[split][i][c] = sum over the split's rows r of U[r][i] R[r][c].
// Wave w owns columns 64 bx + 16 w + j (j = lane % 16); lane (j + 16 g)
// supplies rows 8 g .. 8 g + 7 of each slab of its column.
template <int NSUB>
__device__ __forceinline__ void contract_ut_r_body(const float* __restrict__ R, int64_t m, int64_t n,
                                   const uint32_t* __restrict__ Ucodes, int64_t wm, int bb,
                                   int64_t rows_per_split, float* __restrict__ Pt_part, int bx, int by,
                                   TernStage<NSUB>& st) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int64_t col = (int64_t)bx * 64 + 16 * w + j;
  const bool colok = col < n;
  const float* Rc = R + (colok ? col : 0);
  const int64_t r_begin = (int64_t)by * rows_per_split;
  const int64_t r_end = min(m, r_begin + rows_per_split);
  f4 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = f4{0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  for (int64_t cb = r_begin; cb < r_end; cb += kAC, buf ^= 1) {
    float xv[kAC / 32][8];
#pragma unroll
    for (int s = 0; s < kAC / 32; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t row = cb + 32 * s + 8 * g + e;
        const bool ok = row < r_end && colok;
        const float x = Rc[(ok ? row : r_begin) * n];
        xv[s][e] = ok ? x : 0.f;
      }
    stage_decode<NSUB>(st, buf, Ucodes, wm, bb, cb >> 4);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kAC / 32; ++s) slab_mfma<NSUB>(st, buf, s, j, g, xv[s], acc);
  }
  // D[i][c]: lane holds components 16 s + 4 g + v, column j
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int comp = 16 * s + 4 * g + v;
      if (comp < bb && colok) Pt_part[((int64_t)by * bb + comp) * n + col] = acc[s][v];
    }
  }
}

// Qt_part[split][i][r] = sum over the split's columns c of R[r][c] V[c][i]
// (with W: fl(R[r][c] wt[c]) V[c][i], §2.5).  Wave w owns rows
// 64 bx + 16 w + j (j = lane % 16); lane (j + 16 g) loads columns
// 8 g .. 8 g + 7 of each slab of its row as two float4.
template <int NSUB, bool W>
__device__ __forceinline__ void contract_r_v_body(const float* __restrict__ R, int64_t m, int64_t n,
                                  const uint32_t* __restrict__ Vcodes, int64_t wn, int bb,
                                  int64_t cols_per_split, float* __restrict__ Qt_part, int bx, int by,
                                  const float* __restrict__ wt, TernStage<NSUB>& st) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int64_t row = (int64_t)bx * 64 + 16 * w + j;
  const bool rowok = row < m;
  const float* Rr = R + (rowok ? row : 0) * n;
  const int64_t c_begin = (int64_t)by * cols_per_split;
  const int64_t c_end = min(n, c_begin + cols_per_split);
  const bool vec_ok = (n % 4) == 0;
  f4 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = f4{0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  for (int64_t cb = c_begin; cb < c_end; cb += kAC, buf ^= 1) {
    float xv[kAC / 32][8];
#pragma unroll
    for (int s = 0; s < kAC / 32; ++s) {
      const int64_t cc = cb + 32 * s + 8 * g;
      if (vec_ok && cc + 7 < c_end) {
        const float4 x0 = *reinterpret_cast<const float4*>(Rr + cc);
        const float4 x1 = *reinterpret_cast<const float4*>(Rr + cc + 4);
        xv[s][0] = x0.x; xv[s][1] = x0.y; xv[s][2] = x0.z; xv[s][3] = x0.w;
        xv[s][4] = x1.x; xv[s][5] = x1.y; xv[s][6] = x1.z; xv[s][7] = x1.w;
        if constexpr (W) {
          const float4 y0 = *reinterpret_cast<const float4*>(wt + cc);
          const float4 y1 = *reinterpret_cast<const float4*>(wt + cc + 4);
          xv[s][0] *= y0.x; xv[s][1] *= y0.y; xv[s][2] *= y0.z; xv[s][3] *= y0.w;
          xv[s][4] *= y1.x; xv[s][5] *= y1.y; xv[s][6] *= y1.z; xv[s][7] *= y1.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = cc + e < c_end;
          float x = Rr[ok ? cc + e : c_begin];
          if constexpr (W) x *= wt[ok ? cc + e : c_begin];
          xv[s][e] = ok ? x : 0.f;
        }
      }
      if (!rowok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[s][e] = 0.f;
      }
    }
    stage_decode<NSUB>(st, buf, Vcodes, wn, bb, cb >> 4);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kAC / 32; ++s) slab_mfma<NSUB>(st, buf, s, j, g, xv[s], acc);
  }
  // D[i][r]: lane holds components 16 s + 4 g + v, row 64 bx + 16 w + j
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int comp = 16 * s + 4 * g + v;
      if (comp < bb && rowok) Qt_part[((int64_t)by * bb + comp) * m + row] = acc[s][v];
    }
  }
}



// ---------------------------------------------------------------------------
// Decorrelation inverse for a weighted Gram (b <= 64), and for an integer one
// whose contraction is 2^23 long or more (the exact-residual form below
// covers every other b <= 64): X = (G + eps I)^-1, eps = 1e-6 trace(G)/b,
// by the Newton-Schulz iteration  R = I - G'X,  X <- X + X R  on bf16 MFMA in
// one workgroup (256 threads; wave w owns the 16-row tile band w), followed
// by one fp64 refinement.  Since
// R_{k+1} = R_k^2, the Frobenius norm of R squares each step while it is
// below 1.  The start is the previous inverse of the same side (consecutive
// ALS iterations change the codes little), else the Jacobi guess
// X0 = diag(G')^-1; a warm start whose residual norm is not below 1 (below 1
// the iteration is sure to converge) is replaced by the Jacobi guess, so is a
// warm start whose residual grows, and a Jacobi start whose residual grows by
// X0 = I / ||G'||_inf, which converges for every symmetric positive definite G'.  All loads
// are issued first; each lane keeps its 16 entries of X and R in fp32
// registers (the MFMA output layout) and stores their bf16 parts in LDS; the
// residual norm is summed in fp32 (wave DPP sums, the wave partials published
// with R by one barrier), and a step costs three barriers.  The
// iteration stops when ||R||_F < 1e-4, after the update of a step that found
// ||R||_F < 1e-2 (the next residual is its square, so it is not computed), or
// once ||R||_F < 1e-3 stops falling by more than half (the fp32 floor); a run that does not get there within 40
// steps is counted in stats[EXTERND_STAT_INVERSE_UNCONVERGED]; the steps
// taken and the replaced warm starts are counted too.  The result is within
// 1e-4 relative of the exact inverse (usually far closer: each step squares
// the residual); the targets it decorrelates are then ternarized, which only
// an entry that close to its threshold would notice.  G (integer valued)
// is zeroed after being read so the next Gram accumulation starts from zero.
// ---------------------------------------------------------------------------
constexpr int kNsB = 64;
// The products run on bf16 MFMA (16x16x32) with every fp32 operand split
// exactly into three bf16 parts (x = h + m + l, 8 significant bits each),
// taking the six products of parts whose order of magnitude reaches 2^-16
// (hh, hm, mh, hl, lh, mm): as accurate as an fp32 product.  (Fewer parts in
// the update X R let the slow start from the scaled identity diverge on
// nearly singular Grams.)  X and R are kept transposed (Xt[c][k] = X[k][c]):
// as B operands they are read along rows, X as the A operand of X R down
// columns; G' is symmetric, so its store serves either way.  Each 64 x 64
// part is stored without padding, the 16-byte chunks of row r permuted by
// r mod 8, so the 16 rows one operand load touches fall in different banks.
struct NsShared {
  unsigned short Gp[3][kNsB * kNsB];   // parts of G'
  unsigned short Xt[3][kNsB * kNsB];   // parts of X, transposed
  unsigned short Rt[3][kNsB * kNsB];   // parts of R, transposed
  float red[kCT / kWave];              // per-wave partials of ||R||_F^2
  double dred[kCT / kWave];
  double diag64[kNsB];                 // G_ii + eps in fp64 (the refinement's diagonal)
};
// Index of element (row, k) of a stored part.
__device__ inline int ns_at(int row, int k) { return row * kNsB + ((((k >> 3) ^ (row & 7))) << 3) + (k & 7); }
// Row stride (fp32 words) of the refinement's fp32 copies of G' and X.
constexpr int kNsPad = 68;
static_assert(kNsB * kNsPad * 4 <= 3 * kNsB * kNsB * 2, "an fp32 copy fits in the space of three bf16 parts");

__device__ inline double ns_block_max(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int q = 1; q < kCT / kWave; ++q) r = fmax(r, red[q]);
  return r;
}

// The three bf16 parts of x (bit patterns in the low halves): x = h + m + l exactly.
__device__ inline void ns_split3(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t u = __float_as_uint(x);
  const float r = x - __uint_as_float(u & 0xFFFF0000u);
  const uint32_t v = __float_as_uint(r);
  const float q = r - __uint_as_float(v & 0xFFFF0000u);
  h = u >> 16;
  m = v >> 16;
  l = __float_as_uint(q) >> 16;
}

// The lane's 16 entries val[J][v], at (row 16 w + 4 g + v, column 16 J + j),
// stored transposed as three parts: dst[p] element (16 J + j, 16 w + 4 g + v),
// four consecutive entries per 8-byte store.
__device__ inline void ns_store_t(unsigned short (*dst)[kNsB * kNsB], const f4 (&val)[4], int w, int j, int g) {
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    uint32_t hp[4], mp[4], lp[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) ns_split3(val[J][v], hp[v], mp[v], lp[v]);
    const int at = ns_at(16 * J + j, 16 * w + 4 * g);
    *reinterpret_cast<uint2*>(&dst[0][at]) = uint2{hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16)};
    *reinterpret_cast<uint2*>(&dst[1][at]) = uint2{mp[0] | (mp[1] << 16), mp[2] | (mp[3] << 16)};
    *reinterpret_cast<uint2*>(&dst[2][at]) = uint2{lp[0] | (lp[1] << 16), lp[2] | (lp[3] << 16)};
  }
}

// Eight consecutive k (k0 a multiple of 8) of row `row`.
__device__ inline bf16x8 ns_ld(const unsigned short* buf, int row, int k0) {
  return *reinterpret_cast<const bf16x8*>(&buf[ns_at(row, k0)]);
}
// Elements (k0 .. k0 + 7, col): eight consecutive k down column col.
__device__ inline bf16x8 ns_ld_col(const unsigned short* buf, int k0, int col) {
  uint32_t q[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    q[e] = (uint32_t)buf[ns_at(k0 + 2 * e, col)] | ((uint32_t)buf[ns_at(k0 + 2 * e + 1, col)] << 16);
  return __builtin_bit_cast(bf16x8, u32x4{q[0], q[1], q[2], q[3]});
}
__device__ inline f4 ns_mfma6(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f4 acc) {
  acc = mfma16x16x32bf16(a[0], b[0], acc);
  acc = mfma16x16x32bf16(a[0], b[1], acc);
  acc = mfma16x16x32bf16(a[1], b[0], acc);
  acc = mfma16x16x32bf16(a[0], b[2], acc);
  acc = mfma16x16x32bf16(a[2], b[0], acc);
  acc = mfma16x16x32bf16(a[1], b[1], acc);
  return acc;
}

// acc[J] += (G' X)(rows 16 w .., columns 16 J ..): A = G' rows, B[k][c] =
// X[k][c] = Xt[c][k]; lane (i + 16 g) supplies k = 32 kc + 8 g .. + 7.
__device__ inline void ns_gemm_gx(const NsShared& sh, int w, int i, int g, f4 (&acc)[4]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int k0 = 32 * kc + 8 * g;
    bf16x8 a[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) a[p] = ns_ld(sh.Gp[p], 16 * w + i, k0);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      bf16x8 b[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) b[p] = ns_ld(sh.Xt[p], 16 * J + i, k0);
      acc[J] = ns_mfma6(a, b, acc[J]);
    }
  }
}
// acc[J] += (X R)(rows 16 w .., columns 16 J ..): A[r][k] = X[r][k] = Xt[k][r]
// (down a column of the transposed store), B[k][c] = R[k][c] = Rt[c][k].
__device__ inline void ns_gemm_xr(const NsShared& sh, int w, int i, int g, f4 (&acc)[4]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int k0 = 32 * kc + 8 * g;
    bf16x8 a[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) a[p] = ns_ld_col(sh.Xt[p], k0, 16 * w + i);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      bf16x8 b[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) b[p] = ns_ld(sh.Rt[p], 16 * J + i, k0);
      acc[J] = ns_mfma6(a, b, acc[J]);
    }
  }
}

template <typename GT>
__device__ __forceinline__ void ns_inverse_body(GT* __restrict__ G, int bb, float* __restrict__ X,
                                                int* __restrict__ warm_flag,
                                                long long* __restrict__ stats, NsShared& sh) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
  const int i16 = lane & 15, g = lane >> 4;
  const int warm = *warm_flag;
  // this lane's entries: (r, c) = (16 w + 4 g + v, 16 J + i16); every load first
  GT gv[4][4];
  f4 xv[4];
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
      gv[J][v] = (r < bb && c < bb) ? G[r * bb + c] : (GT)0;
    }
  if (warm) {
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
        xv[J][v] = (r < bb && c < bb) ? X[r * bb + c] : ((r == c) ? 1.f : 0.f);
      }
  }
  // trace (each diagonal entry is held by one lane), eps = 1e-6 trace / b
  double trp = 0.0;
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
      if (r < bb && c < bb) {
        consume_gram(G, r * bb + c);
        if (r == c) trp = (double)gv[J][v];
      }
    }
  trp = wave_sum_to63(trp);
  if (lane == kWave - 1) sh.dred[w] = trp;
  __syncthreads();
  double tr = sh.dred[0];
#pragma unroll
  for (int q = 1; q < kCT / kWave; ++q) tr += sh.dred[q];
  const double eps64 = 1e-6 * tr / bb;
  const float eps = (float)eps64;
  // the exact diagonal of G' for the fp64 refinement (1 beyond bb)
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
      if (r == c) sh.diag64[r] = r < bb ? (double)gv[J][v] + eps64 : 1.0;
    }
  // G' = G + eps I (the identity beyond bb), fp32, then its parts in LDS
  f4 gp[4];
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
      float x = (r == c) ? 1.f : 0.f;
      if (r < bb && c < bb) {
        x = (float)gv[J][v];
        if (r == c) x += eps;
      }
      gp[J][v] = x;
    }
  ns_store_t(sh.Gp, gp, w, i16, g);
  // X0 = diag(1 / G'_ii): the Gram of decorrelated ternary columns is close
  // to diagonal, so this is usually far better than the scaled identity; it
  // can diverge when the columns are strongly correlated (the residual then
  // grows), and the scaled identity takes over.
  auto init_jacobi = [&]() {
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
        xv[J][v] = (r == c) ? 1.f / gp[J][v] : 0.f;
      }
  };
  // X0 = I / ||G'||_inf (the largest absolute row sum), for a cold start or
  // a rejected warm one
  auto init_scaled = [&]() {
    double rs[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double a = 0.0;
#pragma unroll
      for (int J = 0; J < 4; ++J) a += fabs((double)gp[J][v]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o);   // the 16 lanes of the row
      rs[v] = a;
    }
    const double rmax = fmax(fmax(rs[0], rs[1]), fmax(rs[2], rs[3]));
    const float alpha = (float)(1.0 / ns_block_max(rmax, sh.dred));
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
        xv[J][v] = (r == c) ? alpha : 0.f;
      }
  };
  int start = warm ? 0 : 1;   // 0 warm, 1 Jacobi, 2 scaled identity
  if (!warm) init_jacobi();
  ns_store_t(sh.Xt, xv, w, i16, g);
  __syncthreads();
  float prev = 3.0e38f;
  bool conv = false, restarted = false;
  int iters_done = 0, since_start = 0;
  for (int it = 0; it < 40; ++it) {
    ++iters_done;
    f4 acc[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) acc[J] = f4{0.f, 0.f, 0.f, 0.f};
    ns_gemm_gx(sh, w, i16, g, acc);
    float rp = 0.f;
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
        const float rv = ((r == c) ? 1.f : 0.f) - acc[J][v];
        acc[J][v] = rv;
        rp = fmaf(rv, rv, rp);
      }
    ns_store_t(sh.Rt, acc, w, i16, g);
    rp = wave_sum_to63(rp);
    if (lane == kWave - 1) sh.red[w] = rp;
    __syncthreads();   // publishes R and the partial norms; every read of Xt by the product done
    float rn2 = sh.red[0];
#pragma unroll
    for (int q = 1; q < kCT / kWave; ++q) rn2 += sh.red[q];
    if (rn2 < 1e-8f) {
      conv = true;
      break;
    }
    const bool bad = !(rn2 < 1e30f) || (start == 0 && since_start == 0 && rn2 >= 1.f) ||
                     (start < 2 && since_start > 0 && rn2 > prev);
    if (bad) {
      if (start == 2) break;  // not finite from the scaled identity: give up
      restarted = true;       // poor warm start: Jacobi; diverging Jacobi: scaled identity
      if (start == 0) init_jacobi();
      else init_scaled();
      ns_store_t(sh.Xt, xv, w, i16, g);
      __syncthreads();
      ++start;
      since_start = 0;
      prev = 3.0e38f;
      continue;
    }
    ++since_start;
    if (rn2 < 1e-6f && rn2 > 0.25f * prev) {
      conv = true;
      break;
    }
    prev = rn2;
    // below 1e-2 the step's own result has residual R^2 < 1e-4: no check after it
    const bool last = rn2 < 1e-4f;
    // X_next = X + X R
    f4 y[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) y[J] = f4{0.f, 0.f, 0.f, 0.f};
    ns_gemm_xr(sh, w, i16, g, y);
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) xv[J][v] += y[J][v];
    __syncthreads();   // every read of Xt and Rt done
    ns_store_t(sh.Xt, xv, w, i16, g);
    __syncthreads();
    if (last) {
      conv = true;
      break;
    }
  }
  // fp64 refinement.  The fp32 iteration above cannot certify better than
  // about 1e-4 (its residual is itself computed in fp32), so the residual
  // R = I - G'X of the fp32 X is formed exactly enough in fp64 (fp64 MFMA
  // 16x16x4 on fp32 copies of G' and X, with the exact fp64 diagonal of G':
  // every product is exact) and one more step X <- X + X R is
  // taken, which leaves a residual of ||R||_F^2 (the update itself is the
  // six-product bf16 form: it only needs the small correction X R to a few
  // digits).  A step is accepted once the fp64 residual is below 1e-3, so
  // the inverse is then known to about 1e-6 relative; otherwise (at most
  // three rounds) it is counted as unconverged.  The fp64 MFMA layout: lane
  // (j + 16 kk) supplies A[j][kk] and B[kk][j] of each 4-long k slice, and
  // output register v of lane (j + 16 g) is entry (g + 4 v, j).
  bool conv64 = false;
  if (conv) {
    __syncthreads();   // every read of Gp, Xt, Rt and red by the loop done
    // fp32 copies for the fp64 products: G' row-major over the parts of G'
    // (no longer needed), X transposed over the parts of R (rewritten
    // below); rows padded to 68 words, so the 16 x 4 lanes of an operand
    // load (row 16 w + i or 16 J + j, word 4 q + kk) hit 64 different banks
    float* g32 = reinterpret_cast<float*>(&sh.Gp[0][0]);
    float* xt32 = reinterpret_cast<float*>(&sh.Rt[0][0]);
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) g32[(16 * w + 4 * g + v) * kNsPad + 16 * J + i16] = gp[J][v];
    for (int round = 0; round < 3 && !conv64; ++round) {
#pragma unroll
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) xt32[(16 * J + i16) * kNsPad + 16 * w + 4 * g + v] = xv[J][v];
      __syncthreads();
      d4 racc[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) racc[J] = d4{0.0, 0.0, 0.0, 0.0};
      const int kk = g;   // this lane's k within a slice
      const int arow = 16 * w + i16;
      float av[kNsB / 4], bv[kNsB / 4][4];
#pragma unroll
      for (int q = 0; q < kNsB / 4; ++q) {
        av[q] = g32[arow * kNsPad + 4 * q + kk];
#pragma unroll
        for (int J = 0; J < 4; ++J) bv[q][J] = xt32[(16 * J + i16) * kNsPad + 4 * q + kk];
      }
#pragma unroll
      for (int q = 0; q < kNsB / 4; ++q) {
        const int kcol = 4 * q + kk;
        const double a = arow == kcol ? sh.diag64[arow] : (double)av[q];
#pragma unroll
        for (int J = 0; J < 4; ++J) racc[J] = mfma16x16x4f64(a, (double)bv[q][J], racc[J]);
      }
      double rp = 0.0;
#pragma unroll
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 16 * w + g + 4 * v, c = 16 * J + i16;
          const double rv = ((r == c) ? 1.0 : 0.0) - racc[J][v];
          racc[J][v] = rv;
          rp = fma(rv, rv, rp);
        }
      rp = wave_sum_to63(rp);
      if (lane == kWave - 1) sh.dred[w] = rp;
      __syncthreads();   // every read of xt32 done before Rt is rewritten
      // R (rounded to fp32: it only enters the small correction) as
      // transposed parts: element (c, r) of Rt holds R[r][c]
#pragma unroll
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint32_t hp, mp, lp;
          ns_split3((float)racc[J][v], hp, mp, lp);
          const int at = ns_at(16 * J + i16, 16 * w + g + 4 * v);
          sh.Rt[0][at] = (unsigned short)hp;
          sh.Rt[1][at] = (unsigned short)mp;
          sh.Rt[2][at] = (unsigned short)lp;
        }
      __syncthreads();
      double rn64 = sh.dred[0];
#pragma unroll
      for (int q = 1; q < kCT / kWave; ++q) rn64 += sh.dred[q];
      if (!(rn64 < 0.25)) break;   // too far for a single step: leave it counted
      conv64 = rn64 < 1e-6;        // ||R||_F < 1e-3
      f4 y[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) y[J] = f4{0.f, 0.f, 0.f, 0.f};
      ns_gemm_xr(sh, w, i16, g, y);
#pragma unroll
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) xv[J][v] += y[J][v];
      __syncthreads();   // every read of Xt, Rt and dred done
      if (!conv64) ns_store_t(sh.Xt, xv, w, i16, g);   // published by the next round's barrier
    }
  }
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * w + 4 * g + v, c = 16 * J + i16;
      if (r < bb && c < bb) X[r * bb + c] = xv[J][v];
    }
  if (t == 0) {
    *warm_flag = 1;
    if (!conv64) atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_INVERSE_UNCONVERGED), 1ull);
    atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_NS_ITERATIONS), (unsigned long long)iters_done);
    if (restarted) atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_NS_RESTARTS), 1ull);
  }
}

// ---------------------------------------------------------------------------
// (G + eps I)^-1 of an exact integer Gram, b <= 64, in one workgroup of four
// waves: Newton-Schulz, X <- X + X R, in which every residual R = I - G'X is
// computed exactly.  The weighted Gram (not integer) keeps the form above.
//
// Layout.  Wave w owns the columns 16 w .. 16 w + 15 of X and of R: lane
// j + 16 g holds the 16 entries (rho(g, q), 16 w + j), q = 0 .. 15, with
// rho(g, q) = 16 (q / 4) + 4 g + q % 4 -- the MFMA accumulator layout of the
// column block's four 16 x 16 tiles.  Every product here is Y[:, w] =
// A Z[:, w] with Z such a column block, and the contracted index is ordered
// to suit it: operand slot (lane group g, element e) of chunk c of the
// 16x16x32 bf16 MFMA stands for k = rho(g, 8 c + e), and slot (g, byte e) of
// the 16x16x64 int8 MFMA for k = rho(g, e).  (Both MFMAs give the same
// (lane group, element) to the same k in A and in B, so any such order
// gives the full sum.)  The B operand is then the wave's own registers,
// unmoved, and the result lands in the same layout.  The A operand entry of
// output tile row I is A[16 I + i][rho(g, .)], which for a symmetric A is
// exactly what lane i + 16 g of wave I holds: G is symmetric, and so is X up
// to rounding (the exact iteration keeps symmetry; a perturbation of X only
// changes the iterate, and the residual is always that of the X held).
//
// Exact residual.  |G_ij| <= L, the length of the contracted dimension
// (below 2^23 here).  Per column, X is rounded to fixed point, Xq =
// rint(X 2^s) with |Xq| < 2^30, which is X up to 2^-31 of the column's
// largest entry (finer than fp32 keeps it); with L > 32639 the grid is 2^22
// (within 2^-23).  G's balanced base-256 digits (two; three when L > 32639)
// and Xq's (four; three) are multiplied on int8 MFMA, each int32 sum below
// 3 * 64 * 128^2, and the digit products of one weight 256^d are
// accumulated together.  Their recombination is an integer below 2^52,
// formed in fp64 without rounding, so R = I - (G Xq + eps Xq) 2^-s carries
// only the rounding of that last step.  (On a nearly singular G' no fp32 X
// reaches a small residual: the iterate with the smallest one is returned
// and the inverse is counted as unconverged.)
//
// A step: X rounded and the three bf16 parts of X written to LDS (two
// buffers); R from registers alone; the partials of ||R||_F^2 to LDS; one
// barrier; then, unless the iteration stops, X <- X + X R on bf16 MFMA with
// both operands in three exact parts (A = the parts of X from LDS, B = the
// parts of R in registers).  Stopping rule: ||R||_F < 1e-6 accepts X as it
// is; ||R||_F < 1e-3 takes one more step (residual about ||R||_F^2) and
// accepts.  Starts: the previous inverse of the same side when its residual
// is below 1, else the Jacobi guess diag(G')^-1, else I / ||G'||_inf (the
// last converges for any SPD matrix); a residual that grows restarts.
// ---------------------------------------------------------------------------
typedef int i4v __attribute__((ext_vector_type(4)));
// Gram entries below this bound have three balanced base-256 digits; longer
// contractions use the fp32 iteration with the fp64 refinement above.
constexpr int64_t kNsxMaxL = 1 << 23;

constexpr int kGlPad = 68;   // row stride of the Gram in LDS: the accesses below are conflict-free
// the ten 16 x 16 tiles (I, J), I <= J, of a symmetric 64 x 64 Gram
constexpr int kTileI[10] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3};
constexpr int kTileJ[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
struct NsxShared {
  union {   // G is read into registers before X's parts are first written (two barriers apart)
    u32x4 xp[2][kCT / kWave][3][2][kWave];   // [buffer][wave][part][chunk][lane]: the parts of X
    int gl[64 * kGlPad];                     // G, summed over the waves' quarters of the codes
  };
  i4v ga[kCT / kWave][3][kWave];           // [tile row][digit][lane]: G's digits, the A operand
  float xbest[kCT / kWave][16][kWave];     // the iterate with the smallest residual so far
  double red[2][kCT / kWave];              // per-wave partials of ||R||_F^2
};

__device__ inline int nsx_row(int g, int q) { return 16 * (q >> 2) + 4 * g + (q & 3); }

// out[d] = byte d of a0, a1, a2, a3 (in that order): a 4 x 4 byte transpose.
__device__ inline void bytes_transpose4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// The int8 operands of 16 integers of magnitude at most 0x7F7F7F7F: d[a]
// holds their balanced base-256 digit a (value = sum_a 256^a d_a, each d_a in
// [-128, 127]), byte q of the 16 for value q.  Adding 0x80808080 makes every
// digit plus 128 a plain byte; the xor takes the 128 off again.
template <int ND>
__device__ inline void digits(const int (&v)[16], i4v (&d)[ND]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t o[4];
    bytes_transpose4(((uint32_t)v[4 * r] + 0x80808080u) ^ 0x80808080u,
                     ((uint32_t)v[4 * r + 1] + 0x80808080u) ^ 0x80808080u,
                     ((uint32_t)v[4 * r + 2] + 0x80808080u) ^ 0x80808080u,
                     ((uint32_t)v[4 * r + 3] + 0x80808080u) ^ 0x80808080u, o);
#pragma unroll
    for (int a = 0; a < ND; ++a) d[a][r] = (int)o[a];
  }
}

__device__ inline i4v mfma_i8(i4v a, i4v b, i4v c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }

// Eight consecutive values (8 c .. 8 c + 7) of a lane's 16 as the three bf16
// parts of a 16x16x32 operand chunk.
__device__ inline void nsx_parts(const float (&x)[16], int c, u32x4 (&p)[3]) {
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ns_split3(x[8 * c + e], h[e], m[e], l[e]);
  p[0] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  p[1] = u32x4{m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16)};
  p[2] = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
}

// The 2-bit codes of a word as the int8 operand: byte 4 q + b holds code
// 4 b + q of the word (the same order in A and B, so the products pair up).
__device__ inline i4v nsx_unpack(uint32_t w) {
  constexpr uint32_t kLut = 0xFF000100u;   // code 0 -> 0, 1 -> +1, 2 -> 0, 3 -> -1
  i4v r;
  r.x = (int)__builtin_amdgcn_perm(0u, kLut, w & 0x03030303u);
  r.y = (int)__builtin_amdgcn_perm(0u, kLut, (w >> 2) & 0x03030303u);
  r.z = (int)__builtin_amdgcn_perm(0u, kLut, (w >> 4) & 0x03030303u);
  r.w = (int)__builtin_amdgcn_perm(0u, kLut, (w >> 6) & 0x03030303u);
  return r;
}

// The Gram blocks [b0, b1) of four code words (see nsx_inverse_body): lane
// i + 16 g reads block b0 + g, b0 + g + 4, ... of the components 16 I + i.
// All loads of a batch are issued unconditionally from clamped addresses and
// only masked where they are used, so they are in flight together.
template <bool VEC>
__device__ __forceinline__ void nsx_gram_accumulate(const uint32_t* __restrict__ codes, int64_t wl, int bb,
                                                    int64_t b0, int64_t b1, int j, int g, i4v (&acc)[10]) {
  const uint32_t* src[4];
  bool has[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    has[I] = 16 * I + j < bb;
    src[I] = codes + (int64_t)(has[I] ? 16 * I + j : 0) * wl;
  }
  constexpr int kGS = 4;   // rounds of four blocks per batch
  for (int64_t sb = b0; sb < b1; sb += 4 * kGS) {
    uint32_t cw[kGS][4][4];   // [round group][I][word]
#pragma unroll
    for (int st = 0; st < kGS; ++st) {
      const int64_t kb = sb + 4 * st + g;
      const int64_t kc = kb < b1 ? kb : b0;   // a block of the wave's range
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if constexpr (VEC) {
          const uint4 v = *reinterpret_cast<const uint4*>(src[I] + 4 * kc);
          cw[st][I][0] = v.x;
          cw[st][I][1] = v.y;
          cw[st][I][2] = v.z;
          cw[st][I][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t wd = 4 * kc + e;
            cw[st][I][e] = src[I][wd < wl ? wd : wl - 1];
          }
        }
      }
    }
#pragma unroll
    for (int st = 0; st < kGS; ++st) {
      if (sb + 4 * st < b1) {   // wave-uniform
        const int64_t kb = sb + 4 * st + g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool okw = kb < b1 && 4 * kb + e < wl;
          i4v u[4];
#pragma unroll
          for (int I = 0; I < 4; ++I) u[I] = nsx_unpack(okw && has[I] ? cw[st][I][e] : 0u);
#pragma unroll
          for (int tt = 0; tt < 10; ++tt) acc[tt] = mfma_i8(u[kTileI[tt]], u[kTileJ[tt]], acc[tt]);
        }
      }
    }
  }
}

// THREE: the contraction is longer than 32639 (G's entries take three
// digits); a template parameter, so that no branch splits the step's tile
// rows into separate basic blocks.
template <bool THREE>
__device__ __forceinline__ void nsx_inverse_body(const uint32_t* __restrict__ codes, int64_t wl, int bb,
                                                 float* __restrict__ X, int* __restrict__ warm_flag,
                                                 long long* __restrict__ stats, NsxShared& sh) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), w = t / kWave;
  const int j = lane & 15, g = lane >> 4;
  const int col = 16 * w + j;
  // the previous inverse, read now (from clamped addresses) and taken below
  // when it is the warm start: its loads fly with the Gram's
  const int warm = *warm_flag;
  float xv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = nsx_row(g, q);
    xv[q] = X[min(r, bb - 1) * bb + min(col, bb - 1)];
  }
  // ---- G = C^T C of the bb code rows (components), exact, on int8 MFMA ----
  // The code words are taken in blocks of four (64 entries); wave w takes a
  // quarter of the blocks, lane group g the blocks g, g + 4, ... of it.  Lane
  // i + 16 g reads the block of components 16 I + i (I = 0 .. 3) with one
  // 16-byte load each, and word e of it is the lane's operand slot in MFMA
  // round e: A of tile row I and B of tile column I at once.  Every round
  // pairs, in every slot, the same code row of the two components, so the
  // rounds sum G over all rows.  The ten tiles I <= J are accumulated and
  // added, mirrored, into the LDS Gram (codes beyond bb are zero, so are
  // their rows and columns).
  for (int e = t; e < 64 * kGlPad; e += kCT) sh.gl[e] = 0;
  {
    const int64_t nblk = (wl + 3) / 4;
    const int64_t b0 = nblk * w / 4, b1 = nblk * (w + 1) / 4;
    // 16-byte loads when every block is aligned and whole, else word loads
    const bool vec = ((reinterpret_cast<uintptr_t>(codes) & 15) == 0) && ((wl & 3) == 0);
    i4v acc[10];
#pragma unroll
    for (int u = 0; u < 10; ++u) acc[u] = i4v{0, 0, 0, 0};
    if (vec) nsx_gram_accumulate<true>(codes, wl, bb, b0, b1, j, g, acc);
    else nsx_gram_accumulate<false>(codes, wl, bb, b0, b1, j, g, acc);
    __syncthreads();   // the LDS Gram is zero
#pragma unroll
    for (int tt = 0; tt < 10; ++tt) {
      const int I = kTileI[tt], J = kTileJ[tt];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * I + 4 * g + v, c = 16 * J + j;   // entry (r, c) of tile (I, J)
        atomicAdd(&sh.gl[r * kGlPad + c], acc[tt][v]);
        if (I != J) atomicAdd(&sh.gl[c * kGlPad + r], acc[tt][v]);
      }
    }
    __syncthreads();   // G complete
  }
  // Wave w takes column block w of G (row block w by symmetry): entries
  // (rho(g, q), 16 w + j), the identity beyond bb.  It leaves their digits in
  // LDS as the A operand of tile row w, with its part of the trace, of
  // ||G'||_inf, and the diagonal entry G_cc this lane's column meets
  // (q = 4 w + j % 4 when g = j / 4).
  int gv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) gv[q] = sh.gl[nsx_row(g, q) * kGlPad + col];
  double trp = 0.0, rsum = 0.0, gdiag = 1.0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int c = nsx_row(g, q);
    if (c == col) {
      if (col >= bb) gv[q] = 1;
      else trp += (double)gv[q];
      gdiag = (double)gv[q];   // held by the lane with g = j / 4 only
    }
    rsum += fabs((double)gv[q]);
  }
  {
    i4v d[3];
    digits<3>(gv, d);
#pragma unroll
    for (int a = 0; a < 3; ++a) sh.ga[w][a][lane] = d[a];
  }
  trp = wave_sum_to63(trp);
  rsum += __shfl_xor(rsum, 16);
  rsum += __shfl_xor(rsum, 32);
  // the largest row sum of the wave's rows (eps is added below, to each row < bb)
  double rmax = rsum;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) rmax = fmax(rmax, __shfl_xor(rmax, o));
  if (lane == kWave - 1) {
    sh.red[0][w] = trp;
    sh.red[1][w] = rmax;
  }
  __syncthreads();   // digits, trace and row-sum partials visible
  const double tr = (sh.red[0][0] + sh.red[0][1]) + (sh.red[0][2] + sh.red[0][3]);
  const double eps64 = 1e-6 * tr / bb;
  // ||G'||_inf: every row sum gains eps at most (rows below bb), an upper
  // bound is all the scaled start needs
  const double rmax_all = fmax(fmax(sh.red[1][0], sh.red[1][1]), fmax(sh.red[1][2], sh.red[1][3])) + eps64;
  if (col < bb) gdiag += eps64;
  const float alpha = (float)(1.0 / rmax_all);
  auto init_jacobi = [&]() {
#pragma unroll
    for (int q = 0; q < 16; ++q) xv[q] = nsx_row(g, q) == col ? (float)(1.0 / gdiag) : 0.f;
  };
  auto init_scaled = [&]() {
#pragma unroll
    for (int q = 0; q < 16; ++q) xv[q] = nsx_row(g, q) == col ? alpha : 0.f;
  };
  if (warm) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = nsx_row(g, q);
      if (!(r < bb && col < bb)) xv[q] = r == col ? 1.f : 0.f;
    }
  } else {
    init_jacobi();
  }
  __syncthreads();   // red[] is reused by the iteration
  int start = warm ? 0 : 1;   // 0 warm, 1 Jacobi, 2 scaled identity
  double prev = 1e300, best = 1e300;
  bool conv = false, restarted = false;
  int evals = 0, since_start = 0, buf = 0;
  for (int it = 0; it < 40; ++it) {
    ++evals;
    // the lane's indices again, opaque: the per-entry masks built from them
    // stay in the step instead of being held (or spilled) across the loop
    const int to = xchg::opaque_tid();
    const int lane = to & (kWave - 1), w = to / kWave;
    const int g = lane >> 4, col = 16 * w + (lane & 15);
    // ---- X to fixed point per column: Xq = rint(X 2^s), |Xq| < 2^30 (2^22
    // with three digits of G); X itself stays as it is ----
    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, fabsf(xv[q]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool okx = mx > 0.f && mx < 3.0e38f;   // false for inf and NaN too
    const int s = okx ? (THREE ? 21 : 29) - ilogbf(mx) : 0;
    int xq[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) xq[q] = okx ? __float2int_rn(ldexpf(xv[q], s)) : 0;
    i4v xd[4];
    digits<4>(xq, xd);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 p[3];
      nsx_parts(xv, c, p);
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) sh.xp[buf][w][pp][c][lane] = p[pp];
    }
    // ---- R = I - (G Xq + eps Xq) 2^-s, exact up to the final rounding ----
    const double sc = ldexp(1.0, -s);
    double rp = okx ? 0.0 : __builtin_nan("");
    float rf[16];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      i4v acc[5], ga[3];
#pragma unroll
      for (int d = 0; d < 5; ++d) acc[d] = i4v{0, 0, 0, 0};
#pragma unroll
      for (int a = 0; a < 3; ++a) ga[a] = sh.ga[I][a][lane];
      // digit products of weight 256^d into acc[d]: two digits of G by
      // four of Xq, or three by three
      // (ordered so that products into one accumulator are four apart)
      acc[0] = mfma_i8(ga[0], xd[0], acc[0]);
      acc[1] = mfma_i8(ga[0], xd[1], acc[1]);
      acc[2] = mfma_i8(ga[0], xd[2], acc[2]);
      if constexpr (THREE) {
        acc[3] = mfma_i8(ga[1], xd[2], acc[3]);
        acc[4] = mfma_i8(ga[2], xd[2], acc[4]);
        acc[1] = mfma_i8(ga[1], xd[0], acc[1]);
        acc[2] = mfma_i8(ga[1], xd[1], acc[2]);
        acc[3] = mfma_i8(ga[2], xd[1], acc[3]);
        acc[2] = mfma_i8(ga[2], xd[0], acc[2]);
      } else {
        acc[3] = mfma_i8(ga[0], xd[3], acc[3]);
        acc[4] = mfma_i8(ga[1], xd[3], acc[4]);
        acc[1] = mfma_i8(ga[1], xd[0], acc[1]);
        acc[2] = mfma_i8(ga[1], xd[1], acc[2]);
        acc[3] = mfma_i8(ga[1], xd[2], acc[3]);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = 4 * I + v, r = nsx_row(g, q);
        const int lo = acc[0][v] + (int)((uint32_t)acc[1][v] << 8);
        const int hi = acc[2][v] + (int)((uint32_t)acc[3][v] << 8);
        double T = fma((double)hi, 65536.0, (double)lo);
        T = fma((double)acc[4][v], 4294967296.0, T);
        const double gx = fma(r < bb ? eps64 : 0.0, (double)xq[q], T) * sc;
        const double rv = (r == col ? 1.0 : 0.0) - gx;
        rp = fma(rv, rv, rp);
        rf[q] = (float)rv;
      }
    }
    rp = wave_sum_to63(rp);
    if (lane == kWave - 1) sh.red[buf][w] = rp;
    __syncthreads();   // the parts of X and the norm partials are visible
    const double rn2 = (sh.red[buf][0] + sh.red[buf][1]) + (sh.red[buf][2] + sh.red[buf][3]);
    if (rn2 < best) {   // kept for an iteration that does not converge
      best = rn2;
#pragma unroll
      for (int q = 0; q < 16; ++q) sh.xbest[w][q][lane] = xv[q];
    }
    if (rn2 < 1e-12) {   // ||R||_F < 1e-6: X as it is
      conv = true;
      break;
    }
    const bool bad = !(rn2 < 1e30) || (start == 0 && since_start == 0 && rn2 >= 1.0) ||
                     (start < 2 && since_start > 0 && rn2 > prev);
    if (bad) {
      if (start == 2) break;   // not finite from the scaled identity: give up
      restarted = true;        // poor warm start: Jacobi; diverging Jacobi: scaled identity
      if (start == 0) init_jacobi();
      else init_scaled();
      ++start;
      since_start = 0;
      prev = 1e300;
      buf ^= 1;
      continue;
    }
    ++since_start;
    prev = rn2;
    const bool last = rn2 < 1e-6;   // ||R||_F < 1e-3: one more step, then accept
    // ---- X <- X + X R ----
    u32x4 rb[2][3];
#pragma unroll
    for (int c = 0; c < 2; ++c) nsx_parts(rf, c, rb[c]);
    // the four tile rows' accumulators take turns, so consecutive MFMAs are
    // independent; the products of ns_mfma6 grouped by the part of X
    f4 y[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) y[I] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 b[3];
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) b[pp] = __builtin_bit_cast(bf16x8, rb[c][pp]);
#pragma unroll
      for (int pa = 0; pa < 3; ++pa) {
        bf16x8 a[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) a[I] = __builtin_bit_cast(bf16x8, sh.xp[buf][I][pa][c][lane]);
#pragma unroll
        for (int pb = 0; pb < 3 - pa; ++pb)   // parts pa + pb <= 2: down to 2^-16
#pragma unroll
          for (int I = 0; I < 4; ++I) y[I] = mfma16x16x32bf16(a[I], b[pb], y[I]);
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) xv[q] += y[q >> 2][q & 3];
    buf ^= 1;
    if (last) {
      conv = true;
      break;
    }
  }
  if (!conv) {   // the best iterate met (each lane reads back its own entries)
#pragma unroll
    for (int q = 0; q < 16; ++q) xv[q] = sh.xbest[w][q][lane];
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = nsx_row(g, q);
    if (r < bb && col < bb) X[r * bb + col] = xv[q];
  }
  if (t == 0) {
    *warm_flag = 1;
    if (!conv) atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_INVERSE_UNCONVERGED), 1ull);
    atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_NS_ITERATIONS), (unsigned long long)evals);
    if (restarted) atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_NS_RESTARTS), 1ull);
  }
}

// One launch per half-step (1-D grid, roles by block index, in dispatch
// order):
//   [0, ngram)        Gram tiles: (tile, split) of the exact Gram of the codes,
//                     added into G with atomics; each then bumps *gram_done
//                     (release).  Only for b > 64 and for contractions of
//                     2^23 and more: up to b = 64 the inverse workgroup forms
//                     the Gram itself and ngram is 0;
//   ngram             the inverse of G' (weighted: G given): the exact-residual
//                     Newton-Schulz up to b = 64 (the fp32 one with the fp64
//                     refinement for a weighted Gram or a contraction of 2^23
//                     and more), the fp64 MFMA block sweep beyond; with Gram
//                     tiles, after *gram_done has reached gram_target
//                     (acquire; a bounded wait, counted in stats[TIMEOUTS] if
//                     it runs out);
//   the rest          the contraction, (bx, by) = (c % tiles, c / tiles).
// Only the inverse waits, and no other workgroup waits on anything, so every
// Gram workgroup runs to completion whatever order the workgroups are
// dispatched in, and the wait ends.  HIP promises no dispatch order; the
// Gram tiles have the lowest indices so that, with the in-index-order
// dispatch of a 1-D grid seen on this hardware, they start first and the
// inverse waits least.  The wait is bounded as well.  The roles share one
// LDS union.  *gram_done counts up over the whole decomposition; the host
// passes the running target.
constexpr unsigned kGramSpinLimit = 1u << 22;

template <int NSUB>
union HalfStepLds {
  NsShared ns;
  NsxShared nsx;
  TernStage<NSUB> cs;
  uint32_t rows[32][kGramChunk + 1];
};
template <>
union HalfStepLds<8> {   // b > 64: the sweep inverse brings its own LDS
  TernStage<8> cs;
  uint32_t rows[32][kGramChunk + 1];
};

template <bool UT, bool W, int NSUB>
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(2))) void k_contract_with_inverse(
    const float* __restrict__ R, int64_t m, int64_t n, const uint32_t* __restrict__ codes, int64_t wl,
    int bb, int64_t per_split, float* __restrict__ Part, void* __restrict__ G,
    float* __restrict__ Ginv, int* __restrict__ warm_flag, long long* __restrict__ stats,
    const float* __restrict__ wt, int ngram, int gsplits, int tiles,
    unsigned long long* __restrict__ gram_done, unsigned long long gram_target) {
  static_assert(!(UT && W), "weights apply to the V-side contraction only");
  __shared__ HalfStepLds<NSUB> lds;
  const int idx = (int)blockIdx.x;
  if (idx < ngram) {
    if constexpr (!W) {
      // gram_words(bb), as a constant: NSUB > 4 exactly when bb > 64
      gram_tile_body(codes, wl, bb, static_cast<int*>(G), idx / gsplits, idx % gsplits, NSUB > 4 ? 64 : 32,
                     lds.rows);
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(gram_done, 1ull, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (idx == ngram) {
    if (ngram > 0) {
      if (threadIdx.x == 0) {
        unsigned spins = 0;
        while (__hip_atomic_load(gram_done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < gram_target) {
          if (++spins > kGramSpinLimit) {
            atomicAdd(reinterpret_cast<unsigned long long*>(stats + EXTERND_STAT_TIMEOUTS), 1ull);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
    }
    if constexpr (NSUB == 8) {   // b > 64: the fp64 sweep; *warm_flag gets 1 if G' is not SPD
      if constexpr (W) spd_inverse_body<8, double>(static_cast<double*>(G), bb, Ginv, warm_flag);
      else spd_inverse_body<8, int>(static_cast<int*>(G), bb, Ginv, warm_flag);
    } else {
      if constexpr (W) ns_inverse_body(static_cast<double*>(G), bb, Ginv, warm_flag, stats, lds.ns);
      else if ((UT ? m : n) > 32639 && (UT ? m : n) < kNsxMaxL) nsx_inverse_body<true>(codes, wl, bb, Ginv, warm_flag, stats, lds.nsx);
      else if ((UT ? m : n) < kNsxMaxL) nsx_inverse_body<false>(codes, wl, bb, Ginv, warm_flag, stats, lds.nsx);
      else ns_inverse_body(static_cast<int*>(G), bb, Ginv, warm_flag, stats, lds.ns);
    }
    return;
  }
  const int c = idx - ngram - 1;
  if constexpr (UT) contract_ut_r_body<NSUB>(R, m, n, codes, wl, bb, per_split, Part, c % tiles, c / tiles, lds.cs);
  else contract_r_v_body<NSUB, W>(R, m, n, codes, wl, bb, per_split, Part, c % tiles, c / tiles, wt, lds.cs);
}

// ---------------------------------------------------------------------------
// Decorrelated target: Xt[i][c] = sum_k Ginv[i][k] * (sum_s Part[s][k][c]).
// grid ceil(L/DW), DW = 16 or 32 columns; 256 threads.  The split partials
// are summed in split order into an LDS tile of bb x DW (rows bb .. up to a
// multiple of 4 are zero), then the product runs on fp32 MFMA (16x16x4):
// wave w takes the 16-row tiles w and w + 4 and every 16-column tile.  Ginv is symmetric, so
// the A operand of lane (i + 16k), Ginv[16 I + i][4 s + k], is read as
// Ginv[4 s + k][16 I + i]: 16 lanes read 64 contiguous bytes.  Writes the
// plain sums too (Sum[k][c]) when `sum_out` is non-null.
// ---------------------------------------------------------------------------
template <int kDecW, int kRows>
__global__ __launch_bounds__(256) void k_decorrelate(const float* __restrict__ Part, int S, int bb,
                                                     int64_t L, const float* __restrict__ Ginv,
                                                     float* __restrict__ Xt, float* __restrict__ sum_out) {
  static_assert(kRows == 64 || kRows == kMaxB, "row capacity");
  __shared__ float Ps[kRows][kDecW + 1];
  const int t = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kDecW;
  const int kb4 = (bb + 3) & ~3;
  const int lane = t & 63, w = t >> 6;
  const int j = lane & 15, k = lane >> 4;
  const int rt = (bb + 15) / 16;
  // With 64 rows each wave needs one row tile of the inverse (16 values per
  // lane): its loads are issued here, with the split partials', so that the
  // two first reads of data the previous launch wrote overlap.  (With 128
  // rows, 32 values per lane for each of two row tiles: loaded below.)
  float av0[16];
  if constexpr (kRows == 64) {
    const int row = 16 * w + j;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int kk = 4 * q + k;
      const bool ok = kk < bb && row < bb && w < rt;
      const float a = Ginv[ok ? (int64_t)kk * bb + row : 0];
      av0[q] = ok ? a : 0.f;
    }
  }
  // the split sums, in split order: every entry of this thread (E of them)
  // loads QB splits before any is added
  constexpr int E = kRows * kDecW / 256;
  constexpr int QB = kDecW == 32 ? 4 : 8;
  float acc_s[E];
#pragma unroll
  for (int u = 0; u < E; ++u) acc_s[u] = 0.f;
  for (int q0 = 0; q0 < S; q0 += QB) {
    float v[E][QB];
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int e = t + 256 * u;
      const int kk = e / kDecW, cc = e % kDecW;
      const int64_t c = c0 + cc;
      const bool ok = kk < bb && c < L;
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const bool okq = ok && q0 + q < S;
        const float x = Part[okq ? ((int64_t)(q0 + q) * bb + kk) * L + c : 0];
        v[u][q] = okq ? x : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < E; ++u)
#pragma unroll
      for (int q = 0; q < QB; ++q) acc_s[u] += v[u][q];
  }
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const int e = t + 256 * u;
    const int kk = e / kDecW, cc = e % kDecW;
    const int64_t c = c0 + cc;
    if (kk < kb4) Ps[kk][cc] = acc_s[u];
    if (sum_out && kk < bb && c < L) sum_out[(int64_t)kk * L + c] = acc_s[u];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int I = w + 4 * r;
    if (I >= rt) continue;   // uniform per wave
    const int row = 16 * I + j;   // A operand row of this lane
    constexpr int CT = kDecW / 16;
    f4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
    // every A operand of the row tile first (at most kRows / 4 per lane)
    float av[kRows / 4];
    if constexpr (kRows == 64) {
#pragma unroll
      for (int q = 0; q < 16; ++q) av[q] = av0[q];
    } else {
#pragma unroll
      for (int q = 0; q < kRows / 4; ++q) {
        const int kk = 4 * q + k;
        const bool ok = kk < bb && row < bb;
        const float a = Ginv[ok ? (int64_t)kk * bb + row : 0];
        av[q] = ok ? a : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < kRows / 4; ++q) {
      if (4 * q >= kb4) break;   // uniform
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma16x16x4(av[q], Ps[4 * q + k][16 * ct + j], acc[ct]);
    }
    // D[4k + v][j]: row 16 I + 4 k + v, column 16 ct + j
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int64_t c = c0 + 16 * ct + j;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * I + 4 * k + v;
        if (i < bb && c < L) Xt[(int64_t)i * L + c] = acc[ct][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// T_tau (§2.2) of every row of Xt (bb rows of length L): one workgroup per
// row.  Codes go to out_codes row i (row stride wl words); nnz[i] gets the
// count; fallbacks counted in *fb.
// ---------------------------------------------------------------------------
constexpr int kTT = 512;

__global__ __launch_bounds__(kTT) void k_row_ternarize(const float* __restrict__ Xt, int64_t L, float tau,
                                                       uint32_t* __restrict__ out_codes, int64_t wl,
                                                       int* __restrict__ nnz, long long* __restrict__ fb,
                                                       long long* __restrict__ nnz_sum,
                                                       const float* __restrict__ Qrows,
                                                       double* __restrict__ rhs_out) {
  __shared__ double scratch[kTT / kWave];
  const int i = blockIdx.x;
  const float* x = Xt + (int64_t)i * L;
  const float* qr = rhs_out ? Qrows + (int64_t)i * L : nullptr;
  uint32_t* codes = out_codes + (int64_t)i * wl;
  const int t = threadIdx.x;
  float mx = 0.f;
  for (int64_t j = t; j < L; j += kTT) mx = fmaxf(mx, fabsf(x[j]));
  const float M = block_max<kTT>(mx, reinterpret_cast<float*>(scratch));
  if (M == 0.f) {
    for (int64_t w = t; w < wl; w += kTT) codes[w] = (w == 0) ? 1u : 0u;
    if (t == 0) {
      if (rhs_out) rhs_out[i] = (double)qr[0];
      nnz[i] = 1;
      atomicAdd(reinterpret_cast<unsigned long long*>(fb), 1ull);
      atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), 1ull);
    }
    return;
  }
  const int s = fixed_point_shift(M, (int)L);
  double q = 0.0;
  for (int64_t j = t; j < L; j += kTT) q += fixed_point_q(fabsf(x[j]), s);
  const double Q = block_sum<kTT>(q, scratch);
  const double thr = fixed_point_threshold(Q, s, tau, L);
  const uint32_t tb = threshold_bits(thr);
  int cnt = 0;
  double rq = 0.0;   // u_i . q_i over this thread's kept entries (joint scale rhs)
  for (int64_t w = t; w < wl; w += kTT) {
    uint32_t word = 0;
    for (int e = 0; e < 16; ++e) {
      const int64_t j = w * 16 + e;
      if (j < L) {
        const float v = x[j];
        if ((__float_as_uint(v) & 0x7fffffffu) > tb) {
          word |= code_of(v) << (2 * e);
          ++cnt;
          if (qr) rq += v > 0.f ? (double)qr[j] : -(double)qr[j];
        }
      }
    }
    codes[w] = word;
  }
  const uint32_t Mb = __float_as_uint(M);
  if (Mb > tb) {
    const int total = block_sum<kTT>(cnt, reinterpret_cast<int*>(scratch));
    if (rhs_out) {
      const double r = block_sum<kTT>(rq, scratch);
      if (t == 0) rhs_out[i] = r;
    }
    if (t == 0) {
      nnz[i] = total;
      atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), (unsigned long long)total);
    }
    return;
  }
  int first = INT32_MAX;
  for (int64_t j = t; j < L; j += kTT)
    if (fabsf(x[j]) == M) { first = (int)j; break; }
  const int idx = block_min_i<kTT>(first, reinterpret_cast<int*>(scratch));
  __syncthreads();
  if (t == 0) {
    codes[idx >> 4] = code_of(x[idx]) << (2 * (idx & 15));
    if (rhs_out) rhs_out[i] = x[idx] > 0.f ? (double)qr[idx] : -(double)qr[idx];
    nnz[i] = 1;
    atomicAdd(reinterpret_cast<unsigned long long*>(fb), 1ull);
    atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), 1ull);
  }
}

// The same for rows of L <= 512 K with the row held in registers: one read of
// the row, and the codes packed from wave ballots (wave w of pass j covers
// entries 512 j + 64 w .. + 63, i.e. code words 32 j + 4 w .. + 3).  The
// maximum and the fixed-point sum are reduced by DPP inside each wave and
// one LDS atomic per wave (one barrier each; the sum's terms are exact
// integers, so the order of the atomics cannot change it); the counts come
// from the ballots, and the joint right-hand side is summed by DPP inside
// each wave and by thread 0 over the waves in index order.
__device__ inline uint32_t spread_bits16(uint32_t v) {   // bit e -> bit 2e
  v &= 0xffffu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  v = (v | (v << 4)) & 0x0F0F0F0Fu;
  v = (v | (v << 2)) & 0x33333333u;
  v = (v | (v << 1)) & 0x55555555u;
  return v;
}

template <int K>
__global__ __launch_bounds__(kTT) void k_row_ternarize_reg(const float* __restrict__ Xt, int64_t L, float tau,
                                                           uint32_t* __restrict__ out_codes, int64_t wl,
                                                           int* __restrict__ nnz, long long* __restrict__ fb,
                                                           long long* __restrict__ nnz_sum,
                                                           const float* __restrict__ Qrows,
                                                           double* __restrict__ rhs_out) {
  constexpr int W = kTT / kWave;
  __shared__ int scratch[W];
  __shared__ int wcnt[W];
  __shared__ double wrq[W];
  __shared__ unsigned s_max;   // bits of the largest |x| (LDS atomic max)
  __shared__ double s_sum;     // the fixed-point sum (LDS atomic add of exact integers)
  const int i = blockIdx.x;
  const float* x = Xt + (int64_t)i * L;
  const float* qr = rhs_out ? Qrows + (int64_t)i * L : nullptr;
  uint32_t* codes = out_codes + (int64_t)i * wl;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  if (t == 0) {
    s_max = 0u;
    s_sum = 0.0;
  }
  float v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t idx = t + (int64_t)kTT * j;
    const float a = x[idx < L ? idx : 0];
    v[j] = idx < L ? a : 0.f;
  }
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) mx = fmaxf(mx, fabsf(v[j]));
  const float wm = wave_max_to63(mx);
  // one LDS atomic per wave; a wave whose entries are all NaN adds nothing,
  // as a NaN operand of fmaxf adds nothing
  if (lane == kWave - 1) atomicMax(&s_max, wm == wm ? __float_as_uint(wm) : 0u);
  __syncthreads();
  const float M = __uint_as_float(s_max);
  if (M == 0.f) {
    for (int64_t q = t; q < wl; q += kTT) codes[q] = (q == 0) ? 1u : 0u;
    if (t == 0) {
      if (rhs_out) rhs_out[i] = (double)qr[0];
      nnz[i] = 1;
      atomicAdd(reinterpret_cast<unsigned long long*>(fb), 1ull);
      atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), 1ull);
    }
    return;
  }
  const int s = fixed_point_shift(M, (int)L);
  double q = 0.0;
#pragma unroll
  for (int j = 0; j < K; ++j) q += fixed_point_q(fabsf(v[j]), s);
  // the terms are integers whose total is below 2^52: any order of the adds
  // gives the same sum
  const double qw = wave_sum_to63(q);
  if (lane == kWave - 1) atomicAdd(&s_sum, qw);
  __syncthreads();
  const double thr = fixed_point_threshold(s_sum, s, tau, L);
  const uint32_t tb = threshold_bits(thr);
  int cnt = 0;       // this wave's kept entries (wave-uniform, from the ballots)
  double rq = 0.0;   // u_i . q_i over this thread's kept entries (joint scale rhs)
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t idx = t + (int64_t)kTT * j;
    const bool keep = idx < L && (__float_as_uint(v[j]) & 0x7fffffffu) > tb;
    const unsigned long long nz = __ballot(keep);
    const unsigned long long ng = __ballot(keep && v[j] < 0.f);
    cnt += __popcll(nz);
    if (qr && keep) rq += v[j] > 0.f ? (double)qr[idx] : -(double)qr[idx];
    if (lane < 4) {
      const int64_t wd = (int64_t)32 * j + 4 * w + lane;
      if (wd < wl)
        codes[wd] = spread_bits16((uint32_t)(nz >> (16 * lane))) | (spread_bits16((uint32_t)(ng >> (16 * lane))) << 1);
    }
  }
  if (__float_as_uint(M) > tb) {
    // per-wave parts in fixed order: DPP inside the wave, waves in index order
    const double rqw = rhs_out ? wave_sum_to63(rq) : 0.0;
    if (lane == kWave - 1) {
      wcnt[w] = cnt;
      wrq[w] = rqw;
    }
    __syncthreads();
    if (t == 0) {
      int total = 0;
      double r = 0.0;
#pragma unroll
      for (int u = 0; u < W; ++u) {
        total += wcnt[u];
        r += wrq[u];
      }
      if (rhs_out) rhs_out[i] = r;
      nnz[i] = total;
      atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), (unsigned long long)total);
    }
    return;
  }
  int first = INT32_MAX;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t idx = t + (int64_t)kTT * j;
    if (idx < L && fabsf(v[j]) == M) first = min(first, (int)idx);
  }
  const int idx = block_min_i<kTT>(first, scratch);
  __syncthreads();   // the zero code words written above are visible block-wide below
  if (t == 0) {
    codes[idx >> 4] = code_of(x[idx]) << (2 * (idx & 15));
    if (rhs_out) rhs_out[i] = x[idx] > 0.f ? (double)qr[idx] : -(double)qr[idx];
    nnz[i] = 1;
    atomicAdd(reinterpret_cast<unsigned long long*>(fb), 1ull);
    atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), 1ull);
  }
}

// ---------------------------------------------------------------------------
// The optimal ternary projection (§2.2) of every row of Xt, the alternative
// to T_tau; outputs as for k_row_ternarize.
// ---------------------------------------------------------------------------
template <int PMAX>
__global__ __launch_bounds__(kTT) void k_row_project(const float* __restrict__ Xt, int64_t L,
                                                     uint32_t* __restrict__ out_codes, int64_t wl,
                                                     int* __restrict__ nnz, long long* __restrict__ fb,
                                                     long long* __restrict__ nnz_sum,
                                                     const float* __restrict__ Qrows,
                                                     double* __restrict__ rhs_out) {
  __shared__ uint64_t keys[PMAX];
  __shared__ ProjScratch sc;
  __shared__ double scratch[kTT / kWave];
  const int i = blockIdx.x;
  const float* x = Xt + (int64_t)i * L;
  const float* qr = rhs_out ? Qrows + (int64_t)i * L : nullptr;
  uint32_t* codes = out_codes + (int64_t)i * wl;
  const int t = threadIdx.x;
  float mx = 0.f;
  for (int64_t j = t; j < L; j += kTT) mx = fmaxf(mx, fabsf(x[j]));
  const float M = block_max<kTT>(mx, reinterpret_cast<float*>(scratch));
  if (M == 0.f) {
    for (int64_t w = t; w < wl; w += kTT) codes[w] = (w == 0) ? 1u : 0u;
    if (t == 0) {
      if (rhs_out) rhs_out[i] = (double)qr[0];
      nnz[i] = 1;
      atomicAdd(reinterpret_cast<unsigned long long*>(fb), 1ull);
      atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), 1ull);
    }
    return;
  }
  const uint64_t K = projection_threshold<kTT>(x, (int)L, M, keys, sc);
  int cnt = 0;
  double rq = 0.0;
  for (int64_t w = t; w < wl; w += kTT) {
    uint32_t word = 0;
    for (int e = 0; e < 16; ++e) {
      const int64_t j = w * 16 + e;
      if (j < L) {
        const float v = x[j];
        if (proj_key(v, (int)j) >= K) {
          word |= code_of(v) << (2 * e);
          ++cnt;
          if (qr) rq += v > 0.f ? (double)qr[j] : -(double)qr[j];
        }
      }
    }
    codes[w] = word;
  }
  const int total = block_sum<kTT>(cnt, reinterpret_cast<int*>(scratch));
  if (rhs_out) {
    const double r = block_sum<kTT>(rq, scratch);
    if (t == 0) rhs_out[i] = r;
  }
  if (t == 0) {
    nnz[i] = total;
    atomicAdd(reinterpret_cast<unsigned long long*>(nnz_sum), (unsigned long long)total);
  }
}

// ---------------------------------------------------------------------------
// Joint scale solve (§2.4): rhs_j = u_j . q_j with q_j the last Q column,
// M = (U^T U) o (V^T V), d = M^-1 rhs in fp64.  M is inverted without a
// ridge; if it is not positive definite (a pivot is not positive, the same
// test a Cholesky factorisation makes) it is inverted again with the ridge
// and the retry is counted.  d -> D[c0 + j]; ||R||^2 prediction -= d . rhs.
// ---------------------------------------------------------------------------
// GVw (optional): the weighted Gram V^T diag(wt) V in place of GV (§2.5).
template <int T>  // bb <= 16 T
__global__ __launch_bounds__(kCholT) void k_joint_solve(int* __restrict__ GU, int* __restrict__ GV,
                                                        const double* __restrict__ GVw,
                                                        int bb, const double* __restrict__ rhs_in,
                                                        float* __restrict__ Dout, double* __restrict__ dscratch,
                                                        double* __restrict__ trace_state,
                                                        double* __restrict__ trace, int64_t blk,
                                                        long long* __restrict__ st, const int* __restrict__ nnz,
                                                        int bstride, const double* __restrict__ dpart,
                                                        int64_t ndpart, const double* __restrict__ dold,
                                                        int* __restrict__ accept,
                                                        const double* __restrict__ mpart, int64_t nmpart) {
  constexpr int TR = (T + 3) / 4;
  __shared__ SweepShared<T> sh;
  __shared__ double rhs[kMaxB];
  __shared__ double dsol[kMaxB];
  __shared__ double s_diag[kMaxB];
  __shared__ double s_tr;
  __shared__ double red[kCholT / kWave];
  const int t = threadIdx.x, w = t >> 6;
  for (int j = t; j < bb; j += kCholT) rhs[j] = rhs_in[j];
  // Loops over partials written by other launches: eight loads in flight
  // per thread (clamped addresses, masked at use), not one round trip each.
  constexpr int kLd = 8;
  // sweep visit: the exact rise of ||R||^2 when the stored block was added back
  double added = 0.0;
  if (dpart) {
    double p = 0.0;
    for (int64_t j0 = t; j0 < ndpart; j0 += (int64_t)kLd * kCholT) {
      double x[kLd];
#pragma unroll
      for (int u = 0; u < kLd; ++u) {
        const int64_t j = j0 + (int64_t)u * kCholT;
        x[u] = dpart[j < ndpart ? j : 0];
      }
#pragma unroll
      for (int u = 0; u < kLd; ++u)
        if (j0 + (int64_t)u * kCholT < ndpart) p += x[u];   // the same order as one at a time
    }
    added = block_sum<kCholT>(p, red);
  }
  // the single-entry bound of the residual this block was fitted to, from
  // the per-wave partials of the launch that last wrote it (appendix §7)
  double bmx = 0.0;
  for (int64_t j0 = t; j0 < nmpart; j0 += (int64_t)kLd * kCholT) {
    double x[kLd];
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int64_t j = j0 + (int64_t)u * kCholT;
      x[u] = mpart[j < nmpart ? j : 0];
    }
#pragma unroll
    for (int u = 0; u < kLd; ++u)
      if (j0 + (int64_t)u * kCholT < nmpart) bmx = fmax(bmx, x[u]);
  }
  const double bound = block_max_f64<kCholT>(bmx, red);
  // M = (U^T U) o (V^T V); solve without a ridge, retry once with one
  d4 acc[TR][T];
  bool ok = false;
#pragma unroll
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (ok) break;   // uniform
    // up to b = 64 every entry is loaded from a clamped index,
    // unconditionally, then masked, so that the loads are in flight together;
    // at b = 128 that many live loads would spill, and they are taken one by one
#pragma unroll
    for (int r = 0; r < TR; ++r)
#pragma unroll
      for (int J = 0; J < T; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = sweep_row(r, v), j = sweep_col(J);
          const bool in = w + 4 * r < T && i < bb && j < bb;
          if constexpr (T <= 4) {
            const int ix = in ? i * bb + j : 0;
            const double gu = (double)GU[ix];
            const double gv = GVw ? GVw[ix] : (double)GV[ix];
            acc[r][J][v] = in ? gu * gv : (i == j ? 1.0 : 0.0);
          } else {
            acc[r][J][v] = in ? (double)GU[i * bb + j] * (GVw ? GVw[i * bb + j] : (double)GV[i * bb + j])
                              : (i == j ? 1.0 : 0.0);
          }
        }
#pragma unroll
    for (int r = 0; r < TR; ++r)
#pragma unroll
      for (int J = 0; J < T; ++J)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = sweep_row(r, v), j = sweep_col(J);
          if (w + 4 * r < T && i < bb && i == j) s_diag[i] = acc[r][J][v];
        }
    __syncthreads();
    if (attempt == 1) {
      if (t == 0) {
        double tr = 0.0;
        for (int i = 0; i < bb; ++i) tr += s_diag[i];
        s_tr = tr;
        atomicAdd(reinterpret_cast<unsigned long long*>(st + EXTERND_STAT_RIDGE_RETRIES), 1ull);
      }
      __syncthreads();
      const double eps = 1e-6 * s_tr / bb;
#pragma unroll
      for (int r = 0; r < TR; ++r)
#pragma unroll
        for (int J = 0; J < T; ++J)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (sweep_row(r, v) == sweep_col(J) && sweep_col(J) < bb) acc[r][J][v] += eps;
    }
    ok = sweep_inverse<T>(acc, bb, sh);
    __syncthreads();
  }
  // d = M^-1 rhs: per lane the sum over its columns of every tile of the row,
  // then over the 16 lanes of its group (xor butterfly, fixed order)
#pragma unroll
  for (int r = 0; r < TR; ++r) {
    if (w + 4 * r >= T) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double s = 0.0;
#pragma unroll
      for (int J = 0; J < T; ++J) {
        const int j = sweep_col(J);
        if (j < bb) s = fma(acc[r][J][v], rhs[j], s);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
      const int i = sweep_row(r, v);
      if ((t & 15) == 0 && i < bb) dsol[i] = s;
    }
  }
  __syncthreads();
  // the block's code counts, summed over the block (exact integers)
  long long nbl = 0, ncl = 0;
  if (!dpart && t < bb) {
    nbl = nnz[t];
    ncl = nnz[bstride + t];
  }
  const long long nb_sum = block_sum<kCholT>(nbl, reinterpret_cast<long long*>(red));
  const long long nc_sum = block_sum<kCholT>(ncl, reinterpret_cast<long long*>(red));
  if (t == 0) {
    double dec = 0.0;
    for (int i = 0; i < bb; ++i) dec += dsol[i] * rhs[i];
    // On a sweep visit the refit replaces the stored block when it lowers
    // ||R||^2 at least as much as the stored block did; otherwise the stored
    // block (codes restored by k_sweep_restore) is deflated again.
    const bool take = !dpart || dec >= added;
    if (take) {
      for (int i = 0; i < bb; ++i) {
        Dout[i] = (float)dsol[i];
        dscratch[i] = (double)(float)dsol[i];
      }
    } else {
      for (int i = 0; i < bb; ++i) dscratch[i] = dold[i];
      atomicAdd(reinterpret_cast<unsigned long long*>(st + EXTERND_STAT_SWEEP_KEPT_OLD), 1ull);
    }
    if (accept) *accept = take ? 1 : 0;
    // Single-entry safeguard check (appendix §7): would the best single entry
    // of the residual this block was fitted to, max_ij w_j R_ij^2, have
    // lowered ||R||^2 more than the block did?  Counted on extraction only.
    if (!dpart && dec < bound)
      atomicAdd(reinterpret_cast<unsigned long long*>(st + EXTERND_STAT_SAFEGUARD), 1ull);
    const double tnew = take ? trace_state[0] + added - dec : trace_state[0];
    trace_state[0] = tnew;
    if (trace) trace[blk] = tnew;
    if (!dpart) {
      st[EXTERND_STAT_NNZ_B] += nb_sum;
      st[EXTERND_STAT_NNZ_C] += nc_sum;
    }
  }
  for (int e = t; e < bb * bb; e += kCholT) {
    GU[e] = 0;
    GV[e] = 0;
  }
}

// ---------------------------------------------------------------------------
// Rank-b deflation R <- R - U diag(d) V^T on bf16 MFMA (16x16x32).  Each
// fp32 scale is split exactly as d = h + mid + lo (three bf16, as in the
// contractions), so every product of a ternary entry with a part is exact
// and the three passes accumulate in fp32.  A workgroup takes a 64 x 64
// tile: the block's codes for its rows (U) and columns (V) are decoded into
// LDS once, U as bf16 [row][component] and V times each part of d as
// [part][column][component], so the operands of lane (i + 16 g) are 8
// consecutive components (16 bytes).  Wave w owns rows 16 w .. 16 w + 15 of
// the tile and its four 16-column sub-tiles.  With a negated d the same
// kernel adds a block back.  When dpart is given, each workgroup also writes
// the exact change of ||R||^2 over its tile (sum of new^2 - old^2 in fp64,
// fixed order; weighted by wt[col] when given) to dpart[tile].
// ---------------------------------------------------------------------------
constexpr int kDfS = kMaxB + 8;   // bf16 per staged row (16 bytes of padding: conflict-free reads)

struct DeflateLds {
  unsigned short u[64][kDfS];      // U[r0 + row][component]
  unsigned short v[3][64][kDfS];   // part p of d times V[c0 + col][component]
};

__global__ __launch_bounds__(256) void k_block_deflate(float* __restrict__ R, int64_t m, int64_t n,
                                                       const uint32_t* __restrict__ Ucodes, int64_t wm,
                                                       const uint32_t* __restrict__ Vcodes, int64_t wn,
                                                       const double* __restrict__ d, int bb,
                                                       double* __restrict__ dpart, const float* __restrict__ wt,
                                                       double* __restrict__ mpart) {
  __shared__ DeflateLds st;
  __shared__ double red[256 / kWave];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int kb = (bb + 31) & ~31;   // components padded to whole 32-long slabs (zero codes)
  // this thread's 16 residual entries, loaded first so that their latency
  // overlaps the staging and the products: row r0 + 16 w + 4 g + v, column
  // c0 + 16 s + i
  float old[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t col = c0 + 16 * s + i;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = r0 + 16 * w + 4 * g + v;
      const bool ok = row < m && col < n;
      const float x = R[ok ? row * n + col : 0];
      old[s][v] = ok ? x : 0.f;
    }
  }
  // stage: 4 code words (64 rows or columns) per component and side
  for (int e = t; e < 2 * kb * 4; e += 256) {
    const bool vside = e >= kb * 4;
    const int ee = vside ? e - kb * 4 : e;
    const int comp = ee >> 2, wi = ee & 3;
    const int64_t w0 = (vside ? c0 : r0) / 16 + wi;
    const int64_t wl = vside ? wn : wm;
    const bool ok = comp < bb && w0 < wl;
    const uint32_t x = (vside ? Vcodes : Ucodes)[ok ? (int64_t)comp * wl + w0 : 0];
    uint32_t o[8];
    decode16(ok ? x : 0u, o);
    if (!vside) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        st.u[16 * wi + 2 * p][comp] = (unsigned short)(o[p] & 0xFFFFu);
        st.u[16 * wi + 2 * p + 1][comp] = (unsigned short)(o[p] >> 16);
      }
    } else {
      // the parts of d[comp] as bf16 bits (d = h + mid + lo exactly)
      const float df = ok ? (float)d[comp] : 0.f;
      const uint32_t u0 = __float_as_uint(df);
      const float r1 = df - __uint_as_float(u0 & 0xFFFF0000u);
      const uint32_t u1 = __float_as_uint(r1);
      const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
      const uint32_t part[3] = {u0 >> 16, u1 >> 16, __float_as_uint(r2) >> 16};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t tv = (o[p] >> (16 * h)) & 0xFFFFu;   // 0, 0x3F80 or 0xBF80
#pragma unroll
          for (int q = 0; q < 3; ++q)
            st.v[q][16 * wi + 2 * p + h][comp] = (unsigned short)(tv ? (part[q] ^ (tv & 0x8000u)) : 0u);
        }
      }
    }
  }
  __syncthreads();
  f4 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = f4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < kb; k0 += 32) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&st.u[16 * w + i][k0 + 8 * g]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        acc[s] = mfma16x16x32bf16(a, *reinterpret_cast<const bf16x8*>(&st.v[q][16 * s + i][k0 + 8 * g]), acc[s]);
  }
  // D[4g + v][i]: row r0 + 16 w + 4 g + v, column c0 + 16 s + i
  double change = 0.0, mx = 0.0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t col = c0 + 16 * s + i;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = r0 + 16 * w + 4 * g + v;
      if (row < m && col < n) {
        const float upd = old[s][v] - acc[s][v];
        R[row * n + col] = upd;
        const double ch = (double)upd * (double)upd - (double)old[s][v] * (double)old[s][v];
        change += wt ? ch * (double)wt[col] : ch;
        const double e = (double)upd * (double)upd;
        mx = fmax(mx, wt ? e * (double)wt[col] : e);
      }
    }
  }
  // the single-entry bound of the new residual (appendix §7), for the next block's check
  if (mpart) wave_max_nonneg_part(mx, mpart);
  if (dpart) {
    const double tot = block_sum<256>(change, red);
    if (threadIdx.x == 0) dpart[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = tot;
  }
}

// ---------------------------------------------------------------------------
// Refinement sweeps (§2.4).  Before a block is revisited its codes and
// scales are saved (the refit overwrites the codes in place), -d is staged
// for adding it back, and the Newton-Schulz warm starts are reset.
// ---------------------------------------------------------------------------
__global__ void k_sweep_prepare(int bb, const uint32_t* __restrict__ Uc, int64_t wm,
                                const uint32_t* __restrict__ Vc, int64_t wn, const float* __restrict__ D,
                                uint32_t* __restrict__ saved, double* __restrict__ dold,
                                double* __restrict__ dneg, int* __restrict__ warm_flags) {
  const int64_t nu = (int64_t)bb * wm, total = nu + (int64_t)bb * wn;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t0 < 2) warm_flags[t0] = 0;
  if (t0 < bb) {
    dold[t0] = (double)D[t0];
    dneg[t0] = -(double)D[t0];
  }
  for (int64_t idx = t0; idx < total; idx += (int64_t)gridDim.x * blockDim.x)
    saved[idx] = idx < nu ? Uc[idx] : Vc[idx - nu];
}

// Put the saved codes back when the joint solve kept the stored block.
__global__ void k_sweep_restore(const int* __restrict__ accept, int bb, uint32_t* __restrict__ Uc, int64_t wm,
                                uint32_t* __restrict__ Vc, int64_t wn, const uint32_t* __restrict__ saved) {
  if (*accept) return;
  const int64_t nu = (int64_t)bb * wm, total = nu + (int64_t)bb * wn;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    if (idx < nu) Uc[idx] = saved[idx];
    else Vc[idx - nu] = saved[idx];
  }
}

// Nonzero codes in `words` 2-bit code words, added to *count (exact).
__global__ void k_count_nonzero(const uint32_t* __restrict__ codes, int64_t words, long long* __restrict__ count) {
  long long c = 0;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words; w += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t x = codes[w];
    c += __popc((x | (x >> 1)) & 0x55555555u);
  }
  c = wave_sum(c);
  if ((threadIdx.x & (kWave - 1)) == 0 && c)
    atomicAdd(reinterpret_cast<unsigned long long*>(count), (unsigned long long)c);
}

__global__ void k_zero_i32(int* p, int64_t count) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = 0;
}
__global__ void k_set_trace(double* ts, const double* a2) {
  if (threadIdx.x == 0 && blockIdx.x == 0) ts[0] = *a2;
}
__global__ void k_block_finish(const double* __restrict__ a2, const double* __restrict__ r2,
                               const long long* __restrict__ nonfinite, double* __restrict__ energy,
                               const long long* __restrict__ local, long long* __restrict__ stats) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double e;
  if (*nonfinite > 0 || local[EXTERND_STAT_TIMEOUTS] > 0) e = __longlong_as_double(0x7ff8000000000000ll);
  else if (*a2 == 0.0) e = 1.0;
  else e = 1.0 - *r2 / *a2;
  *energy = e;
  if (stats) {
    for (int i = 0; i < EXTERND_STATS_LEN; ++i) stats[i] = local[i];
    stats[EXTERND_STAT_MODE] = 2;
  }
}

inline unsigned grid1d(int64_t count, int threads, int64_t cap = 8192) {
  int64_t g = (count + threads - 1) / threads;
  return (unsigned)std::max<int64_t>(1, std::min(g, cap));
}

// Per-wave partial maxima of the single-entry bound a block decomposition
// keeps: enough for the norm pass over A (at most 4096 workgroups) and for
// a deflation (one 64 x 64 tile per workgroup), 4 waves each.
inline int64_t sg_partials(int64_t m, int64_t n) {
  return wave_partials(std::max<int64_t>(4096, ((n + 63) / 64) * ((m + 63) / 64)), 256);
}

struct BlockLayout {
  int S1, S2;            // K splits of the two contractions
  int64_t rows_split, cols_split;
  size_t bytes;
};

BlockLayout layout_for(int64_t m, int64_t n, int b) {
  BlockLayout L{};
  const int64_t tiles1 = (n + 63) / 64, tiles2 = (m + 63) / 64;
  // contraction workgroups per launch: about two per CU; for b <= 64, where
  // the inverse bounds the launch, about one (fewer split partials for the
  // decorrelation to sum)
  const int64_t target = b <= 64 ? 256 : 512;
  int64_t s1 = std::max<int64_t>(1, std::min<int64_t>((target + tiles1 - 1) / tiles1, (m + 255) / 256));
  int64_t s2 = std::max<int64_t>(1, std::min<int64_t>((target + tiles2 - 1) / tiles2, (n + 255) / 256));
  // splits are whole 256-long chunks of the contracted dimension when they
  // can be (the contraction stages codes per chunk), else multiples of 16
  auto round_split = [](int64_t len) {
    return len >= kChunk ? (len + kChunk - 1) / kChunk * kChunk : (len + 15) / 16 * 16;
  };
  L.rows_split = round_split((m + s1 - 1) / s1);
  L.cols_split = round_split((n + s2 - 1) / s2);
  L.S1 = (int)((m + L.rows_split - 1) / L.rows_split);
  L.S2 = (int)((n + L.cols_split - 1) / L.cols_split);
  size_t by = 0;
  by += sizeof(float) * (size_t)(m * n);                    // R
  by += sizeof(float) * (size_t)L.S1 * b * n;               // Pt partials
  by += sizeof(float) * (size_t)L.S2 * b * m;               // Qt partials
  by += sizeof(float) * (size_t)b * (n + m);                // Vt, Ut
  by += sizeof(float) * (size_t)b * m;                      // Qt (last sum)
  by += sizeof(float) * (size_t)2 * b * b;                  // Ginv of the U and V sides
  by += sizeof(int) * (size_t)b * b * 4;                    // Grams
  by += sizeof(int) * (size_t)b * 2;                        // nnz
  by += sizeof(double) * (size_t)(2 * b + 4096 + 16);       // d, rhs, norm partials, scalars
  by += sizeof(long long) * EXTERND_STATS_LEN + sizeof(int) * 4;
  by += sizeof(uint32_t) * (size_t)b * ((m + 15) / 16 + (n + 15) / 16);   // sweeps: saved codes
  by += sizeof(double) * (size_t)(2 * b + ((n + 63) / 64) * ((m + 63) / 64)) + sizeof(int);
  // importance weights: column weights, weighted Gram and its split partials
  by += sizeof(float) * (size_t)n;
  by += sizeof(double) * (size_t)b * b * (1 + ((n + 15) / 16 + kGramSplit - 1) / kGramSplit);
  by += sizeof(unsigned long long) * 2;   // Gram tile counters
  by += sizeof(double) * (size_t)sg_partials(m, n);   // single-entry bound partials
  by += 32 * 256;   // alignment slack of the bump allocations
  L.bytes = by;
  return L;
}

inline char* bump(char*& p, size_t bytes) {
  char* r = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 255) & ~(uintptr_t)255);
  p = r + bytes;
  return r;
}


// The decorrelation: 32-column tiles for b > 64 on rows longer than 4096
// (the product dominates), 16-column ones otherwise (more workgroups for the
// split sums), each sized for its largest block.
inline void launch_decorrelate(int bb, hipStream_t s, const float* Part, int S, int64_t L, const float* Ginv,
                               float* Xt, float* sum_out) {
  if (bb > 64 && L <= 4096)   // short rows: few 32-column tiles, so 16
    hipLaunchKernelGGL((k_decorrelate<16, kMaxB>), dim3((unsigned)((L + 15) / 16)), dim3(256), 0, s, Part, S, bb, L, Ginv, Xt, sum_out);
  else if (bb > 64)
    hipLaunchKernelGGL((k_decorrelate<32, kMaxB>), dim3((unsigned)((L + 31) / 32)), dim3(256), 0, s, Part, S, bb, L, Ginv, Xt, sum_out);
  else
    hipLaunchKernelGGL((k_decorrelate<16, 64>), dim3((unsigned)((L + 15) / 16)), dim3(256), 0, s, Part, S, bb, L, Ginv, Xt, sum_out);
}

// The combined launch, by sub-tile count.  ngram Gram tiles
// (0 when G is computed beforehand), one inverse, tiles x splits contraction
// workgroups.
template <bool UT, bool W>
void launch_combined(int bb, int tiles, int splits, int ngram, int gsplits, hipStream_t s, const float* R, int64_t m,
                     int64_t n, const uint32_t* codes, int64_t wl, int64_t per_split, float* Part, void* G,
                     float* Ginv, int* warm, long long* st, const float* wt, unsigned long long* gram_done,
                     unsigned long long gram_target) {
  const int nsub = (bb + 15) / 16;
  const dim3 grid((unsigned)(ngram + 1 + tiles * splits));
  if (nsub > 4)
    hipLaunchKernelGGL((k_contract_with_inverse<UT, W, 8>), grid, dim3(kCT), 0, s, R, m, n, codes, wl, bb, per_split, Part, G, Ginv, warm, st, wt, ngram, gsplits, tiles, gram_done, gram_target);
  else if (nsub == 1)
    hipLaunchKernelGGL((k_contract_with_inverse<UT, W, 1>), grid, dim3(kCT), 0, s, R, m, n, codes, wl, bb, per_split, Part, G, Ginv, warm, st, wt, ngram, gsplits, tiles, gram_done, gram_target);
  else if (nsub == 2)
    hipLaunchKernelGGL((k_contract_with_inverse<UT, W, 2>), grid, dim3(kCT), 0, s, R, m, n, codes, wl, bb, per_split, Part, G, Ginv, warm, st, wt, ngram, gsplits, tiles, gram_done, gram_target);
  else
    hipLaunchKernelGGL((k_contract_with_inverse<UT, W, 4>), grid, dim3(kCT), 0, s, R, m, n, codes, wl, bb, per_split, Part, G, Ginv, warm, st, wt, ngram, gsplits, tiles, gram_done, gram_target);
}

}  // namespace

size_t block_workspace_bytes(int64_t m, int64_t n, int b) { return layout_for(m, n, b).bytes; }

hipError_t run_block(const BlockArgs& a, void* ws, hipStream_t s) {
  const int64_t m = a.m, n = a.n, k = a.k;
  const int b = a.b;
  if (b > kMaxB || b < 2) return hipErrorInvalidValue;
  const BlockLayout L = layout_for(m, n, b);
  const int64_t wm = (m + 15) / 16, wn = (n + 15) / 16;
  char* p = static_cast<char*>(ws);
  float* R = reinterpret_cast<float*>(bump(p, sizeof(float) * m * n));
  float* Pt_part = reinterpret_cast<float*>(bump(p, sizeof(float) * L.S1 * b * n));
  float* Qt_part = reinterpret_cast<float*>(bump(p, sizeof(float) * L.S2 * b * m));
  float* Vt = reinterpret_cast<float*>(bump(p, sizeof(float) * b * n));
  float* Ut = reinterpret_cast<float*>(bump(p, sizeof(float) * b * m));
  float* Qt = reinterpret_cast<float*>(bump(p, sizeof(float) * b * m));
  float* GinvU = reinterpret_cast<float*>(bump(p, sizeof(float) * 2 * b * b));   // U side, V side
  float* GinvV = GinvU + b * b;
  int* GU = reinterpret_cast<int*>(bump(p, sizeof(int) * 4 * b * b));  // GU, GV, GUf, GVf
  int* GV = GU + b * b;
  int* GUf = GU + 2 * b * b;
  int* GVf = GU + 3 * b * b;
  int* nnz = reinterpret_cast<int*>(bump(p, sizeof(int) * b * 2));
  double* dvec = reinterpret_cast<double*>(bump(p, sizeof(double) * b));
  double* rhs = reinterpret_cast<double*>(bump(p, sizeof(double) * b));
  double* npart = reinterpret_cast<double*>(bump(p, sizeof(double) * 4096));
  double* scal = reinterpret_cast<double*>(bump(p, sizeof(double) * 16));
  long long* st = reinterpret_cast<long long*>(bump(p, sizeof(long long) * EXTERND_STATS_LEN));
  int* fail = reinterpret_cast<int*>(bump(p, sizeof(int) * 4));
  int* warm = fail + 2;   // Newton-Schulz warm-start flags, U side and V side
  // refinement sweeps: saved codes and scales of the visited block, -d, the
  // per-tile rise of ||R||^2 from adding it back, the keep/replace flag
  uint32_t* saved = reinterpret_cast<uint32_t*>(bump(p, sizeof(uint32_t) * b * (wm + wn)));
  double* dold = reinterpret_cast<double*>(bump(p, sizeof(double) * b));
  double* dneg = reinterpret_cast<double*>(bump(p, sizeof(double) * b));
  double* dpart = reinterpret_cast<double*>(bump(p, sizeof(double) * ((n + 63) / 64) * ((m + 63) / 64)));
  int* accept = reinterpret_cast<int*>(bump(p, sizeof(int)));
  // Gram tiles finished inside the combined launches (U side, V side),
  // counting up over the whole decomposition
  unsigned long long* gram_done = reinterpret_cast<unsigned long long*>(bump(p, sizeof(unsigned long long) * 2));
  // per-wave partial maxima of the single-entry bound max_ij w_j R_ij^2 of
  // the current residual (appendix §7): left by the norm pass over A, then
  // by each deflation; sg_n of them are valid
  const dim3 defl_grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
  double* sg_part = reinterpret_cast<double*>(bump(p, sizeof(double) * sg_partials(m, n)));
  int64_t sg_n = 0;
  unsigned long long gram_issued[2] = {0ull, 0ull};
  // importance weighting (§2.5): column weights wt, the weighted V-side Gram
  // V^T diag(wt) V and its per-split partials
  const bool W = a.importance != nullptr;
  const int wsplits = (int)((wn + kGramSplit - 1) / kGramSplit);
  float* wt = reinterpret_cast<float*>(bump(p, sizeof(float) * n));
  double* GVw = reinterpret_cast<double*>(bump(p, sizeof(double) * b * b));
  double* Gwpart = reinterpret_cast<double*>(bump(p, sizeof(double) * b * b * wsplits));
  if (!W) wt = nullptr;
  double* a2 = scal;
  double* r2 = scal + 1;
  double* tstate = scal + 2;

  hipError_t e;
  if ((e = launch_fill_i64(st, EXTERND_STATS_LEN, 0, s)) != hipSuccess) return e;
  if (W && (e = launch_importance_weights(a.importance, n, a.lambda, wt, st + EXTERND_STAT_NONFINITE, s)) != hipSuccess)
    return e;
  if ((e = launch_fill_i64(reinterpret_cast<long long*>(gram_done), 2, 0, s)) != hipSuccess) return e;
  if ((e = launch_norm2(a.A, m * n, npart, 4096, a2, st + EXTERND_STAT_NONFINITE, s, wt, n, sg_part, &sg_n)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(k_set_trace, dim3(1), dim3(1), 0, s, tstate, a2);
  if ((e = launch_copy_f32(a.A, R, m * n, s)) != hipSuccess) return e;

  hipLaunchKernelGGL(k_zero_i32, dim3(grid1d((int64_t)4 * b * b, 256)), dim3(256), 0, s, GU, (int64_t)4 * b * b);
  const int64_t ndpart = (int64_t)defl_grid.x * defl_grid.y;

  // The block iterations from the U held in Uc, then the joint scale solve
  // (d -> Dout) and the deflation.  trace/tidx: where the predicted ||R||^2
  // goes (may be null).  On a sweep visit dpart holds the exact rise of
  // ||R||^2 from adding the stored block back, dold its scales and saved its
  // codes; the solve keeps whichever block lowers ||R||^2 more.
  // cap (optional): record iteration cap->iteration of this block and the
  // final right-hand side (test capture, extraction only).
  auto fit_block = [&](int bb, uint32_t* Uc, uint32_t* Vc, float* Dout, double* trace, int64_t tidx,
                       const double* dpart, const double* dold, const uint32_t* saved,
                       const externd_block_capture* cap) -> hipError_t {
    // column-wise ternarizer: T_tau, or the optimal projection (§2.2)
    auto row_tern = [&](const float* Xt, int64_t L, uint32_t* codes, int64_t wl, int* nz, long long* nz_sum,
                        const float* Qrows, double* rhs_out) {
      if (!a.projection && L <= 5 * kTT)
        hipLaunchKernelGGL(k_row_ternarize_reg<5>, dim3(bb), dim3(kTT), 0, s, Xt, L, a.tau, codes, wl, nz, st + EXTERND_STAT_FALLBACKS, nz_sum, Qrows, rhs_out);
      else if (!a.projection && L <= 20 * kTT)
        hipLaunchKernelGGL(k_row_ternarize_reg<20>, dim3(bb), dim3(kTT), 0, s, Xt, L, a.tau, codes, wl, nz, st + EXTERND_STAT_FALLBACKS, nz_sum, Qrows, rhs_out);
      else if (!a.projection)
        hipLaunchKernelGGL(k_row_ternarize, dim3(bb), dim3(kTT), 0, s, Xt, L, a.tau, codes, wl, nz, st + EXTERND_STAT_FALLBACKS, nz_sum, Qrows, rhs_out);
      else if (L <= 4096)
        hipLaunchKernelGGL(k_row_project<4096>, dim3(bb), dim3(kTT), 0, s, Xt, L, codes, wl, nz, st + EXTERND_STAT_FALLBACKS, nz_sum, Qrows, rhs_out);
      else
        hipLaunchKernelGGL(k_row_project<kProjMaxN>, dim3(bb), dim3(kTT), 0, s, Xt, L, codes, wl, nz, st + EXTERND_STAT_FALLBACKS, nz_sum, Qrows, rhs_out);
    };
    const int nt = (bb + 15) / 16;
    const int gw = gram_words(bb);
    const dim3 gram_u((unsigned)(nt * (nt + 1) / 2), (unsigned)((wm + gw - 1) / gw));
    const dim3 gram_v((unsigned)(nt * (nt + 1) / 2), (unsigned)((wn + gw - 1) / gw));
    const bool own_gu = bb <= 64 && m < kNsxMaxL, own_gv = bb <= 64 && n < kNsxMaxL;
    hipError_t ce = hipSuccess;
    auto cap_copy = [&](const void* src, void* dst, int64_t words) {   // 4-byte words
      if (dst && ce == hipSuccess)
        ce = launch_copy_f32(static_cast<const float*>(src), static_cast<float*>(dst), words, s);
    };
    if (cap) cap_copy(R, cap->R, m * n);
    for (int it = 0; it < a.iters; ++it) {
      const bool capit = cap && it == cap->iteration;
      if (capit) cap_copy(Uc, cap->U_in, (int64_t)bb * wm);
      // V <- T_col( P (U^T U + eps I)^-1 ),  P = R^T U.  The Gram and its
      // inverse depend only on U's codes, so they run as the first
      // workgroups of the contraction launch, concurrently with it
      // (Newton-Schulz up to b = 64, the fp64 sweep beyond).
      {
        // the Gram of U is computed inside the launch, ahead of its inverse:
        // by the inverse workgroup itself up to b = 64 (contractions shorter
        // than 2^23), else by Gram workgroups
        const int ng = own_gu ? 0 : (int)(gram_u.x * gram_u.y);
        gram_issued[0] += (unsigned long long)ng;
        launch_combined<true, false>(bb, (int)((n + 63) / 64), L.S1, ng, (int)gram_u.y, s, R, m, n, Uc, wm, L.rows_split, Pt_part, (void*)GU, GinvU, bb <= 64 ? warm : fail, st, (const float*)nullptr, gram_done, gram_issued[0]);
      }
      if (capit) cap_copy(GinvU, cap->GinvU, (int64_t)bb * bb);
      launch_decorrelate(bb, s, Pt_part, L.S1, n, GinvU, Vt, capit ? cap->P : (float*)nullptr);
      row_tern(Vt, n, Vc, wn, nnz + b, st + EXTERND_STAT_SUM_NNZ_V, (const float*)nullptr, (double*)nullptr);
      if (capit) {
        cap_copy(Vt, cap->Vt, (int64_t)bb * n);
        cap_copy(Vc, cap->V, (int64_t)bb * wn);
      }
      // U <- T_col( Q (V^T V + eps I)^-1 ),  Q = R V;  weighted (§2.5):
      // Q = R diag(wt) V and the Gram V^T diag(wt) V
      if (W) {
        hipLaunchKernelGGL(k_gram_w_partial, dim3(gram_v.x, (unsigned)wsplits), dim3(256), 0, s, Vc, wn, bb, wt, n, Gwpart);
        hipLaunchKernelGGL(k_gram_w_reduce, dim3((unsigned)((bb * bb + 255) / 256)), dim3(256), 0, s, Gwpart, wsplits, bb, GVw);
        launch_combined<false, true>(bb, (int)((m + 63) / 64), L.S2, 0, 1, s, R, m, n, Vc, wn, L.cols_split, Qt_part, (void*)GVw, GinvV, bb <= 64 ? warm + 1 : fail, st, (const float*)wt, gram_done + 1, 0ull);
      } else {
        const int ng = own_gv ? 0 : (int)(gram_v.x * gram_v.y);
        gram_issued[1] += (unsigned long long)ng;
        launch_combined<false, false>(bb, (int)((m + 63) / 64), L.S2, ng, (int)gram_v.y, s, R, m, n, Vc, wn, L.cols_split, Qt_part, (void*)GV, GinvV, bb <= 64 ? warm + 1 : fail, st, (const float*)nullptr, gram_done + 1, gram_issued[1]);
      }
      if (capit) cap_copy(GinvV, cap->GinvV, (int64_t)bb * bb);
      launch_decorrelate(bb, s, Qt_part, L.S2, m, GinvV, Ut, Qt);
      row_tern(Ut, m, Uc, wm, nnz, st + EXTERND_STAT_SUM_NNZ_U, (const float*)Qt, it == a.iters - 1 ? rhs : (double*)nullptr);
      if (capit) {
        cap_copy(Qt, cap->Q, (int64_t)bb * m);
        cap_copy(Ut, cap->Ut, (int64_t)bb * m);
        cap_copy(Uc, cap->U_out, (int64_t)bb * wm);
      }
    }
    if (cap && cap->rhs && ce == hipSuccess) ce = launch_copy_f64(rhs, cap->rhs, bb, s);
    if (ce != hipSuccess) return ce;
    // joint scales from the final U, V and the last Q = R V (weighted: the
    // last V-side Gram GVw already belongs to the final V)
    hipLaunchKernelGGL(k_gram, gram_u, dim3(256), 0, s, Uc, wm, bb, GUf, gw);
    if (!W) hipLaunchKernelGGL(k_gram, gram_v, dim3(256), 0, s, Vc, wn, bb, GVf, gw);
    int* acc = dpart ? accept : nullptr;
    const double* gvw = W ? GVw : nullptr;
    if (bb <= 16)
      hipLaunchKernelGGL(k_joint_solve<1>, dim3(1), dim3(kCholT), 0, s, GUf, GVf, gvw, bb, rhs, Dout, dvec, tstate, trace, tidx, st, nnz, b, dpart, ndpart, dold, acc, (const double*)sg_part, sg_n);
    else if (bb <= 32)
      hipLaunchKernelGGL(k_joint_solve<2>, dim3(1), dim3(kCholT), 0, s, GUf, GVf, gvw, bb, rhs, Dout, dvec, tstate, trace, tidx, st, nnz, b, dpart, ndpart, dold, acc, (const double*)sg_part, sg_n);
    else if (bb <= 64)
      hipLaunchKernelGGL(k_joint_solve<4>, dim3(1), dim3(kCholT), 0, s, GUf, GVf, gvw, bb, rhs, Dout, dvec, tstate, trace, tidx, st, nnz, b, dpart, ndpart, dold, acc, (const double*)sg_part, sg_n);
    else
      hipLaunchKernelGGL(k_joint_solve<8>, dim3(1), dim3(kCholT), 0, s, GUf, GVf, gvw, bb, rhs, Dout, dvec, tstate, trace, tidx, st, nnz, b, dpart, ndpart, dold, acc, (const double*)sg_part, sg_n);
    if (dpart)
      hipLaunchKernelGGL(k_sweep_restore, dim3(grid1d((int64_t)bb * (wm + wn), 256)), dim3(256), 0, s, accept, bb, Uc, wm, Vc, wn, saved);
    hipLaunchKernelGGL(k_block_deflate, defl_grid, dim3(256), 0, s, R, m, n, Uc, wm, Vc, wn, dvec, bb, (double*)nullptr, (const float*)wt, sg_part);
    sg_n = wave_partials((int64_t)defl_grid.x * defl_grid.y, 256);
    return hipGetLastError();
  };

  const int64_t nblocks = (k + b - 1) / b;
  for (int64_t blk = 0; blk < nblocks; ++blk) {
    const int64_t c0 = blk * b;
    const int bb = (int)std::min<int64_t>(b, k - c0);
    hipLaunchKernelGGL(k_block_start, dim3(grid1d((int64_t)bb * wm, 256)), dim3(256), 0, s, a.seed, c0, bb, m, a.B2, warm);
    const externd_block_capture* cap = (a.cap && a.cap->block == blk) ? a.cap : nullptr;
    if ((e = fit_block(bb, a.B2 + c0 * wm, a.C2 + c0 * wn, a.D + c0, a.trace, blk, nullptr, nullptr, nullptr, cap)) !=
        hipSuccess)
      return e;
  }
  // Refinement sweeps (§2.4): add each block back, refit it from its stored
  // U, keep the better of the two.
  for (int sw = 0; sw < a.sweeps; ++sw) {
    for (int64_t blk = 0; blk < nblocks; ++blk) {
      const int64_t c0 = blk * b;
      const int bb = (int)std::min<int64_t>(b, k - c0);
      uint32_t* Uc = a.B2 + c0 * wm;
      uint32_t* Vc = a.C2 + c0 * wn;
      hipLaunchKernelGGL(k_sweep_prepare, dim3(grid1d((int64_t)bb * (wm + wn), 256)), dim3(256), 0, s, bb, Uc, wm, Vc, wn, a.D + c0, saved, dold, dneg, warm);
      hipLaunchKernelGGL(k_block_deflate, defl_grid, dim3(256), 0, s, R, m, n, Uc, wm, Vc, wn, dneg, bb, dpart, (const float*)wt, sg_part);
      sg_n = wave_partials((int64_t)defl_grid.x * defl_grid.y, 256);
      double* tr = (blk == nblocks - 1) ? a.sweep_trace : nullptr;
      if ((e = fit_block(bb, Uc, Vc, a.D + c0, tr, sw, dpart, dold, saved, nullptr)) != hipSuccess) return e;
    }
  }
  if (a.sweeps > 0 && k > 0) {
    // the factors changed: count their nonzeros afresh
    if ((e = launch_fill_i64(st + EXTERND_STAT_NNZ_B, 2, 0, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_count_nonzero, dim3(grid1d(k * wm, 256, 1024)), dim3(256), 0, s, a.B2, k * wm, st + EXTERND_STAT_NNZ_B);
    hipLaunchKernelGGL(k_count_nonzero, dim3(grid1d(k * wn, 256, 1024)), dim3(256), 0, s, a.C2, k * wn, st + EXTERND_STAT_NNZ_C);
  }
  if ((e = launch_fill_i64(st + EXTERND_STAT_ITERATIONS, 1, (long long)(nblocks * a.iters * (1 + a.sweeps)), s)) != hipSuccess)
    return e;
  if ((e = launch_norm2(R, m * n, npart, 4096, r2, nullptr, s, wt, n)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_block_finish, dim3(1), dim3(1), 0, s, a2, r2, st + EXTERND_STAT_NONFINITE, a.energy, st, a.stats);
  if (a.norm_a2 && (e = launch_copy_f64(a2, a.norm_a2, 1, s)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace externd
