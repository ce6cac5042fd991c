// Inference with the factors on int8 MFMA (ExTernD §2.6): y = B (diag(D) (C x))
// with B stored row by row (m rows of ceil(k/16) code words, the transpose of
// the component-major B2 the decomposition writes; k_codes_transpose makes
// it once per factorisation).  Both products are then "row-major code matrix
// times a vector", computed by one kernel:
//
//   out_r = f( sum_k S[r][k] v_k ),  S ternary,
//
// with the vector in fixed point: X_k = rint(v_k 2^s), s = 29 - floor(log2
// max|v|), so |X_k| < 2^30, split into four balanced int8 digits
// (X = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3, each digit in [-128, 127]).  The
// products c_rk d_j(X_k) are exact int8 products summed exactly in int32 by
// v_mfma_i32_16x16x64_i8 (|sum| <= 128 K), the digits are recombined in
// int64 (exact while K <= 2^21), and one conversion out of fixed point
// remains: the result is the exact sum for the rounded vector, independent of
// any summation order.  The rounding of v to fixed point moves each entry by
// at most 2^-30 of max|v|.
//
// Operands of one MFMA (16 rows x 64 columns): lane (r + 16 g) holds 16 codes
// of row r, the word 8 g + s of the current 32-word stretch of the row at
// step s, unpacked to int8 by a byte permute (v_perm_b32 as a table of the
// four code values); byte 4q + b of the unpacked word holds code 4b + q.  The
// B operand of lane (j + 16 g) holds digit j of the 16 vector entries of the
// same word in the same byte order (lanes j >= 4 read 16 zero bytes: 4 of
// the 16 output columns are used).  Both operands use the same (lane group,
// byte) slot for the same column, and the result D[i][j] lands in lane
// j + 16 (i / 4), register i % 4 (checked on the hardware).  The digits live
// in LDS, built once per vector chunk by every workgroup: 64 bytes per code
// word (the 16 bytes of digit j at 16 j), blocks of 16 words padded to
// 1088 bytes so that the four lane groups, 16 words apart, read different
// banks.
#include "device_common.hpp"
#include "kernels.hpp"

namespace externd {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kRDig = 4;                 // int8 digits of the fixed-point vector
constexpr int kRPf = 2;                  // 32-word stretches of a row in flight per lane (2 measured best: 1, 3, 4, 6 slower)
constexpr int kRMaxRows = 1 << 21;       // vector length bound for the exact int64 recombination
constexpr int kRBlk = 1088;              // LDS bytes per 16 code words of digits (1024 + 64 skew)

constexpr int kRZero = 512;              // zero bytes after the digits (the B operand of lanes j >= 4)

// LDS bytes of the digits of a chunk of CH vector entries, and of the zero block after them
template <int CH>
constexpr int planes_bytes() { return CH / 256 * kRBlk + kRZero; }
__device__ inline int word_off(int W) { return (W >> 4) * kRBlk + (W & 15) * 64; }

// Eight zero code words: the load of a lane with nothing to read (a row past
// the end, a stretch past its part), so every lane issues the same loads.
__device__ uint32_t kZeroWords[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};   // never written

// 16 codes of one word as int8 values {-1, 0, +1}, byte 4q + b = code 4b + q.
__device__ inline v4i unpack_codes(uint32_t w) {
  constexpr uint32_t kLut = 0xFF000100u;   // byte c = value of code c: 00 -> 0, 01 -> 1, 11 -> -1
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(0u, kLut, w & 0x03030303u);
  r.y = (int)__builtin_amdgcn_perm(0u, kLut, (w >> 2) & 0x03030303u);
  r.z = (int)__builtin_amdgcn_perm(0u, kLut, (w >> 4) & 0x03030303u);
  r.w = (int)__builtin_amdgcn_perm(0u, kLut, (w >> 6) & 0x03030303u);
  return r;
}

// Write the digits of vector entries [k0, k0 + CH) into LDS: for word W of
// the chunk, bytes word_off(W) + 16 j .. + 15 hold digit j of entries
// 16 W .. 16 W + 15, byte 4q + b holding entry 16 W + 4 b + q.  Entries
// past K are 0.  Balanced base-256 digits of X come out of one add: the bytes
// of X + 0x80808080 are the digits plus 128 each (no byte overflows, since
// |X| < 2^30), so flipping each byte's top bit gives them as int8.
template <int CH, int NT>
__device__ inline void build_digits(const float* __restrict__ v, int64_t K, int64_t k0, int s, int8_t* lds) {
  const bool vec = ((reinterpret_cast<uintptr_t>(v) & 15) == 0);
  for (int W = threadIdx.x; W < CH / 16; W += NT) {
    const int64_t kb = k0 + 16 * (int64_t)W;
    float x[16];
    if (vec && kb + 16 <= K) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float4 q4 = reinterpret_cast<const float4*>(v + kb)[f];
        x[4 * f] = q4.x; x[4 * f + 1] = q4.y; x[4 * f + 2] = q4.z; x[4 * f + 3] = q4.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) x[c] = kb + c < K ? v[kb + c] : 0.f;
    }
    uint32_t y[16];   // byte j of y[c]: digit j of entry c
#pragma unroll
    for (int c = 0; c < 16; ++c)
      y[c] = ((uint32_t)__float2int_rn(ldexpf(x[c], s)) + 0x80808080u) ^ 0x80808080u;
    uint32_t o[4][4];   // [digit j][dword q]: byte b = digit j of entry 4 b + q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // 4 x 4 byte transpose of (y[q], y[4 + q], y[8 + q], y[12 + q])
      const uint32_t t0 = __builtin_amdgcn_perm(y[4 + q], y[q], 0x05010400u);
      const uint32_t t1 = __builtin_amdgcn_perm(y[4 + q], y[q], 0x07030602u);
      const uint32_t t2 = __builtin_amdgcn_perm(y[12 + q], y[8 + q], 0x05010400u);
      const uint32_t t3 = __builtin_amdgcn_perm(y[12 + q], y[8 + q], 0x07030602u);
      o[0][q] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
      o[1][q] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
      o[2][q] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
      o[3][q] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
    }
    uint4* dst = reinterpret_cast<uint4*>(lds + word_off(W));
#pragma unroll
    for (int j = 0; j < kRDig; ++j) dst[j] = uint4{o[j][0], o[j][1], o[j][2], o[j][3]};
  }
  for (int i = threadIdx.x; i < kRZero / 4; i += NT) reinterpret_cast<uint32_t*>(lds + CH / 256 * kRBlk)[i] = 0u;
}

// out_r = f(sum_k S[r][k] v_k) for the rows of S (R rows, K columns, wK words
// per row), 16 rows per wave, the vector in chunks of CH entries.  A
// workgroup has KP x 4 waves: wave w takes row block w % 4 and part w / 4 of
// each chunk's words (KP parts), and the parts' int32 sums are added through
// LDS (exact, so in any order).  f: with D, out_r = fl32(D_r x) (and the
// workgroup's largest |out| goes to vmax_out); without, out_r = fl32(x).  The
// fixed-point scale comes from max|v|: read from vmax_in (nvmax float bit
// patterns) when given, else scanned here.  A non-finite max makes every
// output NaN.
// One wave's share of one chunk: its rows' words [w0, w1), nst stretches of
// 32 words, the lane group taking words 8 g .. 8 g + 7 of each stretch.
struct RowPart {
  const uint32_t* rp;   // this lane's row (row 0 when the row is past the end)
  int64_t w0, w1;
  int nst, wofs;        // stretches; word of the chunk where the part starts
  bool rowok;
};

// The lane's 8 words of stretch st; branch-free: a lane with nothing to read
// loads the zero words.
template <bool AL>
__device__ inline void load_stretch(const RowPart& pt, int st, int g, uint32_t (&wd)[8]) {
  const int64_t wb = pt.w0 + 32 * (int64_t)st + 8 * g;
  if constexpr (AL) {
    const bool ok = pt.rowok && st < pt.nst && wb < pt.w1;   // w1 is a multiple of 8 here
    const uint4* p4 = reinterpret_cast<const uint4*>(ok ? pt.rp + wb : kZeroWords);
    const uint4 a = p4[0], b = p4[1];
    wd[0] = a.x; wd[1] = a.y; wd[2] = a.z; wd[3] = a.w;
    wd[4] = b.x; wd[5] = b.y; wd[6] = b.z; wd[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = pt.rowok && st < pt.nst && wb + e < pt.w1;
      wd[e] = *(ok ? pt.rp + wb + e : kZeroWords + e);
    }
  }
}

// A workgroup takes RB 16-row blocks, each split over KP waves by K part.
// AL: every row starts 16-byte aligned and holds a multiple of 8 words, so a
// lane's 8 words of a 32-word stretch are two aligned 16-byte loads that
// never cross the end of its part; otherwise eight single-word loads.  FULL
// (with AL): every part of every chunk is a whole number of 64-word
// stretches, read 256 bytes per row at a time (the lane group taking 16 of
// the 64 words), which streams faster than shorter runs.  Then nothing needs
// masking: a row past the end reads the last row and a prefetch past the
// part's end re-reads its last stretch (their products land in rows that
// are never written out or are never computed), and lanes j >= 4 read digit
// j % 4 (their output columns are never read), so the inner loop is loads,
// unpacks, LDS reads and MFMAs only.
template <int CH, int KP, int RB, bool AL, bool FULL>
__global__ __launch_bounds__(KP * RB * kWave) void k_rows_gemv(
    const uint32_t* __restrict__ S, int64_t R, int64_t K, int64_t wK, const float* __restrict__ v,
    const uint32_t* __restrict__ vmax_in, int nvmax, const float* __restrict__ D, float* __restrict__ out,
    uint32_t* __restrict__ vmax_out) {
  constexpr int NT = KP * RB * kWave, NW = NT / kWave;
  __shared__ __align__(16) int8_t digits[planes_bytes<CH>()];
  __shared__ __align__(16) v4i part_acc[KP > 1 ? (KP - 1) * RB * kWave : 1];
  __shared__ uint32_t red[NW];
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const int slot = wv % RB, part = wv / RB;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t nrb = (R + 15) / 16;
  const int64_t nchunks = (K + CH - 1) / CH;
  const int64_t per_round = (int64_t)gridDim.x * RB;
  const int64_t rounds = (nrb + per_round - 1) / per_round;
  auto part_of = [&](int64_t rd, int64_t ch) {
    RowPart pt;
    const int64_t rb = rd * per_round + (int64_t)blockIdx.x * RB + slot;
    const int64_t row = 16 * rb + r16;
    pt.rowok = rb < nrb && row < R;
    const int64_t c0 = ch * (CH / 16), c1 = min(wK, c0 + CH / 16);
    constexpr int SW = FULL ? 64 : 32;   // words per stretch
    const int64_t pw = ((c1 - c0 + SW * KP - 1) / (SW * KP)) * SW;   // words per part, whole stretches
    pt.w0 = c0 + part * pw;
    pt.w1 = min(c1, pt.w0 + pw);
    pt.nst = pt.w1 > pt.w0 ? (int)((pt.w1 - pt.w0 + SW - 1) / SW) : 0;
    pt.wofs = (int)(pt.w0 - c0);
    pt.rp = S + (pt.rowok ? row : 0) * wK;
    return pt;
  };
  // the first stretches of the first round and chunk are in flight before the
  // scale and the digits are worked out
  constexpr int RW = FULL ? 16 : 8;   // words per lane per stretch
  uint32_t ring[kRPf][RW];
  RowPart pt = part_of(0, 0);
  // the FULL path's loads: 16 words w0 + 64 st + 16 g .. + 15 of the (clamped) row
  auto load_fast = [&](const uint32_t* lp, int st, int nst, uint32_t (&wd)[RW]) {
    const uint4* p4 = reinterpret_cast<const uint4*>(lp + 64 * min(st, nst - 1));
#pragma unroll
    for (int u = 0; u < RW / 4; ++u) {
      const uint4 a = p4[u];
      wd[4 * u] = a.x; wd[4 * u + 1] = a.y; wd[4 * u + 2] = a.z; wd[4 * u + 3] = a.w;
    }
  };
  if constexpr (FULL) {
    const int64_t rb0 = (int64_t)blockIdx.x * RB + slot;
    if (rb0 < nrb && pt.nst > 0) {
      const uint32_t* lp = S + min(16 * rb0 + r16, R - 1) * wK + pt.w0 + 16 * g;
#pragma unroll
      for (int p = 0; p < kRPf; ++p) load_fast(lp, p, pt.nst, ring[p]);
    }
  } else {
#pragma unroll
    for (int p = 0; p < kRPf; ++p) load_stretch<AL>(pt, p, g, ring[p]);
  }

  // ---- the scale ----
  uint32_t mb = 0u;
  if (vmax_in) {
    for (int i = t; i < nvmax; i += NT) mb = max(mb, vmax_in[i]);
  } else if ((reinterpret_cast<uintptr_t>(v) & 15) == 0) {
    // float4 loads, four in flight per thread
    const int64_t K4 = K / 4;
    const float4* v4 = reinterpret_cast<const float4*>(v);
    int64_t i = t;
    for (; i + 3 * NT < K4; i += 4 * NT) {
      float4 b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = v4[i + u * NT];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        mb = max(mb, max(max(__float_as_uint(b[u].x) & 0x7fffffffu, __float_as_uint(b[u].y) & 0x7fffffffu),
                         max(__float_as_uint(b[u].z) & 0x7fffffffu, __float_as_uint(b[u].w) & 0x7fffffffu)));
    }
    for (; i < K4; i += NT) {
      const float4 b = v4[i];
      mb = max(mb, max(max(__float_as_uint(b.x) & 0x7fffffffu, __float_as_uint(b.y) & 0x7fffffffu),
                       max(__float_as_uint(b.z) & 0x7fffffffu, __float_as_uint(b.w) & 0x7fffffffu)));
    }
    for (int64_t r = 4 * K4 + t; r < K; r += NT) mb = max(mb, __float_as_uint(v[r]) & 0x7fffffffu);
  } else {
    for (int64_t i = t; i < K; i += NT) mb = max(mb, __float_as_uint(v[i]) & 0x7fffffffu);
  }
  mb = wave_umax_to63(mb);
  if (lane == kWave - 1) red[wv] = mb;
  __syncthreads();
  mb = red[0];
#pragma unroll
  for (int q = 1; q < NW; ++q) mb = max(mb, red[q]);
  const bool bad = mb >= 0x7f800000u;   // Inf or NaN in the vector
  const int s = (mb == 0u || bad) ? 0 : 29 - ilogbf(__uint_as_float(mb));

  uint32_t omax = 0u;
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t rb = rd * per_round + (int64_t)blockIdx.x * RB + slot;
    v4i acc = {0, 0, 0, 0};
    for (int64_t ch = 0; ch < nchunks; ++ch) {
      if (nchunks > 1 || rd == 0) {
        __syncthreads();   // every read of the previous digits done
        build_digits<CH, NT>(v, K, ch * CH, s, digits);
        __syncthreads();
      }
      if (rb >= nrb) continue;   // uniform per wave
      if (rd != 0 || ch != 0) pt = part_of(rd, ch);
      const int nst = pt.nst, wofs = pt.wofs;
      if constexpr (FULL) {
        // digits of word wofs + 64 st + 16 g + e at word_off(wofs + 16 g) + 4352 st + 64 e
        const uint32_t* lp = S + min(16 * rb + r16, R - 1) * wK + pt.w0 + 16 * g;
        const int8_t* bp0 = digits + word_off(wofs + 16 * g) + 16 * (r16 & 3);
        if (rd != 0 || ch != 0) {
#pragma unroll
          for (int p = 0; p < kRPf; ++p) load_fast(lp, p, nst, ring[p]);
        }
        for (int st0 = 0; st0 < nst; st0 += kRPf) {
#pragma unroll
          for (int p = 0; p < kRPf; ++p) {
            const int st = st0 + p;
            if (st < nst) {   // uniform per wave
              const int8_t* bp = bp0 + 4 * kRBlk * st;
#pragma unroll
              for (int e = 0; e < RW; ++e) {
                const v4i a = unpack_codes(ring[p][e]);
                const v4i b = *reinterpret_cast<const v4i*>(bp + 64 * e);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
              }
            }
            load_fast(lp, st + kRPf, nst, ring[p]);
          }
        }
        continue;
      } else {
      if (rd != 0 || ch != 0) {
#pragma unroll
        for (int p = 0; p < kRPf; ++p) load_stretch<AL>(pt, p, g, ring[p]);
      }
      // this lane's B operand: digit r16 of the word, or the zero block (for every e)
      const int zero_off = CH / 256 * kRBlk;
      for (int st0 = 0; st0 < nst; st0 += kRPf) {
#pragma unroll
        for (int p = 0; p < kRPf; ++p) {
          const int st = st0 + p;
          if (st < nst) {   // uniform per wave
            const int8_t* bp = digits + (r16 < kRDig ? word_off(wofs + 32 * st + 8 * g) + 16 * r16 : zero_off);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const v4i a = unpack_codes(ring[p][e]);
              const v4i b = *reinterpret_cast<const v4i*>(bp + 64 * e);
              acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
            }
          }
          load_stretch<AL>(pt, st + kRPf, g, ring[p]);
        }
      }
      }
    }
    if constexpr (KP > 1) {
      // add the parts' sums (exact integers)
      if (part > 0 && rb < nrb) part_acc[((part - 1) * RB + slot) * kWave + lane] = acc;
      __syncthreads();
      if (part == 0 && rb < nrb) {
#pragma unroll
        for (int q = 1; q < KP; ++q) acc += part_acc[((q - 1) * RB + slot) * kWave + lane];
      }
      __syncthreads();
    }
    if (rb >= nrb || part != 0) continue;
    // ---- recombine the digits: lane (j + 16 gq) holds digit j of rows 4 gq + e ----
    const int av[4] = {acc.x, acc.y, acc.z, acc.w};
    int64_t T[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d1 = __shfl(av[e], lane + 1, kWave);
      const int d2 = __shfl(av[e], lane + 2, kWave);
      const int d3 = __shfl(av[e], lane + 3, kWave);
      T[e] = (int64_t)av[e] + ((int64_t)d1 << 8) + ((int64_t)d2 << 16) + ((int64_t)d3 << 24);
    }
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t orow = 16 * rb + 4 * g + e;
        if (orow < R) {
          const double x = ldexp((double)T[e], -s);
          float o;
          if (bad) o = __uint_as_float(0x7fc00000u);
          else if (D) o = (float)((double)D[orow] * x);
          else o = (float)x;
          out[orow] = o;
          omax = max(omax, __float_as_uint(o) & 0x7fffffffu);
        }
      }
    }
  }
  if (vmax_out) {
    omax = wave_umax_to63(omax);
    __syncthreads();
    if (lane == kWave - 1) red[wv] = omax;
    __syncthreads();
    if (t == 0) {
      uint32_t r = red[0];
#pragma unroll
      for (int q = 1; q < NW; ++q) r = max(r, red[q]);
      vmax_out[blockIdx.x] = r;
    }
  }
}

// dst (cols x rows codes, ceil(rows/16) words per row) = transpose of src
// (rows x cols codes, ceil(cols/16) words per row).  One thread per 16 x 16
// block of codes.
__global__ void k_codes_transpose(const uint32_t* __restrict__ src, int64_t rows, int64_t cols,
                                  uint32_t* __restrict__ dst) {
  const int64_t wc = (cols + 15) / 16, wr = (rows + 15) / 16;
  const int64_t nblk = wr * wc;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t a = idx / wc, b = idx % wc;   // src row block a, src word b
    uint32_t in[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) in[r] = 16 * a + r < rows ? src[(16 * a + r) * wc + b] : 0u;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (16 * b + c >= cols) break;
      uint32_t o = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) o |= ((in[r] >> (2 * c)) & 3u) << (2 * r);
      dst[(16 * b + c) * wr + a] = o;
    }
  }
}

__global__ void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Launch shapes (8 waves per workgroup): vectors up to 16384 entries: 8
// row blocks of one K part each, two workgroups per CU when the rows run
// out; longer: 4 row blocks of two K parts, one workgroup per CU.
constexpr int kRB1 = 8, kKP1 = 1, kRB2 = 4, kKP2 = 2;

// Workgroups of one GEMV launch: enough for every 16-row block in one round,
// at most the number that stay resident together.
int rows_grid(int64_t R, int64_t K, int num_cus) {
  const int64_t nrb = (R + 15) / 16;
  const int rbw = K <= 16384 ? kRB1 : kRB2;
  const int per_cu = K <= 16384 ? 2 : 1;
  const int64_t want = (nrb + rbw - 1) / rbw;
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)per_cu * std::max(1, num_cus)));
}

hipError_t launch_rows_gemv(const uint32_t* S, int64_t R, int64_t K, const float* v, const uint32_t* vmax_in,
                            int nvmax, const float* D, float* out, uint32_t* vmax_out, int grid, hipStream_t s) {
  const int64_t wK = (K + 15) / 16;
  const bool al = (wK % 8) == 0 && (reinterpret_cast<uintptr_t>(S) & 15) == 0;
  const dim3 b1(kKP1 * kRB1 * kWave), b2(kKP2 * kRB2 * kWave);
#define EXTERND_ROWS_LAUNCH(CH, KP, RB, AL, FULL, BLK)                                                       \
  hipLaunchKernelGGL((k_rows_gemv<CH, KP, RB, AL, FULL>), dim3(grid), BLK, 0, s, S, R, K, wK, v, vmax_in, nvmax, \
                     D, out, vmax_out)
  if (K <= 16384) {
    if (al && wK % (64 * kKP1) == 0) EXTERND_ROWS_LAUNCH(16384, kKP1, kRB1, true, true, b1);
    else if (al) EXTERND_ROWS_LAUNCH(16384, kKP1, kRB1, true, false, b1);
    else EXTERND_ROWS_LAUNCH(16384, kKP1, kRB1, false, false, b1);
  } else {
    if (al && wK % (64 * kKP2) == 0) EXTERND_ROWS_LAUNCH(32768, kKP2, kRB2, true, true, b2);
    else if (al) EXTERND_ROWS_LAUNCH(32768, kKP2, kRB2, true, false, b2);
    else EXTERND_ROWS_LAUNCH(32768, kKP2, kRB2, false, false, b2);
  }
#undef EXTERND_ROWS_LAUNCH
  return hipGetLastError();
}

}  // namespace

bool apply_rows_fits(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && n >= 1 && k >= 0 && n <= kRMaxRows && k <= kRMaxRows;
}

size_t apply_rows_workspace_bytes(int64_t m, int64_t k, int num_cus) {
  return 256 + sizeof(float) * (size_t)std::max<int64_t>(k, 1) + 256 +
         sizeof(uint32_t) * (size_t)rows_grid(std::max<int64_t>(k, 1), 1, num_cus);
}

hipError_t run_apply_rows(const uint32_t* BT2, const uint32_t* C2, const float* D, int64_t m, int64_t n, int64_t k,
                          const float* x, float* y, void* ws, int num_cus, hipStream_t s) {
  if (k == 0) {
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)std::min<int64_t>((m + 255) / 256, 4096)), dim3(256), 0, s, y, m,
                       0.f);
    return hipGetLastError();
  }
  char* p = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  float* w = reinterpret_cast<float*>(p);
  p = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p + sizeof(float) * k) + 255) & ~(uintptr_t)255);
  uint32_t* wmax = reinterpret_cast<uint32_t*>(p);
  // w = D (C x): rows of C are components (k rows, n columns)
  const int g1 = rows_grid(k, n, num_cus);
  hipError_t e = launch_rows_gemv(C2, k, n, x, nullptr, 0, D, w, wmax, g1, s);
  if (e != hipSuccess) return e;
  // y = B w: rows of B (m rows, k columns), the scale from the first launch's maxima
  const int g2 = rows_grid(m, k, num_cus);
  return launch_rows_gemv(BT2, m, k, w, wmax, g1, nullptr, y, nullptr, g2, s);
}

hipError_t run_codes_transpose(const uint32_t* src, int64_t rows, int64_t cols, uint32_t* dst, hipStream_t s) {
  const int64_t nblk = ((rows + 15) / 16) * ((cols + 15) / 16);
  if (nblk == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((nblk + 255) / 256, 65536);
  hipLaunchKernelGGL(k_codes_transpose, dim3(grid), dim3(256), 0, s, src, rows, cols, dst);
  return hipGetLastError();
}

}  // namespace externd
