// Internal interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <algorithm>

#include "../../include/externd.h"

namespace externd {

// Sets the calling thread's externd_last_error() message; returns status.
int report(int status, const char* msg);

// Arguments of one sequential decomposition (device pointers).
struct SeqArgs {
  const float* A;
  int64_t m, n, k;
  float tau;
  int iters;
  uint64_t seed;
  uint32_t* B2;
  uint32_t* C2;
  float* D;
  double* energy;
  double* trace;
  long long* stats;
  int64_t capture_component;
  float* capture_R;
  float* capture_Rcol;
  float* capture_R_next;
  float* capture_y;
  float* capture_x;
  int8_t* capture_v;
  int8_t* capture_u;
  float* capture_d;
  double* norm_a2;   // optional output: ||A||^2
  const float* importance;   // optional: n per-input-channel second moments h (§2.5)
  float lambda;              // column weights h / max(h) + lambda
  int projection;            // 1: optimal ternary projection instead of T_tau (§2.2)
  int safeguard;             // 1: apply the single-entry safeguard (appendix §7; streaming only)
};

// Arguments of one block-mode decomposition.
struct BlockArgs {
  const float* A;
  int64_t m, n, k;
  int b;
  float tau;
  int iters;
  uint64_t seed;
  uint32_t* B2;
  uint32_t* C2;
  float* D;
  double* energy;
  double* trace;
  long long* stats;
  double* norm_a2;   // optional output: ||A||^2
  int sweeps;          // refinement sweeps after extraction
  double* sweep_trace; // optional output: predicted ||R||^2 after each sweep
  const float* importance;   // optional: n per-input-channel second moments h (§2.5)
  float lambda;              // column weights h / max(h) + lambda
  int projection;            // 1: optimal ternary projection instead of T_tau (§2.2)
  const externd_block_capture* cap;   // optional test capture (host struct of device pointers)
};

// streaming sequential path and single-step kernels (seq_stream.hip)
size_t stream_workspace_bytes(int64_t m, int64_t n);
hipError_t run_stream_seq(const SeqArgs& a, void* ws, hipStream_t s);
int64_t gemv_t_chunks(int64_t m);
hipError_t launch_ternarize(const float* x, int64_t N, float tau, uint32_t* codes, int32_t* nnz,
                            long long* fallbacks, hipStream_t s, const float* wt = nullptr,
                            double* wsum = nullptr, long long* nnz_sum = nullptr);
// Optimal ternary projection of one vector (§2.2), 1 <= N <= kProjMaxN.
constexpr int kProjMaxN = 16384;   // longest vector it takes (128 KB of sort keys in LDS)
hipError_t launch_project(const float* x, int64_t N, uint32_t* codes, int32_t* nnz, long long* fallbacks,
                          hipStream_t s, const float* wt = nullptr, double* wsum = nullptr,
                          long long* nnz_sum = nullptr);
// mpart (optional, only with a dense u, so that every row is read):
// gemv_t_max_partials(m, n) per-wave maxima of w_c R_rc^2 of R after the
// fused deflation.
hipError_t launch_gemv_t(float* R, int64_t m, int64_t n, const uint32_t* u_codes, float* partial,
                         float* y, const float* dprev, const uint32_t* uprev,
                         const uint32_t* vprev, hipStream_t s, double* mpart = nullptr,
                         const float* wt = nullptr);
int64_t gemv_t_max_partials(int64_t m, int64_t n);
hipError_t launch_gemv_n(const float* R, int64_t m, int64_t n, const uint32_t* v_codes, float* x,
                         hipStream_t s, const float* wt = nullptr);
hipError_t launch_deflate(float* R, int64_t m, int64_t n, const uint32_t* u_codes,
                          const uint32_t* v_codes, const float* dptr, hipStream_t s);
// ||A||_F^2 (weighted by wt[column] when given) in a fixed order; mpart
// (optional, room for 4 partial_cap entries) receives per-wave maxima of
// wt_j A_ij^2 and *nmpart their count.
hipError_t launch_norm2(const float* A, int64_t total, double* partial, int64_t partial_cap,
                        double* out, long long* nonfinite, hipStream_t s, const float* wt = nullptr,
                        int64_t ncols = 0, double* mpart = nullptr, int64_t* nmpart = nullptr);
// Column weights wt[j] = h[j] / max(h) + lambda in fp32 (§2.5); negative or
// non-finite h entries are added to *nonfinite.
hipError_t launch_importance_weights(const float* h, int64_t n, float lambda, float* wt,
                                     long long* nonfinite, hipStream_t s);
hipError_t launch_copy_f64(const double* src, double* dst, int64_t count, hipStream_t s);
hipError_t launch_energy_finish(const double* a2, const double* r2, const long long* nonfinite,
                                double* energy, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t v, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t count, float v, hipStream_t s);
hipError_t launch_fill_i64(long long* p, int64_t count, long long v, hipStream_t s);
hipError_t launch_copy_f32(const float* a, float* b, int64_t count, hipStream_t s);

// persistent streaming sequential path (seq_persist.hip): one cooperative
// launch, R in device memory; n % 4 == 0 and the shapes its instantiations cover
bool persist_fits(int64_t m, int64_t n, int num_cus);
size_t persist_workspace_bytes(int64_t m, int64_t n, int64_t k, int num_cus);
hipError_t run_persist_seq(const SeqArgs& a, void* ws, int num_cus, hipStream_t s);

// resident sequential path (seq_resident.hip)
bool resident_fits(int64_t m, int64_t n, int num_cus);
// Placements of the exchange words the resident path tries before the run
// (1: no probe); the workspace holds `cands` placements.
int resident_place_candidates(int64_t m, int64_t n, int64_t k);
size_t resident_workspace_bytes(int64_t m, int64_t n, int64_t k, int cands);
hipError_t run_resident_seq(const SeqArgs& a, void* ws, int cands, int num_cus, hipStream_t s, int* grid_out);
// Set by externd_decompose_noalloc around its call: the resident path then
// uses a single placement, which fits the static scratch.
extern thread_local bool g_single_placement;

// block path (block.hip)
size_t block_workspace_bytes(int64_t m, int64_t n, int b);
hipError_t run_block(const BlockArgs& a, void* ws, hipStream_t s);

// energy / reconstruction from 2-bit factors (factors.hip)
size_t energy_workspace_bytes(int64_t m, int64_t n);
hipError_t run_energy(const float* A, int64_t m, int64_t n, const uint32_t* B2, const uint32_t* C2,
                      const float* D, int64_t k, double* energy, void* ws, hipStream_t s);
hipError_t run_reconstruct(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m,
                           int64_t n, int64_t k, float* out, hipStream_t s);

// inference y = B diag(D) C x with B row by row, on int8 MFMA (apply_rows.hip)
bool apply_rows_fits(int64_t m, int64_t n, int64_t k);
size_t apply_rows_workspace_bytes(int64_t m, int64_t k, int num_cus);
hipError_t run_apply_rows(const uint32_t* BT2, const uint32_t* C2, const float* D, int64_t m, int64_t n, int64_t k,
                          const float* x, float* y, void* ws, int num_cus, hipStream_t s);
hipError_t run_codes_transpose(const uint32_t* src, int64_t rows, int64_t cols, uint32_t* dst, hipStream_t s);

// inference y = B diag(D) C x from 2-bit factors (apply.hip)
size_t apply_workspace_bytes(int64_t m, int64_t k);
hipError_t run_apply(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m, int64_t n, int64_t k,
                     const float* x, float* y, void* ws, hipStream_t s);

}  // namespace externd
