// C ABI of the ExTernD library: argument validation, device checks,
// workspace management and dispatch to the HIP kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/externd.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(EXTERND_EHIP, "%s: %s", where, hipGetErrorString(e));
}

struct DeviceInfo {
  bool checked = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

// Current device must be a gfx950; remembers its compute-unit count.
int check_device(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(EXTERND_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = true;
  }
  if (!d.gfx950) return fail(EXTERND_EUNSUPPORTED, "device %d is not gfx950", dev);
  if (cus) *cus = d.cus;
  return EXTERND_OK;
}

bool bad_size(int64_t m, int64_t n) {
  return m <= 0 || n <= 0 || m > (int64_t(1) << 31) - 1 || n > (int64_t(1) << 31) - 1 ||
         m * n > (int64_t(1) << 40);
}

// The sequential mode a request runs in: AUTO takes the resident kernel when
// the shape fits on chip (not with the projection or an applied safeguard),
// else the persistent streaming kernel when it applies, else the streaming
// kernel chain.  -1 when an explicit mode does not apply to the shape.
int seq_mode(int requested, int64_t m, int64_t n, int cus, bool projection, bool safeguard) {
  const bool res_ok = externd::resident_fits(m, n, cus) && !projection && !safeguard;
  const bool per_ok = externd::persist_fits(m, n, cus) && !projection && !safeguard;
  switch (requested) {
    case EXTERND_MODE_RESIDENT: return res_ok ? EXTERND_MODE_RESIDENT : -1;
    case EXTERND_MODE_PERSISTENT: return per_ok ? EXTERND_MODE_PERSISTENT : -1;
    case EXTERND_MODE_STREAMING: return EXTERND_MODE_STREAMING;
    default: return res_ok ? EXTERND_MODE_RESIDENT : (per_ok ? EXTERND_MODE_PERSISTENT : EXTERND_MODE_STREAMING);
  }
}

// Stream-ordered workspace: allocated on the stream, freed on the stream
// (or borrowed from the caller, then never freed here).
struct Workspace {
  void* ptr = nullptr;
  hipStream_t s = nullptr;
  bool owned = false;
  ~Workspace() {
    if (ptr && owned) (void)hipFreeAsync(ptr, s);
  }
};

int alloc_ws(Workspace& w, size_t bytes, hipStream_t s) {
  w.s = s;
  hipError_t e = hipMallocAsync(&w.ptr, bytes, s);
  if (e != hipSuccess) {
    w.ptr = nullptr;
    return fail(EXTERND_ENOMEM, "hipMallocAsync(%zu): %s", bytes, hipGetErrorString(e));
  }
  w.owned = true;
  return EXTERND_OK;
}

// The caller's workspace when opts provides one (checked against `bytes`),
// else a stream-ordered allocation.
int get_ws(Workspace& w, const externd_opts& o, size_t bytes, hipStream_t s) {
  if (!o.workspace) return alloc_ws(w, bytes, s);
  if (o.workspace_bytes < bytes)
    return fail(EXTERND_ENOMEM, "workspace of %llu bytes < %zu needed",
                (unsigned long long)o.workspace_bytes, bytes);
  w.ptr = o.workspace;
  w.s = s;
  w.owned = false;
  return EXTERND_OK;
}

}  // namespace

namespace externd {
int report(int status, const char* msg) { return fail(status, "%s", msg); }
thread_local bool g_single_placement = false;
}  // namespace externd

extern "C" {

const char* externd_status_string(int status) {
  switch (status) {
    case EXTERND_OK: return "ok";
    case EXTERND_EINVAL: return "invalid argument";
    case EXTERND_ENOMEM: return "out of device memory";
    case EXTERND_EHIP: return "HIP runtime error";
    case EXTERND_EUNSUPPORTED: return "unsupported device or shape";
    default: return "unknown status";
  }
}

const char* externd_last_error(void) { return g_last_error.c_str(); }

int externd_apply(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m, int64_t n,
                  int64_t k, const float* x, void* stream, float* y) {
  if (!x || !y) return fail(EXTERND_EINVAL, "null x or y pointer");
  if (bad_size(m, n) || k < 0 || k > (int64_t(1) << 31))
    return fail(EXTERND_EINVAL, "bad shape");
  if (k > 0 && (!B2 || !C2 || !D)) return fail(EXTERND_EINVAL, "null factor pointer");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w;
  if ((st = alloc_ws(w, externd::apply_workspace_bytes(m, k), s)) != EXTERND_OK) return st;
  hipError_t e = externd::run_apply(B2, C2, D, m, n, k, x, y, w.ptr, s);
  if (e != hipSuccess) return hip_fail(e, "apply");
  return EXTERND_OK;
}

int externd_transpose_codes(const uint32_t* src, int64_t rows, int64_t cols, void* stream, uint32_t* dst) {
  if (rows < 0 || cols < 0 || rows > (int64_t(1) << 40) || cols > (int64_t(1) << 40))
    return fail(EXTERND_EINVAL, "bad shape");
  if (rows > 0 && cols > 0 && (!src || !dst)) return fail(EXTERND_EINVAL, "null code pointer");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipError_t e = externd::run_codes_transpose(src, rows, cols, dst, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "transpose_codes");
  return EXTERND_OK;
}

size_t externd_apply_rows_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (bad_size(m, n) || k < 0 || !externd::apply_rows_fits(m, n, k)) return 0;
  int cus = 0;
  if (check_device(&cus) != EXTERND_OK) return 0;
  return externd::apply_rows_workspace_bytes(m, k, cus);
}

int externd_apply_rows(const uint32_t* BT2, const uint32_t* C2, const float* D, int64_t m, int64_t n, int64_t k,
                       const float* x, void* stream, float* y, void* workspace, size_t workspace_bytes) {
  if (!x || !y) return fail(EXTERND_EINVAL, "null x or y pointer");
  if (bad_size(m, n) || k < 0 || !externd::apply_rows_fits(m, n, k))
    return fail(EXTERND_EINVAL, "bad shape (n and k at most 2^21)");
  if (k > 0 && (!BT2 || !C2 || !D)) return fail(EXTERND_EINVAL, "null factor pointer");
  int cus = 0;
  int st = check_device(&cus);
  if (st != EXTERND_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = externd::apply_rows_workspace_bytes(m, k, cus);
  Workspace w;
  if (workspace) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0 || workspace_bytes < need)
      return fail(EXTERND_EINVAL, "workspace must be 256-byte aligned and at least %zu bytes", need);
    w.ptr = workspace;
  } else if ((st = alloc_ws(w, need, s)) != EXTERND_OK) {
    return st;
  }
  hipError_t e = externd::run_apply_rows(BT2, C2, D, m, n, k, x, y, w.ptr, cus, s);
  if (e != hipSuccess) return hip_fail(e, "apply_rows");
  return EXTERND_OK;
}

int64_t externd_rank(int64_t m, int64_t n, float mu) {
  if (m <= 0 || n <= 0 || !std::isfinite(mu) || mu < 0.f) return -1;
  const double v = (double)mu * (double)(m < n ? m : n);
  if (v > 9.0e15) return -1;
  const double whole = std::floor(v);
  return (int64_t)whole + ((v - whole) >= 0.5 ? 1 : 0);
}

int64_t externd_rank_for_energy(const double* trace, int64_t len, int64_t total, int32_t step,
                                double norm_a2, double target, double* energy) {
  if (energy) *energy = std::nan("");
  if (len < 0 || total < 0 || step < 1 || (len > 0 && !trace) || !std::isfinite(target) ||
      !std::isfinite(norm_a2) || norm_a2 < 0.0)
    return (fail(EXTERND_EINVAL, "bad arguments to externd_rank_for_energy"), -2);
  if (norm_a2 == 0.0) {
    if (energy) *energy = 1.0;
    return 0;
  }
  for (int64_t j = 0; j < len; ++j) {
    const double e = 1.0 - trace[j] / norm_a2;
    if (e >= target) {
      if (energy) *energy = e;
      const int64_t c = (j + 1) * (int64_t)step;
      return c < total ? c : total;
    }
  }
  return -1;
}

int32_t externd_block_width(int64_t m, int64_t n, int32_t block) {
  if (block <= 1 || m <= 0 || n <= 0) return 1;
  const int64_t cap = (m < n ? m : n) / 8;
  const int64_t b = block < cap ? block : cap;
  return b >= 2 ? (int32_t)b : 1;
}

int32_t externd_resident_fits(int64_t m, int64_t n) {
  int cus = 0;
  if (check_device(&cus) != EXTERND_OK) return 0;
  return externd::resident_fits(m, n, cus) ? 1 : 0;
}

uint64_t externd_workspace_bytes(int64_t m, int64_t n, float mu, int32_t block, int32_t mode) {
  if (bad_size(m, n)) return (fail(EXTERND_EINVAL, "bad shape"), 0);
  if (!std::isfinite(mu) || mu <= 0.f) return (fail(EXTERND_EINVAL, "mu must be finite and > 0"), 0);
  if (mode < -1 || mode > 2) return (fail(EXTERND_EINVAL, "bad mode %d", mode), 0);
  const int b = externd_block_width(m, n, block);
  if (b > 1) return externd::block_workspace_bytes(m, n, b);
  const int64_t k = externd_rank(m, n, mu);
  if (mode == EXTERND_MODE_STREAMING) return externd::stream_workspace_bytes(m, n);
  int cus = 0;
  if (check_device(&cus) != EXTERND_OK) return 0;
  const int md = seq_mode(mode, m, n, cus, false, false);
  if (md < 0) return (fail(EXTERND_EUNSUPPORTED, "%lld x %lld does not fit the %s kernel", (long long)m, (long long)n,
                           mode == EXTERND_MODE_RESIDENT ? "resident" : "persistent streaming"), 0);
  if (md == EXTERND_MODE_RESIDENT)
    return externd::resident_workspace_bytes(m, n, k, externd::resident_place_candidates(m, n, k));
  if (md == EXTERND_MODE_PERSISTENT) return externd::persist_workspace_bytes(m, n, k, cus);
  return externd::stream_workspace_bytes(m, n);
}

int externd_decompose(const float* A, int64_t m, int64_t n, float mu, float tau, int32_t iters,
                      int32_t block, void* stream, uint32_t* B2, uint32_t* C2, float* D,
                      double* energy, const externd_opts* opts) {
  if (!A || !energy) return fail(EXTERND_EINVAL, "null A or energy pointer");
  if (bad_size(m, n)) return fail(EXTERND_EINVAL, "bad shape %lld x %lld", (long long)m, (long long)n);
  if (!std::isfinite(mu) || mu <= 0.f) return fail(EXTERND_EINVAL, "mu must be finite and > 0");
  if (!std::isfinite(tau) || tau < 0.f) return fail(EXTERND_EINVAL, "tau must be finite and >= 0");
  if (iters < 1) return fail(EXTERND_EINVAL, "iters must be >= 1");
  const int64_t k = externd_rank(m, n, mu);
  if (k < 0 || k > (int64_t(1) << 31)) return fail(EXTERND_EINVAL, "rank out of range");
  if (k > 0 && (!B2 || !C2 || !D)) return fail(EXTERND_EINVAL, "null factor pointer");
  externd_opts o{};
  o.struct_size = sizeof(externd_opts);
  o.mode = EXTERND_MODE_AUTO;
  o.capture_component = -1;
  if (opts) {
    if (opts->struct_size != sizeof(externd_opts))
      return fail(EXTERND_EINVAL, "externd_opts.struct_size %u != %zu", opts->struct_size,
                  sizeof(externd_opts));
    o = *opts;
  }
  if (o.mode < -1 || o.mode > 2) return fail(EXTERND_EINVAL, "bad mode %d", o.mode);
  if (o.sweeps < 0) return fail(EXTERND_EINVAL, "sweeps must be >= 0");
  if (!std::isfinite(o.importance_lambda) || o.importance_lambda < 0.f)
    return fail(EXTERND_EINVAL, "importance_lambda must be finite and >= 0");
  if (o.ternarizer != EXTERND_TERN_MEAN && o.ternarizer != EXTERND_TERN_PROJECTION)
    return fail(EXTERND_EINVAL, "bad ternarizer %d", o.ternarizer);
  const bool projection = o.ternarizer == EXTERND_TERN_PROJECTION;
  if (projection && (m > externd::kProjMaxN || n > externd::kProjMaxN))
    return fail(EXTERND_EUNSUPPORTED, "the optimal projection takes vectors of at most %d entries",
                externd::kProjMaxN);
  if (projection && (o.mode == EXTERND_MODE_RESIDENT || o.mode == EXTERND_MODE_PERSISTENT))
    return fail(EXTERND_EUNSUPPORTED, "the optimal projection runs in streaming or block mode");
  if (o.workspace && (reinterpret_cast<uintptr_t>(o.workspace) & 255u) != 0)
    return fail(EXTERND_EINVAL, "workspace must be 256-byte aligned");
  if (o.safeguard != 0 && o.safeguard != 1) return fail(EXTERND_EINVAL, "bad safeguard %d", o.safeguard);
  const int b = externd_block_width(m, n, block);
  if (b > EXTERND_MAX_BLOCK)
    return fail(EXTERND_EUNSUPPORTED, "block width %d exceeds the widest supported block, %d", b,
                EXTERND_MAX_BLOCK);
  if (o.sweeps > 0 && b == 1)
    return fail(EXTERND_EINVAL, "refinement sweeps need block mode (block width %d)", b);
  if (o.safeguard && b > 1)
    return fail(EXTERND_EUNSUPPORTED, "the safeguard's replacement runs in the sequential path only");
  if (o.safeguard && projection)
    return fail(EXTERND_EUNSUPPORTED, "the safeguard is not combined with the optimal projection");
  if (o.safeguard && (o.mode == EXTERND_MODE_RESIDENT || o.mode == EXTERND_MODE_PERSISTENT))
    return fail(EXTERND_EUNSUPPORTED, "the safeguard's replacement runs in streaming mode");
  const externd_block_capture* bc = o.block_capture;
  if (bc && b > 1) {
    const int64_t nblocks = (k + b - 1) / b;
    if (bc->block < 0 || bc->block >= nblocks || bc->iteration < 0 || bc->iteration >= iters)
      return fail(EXTERND_EINVAL, "block capture (block %lld, iteration %d) out of range",
                  (long long)bc->block, bc->iteration);
  }
  int cus = 0;
  int st = check_device(&cus);
  if (st != EXTERND_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (b > 1) {
    externd::BlockArgs ba{};
    ba.A = A;
    ba.m = m;
    ba.n = n;
    ba.k = k;
    ba.b = b;
    ba.tau = tau;
    ba.iters = iters;
    ba.seed = o.seed;
    ba.B2 = B2;
    ba.C2 = C2;
    ba.D = D;
    ba.energy = energy;
    ba.trace = o.trace;
    ba.stats = reinterpret_cast<long long*>(o.stats);
    ba.norm_a2 = o.norm_a2;
    ba.sweeps = o.sweeps;
    ba.sweep_trace = o.sweep_trace;
    ba.importance = o.importance;
    ba.lambda = o.importance_lambda;
    ba.projection = projection ? 1 : 0;
    ba.cap = bc;
    Workspace w;
    if ((st = get_ws(w, o, externd::block_workspace_bytes(m, n, b), s)) != EXTERND_OK) return st;
    hipError_t e = externd::run_block(ba, w.ptr, s);
    if (e != hipSuccess) return hip_fail(e, "block decomposition");
    return EXTERND_OK;
  }

  externd::SeqArgs sa{};
  sa.A = A;
  sa.m = m;
  sa.n = n;
  sa.k = k;
  sa.tau = tau;
  sa.iters = iters;
  sa.seed = o.seed;
  sa.B2 = B2;
  sa.C2 = C2;
  sa.D = D;
  sa.energy = energy;
  sa.trace = o.trace;
  sa.stats = reinterpret_cast<long long*>(o.stats);
  sa.norm_a2 = o.norm_a2;
  sa.importance = o.importance;
  sa.lambda = o.importance_lambda;
  sa.projection = projection ? 1 : 0;
  sa.safeguard = o.safeguard;
  const bool any_capture = o.capture_R || o.capture_Rcol || o.capture_R_next || o.capture_y ||
                           o.capture_x || o.capture_v || o.capture_u || o.capture_d;
  sa.capture_component = o.capture_component;
  if (o.capture_component >= 0 && any_capture) {
    if (o.capture_component >= k) return fail(EXTERND_EINVAL, "capture_component >= k");
    sa.capture_R = o.capture_R;
    sa.capture_Rcol = o.capture_Rcol;
    sa.capture_R_next = o.capture_R_next;
    sa.capture_y = o.capture_y;
    sa.capture_x = o.capture_x;
    sa.capture_v = o.capture_v;
    sa.capture_u = o.capture_u;
    sa.capture_d = o.capture_d;
  } else {
    sa.capture_component = -1;
  }
  const int mode = seq_mode(o.mode, m, n, cus, projection, o.safeguard != 0);
  if (mode < 0)
    return fail(EXTERND_EUNSUPPORTED, "%lld x %lld does not fit the %s kernel", (long long)m, (long long)n,
                o.mode == EXTERND_MODE_RESIDENT ? "resident" : "persistent streaming");
  Workspace w;
  hipError_t e;
  if (mode == EXTERND_MODE_RESIDENT) {
    const int cands = externd::g_single_placement ? 1 : externd::resident_place_candidates(m, n, k);
    if ((st = get_ws(w, o, externd::resident_workspace_bytes(m, n, k, cands), s)) != EXTERND_OK) return st;
    int grid = 0;
    e = externd::run_resident_seq(sa, w.ptr, cands, cus, s, &grid);
    if (e != hipSuccess) return hip_fail(e, "resident decomposition");
  } else if (mode == EXTERND_MODE_PERSISTENT) {
    if ((st = get_ws(w, o, externd::persist_workspace_bytes(m, n, k, cus), s)) != EXTERND_OK) return st;
    e = externd::run_persist_seq(sa, w.ptr, cus, s);
    if (e != hipSuccess) return hip_fail(e, "persistent streaming decomposition");
  } else {
    if ((st = get_ws(w, o, externd::stream_workspace_bytes(m, n), s)) != EXTERND_OK) return st;
    e = externd::run_stream_seq(sa, w.ptr, s);
    if (e != hipSuccess) return hip_fail(e, "streaming decomposition");
  }
  return EXTERND_OK;
}

int externd_energy(const float* A, int64_t m, int64_t n, const uint32_t* B2, const uint32_t* C2,
                   const float* D, int64_t k, void* stream, double* energy) {
  if (!A || !energy) return fail(EXTERND_EINVAL, "null A or energy pointer");
  if (bad_size(m, n) || k < 0) return fail(EXTERND_EINVAL, "bad shape");
  if (k > 0 && (!B2 || !C2 || !D)) return fail(EXTERND_EINVAL, "null factor pointer");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w;
  if ((st = alloc_ws(w, externd::energy_workspace_bytes(m, n), s)) != EXTERND_OK) return st;
  hipError_t e = externd::run_energy(A, m, n, B2, C2, D, k, energy, w.ptr, s);
  if (e != hipSuccess) return hip_fail(e, "energy");
  return EXTERND_OK;
}

int externd_reconstruct(const uint32_t* B2, const uint32_t* C2, const float* D, int64_t m,
                        int64_t n, int64_t k, void* stream, float* A_hat) {
  if (!A_hat) return fail(EXTERND_EINVAL, "null output pointer");
  if (bad_size(m, n) || k < 0) return fail(EXTERND_EINVAL, "bad shape");
  if (k > 0 && (!B2 || !C2 || !D)) return fail(EXTERND_EINVAL, "null factor pointer");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipError_t e = externd::run_reconstruct(B2, C2, D, m, n, k, A_hat, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reconstruct");
  return EXTERND_OK;
}

int externd_ternarize(const float* x, int64_t N, float tau, void* stream, uint32_t* codes,
                      int32_t* nnz) {
  if (!x || !codes) return fail(EXTERND_EINVAL, "null pointer");
  if (N <= 0 || N > (int64_t(1) << 31) - 1) return fail(EXTERND_EINVAL, "bad length");
  if (!std::isfinite(tau) || tau < 0.f) return fail(EXTERND_EINVAL, "tau must be finite and >= 0");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipError_t e = externd::launch_ternarize(x, N, tau, codes, nnz, nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ternarize");
  return EXTERND_OK;
}

int externd_project(const float* x, int64_t N, void* stream, uint32_t* codes, int32_t* nnz) {
  if (!x || !codes) return fail(EXTERND_EINVAL, "null pointer");
  if (N <= 0) return fail(EXTERND_EINVAL, "bad length");
  if (N > externd::kProjMaxN)
    return fail(EXTERND_EUNSUPPORTED, "the optimal projection takes at most %d entries", externd::kProjMaxN);
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipError_t e = externd::launch_project(x, N, codes, nnz, nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "project");
  return EXTERND_OK;
}

int externd_gemv_t(const float* R, int64_t m, int64_t n, const uint32_t* u_codes, void* stream,
                   float* y) {
  if (!R || !u_codes || !y) return fail(EXTERND_EINVAL, "null pointer");
  if (bad_size(m, n)) return fail(EXTERND_EINVAL, "bad shape");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w;
  if ((st = alloc_ws(w, sizeof(float) * (size_t)(externd::gemv_t_chunks(m) * n) + 256, s)) != EXTERND_OK) return st;
  hipError_t e = externd::launch_gemv_t(const_cast<float*>(R), m, n, u_codes,
                                        static_cast<float*>(w.ptr), y, nullptr, nullptr, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "gemv_t");
  return EXTERND_OK;
}

int externd_gemv_n(const float* R, int64_t m, int64_t n, const uint32_t* v_codes, void* stream,
                   float* x) {
  if (!R || !v_codes || !x) return fail(EXTERND_EINVAL, "null pointer");
  if (bad_size(m, n)) return fail(EXTERND_EINVAL, "bad shape");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipError_t e = externd::launch_gemv_n(R, m, n, v_codes, x, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemv_n");
  return EXTERND_OK;
}

int externd_deflate(float* R, int64_t m, int64_t n, const uint32_t* u_codes,
                    const uint32_t* v_codes, float d, void* stream) {
  if (!R || !u_codes || !v_codes) return fail(EXTERND_EINVAL, "null pointer");
  if (bad_size(m, n)) return fail(EXTERND_EINVAL, "bad shape");
  if (!std::isfinite(d)) return fail(EXTERND_EINVAL, "d must be finite");
  int st = check_device(nullptr);
  if (st != EXTERND_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w;
  if ((st = alloc_ws(w, 256, s)) != EXTERND_OK) return st;
  float* dptr = static_cast<float*>(w.ptr);
  hipError_t e = externd::launch_fill_f32(dptr, 1, d, s);
  if (e == hipSuccess) e = externd::launch_deflate(R, m, n, u_codes, v_codes, dptr, s);
  if (e != hipSuccess) return hip_fail(e, "deflate");
  return EXTERND_OK;
}

}  // extern "C"
