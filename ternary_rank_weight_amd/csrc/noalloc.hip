// externd_decompose_noalloc: the sequential decomposition for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  It runs the resident sequential
// path, whose scratch memory (exchange slots, partial sums, flags, the
// safeguard bitmap: 144 KB at 2560 x 2560, k = 5120) lives in the file-scope
// device array `scratch` below instead of a stream-ordered allocation.
//
// `scratch` is a host-side stand-in in host code: its device address on the
// current device is looked up once per device with hipGetSymbolAddress, and
// only that address is ever handed to a kernel.  Every call on a device
// shares that device's array, which keeps the last call's contents; the
// kernels clear what must start at zero (fill kernels, no memset) at the
// start of each call.  Calls that overlap on one device race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(1) << 18;   // 256 KiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up with that
// device current on its first use and kept for later calls.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int externd_decompose_noalloc(const float* A, int64_t m, int64_t n, float mu, float tau,
                                         int32_t iters, int32_t block, void* stream, uint32_t* B2,
                                         uint32_t* C2, float* D, double* energy,
                                         const externd_opts* opts) {
  externd_opts o{};
  o.struct_size = sizeof(externd_opts);
  o.mode = EXTERND_MODE_AUTO;
  o.capture_component = -1;
  if (opts) {
    if (opts->struct_size != sizeof(externd_opts))
      return externd::report(EXTERND_EINVAL, "externd_opts.struct_size does not match this library");
    o = *opts;
  }
  if (o.workspace)
    return externd::report(EXTERND_EINVAL, "externd_decompose_noalloc brings its own scratch: opts.workspace must be NULL");
  if (externd_block_width(m, n, block) > 1 || o.mode == EXTERND_MODE_STREAMING || o.mode == EXTERND_MODE_PERSISTENT)
    return externd::report(EXTERND_EUNSUPPORTED, "externd_decompose_noalloc runs the resident sequential path only");
  o.mode = EXTERND_MODE_RESIDENT;
  // one placement of the exchange words (no placement probe): the size of
  // the static scratch does not grow with the probe's copies
  uint64_t need = externd_workspace_bytes(m, n, mu, block, EXTERND_MODE_RESIDENT);
  if (need > 0) need = externd::resident_workspace_bytes(m, n, externd_rank(m, n, mu), 1);
  if (need > kScratchBytes) {
    char msg[160];
    std::snprintf(msg, sizeof(msg), "needs %llu bytes of scratch, above the static %zu",
                  (unsigned long long)need, kScratchBytes);
    return externd::report(EXTERND_ENOMEM, msg);
  }
  void* p = nullptr;
  const hipError_t e = scratch_address(&p);
  if (e != hipSuccess) {
    char msg[160];
    std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    return externd::report(EXTERND_EHIP, msg);
  }
  // Always with the scratch as the workspace: argument errors (need == 0
  // above) are then reported by the shared validation, and nothing below
  // can fall back to an allocation.
  o.workspace = p;
  o.workspace_bytes = kScratchBytes;
  externd::g_single_placement = true;
  const int st = externd_decompose(A, m, n, mu, tau, iters, block, stream, B2, C2, D, energy, &o);
  externd::g_single_placement = false;
  return st;
}
