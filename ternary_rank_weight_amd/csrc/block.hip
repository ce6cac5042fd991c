// Block ALS path (ExTernD §2.4) — placeholder until the MFMA implementation lands.
#include "device_common.hpp"
#include "kernels.hpp"

namespace externd {

size_t block_workspace_bytes(int64_t m, int64_t n, int b) { return 256; }

hipError_t run_block(const BlockArgs& a, void* ws, hipStream_t s) { return hipErrorNotSupported; }

}  // namespace externd
