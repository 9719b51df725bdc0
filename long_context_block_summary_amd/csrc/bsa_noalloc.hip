// bsa_noalloc.hip -- sparse_decode_step for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc).  The step's workspace -- the block scores, then the split-K
// partials -- lives in a file-scope device array instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "../../include/bsa.h"

namespace {

// One copy per GPU, held until the process ends.  In host code this name is
// only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress below and is the only handle host code passes on.
__device__ __align__(256) unsigned char scratch[BSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The scratch array's device address on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BSA_HIP_ERROR;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();  // leave no sticky error for the caller's next call
      return BSA_HIP_ERROR;
    }
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return BSA_OK;
}

}  // namespace

extern "C" int sparse_decode_step_noalloc(const void* q, const void* k, const void* v,
                                          const void* summaries, const bsa_shape* shape,
                                          const bsa_select_cfg* cfg, int32_t* block_idx,
                                          float scale, float* out, float* lse,
                                          void* hip_stream) {
  const size_t need = bsa_decode_step_workspace_size(shape, cfg);
  if (need == SIZE_MAX) return BSA_INVALID_ARG;
  if (need > (size_t)BSA_NOALLOC_SCRATCH_BYTES) return BSA_UNSUPPORTED;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != BSA_OK) return rc;
  // the step needs no zeroed scratch: every score and partial it reads is
  // written earlier in the same call
  return sparse_decode_step(q, k, v, summaries, shape, cfg, block_idx, scale, out, lse, ws,
                            (size_t)BSA_NOALLOC_SCRATCH_BYTES, hip_stream);
}
