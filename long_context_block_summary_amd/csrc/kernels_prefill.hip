// kernels_prefill.hip -- chunked-prefill variant (not built yet).
#include "../../include/bsa.h"

extern "C" {
size_t bsa_prefill_workspace_size(const bsa_shape*, int32_t, const bsa_prefill_cfg*) { return SIZE_MAX; }
int sparse_prefill_attn(const void*, int32_t, const void*, const void*, const float*, const void*,
                        const void*, const void*, const void*, const bsa_shape*,
                        const bsa_prefill_cfg*, float, float*, float*, int32_t*, void*, size_t,
                        void*) {
  return BSA_UNSUPPORTED;
}
}
