// gdn_prefill.hip -- chunked prefill of the gated delta rule (gfx950).
// Placeholder entry points: every call reports GDN_EUNSUPPORTED until the
// chunked kernels are in place.
#include <hip/hip_runtime.h>

#include "gdn.h"

extern "C" size_t gdn_prefill_workspace_bytes(int32_t, int32_t, int32_t,
                                              int32_t, int32_t, int32_t) {
  return 0;
}

extern "C" int gdn_prefill_chunked(int32_t, int32_t, int32_t, int32_t,
                                   int32_t, int32_t, int32_t, const void*,
                                   const void*, const void*, int,
                                   const float*, const float*, const float*,
                                   float*, float*, float*, void*, size_t,
                                   float, int, void*) {
  return GDN_EUNSUPPORTED;
}
