// Batched per-phase decoder for large d_model (not built yet: reports unsupported).
#include "device_common.h"
#include "rlt_internal.h"

namespace rlt {

bool dec_batched_supported(const ModelLayout& m) {
  (void)m;
  return false;
}

size_t dec_batched_scratch_bytes(const ModelLayout& m, int B, int T) {
  (void)m; (void)B; (void)T;
  return 0;
}

hipError_t run_dec_batched(const ModelLayout& m, const StateLayout& s, const char* ws, char* state, float* s_out,
                           int t0, int n, hipStream_t st) {
  (void)m; (void)s; (void)ws; (void)state; (void)s_out; (void)t0; (void)n; (void)st;
  return hipErrorInvalidValue;
}

}  // namespace rlt
