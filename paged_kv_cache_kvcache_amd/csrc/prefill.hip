// pa_prefill_varlen (placeholder until the MFMA kernel lands).
#include "common.hpp"

extern "C" int pa_prefill_varlen(const void*, const void*, const void*, const int32_t*,
                                 const int32_t*, int32_t, int32_t, int32_t, const int32_t*,
                                 int32_t, float, void*, const pa_desc* desc, void*) {
  int rc = pa::check_desc(desc);
  if (rc) return rc;
  return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill_varlen: not built yet");
}
