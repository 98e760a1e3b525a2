// Causal block-sparse GSA prefill (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "gsa.h"
#include "gsa_plan.hpp"

using namespace gsa;

extern "C" gsa_status_t gsa_prefill_workspace_size(const gsa_prefill_params* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(GSA_ERR_INVALID_ARG, "bytes is NULL");
  PrefillPlan pl;
  gsa_status_t s = plan_prefill(p, &pl);
  if (s != GSA_OK) return s;
  *bytes = pl.total;
  return GSA_OK;
}

extern "C" gsa_status_t gsa_prefill_blocksparse(const gsa_prefill_params* p, const void* q,
                                                const void* k_cache, const void* v_cache, float* out,
                                                int32_t* sel, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  clear_error();
  PrefillPlan pl;
  gsa_status_t s = plan_prefill(p, &pl);
  if (s != GSA_OK) return s;
  return fail(GSA_ERR_UNSUPPORTED, "prefill kernel not built yet");
}
