// Chunked causal prefill (placeholder until the kernels land).
#include "tt_device.hpp"
#include "tt_internal.hpp"

namespace tt {

int plan_prefill(int B, int H, int N, int dk, int dv, int n, int chunk, tt_dtype dt, PrefillPlan* p) {
  (void)dt;
  if (chunk != 64) return fail(TT_ERR_UNSUPPORTED, "chunk=%d not compiled (64 only)", chunk);
  p->W = rows_for(dk, n);
  p->Wpad = (p->W + 31) / 32 * 32;
  p->chunk = chunk;
  p->span = N;
  p->nspan = 1;
  p->ngroups = 1;
  p->ws_floats = 0;
  (void)B; (void)H; (void)dv;
  return TT_OK;
}

hipError_t launch_prefill(const void*, const void*, const void*, tt_dtype, int, int, int, int, const PrefillPlan&,
                          float*, float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace tt
