// The sweep-kernel prefill path compiled for chunks of 128 tokens (one unit
// per chunk length, so that the instantiations build in parallel).
#include "tt_prefill_kernels.hpp"

namespace tt {

hipError_t sweep_shape_chunk128(int dk, int n, tt_dtype dt, int* wp, int* ngroups, int* nrg) {
  return sweep_shape<128>(dk, n, dt, wp, ngroups, nrg);
}

hipError_t sweep_launch_chunk128(const void* Q, const void* K, const void* V, tt_dtype dt, int BH, int N, int dk,
                                int n, const PrefillPlan& p, const float* states_in, float* O, float* den_out,
                                float* states, float* ws, hipStream_t s) {
  return sweep_launch<128>(Q, K, V, dt, BH, N, dk, n, p, states_in, O, den_out, states, ws, s);
}

}  // namespace tt
