// Instances of the paired bf16 forward (V = 128), padded key dim 32.
#include "kda_chunk_fwd_px.h"
#include "kda_launch.h"

namespace kda {

template <>
hipError_t launch_chunk_fwd_px_kd<32>(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                       const float* dt_bias, const void* beta, const float* state_in, float scale,
                                       void* o, float* state_out, int B, int H, int T, int K, int zc, void* work,
                                       unsigned long long spin_ticks, hipStream_t s) {
  return zc ? launch_chunk_fwd_px_inst<32, false>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B,
                                                   H, T, K, work, spin_ticks, s)
            : launch_chunk_fwd_px_inst<32, true>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B,
                                                  H, T, K, work, spin_ticks, s);
}

}  // namespace kda
