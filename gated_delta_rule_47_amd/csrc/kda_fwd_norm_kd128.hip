// Instance of the bf16 forward with the fused output norm, padded key dim 128.
#include "kda_chunk_fwd_pc.h"
#include "kda_launch.h"

namespace kda {

template <>
hipError_t launch_chunk_fwd_norm_kd<128>(const void* q, const void* k, const void* v, const void* z,
                                       const float* A_log, const float* dt_bias, const void* beta,
                                       const float* state_in, float scale, const float* norm_w, float eps, void* o,
                                       float* state_out, int B, int H, int T, int K, int V, void* work,
                                       unsigned long long spin_ticks, hipStream_t s) {
  return launch_chunk_fwd_norm_inst<128>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, norm_w, eps, o, state_out,
                                        B, H, T, K, V, work, spin_ticks, s);
}

size_t norm_workspace_bytes(int B, int H, int T, int V) {
  if (V <= 64 || T < 1) return 0;
  const size_t nck = (size_t)(T + 31) / 32;
  return PN_HEADER + (size_t)B * H * 2 * nck * 256;
}

}  // namespace kda
