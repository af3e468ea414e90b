// Instances of the fused chunked forward for f32 activations, padded key dim 16.
#include "kda_chunk_fwd.h"
#include "kda_launch.h"

namespace kda {

template <>
hipError_t launch_chunk_fwd_kd<float, 16>(int VT, int C, const void* q, const void* k, const void* v, const void* z,
                                      const float* A_log, const float* dt_bias, const void* beta,
                                      const float* state_in, float scale, void* o, float* state_out, float* ckpt,
                                      int B, int H, int T, int K, int V, int zc, hipStream_t s) {
#define KDA_CASE(VT_, C_)                                                                                  \
  if (VT == VT_ && C == C_)                                                                                \
    return launch_chunk_fwd_inst<float, 16, VT_, C_>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o,     \
                                                   state_out, ckpt, B, H, T, K, V, zc, s);
  KDA_CASE(16, 16)
  KDA_CASE(16, 32)
  KDA_CASE(16, 64)
  KDA_CASE(32, 16)
  KDA_CASE(32, 32)
  KDA_CASE(32, 64)
  KDA_CASE(64, 16)
  KDA_CASE(64, 32)
  KDA_CASE(64, 64)
#undef KDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
