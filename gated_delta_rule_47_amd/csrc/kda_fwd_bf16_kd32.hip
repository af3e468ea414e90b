// Instances of the pipelined chunked forward for bf16 activations, padded key dim 32
// (per-channel gate, zc = 1, and scalar-decay gate, zc = 0).
#include "kda_chunk_fwd_pc.h"
#include "kda_launch.h"

namespace kda {

template <>
hipError_t launch_chunk_fwd_pc_kd<32>(int VT, int C, const void* q, const void* k, const void* v, const void* z,
                                      const float* A_log, const float* dt_bias, const void* beta,
                                      const float* state_in, float scale, void* o, float* state_out, int B, int H,
                                      int T, int K, int V, int zc, hipStream_t s) {
#define KDA_CASE(VT_, C_)                                                                                       \
  if (VT == VT_ && C == C_)                                                                                     \
    return zc ? launch_chunk_fwd_pc_inst<32, VT_, C_, false>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o,   \
                                                             state_out, B, H, T, K, V, s)                       \
              : launch_chunk_fwd_pc_inst<32, VT_, C_, true>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o,    \
                                                            state_out, B, H, T, K, V, s);
  KDA_CASE(16, 16)
  KDA_CASE(16, 32)
  KDA_CASE(32, 16)
  KDA_CASE(32, 32)
  KDA_CASE(64, 16)
  KDA_CASE(64, 32)
#undef KDA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
