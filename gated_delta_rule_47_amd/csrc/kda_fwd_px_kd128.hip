// Instances of the paired bf16 forward (V = 128), padded key dim 128.
#include "kda_chunk_fwd_px.h"
#include "kda_launch.h"

namespace kda {

// Workspace of the paired forward: the status header and one ring per pair of a launch
// (launches cover at most PX_MAX_PAIRS heads each and reuse the rings in stream order).
size_t px_workspace_bytes(int KD, int nheads) {
  int pb = 0;
  switch (KD) {
    case 32: pb = PxCfg<32>::PAIR_BYTES; break;
    case 64: pb = PxCfg<64>::PAIR_BYTES; break;
    case 128: pb = PxCfg<128>::PAIR_BYTES; break;
    default: return 0;
  }
  const int np = nheads < PX_MAX_PAIRS ? nheads : PX_MAX_PAIRS;
  return (size_t)PX_HEADER + (size_t)np * pb;
}

template <>
hipError_t launch_chunk_fwd_px_kd<128>(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                       const float* dt_bias, const void* beta, const float* state_in, float scale,
                                       void* o, float* state_out, int B, int H, int T, int K, int zc, void* work,
                                       unsigned long long spin_ticks, hipStream_t s) {
  return zc ? launch_chunk_fwd_px_inst<128, false>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B,
                                                   H, T, K, work, spin_ticks, s)
            : launch_chunk_fwd_px_inst<128, true>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B,
                                                  H, T, K, work, spin_ticks, s);
}

}  // namespace kda
