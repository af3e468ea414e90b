// Host-side launchers of the KDA kernels (definitions in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kda_common.h"

namespace kda {

template <typename Tin>
hipError_t launch_gate(const void* z, const float* A_log, const float* dt_bias, float* g, float* alpha, int B, int H,
                       int T, int K, hipStream_t s);

// Gate adjoint: dz (nullable), dA_log and d_dt_bias (nullable) for a cotangent dg.
size_t gate_bwd_workspace_bytes(int B, int H, int T, int K);
// Device address of the current device's built-in gate-adjoint scratch
// (KDA_GATE_BWD_SCRATCH_BYTES), looked up once per device.
hipError_t gate_bwd_scratch(void** ptr);
template <typename Tin>
hipError_t launch_gate_bwd(const void* z, const float* A_log, const float* dt_bias, const float* dg, float* dz,
                           float* dA_log, float* d_dt_bias, void* workspace, int B, int H, int T, int K,
                           hipStream_t s);

template <typename Tin>
hipError_t launch_step(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                       const float* dt_bias, const void* beta, float* state, float scale, void* o, int B, int H,
                       int K, int V, int zc, hipStream_t s);

// Gate layout of the forward and step launchers: zc = 1, z is (B,H,T,K) and dt_bias (H,K);
// zc = 0, the scalar-decay case, z is (B,H,T) and dt_bias (H).

// Chunked forward: instance chosen by (padded key dim KD, value tile VT, chunk C).
// ckpt (nullable) receives the state at every chunk start: (B,H,ceil(T/C),K,V) fp32.
template <typename Tin, int KD>
hipError_t launch_chunk_fwd_kd(int VT, int C, const void* q, const void* k, const void* v, const void* z,
                               const float* A_log, const float* dt_bias, const void* beta, const float* state_in,
                               float scale, void* o, float* state_out, float* ckpt, int B, int H, int T, int K, int V,
                               int zc, hipStream_t s);

// Pipelined bf16 forward (16 waves, internal blocks of C <= 32 tokens).
template <int KD>
hipError_t launch_chunk_fwd_pc_kd(int VT, int C, const void* q, const void* k, const void* v, const void* z,
                                  const float* A_log, const float* dt_bias, const void* beta, const float* state_in,
                                  float scale, void* o, float* state_out, int B, int H, int T, int K, int V, int zc,
                                  hipStream_t s);

// Paired bf16 forward for V = 128 (two workgroups per head share the gate and WY work
// through a ring in `work`, px_workspace_bytes() of it; see kda_chunk_fwd_px.h).
template <int KD>
hipError_t launch_chunk_fwd_px_kd(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                  const float* dt_bias, const void* beta, const float* state_in, float scale, void* o,
                                  float* state_out, int B, int H, int T, int K, int zc, void* work,
                                  unsigned long long spin_ticks, hipStream_t s);
size_t px_workspace_bytes(int KD, int nheads);

// The bf16 forward with the output RMSNorm fused into its output stage (o holds
// y = o / sqrt(mean_v o^2 + eps) * norm_w[h]); when V > 64 the two value tiles of a head
// exchange per-token sums of squares through `work` (norm_workspace_bytes() of it).
template <int KD>
hipError_t launch_chunk_fwd_norm_kd(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                    const float* dt_bias, const void* beta, const float* state_in, float scale,
                                    const float* norm_w, float eps, void* o, float* state_out, int B, int H, int T,
                                    int K, int V, void* work, unsigned long long spin_ticks, hipStream_t s);
size_t norm_workspace_bytes(int B, int H, int T, int V);

// Forward tiling actually used for (dtype, K, V, chunk): padded key dim, value tile
// and the chunk the kernel blocks by.  Returns false when no instance exists.
struct FwdPlan {
  int KD, VT, C;
};
bool fwd_plan(bool bf16, int K, int V, int chunk, FwdPlan* plan);

// Chunked adjoint on MFMA (fp32 activations), see kda_bwd_chunk.hip.
size_t chunk_bwd_mfma_workspace_bytes(int B, int H, int T, int K, int V);
hipError_t launch_chunk_bwd_mfma(const float* q, const float* k, const float* v, const float* z, const float* A_log,
                                 const float* dt_bias, const float* beta, const float* state_in, float scale,
                                 const float* d_o, const float* d_state_out, float* dq, float* dk, float* dv,
                                 float* dg, float* dbeta, float* dstate_in, void* workspace, int B, int H, int T,
                                 int K, int V, hipStream_t s);


}  // namespace kda
