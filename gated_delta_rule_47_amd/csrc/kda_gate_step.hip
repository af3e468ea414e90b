// Standalone gate kernel and the single-token decode step.
//
// Gate: the released KDA decay form g = -exp(clamp(A_log)) * softplus(z + dt_bias),
// alpha = exp(g) (kdafix page, "Fix 1 -- decay form").  Elementwise, HBM-bound:
// each thread handles one element per grid-stride step; consecutive lanes touch
// consecutive addresses.
//
// Decode step: one token of the gated delta rule per (batch, head), the state read
// and written in place.  The state dominates the traffic (2*K*V*4 bytes per head),
// so one workgroup owns a tile of VTS value columns and all K rows of one head;
// lanes map to consecutive value columns, so every state row access is a
// contiguous VTS*4-byte segment.  The two reductions over K (the delta read
// S'^T k and the output S^T q_hat) are a per-thread partial sum over its rows
// followed by one LDS exchange between the NRG row groups.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

template <typename Tin>
__global__ void __launch_bounds__(256) gate_kernel(const Tin* __restrict__ z, const float* __restrict__ A_log,
                                                   const float* __restrict__ dt_bias, float* __restrict__ g_out,
                                                   float* __restrict__ alpha_out, int H, int T, int K, long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += stride) {
    const int c = (int)(idx % K);
    const int h = (int)((idx / K / T) % H);
    const float mult = gate_multiplier(A_log[h]);
    const float x = to_f<Tin>(z[idx]) + (dt_bias ? dt_bias[h * K + c] : 0.0f);
    const float g = -mult * softplus_f(x, true);
    g_out[idx] = g;
    if (alpha_out) alpha_out[idx] = fast_exp2(g * kLog2e);
  }
}

template <typename Tin, int K, int VTS>
__global__ void __launch_bounds__(256) step_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const Tin* __restrict__ v, const Tin* __restrict__ z,
                                                   const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                                                   const Tin* __restrict__ beta, float* __restrict__ state,
                                                   float scale, Tin* __restrict__ o, int H, int V) {
  constexpr int NRG = cmin(256 / VTS, K);   // row groups
  constexpr int RPT = K / NRG;              // rows per thread
  __shared__ float sAl[K], sK[K], sQ[K], sRed[NRG * VTS];

  const int nvt = V / VTS;
  const int bh = blockIdx.x / nvt;
  const int v0 = (blockIdx.x % nvt) * VTS;
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int vc = tid % VTS;
  const int rg = tid / VTS;

  const float mult = gate_multiplier(A_log[h]);
  for (int c = tid; c < K; c += NRG * VTS) {
    const float x = to_f<Tin>(z[(size_t)bh * K + c]) + (dt_bias ? dt_bias[h * K + c] : 0.0f);
    sAl[c] = fast_exp2(-mult * softplus_f(x, true) * kLog2e);
    sK[c] = to_f<Tin>(k[(size_t)bh * K + c]);
    sQ[c] = scale * to_f<Tin>(q[(size_t)bh * K + c]);
  }
  lds_barrier();

  float* S = state + (size_t)bh * K * V + v0 + vc;
  float s[RPT];
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + NRG * i;
    s[i] = S[(size_t)c * V] * sAl[c];          // S' = diag(alpha) S
    r += s[i] * sK[c];                         // partial S'^T k
  }
  sRed[rg * VTS + vc] = r;
  lds_barrier();
  float rt = 0.0f;
#pragma unroll
  for (int g = 0; g < NRG; ++g) rt += sRed[g * VTS + vc];
  const float e = to_f<Tin>(v[(size_t)bh * V + v0 + vc]) - rt;
  const float b = to_f<Tin>(beta[bh]);
  float ov = 0.0f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + NRG * i;
    s[i] += b * sK[c] * e;                     // S = S' + beta k e^T
    ov += s[i] * sQ[c];                        // partial S^T q_hat
    S[(size_t)c * V] = s[i];
  }
  lds_barrier();
  sRed[rg * VTS + vc] = ov;
  lds_barrier();
  if (rg == 0) {
    float ot = 0.0f;
#pragma unroll
    for (int g = 0; g < NRG; ++g) ot += sRed[g * VTS + vc];
    o[(size_t)bh * V + v0 + vc] = from_f<Tin>(ot);
  }
}

// ------------------------------------------------------------------ launchers
template <typename Tin>
hipError_t launch_gate(const void* z, const float* A_log, const float* dt_bias, float* g, float* alpha,
                       int B, int H, int T, int K, hipStream_t s) {
  const long long n = (long long)B * H * T * K;
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gate_kernel<Tin>, dim3((unsigned)blocks), dim3(256), 0, s, (const Tin*)z, A_log, dt_bias, g,
                     alpha, H, T, K, n);
  return hipGetLastError();
}

template <typename Tin, int K, int VTS>
static hipError_t launch_step_kv(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                 const float* dt_bias, const void* beta, float* state, float scale, void* o, int B,
                                 int H, int V, hipStream_t s) {
  constexpr int NRG = cmin(256 / VTS, K);
  const int grid = B * H * (V / VTS);
  hipLaunchKernelGGL((step_kernel<Tin, K, VTS>), dim3(grid), dim3(NRG * VTS), 0, s, (const Tin*)q, (const Tin*)k,
                     (const Tin*)v, (const Tin*)z, A_log, dt_bias, (const Tin*)beta, state, scale, (Tin*)o, H, V);
  return hipGetLastError();
}

template <typename Tin, int K>
static hipError_t launch_step_k(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                const float* dt_bias, const void* beta, float* state, float scale, void* o, int B,
                                int H, int V, hipStream_t s) {
  switch (V) {
    case 8: return launch_step_kv<Tin, K, 8>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    case 16: return launch_step_kv<Tin, K, 16>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    case 32: return launch_step_kv<Tin, K, 32>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    default: return launch_step_kv<Tin, K, 64>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
  }
}

template <typename Tin>
hipError_t launch_step(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                       const float* dt_bias, const void* beta, float* state, float scale, void* o, int B, int H,
                       int K, int V, hipStream_t s) {
  switch (K) {
    case 8: return launch_step_k<Tin, 8>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    case 16: return launch_step_k<Tin, 16>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    case 32: return launch_step_k<Tin, 32>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    case 64: return launch_step_k<Tin, 64>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
    default: return launch_step_k<Tin, 128>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, s);
  }
}

template hipError_t launch_gate<float>(const void*, const float*, const float*, float*, float*, int, int, int, int,
                                       hipStream_t);
template hipError_t launch_gate<bf16_t>(const void*, const float*, const float*, float*, float*, int, int, int, int,
                                        hipStream_t);
template hipError_t launch_step<float>(const void*, const void*, const void*, const void*, const float*, const float*,
                                       const void*, float*, float, void*, int, int, int, int, hipStream_t);
template hipError_t launch_step<bf16_t>(const void*, const void*, const void*, const void*, const float*,
                                        const float*, const void*, float*, float, void*, int, int, int, int,
                                        hipStream_t);

}  // namespace kda
