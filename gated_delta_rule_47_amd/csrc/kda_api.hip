// C ABI of libkda (see include/kda.h): argument checks, dispatch to kernel
// instances, status codes and call counters.  No allocation, no printing, no
// exceptions across the boundary, no fallback path.
#include <atomic>
#include <stdint.h>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace kda {

static std::atomic<unsigned long long> g_counters[KDA_NUM_COUNTERS];

static int reject(int status) {
  g_counters[KDA_COUNTER_REJECTED].fetch_add(1, std::memory_order_relaxed);
  return status;
}

// Bound of every wait for the partner workgroup, in 100 MHz real-time ticks (1 s).
static std::atomic<unsigned long long> g_spin_ticks{100000000ull};

// A bf16 call with two value tiles of 64 columns and blocks of 32 tokens runs paired.
static bool px_eligible(bool bf16, int V, int chunk) { return bf16 && V == 128 && chunk >= 32; }

static bool valid_dim(int d) { return d == 8 || d == 16 || d == 32 || d == 64 || d == 128; }
static bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64; }
static size_t esize(int dtype) { return dtype == KDA_BF16 ? 2 : 4; }

// True when [a, a+na) and [b, b+nb) share a byte.
static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool fwd_plan(bool bf16, int K, int V, int chunk, FwdPlan* p) {
  if (!valid_dim(K) || !valid_dim(V) || !valid_chunk(chunk)) return false;
  if (bf16) {
    p->KD = K < 32 ? 32 : K;
    p->VT = V < 16 ? 16 : (V > 64 ? 64 : V);
    p->C = chunk > 32 ? 32 : chunk;
  } else {
    p->KD = K < 16 ? 16 : K;
    // 16-column value tiles from K = 64 up: the fp32 kernel is latency-bound per block, so
    // more workgroups per head beat wider tiles (measured: 16% less time at 2 x 16 heads,
    // K = V = 128, T = 8192)
    const int vtmax = p->KD >= 64 ? 16 : 64;
    p->VT = V < 16 ? 16 : (V > vtmax ? vtmax : V);
    p->C = (p->KD == 128 && chunk > 32) ? 32 : chunk;
  }
  return true;
}

static hipError_t launch_fwd(bool bf16, const FwdPlan& p, const void* q, const void* k, const void* v, const void* z,
                             const float* A_log, const float* dt_bias, const void* beta, const float* state_in,
                             float scale, void* o, float* state_out, int B, int H, int T, int K, int V, int zc,
                             hipStream_t s) {
#define KDA_FWD(TYPE, KD_)                                                                                    \
  return launch_chunk_fwd_kd<TYPE, KD_>(p.VT, p.C, q, k, v, z, A_log, dt_bias, beta, state_in, scale, o,     \
                                         state_out, nullptr, B, H, T, K, V, zc, s)
#define KDA_FWD_PC(KD_)                                                                                       \
  return launch_chunk_fwd_pc_kd<KD_>(p.VT, p.C, q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B, \
                                     H, T, K, V, zc, s)
  if (bf16) {
    switch (p.KD) {
      case 32: KDA_FWD_PC(32);
      case 64: KDA_FWD_PC(64);
      case 128: KDA_FWD_PC(128);
    }
  } else {
    switch (p.KD) {
      case 16: KDA_FWD(float, 16);
      case 32: KDA_FWD(float, 32);
      case 64: KDA_FWD(float, 64);
      case 128: KDA_FWD(float, 128);
    }
  }
#undef KDA_FWD
#undef KDA_FWD_PC
  return hipErrorInvalidValue;
}

// Copies state_in to state_out (or zeroes it) for T == 0 with a plain copy kernel.
__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace kda

using namespace kda;

extern "C" {

float kda_read_scale(int K) { return K > 0 ? (float)(1.0 / __builtin_sqrt((double)K)) : 0.0f; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "null pointer";
    case KDA_ERR_SHAPE: return "unsupported shape";
    case KDA_ERR_DTYPE: return "unsupported dtype";
    case KDA_ERR_CHUNK: return "unsupported chunk size";
    case KDA_ERR_ALIAS: return "output aliases an input";
    case KDA_ERR_HIP: return "HIP launch or runtime error";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_ALIGN: return "misaligned activation pointer";
    case KDA_ERR_EXCHANGE: return "the two workgroups of a head failed to exchange blocks (outputs undefined)";
    case KDA_ERR_SCRATCH: return "sizes need more than the built-in scratch of the allocation-free call";
    default: return "unknown status";
  }
}

int kda_get_counters(unsigned long long* out, int n) {
  if (out) {
    for (int i = 0; i < n && i < KDA_NUM_COUNTERS; ++i) out[i] = g_counters[i].load(std::memory_order_relaxed);
  }
  return KDA_NUM_COUNTERS;
}

int kda_gate(const void* z, const float* A_log, const float* dt_bias, float* g_out, float* alpha_out, int B, int H,
             int T, int K, int dtype, void* stream) {
  if (!A_log || (T != 0 && (!z || !g_out))) return reject(KDA_ERR_NULL);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return reject(KDA_ERR_DTYPE);
  if (B < 1 || H < 1 || T < 0 || K < 1) return reject(KDA_ERR_SHAPE);
  const size_t n = (size_t)B * H * T * K;
  if (overlap(g_out, n * 4, z, n * esize(dtype)) || overlap(alpha_out, n * 4, z, n * esize(dtype)) ||
      overlap(g_out, n * 4, alpha_out, n * 4))
    return reject(KDA_ERR_ALIAS);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == KDA_BF16 ? launch_gate<bf16_t>(z, A_log, dt_bias, g_out, alpha_out, B, H, T, K, s)
                                   : launch_gate<float>(z, A_log, dt_bias, g_out, alpha_out, B, H, T, K, s);
  if (e != hipSuccess) return reject(KDA_ERR_HIP);
  g_counters[KDA_COUNTER_GATE].fetch_add(1, std::memory_order_relaxed);
  return KDA_OK;
}

}  // extern "C"

// kda_chunk_fwd (zc = 1: z (B,H,T,K), dt_bias (H,K)) and kda_chunk_fwd_scalar (zc = 0:
// z (B,H,T), dt_bias (H)): checks, then one launch.
static int chunk_fwd_impl(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                          const float* dt_bias, const void* beta, const float* state_in, float scale, int chunk,
                          void* o, float* state_out, void* workspace, size_t workspace_bytes, int B, int H, int T,
                          int K, int V, int dtype, void* stream, int zc) {
  if (!A_log || (T != 0 && (!q || !k || !v || !z || !beta || !o))) return reject(KDA_ERR_NULL);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return reject(KDA_ERR_DTYPE);
  if (B < 1 || H < 1 || T < 0 || !valid_dim(K) || !valid_dim(V)) return reject(KDA_ERR_SHAPE);
  if (!valid_chunk(chunk)) return reject(KDA_ERR_CHUNK);
  const size_t es = esize(dtype);
  // one head's activations are addressed with 32-bit byte offsets (including the
  // reads of up to 64 tokens past T that the range check turns into zeros)
  if ((size_t)(T + 64) * (size_t)(K > V ? K : V) * es > 0x7fffffffu) return reject(KDA_ERR_SHAPE);
  const uintptr_t amask = 2 * es - 1;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (zc ? (uintptr_t)z : 0)) & amask) return reject(KDA_ERR_ALIGN);
  if ((uintptr_t)z & (es - 1)) return reject(KDA_ERR_ALIGN);
  const size_t nk = (size_t)B * H * T * K * es, nv = (size_t)B * H * T * V * es, nb = (size_t)B * H * T * es;
  const size_t nz = zc ? nk : nb;
  const size_t ns = (size_t)B * H * K * V * 4;
  const void* ins[] = {q, k};
  for (const void* p : ins)
    if (overlap(o, nv, p, nk)) return reject(KDA_ERR_ALIAS);
  if (overlap(o, nv, z, nz) || overlap(o, nv, v, nv) || overlap(o, nv, beta, nb) || overlap(o, nv, state_in, ns) ||
      overlap(o, nv, state_out, ns))
    return reject(KDA_ERR_ALIAS);
  for (const void* p : ins)
    if (overlap(state_out, ns, p, nk)) return reject(KDA_ERR_ALIAS);
  if (overlap(state_out, ns, z, nz) || overlap(state_out, ns, v, nv) || overlap(state_out, ns, beta, nb))
    return reject(KDA_ERR_ALIAS);
  if (state_out && state_in && state_out != state_in && overlap(state_out, ns, state_in, ns))
    return reject(KDA_ERR_ALIAS);
  const size_t na = (size_t)H * 4, ndb = (size_t)H * (zc ? K : 1) * 4;
  if (overlap(o, nv, A_log, na) || overlap(o, nv, dt_bias, ndb) || overlap(state_out, ns, A_log, na) ||
      overlap(state_out, ns, dt_bias, ndb))
    return reject(KDA_ERR_ALIAS);
  FwdPlan plan;
  if (!fwd_plan(dtype == KDA_BF16, K, V, chunk, &plan)) return reject(KDA_ERR_SHAPE);
  // paired path: needs the workspace (without one, each value tile recomputes the
  // gate and WY stages of its head)
  const bool paired = T > 0 && workspace && px_eligible(dtype == KDA_BF16, V, chunk);
  if (paired) {
    const size_t need = px_workspace_bytes(plan.KD, B * H);
    if (workspace_bytes < need) return reject(KDA_ERR_WORKSPACE);
    if ((uintptr_t)workspace & 255) return reject(KDA_ERR_ALIGN);
    struct Buf { const void* p; size_t n; };
    const Buf all[] = {{q, nk}, {k, nk}, {v, nv}, {z, nz}, {beta, nb}, {state_in, ns}, {o, nv}, {state_out, ns},
                       {A_log, (size_t)H * 4}, {dt_bias, (size_t)H * (zc ? K : 1) * 4}};
    for (const Buf& b : all)
      if (overlap(workspace, need, b.p, b.n)) return reject(KDA_ERR_ALIAS);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (paired) {
    {
      const unsigned long long spin = g_spin_ticks.load(std::memory_order_relaxed);
#define KDA_FWD_PX(KD_)                                                                                        \
  e = launch_chunk_fwd_px_kd<KD_>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B, H, T, K, zc, \
                                  workspace, spin, s);                                                         \
  break;
      switch (plan.KD) {
        case 32: KDA_FWD_PX(32)
        case 64: KDA_FWD_PX(64)
        case 128: KDA_FWD_PX(128)
        default: e = hipErrorInvalidValue;
      }
#undef KDA_FWD_PX
    }
  } else if (T == 0) {
    if (state_out && state_out != state_in) {
      const long long n = (long long)B * H * K * V;
      hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, state_in, state_out,
                         n);
      e = hipGetLastError();
    }
  } else {
    e = launch_fwd(dtype == KDA_BF16, plan, q, k, v, z, A_log, dt_bias, beta, state_in, scale, o, state_out, B, H, T,
                   K, V, zc, s);
  }
  if (e != hipSuccess) return reject(KDA_ERR_HIP);
  g_counters[KDA_COUNTER_CHUNK_FWD].fetch_add(1, std::memory_order_relaxed);
  return KDA_OK;
}

// kda_chunk_fwd_norm: the checks of kda_chunk_fwd (bf16 only), the weight row and eps,
// the workspace when the two value tiles of a head exchange sums; then the launches.
static int chunk_fwd_norm_impl(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                               const float* dt_bias, const void* beta, const float* state_in, float scale,
                               int chunk, const float* norm_w, float eps, void* o, float* state_out,
                               void* workspace, size_t workspace_bytes, int B, int H, int T, int K, int V, int dtype,
                               void* stream) {
  if (!A_log || (T != 0 && (!q || !k || !v || !z || !beta || !o))) return reject(KDA_ERR_NULL);
  if (dtype != KDA_BF16) return reject(KDA_ERR_DTYPE);
  if (B < 1 || H < 1 || T < 0 || !valid_dim(K) || !valid_dim(V)) return reject(KDA_ERR_SHAPE);
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return reject(KDA_ERR_SHAPE);
  if (!valid_chunk(chunk)) return reject(KDA_ERR_CHUNK);
  if ((size_t)(T + 64) * (size_t)(K > V ? K : V) * 2 > 0x7fffffffu) return reject(KDA_ERR_SHAPE);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)z) & 3) return reject(KDA_ERR_ALIGN);
  if ((uintptr_t)o & 7) return reject(KDA_ERR_ALIGN);
  const size_t nk = (size_t)B * H * T * K * 2, nv = (size_t)B * H * T * V * 2, nb = (size_t)B * H * T * 2;
  const size_t ns = (size_t)B * H * K * V * 4, na = (size_t)H * 4, ndb = (size_t)H * K * 4, nw = (size_t)H * V * 4;
  struct Buf { const void* p; size_t n; };
  const Buf ins[] = {{q, nk}, {k, nk}, {v, nv}, {z, nk}, {beta, nb}, {A_log, na}, {dt_bias, ndb}, {norm_w, nw}};
  for (const Buf& b : ins)
    if (overlap(o, nv, b.p, b.n) || overlap(state_out, ns, b.p, b.n)) return reject(KDA_ERR_ALIAS);
  if (overlap(o, nv, state_in, ns) || overlap(o, nv, state_out, ns)) return reject(KDA_ERR_ALIAS);
  if (state_out && state_in && state_out != state_in && overlap(state_out, ns, state_in, ns))
    return reject(KDA_ERR_ALIAS);
  const size_t need = T > 0 ? norm_workspace_bytes(B, H, T, V) : 0;
  if (need) {
    if (!workspace || workspace_bytes < need) return reject(KDA_ERR_WORKSPACE);
    if ((uintptr_t)workspace & 255) return reject(KDA_ERR_ALIGN);
    const Buf all[] = {{q, nk}, {k, nk}, {v, nv}, {z, nk}, {beta, nb}, {state_in, ns}, {o, nv}, {state_out, ns},
                       {A_log, na}, {dt_bias, ndb}, {norm_w, nw}};
    for (const Buf& b : all)
      if (overlap(workspace, need, b.p, b.n)) return reject(KDA_ERR_ALIAS);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (T == 0) {
    if (state_out && state_out != state_in) {
      const long long n = (long long)B * H * K * V;
      hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, state_in, state_out,
                         n);
      e = hipGetLastError();
    }
  } else {
    const unsigned long long spin = g_spin_ticks.load(std::memory_order_relaxed);
    switch (K < 32 ? 32 : K) {
      case 32:
        e = launch_chunk_fwd_norm_kd<32>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, norm_w, eps, o, state_out,
                                         B, H, T, K, V, workspace, spin, s);
        break;
      case 64:
        e = launch_chunk_fwd_norm_kd<64>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, norm_w, eps, o, state_out,
                                         B, H, T, K, V, workspace, spin, s);
        break;
      default:
        e = launch_chunk_fwd_norm_kd<128>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, norm_w, eps, o,
                                          state_out, B, H, T, K, V, workspace, spin, s);
    }
  }
  if (e != hipSuccess) return reject(KDA_ERR_HIP);
  g_counters[KDA_COUNTER_CHUNK_FWD].fetch_add(1, std::memory_order_relaxed);
  return KDA_OK;
}

// kda_recurrent_step (zc = 1) and kda_recurrent_step_scalar (zc = 0).
static int recurrent_step_impl(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                               const float* dt_bias, const void* beta, float* state, float scale, void* o, int B,
                               int H, int K, int V, int dtype, void* stream, int zc) {
  if (!q || !k || !v || !z || !A_log || !beta || !state || !o) return reject(KDA_ERR_NULL);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return reject(KDA_ERR_DTYPE);
  if (B < 1 || H < 1 || !valid_dim(K) || !valid_dim(V)) return reject(KDA_ERR_SHAPE);
  const size_t es = esize(dtype);
  const size_t nk = (size_t)B * H * K * es, nv = (size_t)B * H * V * es, ns = (size_t)B * H * K * V * 4;
  const size_t nz = zc ? nk : (size_t)B * H * es;
  const size_t nbe = (size_t)B * H * es, na = (size_t)H * 4, ndb = (size_t)H * (zc ? K : 1) * 4;
  if (overlap(o, nv, q, nk) || overlap(o, nv, k, nk) || overlap(o, nv, z, nz) || overlap(o, nv, v, nv) ||
      overlap(o, nv, beta, nbe) || overlap(o, nv, state, ns) || overlap(o, nv, A_log, na) ||
      overlap(o, nv, dt_bias, ndb) || overlap(state, ns, q, nk) || overlap(state, ns, k, nk) ||
      overlap(state, ns, z, nz) || overlap(state, ns, v, nv) || overlap(state, ns, beta, nbe) ||
      overlap(state, ns, A_log, na) || overlap(state, ns, dt_bias, ndb))
    return reject(KDA_ERR_ALIAS);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == KDA_BF16
                     ? launch_step<bf16_t>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, K, V, zc, s)
                     : launch_step<float>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, K, V, zc, s);
  if (e != hipSuccess) return reject(KDA_ERR_HIP);
  g_counters[KDA_COUNTER_RECURRENT_STEP].fetch_add(1, std::memory_order_relaxed);
  return KDA_OK;
}

extern "C" {

size_t kda_chunk_fwd_workspace_bytes(int B, int H, int T, int K, int V, int chunk, int dtype) {
  if (B < 1 || H < 1 || T < 1 || !valid_dim(K) || !valid_dim(V) || !valid_chunk(chunk)) return 0;
  if (!px_eligible(dtype == KDA_BF16, V, chunk)) return 0;
  return px_workspace_bytes(K < 32 ? 32 : K, B * H);
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                  const float* dt_bias, const void* beta, const float* state_in, float scale, int chunk, void* o,
                  float* state_out, void* workspace, size_t workspace_bytes, int B, int H, int T, int K, int V,
                  int dtype, void* stream) {
  return chunk_fwd_impl(q, k, v, z, A_log, dt_bias, beta, state_in, scale, chunk, o, state_out, workspace,
                        workspace_bytes, B, H, T, K, V, dtype, stream, 1);
}

int kda_chunk_fwd_scalar(const void* q, const void* k, const void* v, const void* a, const float* A_log,
                         const float* dt_bias, const void* beta, const float* state_in, float scale, int chunk,
                         void* o, float* state_out, void* workspace, size_t workspace_bytes, int B, int H, int T,
                         int K, int V, int dtype, void* stream) {
  return chunk_fwd_impl(q, k, v, a, A_log, dt_bias, beta, state_in, scale, chunk, o, state_out, workspace,
                        workspace_bytes, B, H, T, K, V, dtype, stream, 0);
}

size_t kda_chunk_fwd_norm_workspace_bytes(int B, int H, int T, int K, int V, int dtype) {
  if (B < 1 || H < 1 || T < 1 || !valid_dim(K) || !valid_dim(V) || dtype != KDA_BF16) return 0;
  return norm_workspace_bytes(B, H, T, V);
}

int kda_chunk_fwd_norm(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                       const float* dt_bias, const void* beta, const float* state_in, float scale, int chunk,
                       const float* norm_weight, float eps, void* o, float* state_out, void* workspace,
                       size_t workspace_bytes, int B, int H, int T, int K, int V, int dtype, void* stream) {
  return chunk_fwd_norm_impl(q, k, v, z, A_log, dt_bias, beta, state_in, scale, chunk, norm_weight, eps, o, state_out,
                             workspace, workspace_bytes, B, H, T, K, V, dtype, stream);
}

int kda_chunk_fwd_status(void* workspace, void* stream) {
  if (!workspace) return reject(KDA_ERR_NULL);
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KDA_ERR_HIP;
  unsigned w = 0;
  if (hipMemcpy(&w, workspace, 4, hipMemcpyDeviceToHost) != hipSuccess) return KDA_ERR_HIP;
  if (w == 0) return KDA_OK;
  const unsigned zero = 0;
  if (hipMemcpy(workspace, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return KDA_ERR_HIP;
  return KDA_ERR_EXCHANGE;
}

int kda_set_exchange_timeout_us(unsigned long long us) {
  g_spin_ticks.store(us > (~0ull) / 100 ? ~0ull : us * 100, std::memory_order_relaxed);
  return KDA_OK;
}

int kda_recurrent_step(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                       const float* dt_bias, const void* beta, float* state, float scale, void* o, int B, int H,
                       int K, int V, int dtype, void* stream) {
  return recurrent_step_impl(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, K, V, dtype, stream, 1);
}

int kda_recurrent_step_scalar(const void* q, const void* k, const void* v, const void* a, const float* A_log,
                              const float* dt_bias, const void* beta, float* state, float scale, void* o, int B,
                              int H, int K, int V, int dtype, void* stream) {
  return recurrent_step_impl(q, k, v, a, A_log, dt_bias, beta, state, scale, o, B, H, K, V, dtype, stream, 0);
}

size_t kda_chunk_bwd_workspace_bytes(int B, int H, int T, int K, int V, int chunk) {
  if (B < 1 || H < 1 || T < 0 || !valid_dim(K) || !valid_dim(V) || !valid_chunk(chunk)) return 0;
  return chunk_bwd_mfma_workspace_bytes(B, H, T, K, V);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                  const float* dt_bias, const void* beta, const float* state_in, float scale, int chunk,
                  const void* d_o, const float* d_state_out, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                  float* dstate_in, void* workspace, size_t workspace_bytes, int B, int H, int T, int K, int V,
                  int dtype, void* stream) {
  if (!A_log || !dstate_in ||
      (T != 0 && (!q || !k || !v || !z || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta)))
    return reject(KDA_ERR_NULL);
  if (dtype != KDA_F32) return reject(KDA_ERR_DTYPE);
  if (B < 1 || H < 1 || T < 0 || !valid_dim(K) || !valid_dim(V)) return reject(KDA_ERR_SHAPE);
  if (!valid_chunk(chunk)) return reject(KDA_ERR_CHUNK);
  if ((size_t)(T + 64) * (size_t)(K > V ? K : V) * 4 > 0x7fffffffu) return reject(KDA_ERR_SHAPE);
  if ((uintptr_t)z & 7) return reject(KDA_ERR_ALIGN);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)d_o) & 15)
    return reject(KDA_ERR_ALIGN);   // read in 16-byte pieces
  if ((long long)B * H > 65535) return reject(KDA_ERR_SHAPE);   // one grid row per head
  const size_t need = chunk_bwd_mfma_workspace_bytes(B, H, T, K, V);
  if (!workspace || workspace_bytes < need) return reject(KDA_ERR_WORKSPACE);
  if ((uintptr_t)workspace & 15) return reject(KDA_ERR_ALIGN);
  const size_t nk = (size_t)B * H * T * K * 4, nv = (size_t)B * H * T * V * 4, nb = (size_t)B * H * T * 4;
  const size_t ns = (size_t)B * H * K * V * 4;
  struct Buf { const void* p; size_t n; };
  const Buf ins[] = {{q, nk}, {k, nk}, {v, nv}, {z, nk}, {beta, nb}, {state_in, ns}, {d_o, nv}, {d_state_out, ns},
                     {workspace, need}};
  const Buf outs[] = {{dq, nk}, {dk, nk}, {dv, nv}, {dg, nk}, {dbeta, nb}, {dstate_in, ns}};
  for (const Buf& a : outs) {
    for (const Buf& b : ins)
      if (overlap(a.p, a.n, b.p, b.n)) return reject(KDA_ERR_ALIAS);
    for (const Buf& b : outs)
      if (&a != &b && overlap(a.p, a.n, b.p, b.n)) return reject(KDA_ERR_ALIAS);
  }
  hipError_t e = launch_chunk_bwd_mfma((const float*)q, (const float*)k, (const float*)v, (const float*)z, A_log,
                                       dt_bias, (const float*)beta, state_in, scale, (const float*)d_o, d_state_out,
                                       dq, dk, dv, dg, dbeta, dstate_in, workspace, B, H, T, K, V,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return reject(KDA_ERR_HIP);
  g_counters[KDA_COUNTER_CHUNK_BWD].fetch_add(1, std::memory_order_relaxed);
  return KDA_OK;
}

size_t kda_gate_bwd_workspace_bytes(int B, int H, int T, int K) { return gate_bwd_workspace_bytes(B, H, T, K); }

}  // extern "C"

// Checks of kda_gate_bwd and kda_gate_bwd_noalloc, then the launch.  `workspace` is
// the caller's buffer or the built-in scratch (need bytes of either are used).
static int gate_bwd_impl(const void* z, const float* A_log, const float* dt_bias, const float* dg, float* dz,
                         float* dA_log, float* d_dt_bias, bool noalloc, void* workspace, size_t workspace_bytes,
                         int B, int H, int T, int K, int dtype, void* stream) {
  if (!A_log || (!dz && !dA_log && !d_dt_bias) || (T != 0 && (!z || !dg))) return reject(KDA_ERR_NULL);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return reject(KDA_ERR_DTYPE);
  if (B < 1 || H < 1 || T < 0 || K < 1) return reject(KDA_ERR_SHAPE);
  const size_t need = gate_bwd_workspace_bytes(B, H, T, K);
  if (noalloc) {
    if (need > KDA_GATE_BWD_SCRATCH_BYTES) return reject(KDA_ERR_SCRATCH);
  } else if (need && (!workspace || workspace_bytes < need)) {
    return reject(KDA_ERR_WORKSPACE);
  }
  const size_t n = (size_t)B * H * T * K;
  struct Buf { const void* p; size_t n; };
  const Buf ins[] = {{z, n * esize(dtype)}, {A_log, (size_t)H * 4}, {dt_bias, (size_t)H * K * 4}, {workspace, need}};
  const Buf outs[] = {{dz, n * 4}, {dA_log, (size_t)H * 4}, {d_dt_bias, (size_t)H * K * 4}};
  for (const Buf& a : outs) {
    for (const Buf& b : ins)
      if (overlap(a.p, a.n, b.p, b.n)) return reject(KDA_ERR_ALIAS);
    for (const Buf& b : outs)
      if (&a != &b && overlap(a.p, a.n, b.p, b.n)) return reject(KDA_ERR_ALIAS);
  }
  // dz may be dg itself (each element is read before it is written, by the same thread),
  // but no other output may touch dg
  if ((dz != dg && overlap(dz, n * 4, dg, n * 4)) || overlap(dA_log, (size_t)H * 4, dg, n * 4) ||
      overlap(d_dt_bias, (size_t)H * K * 4, dg, n * 4))
    return reject(KDA_ERR_ALIAS);
  if (noalloc && need && gate_bwd_scratch(&workspace) != hipSuccess) return reject(KDA_ERR_HIP);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == KDA_BF16
                     ? launch_gate_bwd<bf16_t>(z, A_log, dt_bias, dg, dz, dA_log, d_dt_bias, workspace, B, H, T, K, s)
                     : launch_gate_bwd<float>(z, A_log, dt_bias, dg, dz, dA_log, d_dt_bias, workspace, B, H, T, K, s);
  if (e != hipSuccess) return reject(KDA_ERR_HIP);
  g_counters[KDA_COUNTER_GATE_BWD].fetch_add(1, std::memory_order_relaxed);
  return KDA_OK;
}

extern "C" {

int kda_gate_bwd(const void* z, const float* A_log, const float* dt_bias, const float* dg, float* dz, float* dA_log,
                 float* d_dt_bias, void* workspace, size_t workspace_bytes, int B, int H, int T, int K, int dtype,
                 void* stream) {
  return gate_bwd_impl(z, A_log, dt_bias, dg, dz, dA_log, d_dt_bias, false, workspace, workspace_bytes, B, H, T, K,
                       dtype, stream);
}

int kda_gate_bwd_noalloc(const void* z, const float* A_log, const float* dt_bias, const float* dg, float* dz,
                         float* dA_log, float* d_dt_bias, int B, int H, int T, int K, int dtype, void* stream) {
  return gate_bwd_impl(z, A_log, dt_bias, dg, dz, dA_log, d_dt_bias, true, nullptr, 0, B, H, T, K, dtype, stream);
}

}  // extern "C"
