// Standalone gate kernel and the single-token decode step.
//
// Gate: the released KDA decay form g = -exp(clamp(A_log)) * softplus(z + dt_bias),
// alpha = exp(g) (kdafix page, "Fix 1 -- decay form").  Elementwise, HBM-bound: one
// workgroup per (batch, head, tile of kGateTile tokens), so the head's multiplier and
// each thread's channel bias are read once; consecutive lanes touch consecutive
// addresses of a token row.
//
// Decode step: one token of the gated delta rule per (batch, head), the state read
// and written in place.  The state dominates the traffic (2*K*V*4 bytes per head),
// so one workgroup owns a tile of VTS value columns and all K rows of one head;
// lanes map to consecutive value columns, so every state row access is a
// contiguous VTS*4-byte segment.  The two reductions over K (the delta read
// S'^T k and the output S^T q_hat) are a per-thread partial sum over its rows
// followed by one LDS exchange between the NRG row groups.
#include <mutex>

#include "../../include/kda.h"
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

constexpr int kGateTile = 32;
constexpr int kGate4Threads = 512;            // workgroup size of gate_kernel4

// Thread tid covers channel cb + tid % KC of every (256 / KC)-th token row of the tile,
// for each pass cb of up to 256 channels.
template <typename Tin>
__global__ void __launch_bounds__(256) gate_kernel(const Tin* __restrict__ z, const float* __restrict__ A_log,
                                                   const float* __restrict__ dt_bias, float* __restrict__ g_out,
                                                   float* __restrict__ alpha_out, int H, int T, int K, int ntile) {
  const int wg = blockIdx.x;
  const int bh = wg / ntile, tile = wg - bh * ntile;
  const int h = bh % H;
  const int t0 = tile * kGateTile, t1 = min(T, t0 + kGateTile);
  const float mult = gate_multiplier(A_log[h]);
  const int tid = threadIdx.x;
  for (int cb = 0; cb < K; cb += 256) {
    const int KC = min(K - cb, 256);           // channels of this pass
    const int rpp = 256 / KC;                  // token rows per pass
    const int r = tid / KC, c = cb + tid % KC;
    if (r >= rpp) continue;
    const float db = dt_bias ? dt_bias[h * K + c] : 0.0f;
    for (int t = t0 + r; t < t1; t += rpp) {
      const size_t idx = ((size_t)bh * T + t) * K + c;
      const float g = -mult * softplus_f(to_f<Tin>(z[idx]) + db, true);
      g_out[idx] = g;
      if (alpha_out) alpha_out[idx] = fast_exp2(g * kLog2e);
    }
  }
}

// The same gate for K % 4 == 0 and aligned buffers (g, alpha, dt_bias 16 bytes, z four
// elements).  A tile's rows t0 .. t1-1 are one contiguous range of (t1 - t0) * K elements
// in z, g and alpha; thread tid takes the four-element groups tid, tid + kGate4Threads, ... of that
// range, so the 64 lanes of a wave read and write one gap-free span per instruction (16
// bytes per lane of g and of alpha, 8 or 16 of z).  The group's channel advances by
// kGate4Threads mod (K / 4) groups per pass, without a division.
template <typename Tin, bool FIXED>
__device__ __forceinline__ void gate_range4(const Tin* __restrict__ z, const float* __restrict__ db_h,
                                            float* __restrict__ g_out, float* __restrict__ alpha_out, size_t base,
                                            int ngroups, int K4, float mult) {
  const int step = FIXED ? 0 : kGate4Threads % K4;
  int cg = threadIdx.x % K4;
  float4 d4 = db_h ? *reinterpret_cast<const float4*>(db_h + 4 * cg) : float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
  for (int e = threadIdx.x; e < ngroups; e += kGate4Threads) {
    const size_t idx = base + 4 * (size_t)e;
    float x[4];
    if constexpr (sizeof(Tin) == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(z + idx);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xffff0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      const float4 v4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(z) + idx);
      x[0] = v4.x;
      x[1] = v4.y;
      x[2] = v4.z;
      x[3] = v4.w;
    }
    if (!FIXED && db_h) d4 = *reinterpret_cast<const float4*>(db_h + 4 * cg);
    const float gv[4] = {-mult * softplus_f(x[0] + d4.x, true), -mult * softplus_f(x[1] + d4.y, true),
                         -mult * softplus_f(x[2] + d4.z, true), -mult * softplus_f(x[3] + d4.w, true)};
    *reinterpret_cast<float4*>(g_out + idx) = float4{gv[0], gv[1], gv[2], gv[3]};
    if (alpha_out)
      *reinterpret_cast<float4*>(alpha_out + idx) =
          float4{fast_exp2(gv[0] * kLog2e), fast_exp2(gv[1] * kLog2e), fast_exp2(gv[2] * kLog2e),
                 fast_exp2(gv[3] * kLog2e)};
    if (!FIXED) {
      cg += step;
      if (cg >= K4) cg -= K4;
    }
  }
}

template <typename Tin>
__global__ void __launch_bounds__(kGate4Threads) gate_kernel4(const Tin* __restrict__ z, const float* __restrict__ A_log,
                                                    const float* __restrict__ dt_bias, float* __restrict__ g_out,
                                                    float* __restrict__ alpha_out, int H, int T, int K, int ntile) {
  const int wg = blockIdx.x;
  const int bh = wg / ntile, tile = wg - bh * ntile;
  const int h = bh % H;
  const int t0 = tile * kGateTile, t1 = min(T, t0 + kGateTile);
  const float mult = gate_multiplier(A_log[h]);
  const int K4 = K >> 2;
  const int ngroups = (t1 - t0) * K4;
  const size_t base = ((size_t)bh * T + t0) * K;
  const float* db_h = dt_bias ? dt_bias + (size_t)h * K : nullptr;
  if (kGate4Threads % K4 == 0)                 // each thread keeps one channel group
    gate_range4<Tin, true>(z, db_h, g_out, alpha_out, base, ngroups, K4, mult);
  else
    gate_range4<Tin, false>(z, db_h, g_out, alpha_out, base, ngroups, K4, mult);
}

// Reverse of the gate for a cotangent dg on g.  With x = z + dt_bias and
// m = exp(clamp(A_log)):  dz = -m sigmoid(x) dg  (the slope of softplus is the sigmoid);
// d dt_bias[h][c] = dz summed over batch and time; dA_log[h] = dg g summed over batch,
// time and channel where A_log lies in the closed clamp interval, else 0.
// Pass 1 (elementwise, HBM-bound): one workgroup per (batch, head, tile of
// kGateBwdTile tokens) writes dz and the tile's per-channel sums of dz and dg g to the
// workspace; consecutive lanes take consecutive channels of a token row.  Pass 2: one
// workgroup per head adds the tiles' sums in a fixed order, so the parameter gradients
// do not depend on scheduling.
constexpr int kGateBwdTile = 256;

template <typename Tin>
__global__ void __launch_bounds__(256) gate_bwd_tile_kernel(const Tin* __restrict__ z, const float* __restrict__ A_log,
                                                            const float* __restrict__ dt_bias, const float* dg,
                                                            float* dz, float* __restrict__ part, int H, int T, int K,
                                                            int ntile) {
  __shared__ float s_dz[256], s_gg[256];
  const int wg = blockIdx.x;
  const int bh = wg / ntile, tile = wg % ntile;
  const int h = bh % H;
  const int t0 = tile * kGateBwdTile, t1 = min(T, t0 + kGateBwdTile);
  const float m = gate_multiplier(A_log[h]);
  const int tid = threadIdx.x;
  float* pw = part + (size_t)wg * 2 * K;
  for (int cb = 0; cb < K; cb += 256) {
    const int KC = min(K - cb, 256);          // channels of this pass
    const int rpp = 256 / KC;                 // token rows per pass
    const int r = tid / KC, c = cb + tid % KC;
    float sdz = 0.0f, sgg = 0.0f;
    if (r < rpp) {
      const float db = dt_bias ? dt_bias[h * K + c] : 0.0f;
      for (int t = t0 + r; t < t1; t += rpp) {
        const size_t idx = ((size_t)bh * T + t) * K + c;
        const float x = to_f<Tin>(z[idx]) + db;
        const float dgv = dg[idx];
        const float g = -m * softplus_f(x, true);
        const float sig = fast_rcp(1.0f + fast_exp2(-x * kLog2e));   // 0 as x -> -inf, 1 as x -> inf
        const float d = -m * sig * dgv;
        if (dz) dz[idx] = d;                   // (dz may be dg itself: read above, same thread)
        sdz += d;
        sgg += dgv * g;
      }
    }
    s_dz[tid] = sdz;
    s_gg[tid] = sgg;
    __syncthreads();
    if (tid < KC) {
      float a = 0.0f, e = 0.0f;
      for (int j = 0; j < rpp; ++j) {
        a += s_dz[j * KC + tid];
        e += s_gg[j * KC + tid];
      }
      pw[c] = a;
      pw[K + c] = e;
    }
    __syncthreads();
  }
}

// The same first pass for K % 4 == 0, K / 4 dividing the workgroup size, and aligned
// buffers (dg, dz, dt_bias and the workspace 16 bytes, z four elements): the tile's rows
// are one contiguous range, thread tid takes its four-element groups tid, tid + NT, ...
// (gap-free 16-byte accesses per wave), and since NT is a multiple of K / 4 every group of
// a thread has the same four channels, whose sums it keeps in registers; the threads of a
// channel group then add theirs in a fixed order.
constexpr int kGateBwd4Threads = 1024;

template <typename Tin>
__global__ void __launch_bounds__(kGateBwd4Threads) gate_bwd_tile_kernel4(
    const Tin* __restrict__ z, const float* __restrict__ A_log, const float* __restrict__ dt_bias, const float* dg,
    float* dz, float* __restrict__ part, int H, int T, int K, int ntile) {
  constexpr int NT = kGateBwd4Threads;
  __shared__ float4 s_dz[NT], s_gg[NT];
  const int wg = blockIdx.x;
  const int bh = wg / ntile, tile = wg % ntile;
  const int h = bh % H;
  const int t0 = tile * kGateBwdTile, t1 = min(T, t0 + kGateBwdTile);
  const float m = gate_multiplier(A_log[h]);
  const int tid = threadIdx.x;
  const int K4 = K >> 2;
  const int cg = tid % K4;
  const float4 d4 = dt_bias ? *reinterpret_cast<const float4*>(dt_bias + (size_t)h * K + 4 * cg)
                            : float4{0.0f, 0.0f, 0.0f, 0.0f};
  const float db[4] = {d4.x, d4.y, d4.z, d4.w};
  const int ngroups = (t1 - t0) * K4;
  const size_t base = ((size_t)bh * T + t0) * K;
  float sdz[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sgg[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int e = tid; e < ngroups; e += NT) {
    const size_t idx = base + 4 * (size_t)e;
    float x[4];
    if constexpr (sizeof(Tin) == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(z + idx);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xffff0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      const float4 v4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(z) + idx);
      x[0] = v4.x;
      x[1] = v4.y;
      x[2] = v4.z;
      x[3] = v4.w;
    }
    const float4 g4 = *reinterpret_cast<const float4*>(dg + idx);
    const float dgv[4] = {g4.x, g4.y, g4.z, g4.w};
    float d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xv = x[j] + db[j];
      const float g = -m * softplus_f(xv, true);
      const float sig = fast_rcp(1.0f + fast_exp2(-xv * kLog2e));
      d[j] = -m * sig * dgv[j];
      sdz[j] += d[j];
      sgg[j] += dgv[j] * g;
    }
    if (dz) *reinterpret_cast<float4*>(dz + idx) = float4{d[0], d[1], d[2], d[3]};   // (dz may be dg: read above)
  }
  s_dz[tid] = float4{sdz[0], sdz[1], sdz[2], sdz[3]};
  s_gg[tid] = float4{sgg[0], sgg[1], sgg[2], sgg[3]};
  __syncthreads();
  if (tid < K4) {                              // channel group tid: threads tid, tid + K4, ...
    float4 a = s_dz[tid], b = s_gg[tid];
    for (int r = tid + K4; r < NT; r += K4) {
      const float4 u = s_dz[r], w = s_gg[r];
      a = float4{a.x + u.x, a.y + u.y, a.z + u.z, a.w + u.w};
      b = float4{b.x + w.x, b.y + w.y, b.z + w.z, b.w + w.w};
    }
    float* pw = part + (size_t)wg * 2 * K;
    *reinterpret_cast<float4*>(pw + 4 * tid) = a;
    *reinterpret_cast<float4*>(pw + K + 4 * tid) = b;
  }
}

// Pass 2, one workgroup of 1024 threads per head: thread (s, j) adds column j of the tile
// sums (2K columns: the dz sums, then the dg g sums) over the tiles s, s + 4, ... of each
// batch, 256 columns at a time; the four slices meet in LDS in a fixed order, and the
// dg g column totals are added by a fixed tree, so the result does not depend on
// scheduling.
constexpr int kGateRedCols = 256, kGateRedSlices = 4;

__global__ void __launch_bounds__(kGateRedCols* kGateRedSlices) gate_bwd_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ A_log, float* dA_log, float* d_dt_bias, int B, int H,
    int K, int ntile) {
  __shared__ float s_red[kGateRedSlices][kGateRedCols];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int col = tid % kGateRedCols, sl = tid / kGateRedCols;
  float gg = 0.0f;                             // slice 0: this column's dg g totals
  for (int c0 = 0; c0 < 2 * K; c0 += kGateRedCols) {
    const int j = c0 + col;
    float acc = 0.0f;
    if (j < 2 * K) {
      for (int b = 0; b < B; ++b) {
        const float* pc = part + (size_t)(b * H + h) * ntile * 2 * K + j;
#pragma unroll 8
        for (int tile = sl; tile < ntile; tile += kGateRedSlices) acc += pc[(size_t)tile * 2 * K];
      }
    }
    s_red[sl][col] = acc;
    __syncthreads();
    if (sl == 0 && j < 2 * K) {
      float t = s_red[0][col];
#pragma unroll
      for (int q = 1; q < kGateRedSlices; ++q) t += s_red[q][col];
      if (j < K) {
        if (d_dt_bias) d_dt_bias[h * K + j] = t;
      } else {
        gg += t;
      }
    }
    __syncthreads();
  }
  if (sl == 0) s_red[0][col] = gg;
  __syncthreads();
  for (int w = kGateRedCols / 2; w > 0; w >>= 1) {
    if (sl == 0 && col < w) s_red[0][col] += s_red[0][col + w];
    __syncthreads();
  }
  if (tid == 0 && dA_log) {
    const float a = A_log[h];
    dA_log[h] = (a >= kALogMin && a <= kALogMax) ? s_red[0][0] : 0.0f;
  }
}

template <typename Tin, int K, int VTS>
__global__ void __launch_bounds__(256) step_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const Tin* __restrict__ v, const Tin* __restrict__ z,
                                                   const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                                                   const Tin* __restrict__ beta, float* __restrict__ state,
                                                   float scale, Tin* __restrict__ o, int H, int V, int zc) {
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
    // zc = 0: the scalar-decay layout, one gate input per (b, h) and one bias per head
    const float x = to_f<Tin>(z[zc ? (size_t)bh * K + c : (size_t)bh]) + (dt_bias ? dt_bias[zc ? h * K + c : h] : 0.0f);
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
  const int ntile = (T + kGateTile - 1) / kGateTile;
  const long long blocks = (long long)B * H * ntile;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const uintptr_t al = (uintptr_t)g | (uintptr_t)alpha | (uintptr_t)dt_bias;
  if (K % 4 == 0 && (al & 15) == 0 && ((uintptr_t)z & (4 * sizeof(Tin) - 1)) == 0)
    hipLaunchKernelGGL(gate_kernel4<Tin>, dim3((unsigned)blocks), dim3(kGate4Threads), 0, s, (const Tin*)z, A_log, dt_bias, g,
                       alpha, H, T, K, ntile);
  else
    hipLaunchKernelGGL(gate_kernel<Tin>, dim3((unsigned)blocks), dim3(256), 0, s, (const Tin*)z, A_log, dt_bias, g,
                       alpha, H, T, K, ntile);
  return hipGetLastError();
}

// The gate adjoint's partial sums for callers that cannot allocate: a file-scope
// device array (each GPU the library runs on holds its own copy until the process
// ends).  Its name is only a host-side handle; kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[KDA_GATE_BWD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

hipError_t gate_bwd_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t gate_bwd_workspace_bytes(int B, int H, int T, int K) {
  if (B < 1 || H < 1 || T < 0 || K < 1) return 0;
  const size_t ntile = (size_t)(T + kGateBwdTile - 1) / kGateBwdTile;
  return (size_t)B * H * ntile * 2 * K * sizeof(float);
}

template <typename Tin>
hipError_t launch_gate_bwd(const void* z, const float* A_log, const float* dt_bias, const float* dg, float* dz,
                           float* dA_log, float* d_dt_bias, void* workspace, int B, int H, int T, int K,
                           hipStream_t s) {
  const int ntile = (T + kGateBwdTile - 1) / kGateBwdTile;
  float* part = reinterpret_cast<float*>(workspace);
  if (ntile > 0) {
    const uintptr_t al = (uintptr_t)dg | (uintptr_t)dz | (uintptr_t)dt_bias | (uintptr_t)workspace;
    if (K % 4 == 0 && kGateBwd4Threads % (K / 4) == 0 && (al & 15) == 0 &&
        ((uintptr_t)z & (4 * sizeof(Tin) - 1)) == 0)
      hipLaunchKernelGGL(gate_bwd_tile_kernel4<Tin>, dim3((unsigned)(B * H * ntile)), dim3(kGateBwd4Threads), 0, s,
                         (const Tin*)z, A_log, dt_bias, dg, dz, part, H, T, K, ntile);
    else
      hipLaunchKernelGGL(gate_bwd_tile_kernel<Tin>, dim3((unsigned)(B * H * ntile)), dim3(256), 0, s, (const Tin*)z,
                         A_log, dt_bias, dg, dz, part, H, T, K, ntile);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dA_log || d_dt_bias)                    // (T = 0: both come out zero)
    hipLaunchKernelGGL(gate_bwd_reduce_kernel, dim3((unsigned)H), dim3(kGateRedCols * kGateRedSlices), 0, s, part,
                       A_log, dA_log, d_dt_bias, B, H, K, ntile);
  return hipGetLastError();
}

template hipError_t launch_gate_bwd<float>(const void*, const float*, const float*, const float*, float*, float*,
                                           float*, void*, int, int, int, int, hipStream_t);
template hipError_t launch_gate_bwd<bf16_t>(const void*, const float*, const float*, const float*, float*, float*,
                                            float*, void*, int, int, int, int, hipStream_t);

template <typename Tin, int K, int VTS>
static hipError_t launch_step_kv(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                 const float* dt_bias, const void* beta, float* state, float scale, void* o, int B,
                                 int H, int V, int zc, hipStream_t s) {
  constexpr int NRG = cmin(256 / VTS, K);
  const int grid = B * H * (V / VTS);
  hipLaunchKernelGGL((step_kernel<Tin, K, VTS>), dim3(grid), dim3(NRG * VTS), 0, s, (const Tin*)q, (const Tin*)k,
                     (const Tin*)v, (const Tin*)z, A_log, dt_bias, (const Tin*)beta, state, scale, (Tin*)o, H, V, zc);
  return hipGetLastError();
}

template <typename Tin, int K>
static hipError_t launch_step_k(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                const float* dt_bias, const void* beta, float* state, float scale, void* o, int B,
                                int H, int V, int zc, hipStream_t s) {
  switch (V) {
    case 8: return launch_step_kv<Tin, K, 8>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    case 16: return launch_step_kv<Tin, K, 16>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    case 32: return launch_step_kv<Tin, K, 32>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    default: return launch_step_kv<Tin, K, 64>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
  }
}

template <typename Tin>
hipError_t launch_step(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                       const float* dt_bias, const void* beta, float* state, float scale, void* o, int B, int H,
                       int K, int V, int zc, hipStream_t s) {
  switch (K) {
    case 8: return launch_step_k<Tin, 8>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    case 16: return launch_step_k<Tin, 16>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    case 32: return launch_step_k<Tin, 32>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    case 64: return launch_step_k<Tin, 64>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
    default: return launch_step_k<Tin, 128>(q, k, v, z, A_log, dt_bias, beta, state, scale, o, B, H, V, zc, s);
  }
}

template hipError_t launch_gate<float>(const void*, const float*, const float*, float*, float*, int, int, int, int,
                                       hipStream_t);
template hipError_t launch_gate<bf16_t>(const void*, const float*, const float*, float*, float*, int, int, int, int,
                                        hipStream_t);
template hipError_t launch_step<float>(const void*, const void*, const void*, const void*, const float*, const float*,
                                       const void*, float*, float, void*, int, int, int, int, int, hipStream_t);
template hipError_t launch_step<bf16_t>(const void*, const void*, const void*, const void*, const float*,
                                        const float*, const void*, float*, float, void*, int, int, int, int, int,
                                        hipStream_t);

}  // namespace kda
