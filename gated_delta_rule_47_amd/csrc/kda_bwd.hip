// Adjoint of the KDA forward (fp32): gradients of L = sum(o * d_o) + sum(S_T * d_S_T)
// with respect to q, k, v, the log-decay g, beta and the initial state.
//
// Structure (the adjoint page's split into an intra-chunk part and a reverse
// recurrence over chunks that carries dS):
//   1. the fused chunked forward runs once and stores the state at every chunk
//      start (the checkpoints);
//   2. one workgroup per (batch, head, value tile) walks the chunks in reverse.
//      For each chunk it recomputes the token states inside the chunk from the
//      checkpoint (kept in a per-workgroup scratch: every thread reads back only
//      the state elements it wrote), then runs the token-level reverse recurrence
//         dS += q_hat do^T,  e = v - S'^T k,  de = beta dS^T k,
//         dq = scale S_t do,  dk = beta dS e - S' de,  dv = de,  dbeta = k.dS e,
//         dS' = dS - k de^T,  dg = alpha * rowsum(dS' * S_{t-1}),  dS = alpha dS'
//      with S' = diag(alpha) S_{t-1} and S_t do = S' do + beta k (e.do);
//   3. the row sums over value columns (dq, dk, dg and dS e) are partial per value
//      tile; a last kernel adds the tiles in a fixed order and forms
//      dbeta = k . (dS e).  Nothing uses atomics, so results are deterministic.
//
// Thread layout of step 2: thread (a, b) holds rows 4a..4a+3 and value columns
// 4b..4b+3 of the K x VT tile.  Each wave holds every row of CBW column blocks (lane =
// RB * bw + a, b = CBW * wave + bw), so the sums over rows that each token needs are lane
// exchanges inside one wave (DPP moves and permlane swaps) and no token waits for another
// wave.  The per-row sums over columns (the dq, dk, dg and dS e partials) are summed over
// the wave's columns the same way, kept in a double-buffered LDS ring for RING tokens and
// added over the waves at one barrier per RING tokens.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

constexpr int kBwdVTMax = 32;

// Sum of x over the lanes l ^ m, m = lo, 2 lo, ..., hi / 2 (so every lane of each group
// holds the group's total), without the LDS crossbar: the exchanges are DPP lane moves
// within a row (xor 1 and 2 by quad permutes, xor 8 by rotating the 16-lane row by 8,
// xor 4 by mirroring the 8-lane halves once the quads already hold equal sums) and the
// permlane swaps across rows (xor 16 and 32).  The pairs are exactly those of a
// butterfly, so the sum is the same as with lane shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor_sum(float x, int lo, int hi) {
  for (int m = lo; m < hi; m <<= 1) {
    if (m == 1) {
      x += dpp_partner<0xB1>(x);               // quad_perm [1,0,3,2]
    } else if (m == 2) {
      x += dpp_partner<0x4E>(x);               // quad_perm [2,3,0,1]
    } else if (m == 4 && lo == 1) {
      x += dpp_partner<0x141>(x);              // row_half_mirror: the quads hold equal sums
    } else if (m == 8) {
      x += dpp_partner<0x128>(x);              // row_ror:8 = lane ^ 8 within a row
    } else if (m == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if (m == 32) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
      x += __shfl_xor(x, m);
    }
  }
  return x;
}

template <int K, int VT, int CKMAX>
__global__ void __launch_bounds__(256)
bwd_reverse_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                   const float* __restrict__ z, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                   const float* __restrict__ beta, float scale, const float* __restrict__ d_o,
                   const float* __restrict__ d_state_out, const float* __restrict__ ckpt, float* __restrict__ scratch,
                   float* __restrict__ part, float* __restrict__ dv, float* __restrict__ dstate_in, int H, int T,
                   int V, int CK, int nck, int nvt) {
  constexpr int CB = VT / 4, RB = K / 4;
  constexpr int CBW = CB < 64 / RB ? CB : 64 / RB;   // column blocks per wave
  constexpr int NW = CB / CBW;                         // waves that hold the tile
  constexpr int RING = 4;                              // tokens per partial-sum flush
  static_assert(NW <= 4 && RB * CBW <= 64, "tile too large for one workgroup");
  __shared__ float sAl[CKMAX * K], sK[CKMAX * K], sQ[CKMAX * K];
  __shared__ float sV[CKMAX * VT], sDO[CKMAX * VT], sB[CKMAX];
  __shared__ float sPart[2][RING][NW][4 * K];          // per-wave row partials of RING tokens

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bw = lane / RB;
  const bool act = wave < NW && bw < CBW;
  const int a = act ? lane % RB : 0;      // idle threads alias row block 0 and never store
  const int b = act ? wave * CBW + bw : 0;
  const int bh = blockIdx.x / nvt, vt = blockIdx.x % nvt, h = bh % H, v0 = vt * VT;
  const int BH = gridDim.x / nvt;
  const float mult2 = gate_multiplier(A_log[h]) * kLog2e;
  float* scr = scratch + (size_t)blockIdx.x * CKMAX * K * VT;

  float dS[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dS[i][j] = (act && d_state_out) ? d_state_out[((size_t)bh * K + 4 * a + i) * V + v0 + 4 * b + j] : 0.0f;

  // sums over the tile's rows (all in this wave) and over the wave's columns
  auto row_sum = [&](float x) { return xor_sum(act ? x : 0.0f, 1, RB); };
  auto col_sum = [&](float x) { return xor_sum(act ? x : 0.0f, RB, RB * CBW); };

  // the ring: tokens of the current round go to half `ring` at slot 0, 1, ...; a flush adds
  // the waves' partials of `cnt` tokens (slot d is token t_first - d) into the tile's rows
  int ring = 0;
  auto flush = [&](int cnt, size_t tok_first) {
    lds_barrier();
    for (int idx = tid; idx < cnt * 4 * K; idx += 256) {
      const int d = idx / (4 * K), r = idx % (4 * K);
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += sPart[ring][d][w][r];
      part[(((size_t)vt * BH + bh) * T + tok_first - d) * 4 * K + r] = acc;
    }
    ring ^= 1;
  };

  for (int ci = nck - 1; ci >= 0; --ci) {
    const int tc0 = ci * CK;
    const int n = min(CK, T - tc0);
    lds_barrier();
    for (int idx = tid; idx < n * K; idx += 256) {
      const int t = idx / K, c = idx % K;
      const size_t g = ((size_t)bh * T + tc0 + t) * K + c;
      const float x = z[g] + (dt_bias ? dt_bias[h * K + c] : 0.0f);
      sAl[idx] = fast_exp2(-mult2 * softplus_f(x, true));
      sK[idx] = k[g];
      sQ[idx] = scale * q[g];
    }
    for (int idx = tid; idx < n * VT; idx += 256) {
      const int t = idx / VT, j = idx % VT;
      const size_t g = ((size_t)bh * T + tc0 + t) * V + v0 + j;
      sV[idx] = v[g];
      sDO[idx] = d_o[g];
    }
    for (int t = tid; t < n; t += 256) sB[t] = beta[(size_t)bh * T + tc0 + t];
    const float* ck = ckpt + ((size_t)bh * nck + ci) * K * V;
    float S[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = act ? ck[(size_t)(4 * a + i) * V + v0 + 4 * b + j] : 0.0f;
    lds_barrier();

    // forward recompute: the states after tokens 0..n-2 of this chunk
    for (int t = 0; t < n - 1; ++t) {
      float rp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float al = sAl[t * K + 4 * a + i], kk = sK[t * K + 4 * a + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) { S[i][j] *= al; rp[j] += S[i][j] * kk; }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) rp[j] = row_sum(rp[j]);
      const float bt = sB[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float kk = bt * sK[t * K + 4 * a + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) S[i][j] += kk * (sV[t * VT + 4 * b + j] - rp[j]);
        if (act)
          *reinterpret_cast<floatx4*>(scr + ((size_t)t * K + 4 * a + i) * VT + 4 * b) =
              floatx4{S[i][0], S[i][1], S[i][2], S[i][3]};
      }
    }

    // reverse over the chunk's tokens.  S_{t-1} comes from the checkpoint (t = 0) or from the
    // recomputed states in scratch; the state a token needs is loaded one token ahead, so
    // that the load's latency is not on the token chain.
    auto load_prev = [&](int t, floatx4 (&dst)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!act) {
          dst[i] = zero4();
        } else if (t == 0) {
          dst[i] = *reinterpret_cast<const floatx4*>(ck + (size_t)(4 * a + i) * V + v0 + 4 * b);
        } else {
          dst[i] = *reinterpret_cast<const floatx4*>(scr + ((size_t)(t - 1) * K + 4 * a + i) * VT + 4 * b);
        }
      }
    };
    floatx4 Snext[4];
    load_prev(n - 1, Snext);
    int slot = 0;
    for (int t = n - 1; t >= 0; --t) {
      const size_t tok = (size_t)bh * T + tc0 + t;
      float Sprev[4][4];                           // S_{t-1}, undecayed
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sprev[i][j] = Snext[i][j];
      if (t > 0) load_prev(t - 1, Snext);
      float al[4], kk[4], qh[4], vv[4], dov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        al[i] = sAl[t * K + 4 * a + i];
        kk[i] = sK[t * K + 4 * a + i];
        qh[i] = sQ[t * K + 4 * a + i];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vv[j] = sV[t * VT + 4 * b + j];
        dov[j] = sDO[t * VT + 4 * b + j];
      }
      const float bt = sB[t];
      float ep[4] = {0.f, 0.f, 0.f, 0.f}, dep[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dS[i][j] += qh[i] * dov[j];              // dS += q_hat do^T
          ep[j] += al[i] * Sprev[i][j] * kk[i];    // S'^T k, S' = diag(alpha) S_{t-1}
          dep[j] += dS[i][j] * kk[i];              // dS^T k
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ep[j] = row_sum(ep[j]);
        dep[j] = row_sum(dep[j]);
      }
      float e[4], de[4], edo = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = vv[j] - ep[j];
        de[j] = bt * dep[j];
        edo += e[j] * dov[j];
      }
      float sdo[4], dse[4], sde[4], dgp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sdo[i] = 0.f; dse[i] = 0.f; sde[i] = 0.f; dgp[i] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sd = al[i] * Sprev[i][j];
          sdo[i] += sd * dov[j];
          dse[i] += dS[i][j] * e[j];
          sde[i] += sd * de[j];
          const float dsd = dS[i][j] - kk[i] * de[j];    // dS' = dS - k de^T
          dgp[i] += dsd * Sprev[i][j];
          dS[i][j] = dsd;
        }
      }
      // sums over this wave's value columns; the waves' sums are added at the flush
      edo = col_sum(edo);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sdo[i] = col_sum(sdo[i]);
        dse[i] = col_sum(dse[i]);
        sde[i] = col_sum(sde[i]);
        dgp[i] = col_sum(dgp[i]);
      }
      if (act && bw == 0) {
        float* pp = sPart[ring][slot][wave];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * a + i;
          pp[c] = scale * (sdo[i] + bt * kk[i] * edo);     // dq partial
          pp[K + c] = bt * dse[i] - sde[i];                 // dk partial
          pp[2 * K + c] = al[i] * dgp[i];                   // dg partial
          pp[3 * K + c] = dse[i];                           // (dS e) partial, for dbeta
        }
      }
      if (act && a == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dv[tok * V + v0 + 4 * b + j] = de[j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dS[i][j] *= al[i];    // dS_{t-1} = diag(alpha) dS'
      if (++slot == RING || t == 0) {
        flush(slot, (size_t)tc0 + t + slot - 1);
        slot = 0;
      }
    }
  }
  if (act) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dstate_in[((size_t)bh * K + 4 * a + i) * V + v0 + 4 * b + j] = dS[i][j];
  }
}

// One wave per token row: add the value-tile partials in tile order.
__global__ void __launch_bounds__(256)
bwd_reduce_kernel(const float* __restrict__ part, const float* __restrict__ k, float* __restrict__ dq,
                  float* __restrict__ dk, float* __restrict__ dg, float* __restrict__ dbeta, long long BHT, int K,
                  int nvt) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= BHT) return;
  float acc = 0.0f;
  for (int c = lane; c < K; c += 64) {
    float sq = 0.f, sk = 0.f, sg = 0.f, se = 0.f;
    for (int t = 0; t < nvt; ++t) {
      const float* pp = part + ((size_t)t * BHT + row) * 4 * K;
      sq += pp[c];
      sk += pp[K + c];
      sg += pp[2 * K + c];
      se += pp[3 * K + c];
    }
    dq[row * K + c] = sq;
    dk[row * K + c] = sk;
    dg[row * K + c] = sg;
    acc += k[row * K + c] * se;
  }
  acc = xor_sum(acc, 1, 64);
  if (lane == 0) dbeta[row] = acc;
}

// ------------------------------------------------------------------ host side
struct BwdPlan {
  FwdPlan fwd;
  int VT, nvt, CK, nck;
  size_t off_scratch, off_part, bytes;
};

static bool bwd_plan(int B, int H, int T, int K, int V, int chunk, BwdPlan* p) {
  if (!fwd_plan(false, K, V, chunk, &p->fwd)) return false;
  p->VT = V < kBwdVTMax ? V : kBwdVTMax;
  p->nvt = V / p->VT;
  p->CK = p->fwd.C;
  p->nck = (T + p->CK - 1) / p->CK;
  const size_t BH = (size_t)B * H;
  const size_t ckpt = BH * p->nck * K * V * sizeof(float);
  const int ckmax = K == 128 ? 32 : 64;
  const size_t scratch = BH * p->nvt * (size_t)ckmax * K * p->VT * sizeof(float);
  const size_t part = (size_t)p->nvt * BH * T * 4 * K * sizeof(float);
  p->off_scratch = (ckpt + 255) / 256 * 256;
  p->off_part = (p->off_scratch + scratch + 255) / 256 * 256;
  p->bytes = p->off_part + part;
  return true;
}

size_t bwd_workspace_bytes(int B, int H, int T, int K, int V, int chunk) {
  BwdPlan p;
  return bwd_plan(B, H, T, K, V, chunk, &p) ? p.bytes : 0;
}

template <int K, int VT>
static hipError_t launch_rev(const BwdPlan& p, const float* q, const float* k, const float* v, const float* z,
                             const float* A_log, const float* dt_bias, const float* beta, float scale, const float* d_o,
                             const float* d_state_out, char* ws, float* dv, float* dstate_in, int B, int H, int T,
                             int V, hipStream_t s) {
  constexpr int CKMAX = K == 128 ? 32 : 64;
  hipLaunchKernelGGL((bwd_reverse_kernel<K, VT, CKMAX>), dim3(B * H * p.nvt), dim3(256), 0, s, q, k, v, z, A_log,
                     dt_bias, beta, scale, d_o, d_state_out, (const float*)ws, (float*)(ws + p.off_scratch),
                     (float*)(ws + p.off_part), dv, dstate_in, H, T, V, p.CK, p.nck, p.nvt);
  return hipGetLastError();
}

template <int K>
static hipError_t launch_rev_k(const BwdPlan& p, const float* q, const float* k, const float* v, const float* z,
                               const float* A_log, const float* dt_bias, const float* beta, float scale,
                               const float* d_o, const float* d_state_out, char* ws, float* dv, float* dstate_in,
                               int B, int H, int T, int V, hipStream_t s) {
  switch (p.VT) {
    case 8: return launch_rev<K, 8>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s);
    case 16: return launch_rev<K, 16>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s);
    default: return launch_rev<K, 32>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s);
  }
}

hipError_t launch_chunk_bwd(const float* q, const float* k, const float* v, const float* z, const float* A_log,
                            const float* dt_bias, const float* beta, const float* state_in, float scale, int chunk,
                            const float* d_o, const float* d_state_out, float* dq, float* dk, float* dv, float* dg,
                            float* dbeta, float* dstate_in, void* workspace, int B, int H, int T, int K, int V,
                            hipStream_t s) {
  BwdPlan p;
  if (!bwd_plan(B, H, T, K, V, chunk, &p)) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(workspace);
  hipError_t err = hipSuccess;
  if (T > 0) {
    switch (p.fwd.KD) {
      case 16: err = launch_chunk_fwd_kd<float, 16>(p.fwd.VT, p.fwd.C, q, k, v, z, A_log, dt_bias, beta, state_in, scale, nullptr, nullptr, (float*)ws, B, H, T, K, V, 1, s); break;
      case 32: err = launch_chunk_fwd_kd<float, 32>(p.fwd.VT, p.fwd.C, q, k, v, z, A_log, dt_bias, beta, state_in, scale, nullptr, nullptr, (float*)ws, B, H, T, K, V, 1, s); break;
      case 64: err = launch_chunk_fwd_kd<float, 64>(p.fwd.VT, p.fwd.C, q, k, v, z, A_log, dt_bias, beta, state_in, scale, nullptr, nullptr, (float*)ws, B, H, T, K, V, 1, s); break;
      default: err = launch_chunk_fwd_kd<float, 128>(p.fwd.VT, p.fwd.C, q, k, v, z, A_log, dt_bias, beta, state_in, scale, nullptr, nullptr, (float*)ws, B, H, T, K, V, 1, s); break;
    }
    if (err != hipSuccess) return err;
  }
  switch (K) {
    case 8: err = launch_rev_k<8>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s); break;
    case 16: err = launch_rev_k<16>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s); break;
    case 32: err = launch_rev_k<32>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s); break;
    case 64: err = launch_rev_k<64>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s); break;
    default: err = launch_rev_k<128>(p, q, k, v, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, B, H, T, V, s); break;
  }
  if (err != hipSuccess) return err;
  const long long BHT = (long long)B * H * T;
  if (BHT > 0) {
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((BHT + 3) / 4)), dim3(256), 0, s,
                       (const float*)(ws + p.off_part), k, dq, dk, dg, dbeta, BHT, K, p.nvt);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace kda
