// Chunked adjoint of the KDA forward (fp32): gradients of
//   L = sum(o * d_o) + sum(S_T * d_S_T)
// with respect to q, k, v, the log-decay g, beta and the initial state ("The fused KDA
// adjoint" page, section 1: a token-parallel pass inside each chunk and a sequential
// reverse recurrence over the chunks that carries dS; section 3 for the gradient blocks).
//
// Chunks of C = 32 tokens.  Inside a chunk (tokens t, channels c), with G_t the gate's
// cumulative sum from the chunk start, the reference m = G_15 (the middle of the chunk)
// and E = G - m:
//   L = exp(E), R = exp(-E),  KE = k L,  QE = (scale q) L,  KR = k R,
//   A_tj = KE_t . KR_j (j < t),  P_tj = QE_t . KR_j (j <= t),  T = (I + diag(beta) A)^-1,
//   G0 = exp(m) (chunk start -> reference),  D0 = exp(G_31 - m) (reference -> chunk end).
// The chunk maps its start state S to
//   S~ = diag(G0) S,  Y = V - KE S~,  Z = diag(beta) Y,  U = T Z,
//   O = QE S~ + P U,  S_next = diag(D0) (S~ + KR^T U),
// which is the token recurrence S' = diag(alpha_t) S, S = S' + beta_t k_t (v_t - S'^T k_t)^T,
// o_t = S_t^T (scale q_t), rearranged exactly.  Its reverse, for the cotangent dS_next of
// the chunk-end state and dO:
//   dX = diag(D0) dS_next,  dU = P^T dO + KR dX,  dZ = T^T dU,  dY = diag(beta) dZ,
//   dv = dY,  dS = diag(G0) (dX + QE^T dO - KE^T dY)                          (reverse pass)
//   dP = tril(dO U^T),  dM = -strict_tril(dZ U^T),  dA = diag(beta) dM,
//   dQE = dO S~^T + dP KR,  dKE = -dY S~^T + dA KR,  dKR = U dX^T + dP^T QE + dA^T KE,
//   dbeta_t = Z-term sum_v dZ Y + sum_j dM_tj A_tj,
//   dk = dKE L + dKR R,  dq = scale dQE L,
//   dG = dKE KE + dQE QE - dKR KR,  plus, at the chunk's last token,
//        rowsum(dS_next * S_next) = rowsum(dX * S~) + colsum(KR * (U dX^T)),
//   dg = the reverse cumulative sum of dG over the chunk's tokens          (gradient pass)
// (m is held fixed: the rearrangement does not depend on it, so its own gradient is 0).
//
// Four passes:
//   prep     one workgroup per (head, chunk): the gate, E, KE, QE, KR, A and P on MFMA
//            (v_mfma_f32_16x16x4_f32), T by substitution, G0, D0, beta, into the workspace;
//   forward  one workgroup per (head, 16 value columns), chunks in order: the state at
//            every chunk start (the checkpoints), and Y, U of every chunk;
//   reverse  one workgroup per (head, 16 value columns), chunks in reverse: the chunk-end
//            cotangents, dZ, dv and the initial state's gradient;
//   gradient one workgroup per (head, chunk): every other gradient, from the chunk's
//            checkpoint and chunk-end cotangent, all value columns at once (the sums over
//            value columns stay in the workgroup: no partial buffers, no atomics); a
//            second launch takes the token-path chunks.
// A chunk whose decay inside it exceeds exp(+-60) around the reference (the factors
// would leave fp32) is flagged by prep and evaluated token by token, exactly; the
// cotangent's path through a token does not involve the state, so only the gradient pass
// recomputes states (from the checkpoint, token by token, in grad_token_kernel).
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace cb {

constexpr int C = 32;              // tokens per chunk
constexpr float THRESH = 60.0f;    // |G_t - m| (natural log units) on the MFMA path

__device__ __forceinline__ floatx4 mma(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Per-chunk record of the prep kernel (floats).
template <int KD>
struct Rec {
  static constexpr int KE = 0;
  static constexpr int QE = KE + C * KD;
  static constexpr int KR = QE + C * KD;
  static constexpr int E = KR + C * KD;
  static constexpr int A = E + C * KD;       // [C][C] strictly lower
  static constexpr int P = A + C * C;        // [C][C] lower
  static constexpr int T = P + C * C;        // [C][C] lower, unit diagonal
  static constexpr int BETA = T + C * C;     // [C]
  static constexpr int G0 = BETA + C;        // [KD]
  static constexpr int D0 = G0 + KD;         // [KD]
  static constexpr int FLAG = D0 + KD;       // 1: token path
  static constexpr int SIZE = round_up(FLAG + 1, 64);
};

// Workspace layout (bytes), shared by the host and the kernels.  The per-chunk tensors
// with value columns (the checkpoint and the chunk-end cotangent, K x VP; U, Y and dZ,
// C x VP) are stored by value tile: [chunk][VP / 16][rows][16], so that the sequential
// passes, one workgroup per 16-column tile, write each of them as one contiguous block.
struct Layout {
  size_t rec, ck, dse, u, y, dz, bytes;
};
__host__ __device__ inline Layout layout(int KD, int VP, long long BH, int nck) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rec_f = (size_t)round_up(4 * C * KD + 3 * C * C + C + 2 * KD + 1, 64);
  const size_t nchunks = (size_t)BH * nck;
  Layout l;
  l.rec = 0;
  l.ck = al(l.rec + nchunks * rec_f * 4);
  l.dse = al(l.ck + nchunks * KD * VP * 4);
  l.u = al(l.dse + nchunks * KD * VP * 4);
  l.y = al(l.u + nchunks * C * VP * 4);
  l.dz = al(l.y + nchunks * C * VP * 4);
  l.bytes = al(l.dz + nchunks * C * VP * 4);
  return l;
}

// Offset of (row, column col) in a per-chunk [VP / 16][rows][16] tensor of `rows` rows.
__host__ __device__ __forceinline__ size_t vt_off(int rows, int row, int col) {
  return ((size_t)(col >> 4) * rows + row) * 16 + (col & 15);
}

__device__ __forceinline__ float gate_g(float z, float db, float gm) { return -gm * softplus_f(z + db, true); }
__device__ __forceinline__ float expn(float x) { return fast_exp2(x * kLog2e); }

// ============================================================================ prep
template <int KD>
__global__ void __launch_bounds__(256)
prep_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ z,
            const float* __restrict__ A_log, const float* __restrict__ dt_bias, const float* __restrict__ beta,
            float scale, float* __restrict__ recs, int H, int T, int K, int nck) {
  using Rc = Rec<KD>;
  constexpr int LK = KD + 4, LC = C + 4;
  __shared__ float sG[C][KD + 1];
  __shared__ __attribute__((aligned(16))) float sKE[C * LK];
  __shared__ __attribute__((aligned(16))) float sQE[C * LK];
  __shared__ __attribute__((aligned(16))) float sKR[C * LK];
  __shared__ float sA[C * LC];
  __shared__ float sT[C * LC];
  __shared__ float sX[16 * 16];
  __shared__ float sBeta[C];
  __shared__ int sSlow;
  const int c = blockIdx.x, bh = blockIdx.y, h = bh % H;
  const int t0 = c * C, nval = min(C, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* rec = recs + ((size_t)bh * nck + c) * Rc::SIZE;
  const float gm = gate_multiplier(A_log[h]);
  const size_t row0 = (size_t)bh * T + t0;
  // k and q of the element pass, loaded first so that they arrive during the gate's sum:
  // four channels per thread and float4 i4 = tid + 256 m (K is a multiple of 4)
  constexpr int NI = (C * KD / 4 + 255) / 256;
  float4 kv[NI], qv[NI];
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int i4 = tid + 256 * m, t = (4 * i4) / KD, ch = (4 * i4) % KD;
    kv[m] = qv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i4 < C * KD / 4 && t < nval && ch < K) {
      kv[m] = *reinterpret_cast<const float4*>(k + (row0 + t) * K + ch);
      qv[m] = *reinterpret_cast<const float4*>(q + (row0 + t) * K + ch);
    }
  }
  if (tid == 0) sSlow = 0;
  if (tid < C) sBeta[tid] = tid < nval ? beta[row0 + tid] : 0.0f;
  __syncthreads();
  // the cumulative gate of each channel over the chunk (zero past the chunk's tokens)
  if (tid < KD) {
    const int ch = tid;
    const float db = (dt_bias && ch < K) ? dt_bias[h * K + ch] : 0.0f;
    // the 32 inputs first (independent loads), then the dependent sum
    float zv[C];
#pragma unroll
    for (int t = 0; t < C; ++t) zv[t] = (t < nval && ch < K) ? z[(row0 + t) * K + ch] : 0.0f;
    float G = 0.0f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
      if (t < nval && ch < K) G += gate_g(zv[t], db, gm);
      sG[t][ch] = G;
    }
    const float m = sG[15][ch];
    float mx = 0.0f;
    for (int t = 0; t < C; ++t) mx = fmaxf(mx, fabsf(sG[t][ch] - m));
    if (!(mx <= THRESH)) atomicOr(&sSlow, 1);
    rec[Rc::G0 + ch] = expn(m);
    rec[Rc::D0 + ch] = expn(sG[C - 1][ch] - m);
  }
  __syncthreads();
  const bool slow = sSlow != 0;
  if (tid == 0) rec[Rc::FLAG] = slow ? 1.0f : 0.0f;
  if (tid < C) rec[Rc::BETA + tid] = sBeta[tid];
  if (slow) return;                            // the token path needs nothing else
  // four channels per thread and step: 16-byte stores
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int i4 = tid + 256 * m;
    if (i4 >= C * KD / 4) break;
    const int i = 4 * i4, t = i / KD, ch = i % KD;
    float4 E, ke, qe, kr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = sG[t][ch + j] - sG[15][ch + j];
      const float L = expn(e), Rr = expn(-e);
      E[j] = e;
      ke[j] = kv[m][j] * L;
      qe[j] = scale * qv[m][j] * L;
      kr[j] = kv[m][j] * Rr;
    }
    *reinterpret_cast<float4*>(sKE + t * LK + ch) = ke;
    *reinterpret_cast<float4*>(sQE + t * LK + ch) = qe;
    *reinterpret_cast<float4*>(sKR + t * LK + ch) = kr;
    *reinterpret_cast<float4*>(rec + Rc::KE + i) = ke;
    *reinterpret_cast<float4*>(rec + Rc::QE + i) = qe;
    *reinterpret_cast<float4*>(rec + Rc::KR + i) = kr;
    *reinterpret_cast<float4*>(rec + Rc::E + i) = E;
  }
  __syncthreads();
  // A (strictly lower) and P (lower) on MFMA: 2 x 2 tiles each, two tiles per wave
  for (int tt = wave; tt < 8; tt += 4) {
    const bool isP = tt >= 4;
    const int ti = (tt >> 1) & 1, tj = tt & 1;
    const float* pa = (isP ? sQE : sKE) + 16 * ti * LK;
    const float* pb = sKR + 16 * tj * LK;
    floatx4 acc = zero4();
#pragma unroll 8
    for (int d = 0; d < KD; d += 4)
      acc = mma(pa[(lane & 15) * LK + d + (lane >> 4)], pb[(lane & 15) * LK + d + (lane >> 4)], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * (lane >> 4) + r, j = 16 * tj + (lane & 15);
      const float val = (isP ? j <= i : j < i) ? acc[r] : 0.0f;
      rec[(isP ? Rc::P : Rc::A) + i * C + j] = val;
      if (!isP) sA[i * LC + j] = val;
    }
  }
  __syncthreads();
  // T = M^-1 for M = I + diag(beta) A, in 16-row blocks: M = [[M00, 0], [M10, M11]] gives
  // T00 = M00^-1 and T11 = M11^-1 by forward substitution (waves 0 and 1 side by side, lane
  // l < 16 holding column l: T_il = delta_il - beta_i sum_{j<i} A_ij T_jl), then
  // T10 = -T11 (M10 T00) from two 16 x 16 products; T01 = 0.
  if (wave < 2 && lane < 16) {
    const int I = wave;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * I + i;
      const float bi = sBeta[r];
      float s0 = i == lane ? 1.0f : 0.0f, s1 = 0.0f;
#pragma unroll
      for (int j = 0; j < i; ++j) {
        const float a = -bi * sA[r * LC + 16 * I + j];
        if (j & 1) s1 = fmaf(a, x[j], s1);
        else s0 = fmaf(a, x[j], s0);
      }
      x[i] = s0 + s1;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(16 * I + i) * LC + 16 * I + lane] = x[i];
  }
  __syncthreads();
  const int ti = tid >> 4, tj = tid & 15;      // one element of a 16 x 16 block per thread
  {
    float s = 0.0f;
#pragma unroll
    for (int l = 0; l < 16; ++l) s = fmaf(sA[(16 + ti) * LC + l], sT[l * LC + tj], s);
    sX[ti * 16 + tj] = sBeta[16 + ti] * s;     // M10 T00
  }
  __syncthreads();
  {
    float s = 0.0f;
#pragma unroll
    for (int l = 0; l < 16; ++l) s = fmaf(sT[(16 + ti) * LC + 16 + l], sX[l * 16 + tj], s);
    sT[(16 + ti) * LC + tj] = -s;
    sT[ti * LC + 16 + tj] = 0.0f;
  }
  __syncthreads();
  for (int e = tid; e < C * C; e += 256) rec[Rc::T + e] = sT[(e / C) * LC + e % C];
}

// Column sums over the KD rows of a [KD][16] LDS tile weighted by w[KD]: 256 threads, thread
// (rg, j) adds rows rg, rg + 16, ... of column j; the 16 partials meet in red[16][16].
template <int KD>
__device__ __forceinline__ void colsum16(const float* tile, const float* w, float* red, float* out, int tid) {
  const int j = tid & 15, rg = tid >> 4;
  float s = 0.0f;
#pragma unroll
  for (int r = rg; r < KD; r += 16) s = fmaf(tile[r * 16 + j], w[r], s);
  red[rg * 16 + j] = s;
  __syncthreads();
  if (tid < 16) {
    float a = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) a += red[g * 16 + tid];
    out[tid] = a;
  }
  __syncthreads();
}

// Chunk operands staged through registers: the loads of chunk c+1 are issued before the
// MFMA phases of chunk c (16 bytes per lane) and written to LDS at the start of step c+1,
// so that the sequential passes do not wait on their loads.
template <int N>
struct Stage {
  float4 r[N];
  // src: n float4; r[i] holds element tid + 256 i
  __device__ __forceinline__ void load(const float* src, int n, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = tid + 256 * i;
      r[i] = e < n ? reinterpret_cast<const float4*>(src)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // into a [rows][cols] LDS tile with row stride ld (cols a multiple of 4)
  __device__ __forceinline__ void put(float* dst, int cols, int ld, int n, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = tid + 256 * i;
      if (e < n) {
        const int row = (4 * e) / cols, col = (4 * e) % cols;
        *reinterpret_cast<float4*>(dst + row * ld + col) = r[i];
      }
    }
  }
};

// The 16 value columns of C token rows (0 past the chunk's tokens or past V): lane
// (t = tid / 4, quarter tid % 4), threads 0..127.
__device__ __forceinline__ float4 load_rows16(const float* base, size_t row0, int nval, int V, int v0, int tid) {
  const int t = tid >> 2, j = 4 * (tid & 3);
  if (tid < 4 * C && t < nval && v0 + j < V) return *reinterpret_cast<const float4*>(base + (row0 + t) * V + v0 + j);
  return make_float4(0.f, 0.f, 0.f, 0.f);
}

// ============================================================================ forward
// One workgroup per (head, 16 value columns), chunks in order.  The state tile lives in
// LDS as [KD][16].
template <int KD>
constexpr int fwd_lds_floats() {
  return KD * 16 + 2 * C * (KD + 4) + C * (C + 4) + 4 * C * 16 + 2 * KD + C + 4 + 256 + KD + 16;
}

template <int KD>
__device__ __forceinline__ void fwd_pass(float* __restrict__ lds, int vt, int bh, int BH, const float* __restrict__ k,
                                         const float* __restrict__ v, const float* __restrict__ z,
                                         const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                                         const float* __restrict__ beta, const float* __restrict__ state_in,
                                         char* __restrict__ ws, int H, int T, int K, int V, int VP, int nck) {
  using Rc = Rec<KD>;
  constexpr int LK = KD + 4, LC = C + 4;
  constexpr int NK = C * KD / 4, NI = (NK + 255) / 256;
  float* sS = lds;                             // [KD][16]
  float* sKE = sS + KD * 16;
  float* sKR = sKE + C * LK;
  float* sT = sKR + C * LK;
  float* sZ = sT + C * LC;
  float* sU = sZ + C * 16;
  float* sPart = sU + C * 16;
  float* sMisc = sPart + 2 * C * 16;           // G0, D0, beta, flag
  float* sRed = sMisc + 2 * KD + C + 4;
  float* sVec = sRed + 256;
  float* sE = sVec + KD;
  float* sG0 = sMisc;
  float* sD0 = sMisc + KD;
  float* sBeta = sMisc + 2 * KD;
  const int h = bh % H, v0 = 16 * vt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Layout lo = layout(KD, VP, BH, nck);
  const float* recs = reinterpret_cast<const float*>(ws + lo.rec);
  float* ck = reinterpret_cast<float*>(ws + lo.ck);
  float* ub = reinterpret_cast<float*>(ws + lo.u);
  float* yb = reinterpret_cast<float*>(ws + lo.y);
  const float gm = gate_multiplier(A_log[h]);
  for (int i = tid; i < KD * 16; i += 256) {
    const int ch = i >> 4, j = i & 15;
    sS[i] = (state_in && ch < K && v0 + j < V) ? state_in[((size_t)bh * K + ch) * V + v0 + j] : 0.0f;
  }
  Stage<NI> pKE, pKR;
  Stage<1> pT, pM;
  float4 pV;
  auto issue = [&](int c) __attribute__((always_inline)) {
    const float* rec = recs + ((size_t)bh * nck + c) * Rc::SIZE;
    pKE.load(rec + Rc::KE, NK, tid);
    pKR.load(rec + Rc::KR, NK, tid);
    pT.load(rec + Rc::T, C * C / 4, tid);
    pM.load(rec + Rc::BETA, (C + 2 * KD + 4) / 4, tid);   // beta, G0, D0, flag (contiguous)
    pV = load_rows16(v, (size_t)bh * T + (size_t)c * C, min(C, T - c * C), V, v0, tid);
  };
  if (nck > 0) issue(0);
  for (int c = 0; c < nck; ++c) {
    const int t0 = c * C, nval = min(C, T - t0);
    const size_t row0 = (size_t)bh * T + t0;
    const size_t chunk = (size_t)bh * nck + c;
    __syncthreads();                           // (the previous chunk is done with every buffer)
    pKE.put(sKE, KD, LK, NK, tid);
    pKR.put(sKR, KD, LK, NK, tid);
    pT.put(sT, C, LC, C * C / 4, tid);
    if (tid < (C + 2 * KD + 4) / 4) {
      // record order: beta [C], G0 [KD], D0 [KD], flag; LDS order: G0, D0, beta, flag
      const int e = 4 * tid;
      float* d = e < C ? sBeta + e : (e < C + 2 * KD ? sG0 + (e - C) : sMisc + 2 * KD + C + (e - C - 2 * KD));
      *reinterpret_cast<float4*>(d) = pM.r[0];
    }
    if (tid < 4 * C) *reinterpret_cast<float4*>(sZ + 4 * tid) = pV;
    // checkpoint: the state at the chunk start
    for (int i = tid; i < KD * 4; i += 256) {
      const int ch = i >> 2, j = 4 * (i & 3);
      *reinterpret_cast<float4*>(ck + chunk * KD * VP + vt_off(KD, ch, v0 + j)) =
          *reinterpret_cast<const float4*>(sS + ch * 16 + j);
    }
    __syncthreads();
    if (c + 1 < nck) issue(c + 1);
    const bool slow = sMisc[2 * KD + C] != 0.0f;
    if (!slow) {
      for (int i = tid; i < KD * 16; i += 256) sS[i] *= sG0[i >> 4];   // S~ = diag(G0) S
      __syncthreads();
      // Y = V - KE S~: tiles of 16 tokens, the depth split in halves over the four waves
      {
        const int rt = wave & 1, dh = wave >> 1;
        floatx4 acc = zero4();
        const float* pa = sKE + 16 * rt * LK;
#pragma unroll 8
        for (int d = dh * (KD / 2); d < (dh + 1) * (KD / 2); d += 4)
          acc = mma(pa[(lane & 15) * LK + d + (lane >> 4)], sS[(d + (lane >> 4)) * 16 + (lane & 15)], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sPart[dh * C * 16 + (16 * rt + 4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[r];
      }
      __syncthreads();
      for (int i = tid; i < C * 16; i += 256) {
        const int t = i >> 4, j = i & 15;
        const float y = sZ[i] - sPart[i] - sPart[C * 16 + i];
        yb[chunk * C * VP + vt_off(C, t, v0 + j)] = y;
        sZ[i] = sBeta[t] * y;
      }
      __syncthreads();
      // U = T Z
      if (wave < 2) {
        const int rt = wave;
        floatx4 acc = zero4();
#pragma unroll
        for (int d = 0; d < C; d += 4)
          acc = mma(sT[(16 * rt + (lane & 15)) * LC + d + (lane >> 4)], sZ[(d + (lane >> 4)) * 16 + (lane & 15)], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rt + 4 * (lane >> 4) + r, j = lane & 15;
          sU[t * 16 + j] = acc[r];
        }
      }
      __syncthreads();
      // U for the gradient kernel: the tile's C x 16 block in one contiguous 16-byte-per-lane
      // copy by the waves that did not compute it
      if (tid >= 128) {
        const int i = tid - 128;
        *reinterpret_cast<float4*>(ub + chunk * C * VP + vt_off(C, 0, v0) + 4 * i) =
            *reinterpret_cast<const float4*>(sU + 4 * i);
      }
      // S = diag(D0) (S~ + KR^T U)
      for (int ct = wave; ct < KD / 16; ct += 4) {
        floatx4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sS[(16 * ct + 4 * (lane >> 4) + r) * 16 + (lane & 15)];
#pragma unroll
        for (int d = 0; d < C; d += 4)
          acc = mma(sKR[(d + (lane >> 4)) * LK + 16 * ct + (lane & 15)], sU[(d + (lane >> 4)) * 16 + (lane & 15)], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ch = 16 * ct + 4 * (lane >> 4) + r;
          sS[ch * 16 + (lane & 15)] = sD0[ch] * acc[r];
        }
      }
    } else {
      // token by token: S' = diag(alpha) S, e = v - S'^T k, S = S' + beta k e^T
      for (int t = 0; t < nval; ++t) {
        if (tid < KD) {
          const int ch = tid;
          const float db = (dt_bias && ch < K) ? dt_bias[h * K + ch] : 0.0f;
          const float al = ch < K ? expn(gate_g(z[(row0 + t) * K + ch], db, gm)) : 0.0f;
          sVec[ch] = ch < K ? k[(row0 + t) * K + ch] : 0.0f;
          sRed[ch] = al;                         // (alpha kept here until the scaling below)
        }
        __syncthreads();
        for (int i = tid; i < KD * 16; i += 256) sS[i] *= sRed[i >> 4];
        __syncthreads();
        colsum16<KD>(sS, sVec, sRed, sE, tid);
        const float bt = beta[row0 + t];
        for (int i = tid; i < KD * 16; i += 256) {
          const int ch = i >> 4, j = i & 15;
          const float vv = v0 + j < V ? v[(row0 + t) * V + v0 + j] : 0.0f;
          sS[i] = fmaf(sVec[ch], bt * (vv - sE[j]), sS[i]);
        }
        __syncthreads();
      }
    }
  }
}

// ============================================================================ reverse
// One workgroup per (head, 16 value columns), chunks in reverse; the cotangent tile dS
// lives in LDS as [KD][16].
template <int KD>
constexpr int rev_lds_floats() {
  return KD * 16 + 3 * C * (KD + 4) + 2 * C * (C + 4) + 4 * C * 16 + 2 * KD + C + 4 + 256 + 2 * KD + 16;
}

template <int KD>
__device__ __forceinline__ void rev_pass(float* __restrict__ lds, int vt, int bh, int BH, const float* __restrict__ q,
                                         const float* __restrict__ k, const float* __restrict__ z,
                                         const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                                         const float* __restrict__ beta, float scale, const float* __restrict__ d_o,
                                         const float* __restrict__ d_state_out, char* __restrict__ ws,
                                         float* __restrict__ dv, float* __restrict__ dstate_in, int H, int T, int K,
                                         int V, int VP, int nck) {
  using Rc = Rec<KD>;
  constexpr int LK = KD + 4, LC = C + 4;
  constexpr int NK = C * KD / 4, NI = (NK + 255) / 256;
  float* sD = lds;                             // [KD][16]
  float* sQE = sD + KD * 16;
  float* sKE = sQE + C * LK;
  float* sKR = sKE + C * LK;
  float* sP = sKR + C * LK;
  float* sT = sP + C * LC;
  float* sDO = sT + C * LC;
  float* sDU = sDO + C * 16;                   // two partial sums [2][C][16]
  float* sDZ = sDU + 2 * C * 16;
  float* sMisc = sDZ + C * 16;                 // G0, D0, beta, flag
  float* sRed = sMisc + 2 * KD + C + 4;
  float* sVec = sRed + 256;
  float* sAl = sVec + KD;
  float* sE = sAl + KD;
  float* sG0 = sMisc;
  float* sD0 = sMisc + KD;
  float* sBeta = sMisc + 2 * KD;
  const int h = bh % H, v0 = 16 * vt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Layout lo = layout(KD, VP, BH, nck);
  const float* recs = reinterpret_cast<const float*>(ws + lo.rec);
  float* dse = reinterpret_cast<float*>(ws + lo.dse);
  float* dzb = reinterpret_cast<float*>(ws + lo.dz);
  const float gm = gate_multiplier(A_log[h]);
  for (int i = tid; i < KD * 16; i += 256) {
    const int ch = i >> 4, j = i & 15;
    sD[i] = (d_state_out && ch < K && v0 + j < V) ? d_state_out[((size_t)bh * K + ch) * V + v0 + j] : 0.0f;
  }
  Stage<NI> pQE, pKE, pKR;
  Stage<1> pP, pT, pM;
  float4 pO;
  auto issue = [&](int c) __attribute__((always_inline)) {
    const float* rec = recs + ((size_t)bh * nck + c) * Rc::SIZE;
    pQE.load(rec + Rc::QE, NK, tid);
    pKE.load(rec + Rc::KE, NK, tid);
    pKR.load(rec + Rc::KR, NK, tid);
    pP.load(rec + Rc::P, C * C / 4, tid);
    pT.load(rec + Rc::T, C * C / 4, tid);
    pM.load(rec + Rc::BETA, (C + 2 * KD + 4) / 4, tid);
    pO = load_rows16(d_o, (size_t)bh * T + (size_t)c * C, min(C, T - c * C), V, v0, tid);
  };
  if (nck > 0) issue(nck - 1);
  for (int c = nck - 1; c >= 0; --c) {
    const int t0 = c * C, nval = min(C, T - t0);
    const size_t row0 = (size_t)bh * T + t0;
    const size_t chunk = (size_t)bh * nck + c;
    __syncthreads();
    pQE.put(sQE, KD, LK, NK, tid);
    pKE.put(sKE, KD, LK, NK, tid);
    pKR.put(sKR, KD, LK, NK, tid);
    pP.put(sP, C, LC, C * C / 4, tid);
    pT.put(sT, C, LC, C * C / 4, tid);
    if (tid < (C + 2 * KD + 4) / 4) {
      const int e = 4 * tid;
      float* d = e < C ? sBeta + e : (e < C + 2 * KD ? sG0 + (e - C) : sMisc + 2 * KD + C + (e - C - 2 * KD));
      *reinterpret_cast<float4*>(d) = pM.r[0];
    }
    if (tid < 4 * C) *reinterpret_cast<float4*>(sDO + 4 * tid) = pO;
    // the chunk-end cotangent, for the gradient kernel
    for (int i = tid; i < KD * 4; i += 256) {
      const int ch = i >> 2, j = 4 * (i & 3);
      *reinterpret_cast<float4*>(dse + chunk * KD * VP + vt_off(KD, ch, v0 + j)) =
          *reinterpret_cast<const float4*>(sD + ch * 16 + j);
    }
    __syncthreads();
    if (c > 0) issue(c - 1);
    const bool slow = sMisc[2 * KD + C] != 0.0f;
    if (!slow) {
      for (int i = tid; i < KD * 16; i += 256) sD[i] *= sD0[i >> 4];   // dX = diag(D0) dS
      __syncthreads();
      // dU = P^T dO + KR dX in two partial sums over all four waves: row tile wave & 1;
      // part 0 takes P^T dO and KR dX over the channels [0, D1), part 1 the rest
      {
        constexpr int D1 = KD > 32 ? (KD - 32) / 2 : 0;
        const int rt = wave & 1, part = wave >> 1;
        floatx4 acc = zero4();
        if (part == 0) {
#pragma unroll
          for (int d = 0; d < C; d += 4)
            acc = mma(sP[(d + (lane >> 4)) * LC + 16 * rt + (lane & 15)], sDO[(d + (lane >> 4)) * 16 + (lane & 15)], acc);
#pragma unroll 4
          for (int d = 0; d < D1; d += 4)
            acc = mma(sKR[(16 * rt + (lane & 15)) * LK + d + (lane >> 4)], sD[(d + (lane >> 4)) * 16 + (lane & 15)], acc);
        } else {
#pragma unroll 4
          for (int d = D1; d < KD; d += 4)
            acc = mma(sKR[(16 * rt + (lane & 15)) * LK + d + (lane >> 4)], sD[(d + (lane >> 4)) * 16 + (lane & 15)], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sDU[part * C * 16 + (16 * rt + 4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[r];
      }
      __syncthreads();
      // dZ = T^T dU; dv = diag(beta) dZ
      if (wave < 2) {
        const int rt = wave;
        floatx4 acc = zero4();
#pragma unroll
        for (int d = 0; d < C; d += 4) {
          const int e = (d + (lane >> 4)) * 16 + (lane & 15);
          acc = mma(sT[(d + (lane >> 4)) * LC + 16 * rt + (lane & 15)], sDU[e] + sDU[C * 16 + e], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rt + 4 * (lane >> 4) + r, j = lane & 15;
          sDZ[t * 16 + j] = acc[r];
          if (t < nval && v0 + j < V) dv[(row0 + t) * V + v0 + j] = sBeta[t] * acc[r];
        }
      }
      __syncthreads();
      // dZ for the gradient kernel, copied as U is in the forward pass
      if (tid >= 128) {
        const int i = tid - 128;
        *reinterpret_cast<float4*>(dzb + chunk * C * VP + vt_off(C, 0, v0) + 4 * i) =
            *reinterpret_cast<const float4*>(sDZ + 4 * i);
      }
      // dS = diag(G0) (dX + QE^T dO - KE^T diag(beta) dZ); a wave reads and writes only the
      // rows of its own tiles of dS
      for (int ct = wave; ct < KD / 16; ct += 4) {
        floatx4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = sD[(16 * ct + 4 * (lane >> 4) + r) * 16 + (lane & 15)];
#pragma unroll
        for (int d = 0; d < C; d += 4) {
          const int t = d + (lane >> 4);
          acc = mma(sQE[t * LK + 16 * ct + (lane & 15)], sDO[t * 16 + (lane & 15)], acc);
          acc = mma(-sBeta[t] * sKE[t * LK + 16 * ct + (lane & 15)], sDZ[t * 16 + (lane & 15)], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ch = 16 * ct + 4 * (lane >> 4) + r;
          sD[ch * 16 + (lane & 15)] = sG0[ch] * acc[r];
        }
      }
    } else {
      // token by token: dS += q_hat do^T, de = beta dS^T k, dv = de, dS -= k de^T, dS = diag(alpha) dS
      for (int t = nval - 1; t >= 0; --t) {
        if (tid < KD) {
          const int ch = tid;
          const float db = (dt_bias && ch < K) ? dt_bias[h * K + ch] : 0.0f;
          sAl[ch] = ch < K ? expn(gate_g(z[(row0 + t) * K + ch], db, gm)) : 0.0f;
          sVec[ch] = ch < K ? k[(row0 + t) * K + ch] : 0.0f;
          sRed[ch] = ch < K ? scale * q[(row0 + t) * K + ch] : 0.0f;
        }
        __syncthreads();
        for (int i = tid; i < KD * 16; i += 256) {
          const int ch = i >> 4, j = i & 15;
          const float dov = v0 + j < V ? d_o[(row0 + t) * V + v0 + j] : 0.0f;
          sD[i] = fmaf(sRed[ch], dov, sD[i]);
        }
        __syncthreads();
        colsum16<KD>(sD, sVec, sRed, sE, tid);
        const float bt = beta[row0 + t];
        if (tid < 16 && v0 + tid < V) dv[(row0 + t) * V + v0 + tid] = bt * sE[tid];
        for (int i = tid; i < KD * 16; i += 256) {
          const int ch = i >> 4, j = i & 15;
          sD[i] = sAl[ch] * fmaf(-sVec[ch], bt * sE[j], sD[i]);
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < KD * 16; i += 256) {
    const int ch = i >> 4, j = i & 15;
    if (dstate_in && ch < K && v0 + j < V) dstate_in[((size_t)bh * K + ch) * V + v0 + j] = sD[i];
  }
}

// The two sequential passes do not depend on each other (the reverse pass needs only the
// prep records and d_o), so one launch runs both, 2 VP / 16 workgroups per head: slot
// x < VP / 16 takes the forward pass of value tile x, the others the reverse pass of tile
// x - VP / 16.  Their LDS is one shared buffer, so that a forward and a reverse workgroup
// fit one CU together.  Every value tile of a pass reads the same chunk records; when the
// head count is a multiple of 8, all workgroups of a head go to one XCD (workgroup i runs
// on XCD i % 8), so that the records come from HBM once and from that XCD's L2 after.
template <int KD>
__global__ void __launch_bounds__(256)
seq_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
           const float* __restrict__ z, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
           const float* __restrict__ beta, const float* __restrict__ state_in, float scale,
           const float* __restrict__ d_o, const float* __restrict__ d_state_out, char* __restrict__ ws,
           float* __restrict__ dv, float* __restrict__ dstate_in, int H, int T, int K, int V, int VP, int nck,
           int BH) {
  __shared__ __attribute__((aligned(16))) float lds[cmax(fwd_lds_floats<KD>(), rev_lds_floats<KD>())];
  const int nt = VP / 16, per = 2 * nt;
  const int i = blockIdx.x;
  int bh, x;
  if ((BH & 7) == 0) {
    const int r = i >> 3;                      // rank within XCD i % 8
    bh = (i & 7) + 8 * (r / per);
    x = r % per;
  } else {
    bh = i / per;
    x = i % per;
  }
  if (x < nt)
    fwd_pass<KD>(lds, x, bh, BH, k, v, z, A_log, dt_bias, beta, state_in, ws, H, T, K, V, VP, nck);
  else
    rev_pass<KD>(lds, x - nt, bh, BH, q, k, z, A_log, dt_bias, beta, scale, d_o, d_state_out, ws, dv, dstate_in, H,
                 T, K, V, VP, nck);
}

// ============================================================================ gradient
// One workgroup (8 waves) per (head, chunk), all value columns.  The products over the
// value columns go in slabs of 32 columns through LDS.  The slab buffers and the chunk's
// KE, QE, KR are not needed at the same time and share one LDS region (66 KB in all at
// KD = 128), so two workgroups fit one CU and each hides the other's load latency.
// Chunks on the token path are left to grad_token_kernel.
template <int KD>
struct GradCfg {
  static constexpr int LK = KD + 4, LC = C + 4, LS = 32 + 4;
  static constexpr int NCT = KD / 16;                 // channel tiles
  static constexpr int NTT = 2 * NCT;                 // [token][channel] output tiles
  static constexpr int NTW = (NTT + 7) / 8;           // of them per wave
  static constexpr int NCH = (KD * 8 + 511) / 512;    // float4 of a state slab per thread
  // region X, first the slab (dO, dZ, U over tokens; S~, dX over channels), then KE, QE,
  // KR; at the end dG and KW overwrite KE and QE in place
  static constexpr int X_DO = 0, X_DZ = X_DO + C * LS, X_U = X_DZ + C * LS;
  static constexpr int X_ST = X_U + C * LS, X_DX = X_ST + KD * LS;
  static constexpr int X_KE = 0, X_QE = C * LK, X_KR = 2 * C * LK;
  static constexpr int X_END = cmax(X_DX + KD * LS, 3 * C * LK);
  static constexpr int F_A = X_END, F_DP = F_A + C * LC, F_DA = F_DP + C * LC;
  static constexpr int F_MISC = F_DA + C * LC;        // beta, G0, D0, dbeta, rowsum(dX S~)
  static constexpr int F_TOTAL = F_MISC + C + 2 * KD + C + KD;
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

template <int KD, int VP>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4)))
grad_kernel(const float* __restrict__ d_o, const char* __restrict__ ws, float scale, float* __restrict__ dq,
            float* __restrict__ dk, float* __restrict__ dg, float* __restrict__ dbeta, int T, int K, int V,
            int nck) {
  using Rc = Rec<KD>;
  using G = GradCfg<KD>;
  constexpr int LK = G::LK, LC = G::LC, LS = G::LS, NCH = G::NCH;
  __shared__ __attribute__((aligned(16))) float sm[G::F_TOTAL];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int t0 = c * C, nval = min(C, T - t0);
  const size_t row0 = (size_t)bh * T + t0;
  const size_t chunk = (size_t)bh * nck + c;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Layout lo = layout(KD, VP, (long long)gridDim.y, nck);
  const float* rec = reinterpret_cast<const float*>(ws + lo.rec) + chunk * Rc::SIZE;
  const float* ckp = reinterpret_cast<const float*>(ws + lo.ck) + chunk * KD * VP;
  const float* dsep = reinterpret_cast<const float*>(ws + lo.dse) + chunk * KD * VP;
  const float* up = reinterpret_cast<const float*>(ws + lo.u) + chunk * C * VP;
  const float* yp = reinterpret_cast<const float*>(ws + lo.y) + chunk * C * VP;
  const float* dzp = reinterpret_cast<const float*>(ws + lo.dz) + chunk * C * VP;
  if (rec[Rc::FLAG] != 0.0f) return;           // the token path's chunk

  float* sDO = sm + G::X_DO;
  float* sDZ = sm + G::X_DZ;
  float* sU = sm + G::X_U;
  float* sST = sm + G::X_ST;
  float* sDX = sm + G::X_DX;
  float* sKE = sm + G::X_KE;
  float* sQE = sm + G::X_QE;
  float* sKR = sm + G::X_KR;
  float* sA = sm + G::F_A;
  float* sDP = sm + G::F_DP;
  float* sDA = sm + G::F_DA;
  float* sBeta = sm + G::F_MISC;
  float* sG0 = sBeta + C;
  float* sD0 = sG0 + KD;
  float* sDB = sD0 + KD;
  float* sXS = sDB + C;
  for (int i = tid; i < C * C / 4; i += 512) {
    const int r = (4 * i) / C, col = (4 * i) % C;
    st4(sA + r * LC + col, ld4(rec + Rc::A + 4 * i));
  }
  for (int i = tid; i < KD; i += 512) {
    sG0[i] = rec[Rc::G0 + i];
    sD0[i] = rec[Rc::D0 + i];
  }
  if (tid < C) {
    sBeta[tid] = rec[Rc::BETA + tid];
    sDB[tid] = 0.0f;
  }
  // slab operands in registers: token rows (threads 0..255: token tid / 8, columns
  // 4 (tid % 8) .. +3) and channel rows (float4 i = tid + 512 m: channel i / 8).  The
  // channel rows (the bulk: S~ and dX) of the next slab are loaded while the current one
  // is multiplied; the token rows are loaded when they are needed.
  const int st_t = tid >> 3, st_f = tid & 7;
  float4 rDO, rDZ, rU, rY, rCK[NCH], rDS[NCH];
  auto load_tok = [&](int v0) __attribute__((always_inline)) {
    if (tid < 256) {
      const size_t g = vt_off(C, st_t, v0 + 4 * st_f);
      const bool ok = st_t < nval && v0 + 4 * st_f < V;
      rDO = ok ? ld4(d_o + (row0 + st_t) * V + v0 + 4 * st_f) : make_float4(0.f, 0.f, 0.f, 0.f);
      rDZ = ld4(dzp + g);
      rU = ld4(up + g);
      rY = ld4(yp + g);
    }
  };
  auto load_ch = [&](int v0) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int i = tid + 512 * m;
      if (i < KD * 8) {
        const size_t off = vt_off(KD, i >> 3, v0 + 4 * (i & 7));
        rCK[m] = ld4(ckp + off);
        rDS[m] = ld4(dsep + off);
      }
    }
  };
  // accumulators: dQE, dKE and W = U dX^T on [token][channel] tiles wave + 8 i; dP (waves
  // 0..3) or dM (waves 4..7) on one [token][token] tile
  floatx4 aQ[G::NTW], aK[G::NTW], aW[G::NTW], aPM = zero4();
#pragma unroll
  for (int i = 0; i < G::NTW; ++i) aQ[i] = aK[i] = aW[i] = zero4();
  // elementwise sums: rowsum(dX S~) of the thread's channels, sum_v dZ Y of its token
  float xs[NCH], zy = 0.0f;
#pragma unroll
  for (int m = 0; m < NCH; ++m) xs[m] = 0.0f;
  load_ch(0);
  __syncthreads();                             // sBeta, sG0, sD0
#pragma unroll 1
  for (int v0 = 0; v0 < VP; v0 += 32) {
    if (v0) __syncthreads();                   // (the previous slab is consumed)
    load_tok(v0);
    if (tid < 256) {
      st4(sDO + st_t * LS + 4 * st_f, rDO);
      st4(sDZ + st_t * LS + 4 * st_f, rDZ);
      st4(sU + st_t * LS + 4 * st_f, rU);
      zy += dot4(rDZ, rY);
    }
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int i = tid + 512 * m;
      if (i < KD * 8) {
        const int ch = i >> 3, j = 4 * (i & 7);
        const float g0 = sG0[ch], d0 = sD0[ch];
        const float4 st = make_float4(g0 * rCK[m].x, g0 * rCK[m].y, g0 * rCK[m].z, g0 * rCK[m].w);
        const float4 dx = make_float4(d0 * rDS[m].x, d0 * rDS[m].y, d0 * rDS[m].z, d0 * rDS[m].w);
        st4(sST + ch * LS + j, st);
        st4(sDX + ch * LS + j, dx);
        xs[m] += dot4(st, dx);
      }
    }
    if (v0 + 32 < VP) load_ch(v0 + 32);       // in flight during this slab's products
    __syncthreads();
#pragma unroll
    for (int i = 0; i < G::NTW; ++i) {
      const int tau = wave + 8 * i;
      if (tau < G::NTT) {
        const int rt = tau / G::NCT, ct = tau % G::NCT;
        const int ti = 16 * rt + (lane & 15), ci = 16 * ct + (lane & 15);
        const float nb = -sBeta[ti];
#pragma unroll 2
        for (int d = 0; d < 32; d += 4) {
          const int dd = d + (lane >> 4);
          const float st = sST[ci * LS + dd];
          aQ[i] = mma(sDO[ti * LS + dd], st, aQ[i]);
          aK[i] = mma(nb * sDZ[ti * LS + dd], st, aK[i]);
          aW[i] = mma(sU[ti * LS + dd], sDX[ci * LS + dd], aW[i]);
        }
      }
    }
    {
      const int ti = 16 * ((wave >> 1) & 1) + (lane & 15), tj = 16 * (wave & 1) + (lane & 15);
      const float* pa = wave < 4 ? sDO : sDZ;
      const float sg = wave < 4 ? 1.0f : -1.0f;
#pragma unroll
      for (int d = 0; d < 32; d += 4) {
        const int dd = d + (lane >> 4);
        aPM = mma(sg * pa[ti * LS + dd], sU[tj * LS + dd], aPM);
      }
    }
  }
  // dP (lower) and dA = diag(beta) dM (strictly lower) to LDS; dbeta gets sum_j dM_tj A_tj
  {
    const int ti0 = 16 * ((wave >> 1) & 1), tj0 = 16 * (wave & 1);
    float rs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = ti0 + 4 * (lane >> 4) + r, j = tj0 + (lane & 15);
      if (wave < 4) {
        sDP[i * LC + j] = j <= i ? aPM[r] : 0.0f;
        rs[r] = 0.0f;
      } else {
        const float dm = j < i ? aPM[r] : 0.0f;
        sDA[i * LC + j] = sBeta[i] * dm;
        rs[r] = dm * sA[i * LC + j];
      }
    }
    if (wave >= 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = rs[r];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if ((lane & 15) == 0) atomicAdd(&sDB[ti0 + 4 * (lane >> 4) + r], x);
      }
    }
  }
  // the per-thread sums: rowsum(dX S~) per channel (8 threads a channel), sum_v dZ Y per
  // token (8 threads a token)
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    xs[m] += __shfl_xor(xs[m], 1);
    xs[m] += __shfl_xor(xs[m], 2);
    xs[m] += __shfl_xor(xs[m], 4);
  }
  zy += __shfl_xor(zy, 1);
  zy += __shfl_xor(zy, 2);
  zy += __shfl_xor(zy, 4);
  __syncthreads();                             // the slab region is free; dP, dA complete
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    const int i = tid + 512 * m;
    if (i < KD * 8 && (i & 7) == 0) sXS[i >> 3] = xs[m];
  }
  if (tid < 256 && st_f == 0) atomicAdd(&sDB[st_t], zy);
  for (int i = tid; i < C * KD / 4; i += 512) {
    const int t = (4 * i) / KD, ch = (4 * i) % KD;
    st4(sKE + t * LK + ch, ld4(rec + Rc::KE + 4 * i));
    st4(sQE + t * LK + ch, ld4(rec + Rc::QE + 4 * i));
    st4(sKR + t * LK + ch, ld4(rec + Rc::KR + 4 * i));
  }
  // E of the thread's output elements (for L and R), ahead of the products
  const float* Erec = rec + Rc::E;
  float rE[G::NTW][4];
#pragma unroll
  for (int i = 0; i < G::NTW; ++i) {
    const int tau = wave + 8 * i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rE[i][r] = 0.0f;
      if (tau < G::NTT) {
        const int t = 16 * (tau / G::NCT) + 4 * (lane >> 4) + r, ch = 16 * (tau % G::NCT) + (lane & 15);
        rE[i][r] = Erec[t * KD + ch];
      }
    }
  }
  __syncthreads();
  // second products (depth: the chunk's tokens)
  floatx4 aR[G::NTW];
#pragma unroll
  for (int i = 0; i < G::NTW; ++i) {
    const int tau = wave + 8 * i;
    aR[i] = aW[i];
    if (tau < G::NTT) {
      const int rt = tau / G::NCT, ct = tau % G::NCT;
      const int ti = 16 * rt + (lane & 15), ci = 16 * ct + (lane & 15);
#pragma unroll
      for (int d = 0; d < C; d += 4) {
        const int dd = d + (lane >> 4);
        const float kr = sKR[dd * LK + ci];
        aQ[i] = mma(sDP[ti * LC + dd], kr, aQ[i]);
        aK[i] = mma(sDA[ti * LC + dd], kr, aK[i]);
        aR[i] = mma(sDP[dd * LC + ti], sQE[dd * LK + ci], aR[i]);
        aR[i] = mma(sDA[dd * LC + ti], sKE[dd * LK + ci], aR[i]);
      }
    }
  }
  __syncthreads();                             // every wave is done reading KE, QE, KR
  // the elementwise gradients; dG and KW = KR (U dX^T) replace KE and QE element by element
  float* sDG = sKE;
  float* sKW = sQE;
#pragma unroll
  for (int i = 0; i < G::NTW; ++i) {
    const int tau = wave + 8 * i;
    if (tau < G::NTT) {
      const int rt = tau / G::NCT, ct = tau % G::NCT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rt + 4 * (lane >> 4) + r, ch = 16 * ct + (lane & 15);
        const float ke = sKE[t * LK + ch], qe = sQE[t * LK + ch], kr = sKR[t * LK + ch];
        const float L = expn(rE[i][r]), Rr = expn(-rE[i][r]);
        sDG[t * LK + ch] = aK[i][r] * ke + aQ[i][r] * qe - aR[i][r] * kr;
        sKW[t * LK + ch] = kr * aW[i][r];
        if (t < nval && ch < K) {
          dk[(row0 + t) * K + ch] = aK[i][r] * L + aR[i][r] * Rr;
          dq[(row0 + t) * K + ch] = scale * aQ[i][r] * L;
        }
      }
    }
  }
  __syncthreads();
  // dg: reverse cumulative sum over the chunk's tokens, from the chunk-end term
  if (tid < KD) {
    const int ch = tid;
    float run = sXS[ch];
    for (int t = 0; t < C; ++t) run += sKW[t * LK + ch];
    for (int t = nval - 1; t >= 0; --t) {
      run += sDG[t * LK + ch];
      if (ch < K) dg[(row0 + t) * K + ch] = run;
    }
  }
  if (tid < nval) dbeta[row0 + tid] = sDB[tid];
}

// The gradients of a token-path chunk: an exact token-by-token reverse from the chunk's
// checkpoint S_c and chunk-end cotangent, for t = last .. first, with the states S_{t-1},
// S_t recomputed from S_c.  One workgroup per (head, group of GTOK chunks) takes the
// group's flagged chunks in turn, so that the launch costs little when none is flagged.
constexpr int GTOK = 16;

template <int KD, int VP>
__global__ void __launch_bounds__(512)
grad_token_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                  const float* __restrict__ z, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                  const float* __restrict__ beta, float scale, const float* __restrict__ d_o,
                  const char* __restrict__ ws, float* __restrict__ dq, float* __restrict__ dk,
                  float* __restrict__ dg, float* __restrict__ dbeta, int H, int T, int K, int V, int nck) {
  using Rc = Rec<KD>;
  constexpr int SMEM = 2 * KD * VP + 4 * KD + 4 * VP + 512 + 4;
  __shared__ __attribute__((aligned(16))) float sm[SMEM];
  const int bh = blockIdx.y, h = bh % H;
  const int tid = threadIdx.x;
  const Layout lo = layout(KD, VP, (long long)gridDim.y, nck);
  float* sS = sm;                               // [KD][VP]: S_{t-1}
  float* sD = sS + KD * VP;                     // [KD][VP]: dS
  float* sAl = sD + KD * VP;                    // alpha_t
  float* sK = sAl + KD;                         // k_t
  float* sQ = sK + KD;                          // scale q_t
  float* sX = sQ + KD;                          // scratch per channel
  float* sVv = sX + KD;                         // v_t
  float* sDo = sVv + VP;                        // do_t
  float* sEv = sDo + VP;                        // e (v_t - S'^T k_t)
  float* sDe = sEv + VP;                        // de
  float* sPc = sDe + VP;                        // column-sum partials [512 / VP][VP]
  float* sBt = sPc + 512;                       // beta_t
  const float gm = gate_multiplier(A_log[h]);
  constexpr int RG = 512 / VP;                  // row groups of the column sums
  constexpr int TPC = 512 / KD;                 // threads per channel of the row sums
  const int cend = min(nck, (int)(blockIdx.x + 1) * GTOK);
  for (int c = blockIdx.x * GTOK; c < cend; ++c) {
    const size_t chunk = (size_t)bh * nck + c;
    const float* rec = reinterpret_cast<const float*>(ws + lo.rec) + chunk * Rc::SIZE;
    if (rec[Rc::FLAG] == 0.0f) continue;       // (uniform over the workgroup)
    const float* ckp = reinterpret_cast<const float*>(ws + lo.ck) + chunk * KD * VP;
    const float* dsep = reinterpret_cast<const float*>(ws + lo.dse) + chunk * KD * VP;
    const int t0 = c * C, nval = min(C, T - t0);
    const size_t row0 = (size_t)bh * T + t0;
    auto load_token = [&](int t) {
      if (tid < KD) {
        const int ch = tid;
        const float db = (dt_bias && ch < K) ? dt_bias[h * K + ch] : 0.0f;
        sAl[ch] = ch < K ? expn(gate_g(z[(row0 + t) * K + ch], db, gm)) : 0.0f;
        sK[ch] = ch < K ? k[(row0 + t) * K + ch] : 0.0f;
        sQ[ch] = ch < K ? scale * q[(row0 + t) * K + ch] : 0.0f;
      }
      if (tid < VP) {
        sVv[tid] = tid < V ? v[(row0 + t) * V + tid] : 0.0f;
        sDo[tid] = tid < V ? d_o[(row0 + t) * V + tid] : 0.0f;
      }
      if (tid == 0) sBt[0] = beta[row0 + t];
      __syncthreads();
    };
    // out[col] = sum over rows of w[row] * f(row, col) for f = mat[row][col] * rowscale[row]
    auto colsum = [&](const float* mat, const float* rscale, float* out) {
      const int col = tid % VP, rg = tid / VP;
      float s = 0.0f;
      for (int r = rg; r < KD; r += RG) s = fmaf(mat[r * VP + col] * rscale[r], sK[r], s);
      sPc[rg * VP + col] = s;
      __syncthreads();
      if (tid < VP) {
        float a = 0.0f;
        for (int g = 0; g < RG; ++g) a += sPc[g * VP + tid];
        out[tid] = a;
      }
      __syncthreads();
    };
    // one token forward on sS with the loaded token: S' = alpha S, e = v - S'^T k, S = S' + beta k e^T
    auto token_fwd = [&]() {
      colsum(sS, sAl, sEv);
      const float bt = sBt[0];
      for (int i = tid; i < KD * VP; i += 512) {
        const int r = i / VP, col = i % VP;
        sS[i] = fmaf(sK[r], bt * (sVv[col] - sEv[col]), sAl[r] * sS[i]);
      }
      __syncthreads();
    };
    __syncthreads();                            // (the previous chunk is done with sD)
    for (int i = tid; i < KD * VP; i += 512) sD[i] = dsep[vt_off(KD, i / VP, i % VP)];
    for (int t = nval - 1; t >= 0; --t) {
      for (int i = tid; i < KD * VP; i += 512) sS[i] = ckp[vt_off(KD, i / VP, i % VP)];
      __syncthreads();
      for (int u = 0; u < t; ++u) {
        load_token(u);
        token_fwd();
      }
      load_token(t);                               // sS = S_{t-1}
      colsum(sS, sAl, sEv);                        // S'^T k
      const float bt = sBt[0];
      if (tid < VP) sEv[tid] = sVv[tid] - sEv[tid];   // e
      __syncthreads();
      // dS += q_hat do^T
      for (int i = tid; i < KD * VP; i += 512) sD[i] = fmaf(sQ[i / VP], sDo[i % VP], sD[i]);
      __syncthreads();
      // row sums over the columns: dq = S_t do, dSe = dS e; thread (row tid / TPC, part tid % TPC)
      {
        const int r = tid / TPC, p = tid % TPC;
        float aq = 0.0f, ae = 0.0f;
        for (int col = p; col < VP; col += TPC) {
          const float st = fmaf(sK[r], bt * sEv[col], sAl[r] * sS[r * VP + col]);
          aq = fmaf(st, sDo[col], aq);
          ae = fmaf(sD[r * VP + col], sEv[col], ae);
        }
        for (int m = 1; m < TPC; m <<= 1) {
          aq += __shfl_xor(aq, m);
          ae += __shfl_xor(ae, m);
        }
        if (p == 0) {
          if (r < K) dq[(row0 + t) * K + r] = scale * aq;
          sX[r] = ae;                              // dS e
        }
      }
      __syncthreads();
      // de = beta dS^T k
      {
        const int col = tid % VP, rg = tid / VP;
        float s = 0.0f;
        for (int r = rg; r < KD; r += RG) s = fmaf(sD[r * VP + col], sK[r], s);
        sPc[rg * VP + col] = s;
        __syncthreads();
        if (tid < VP) {
          float a = 0.0f;
          for (int g = 0; g < RG; ++g) a += sPc[g * VP + tid];
          sDe[tid] = bt * a;
        }
        __syncthreads();
      }
      // dbeta = k . dS e; dk = beta dS e - S' de; dS'' = dS - k de^T; dg = alpha rowsum(dS'' S_{t-1})
      {
        const int r = tid / TPC, p = tid % TPC;
        float a1 = 0.0f, a2 = 0.0f;
        for (int col = p; col < VP; col += TPC) {
          const float sp = sAl[r] * sS[r * VP + col];
          a1 = fmaf(sp, sDe[col], a1);
          const float d2 = fmaf(-sK[r], sDe[col], sD[r * VP + col]);
          a2 = fmaf(d2, sS[r * VP + col], a2);
        }
        for (int m = 1; m < TPC; m <<= 1) {
          a1 += __shfl_xor(a1, m);
          a2 += __shfl_xor(a2, m);
        }
        if (p == 0 && r < K) {
          dk[(row0 + t) * K + r] = bt * sX[r] - a1;
          dg[(row0 + t) * K + r] = sAl[r] * a2;
        }
      }
      if (tid < 64) {
        float x = 0.0f;
        for (int r = tid; r < KD; r += 64) x = fmaf(sK[r], sX[r], x);
        for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
        if (tid == 0) dbeta[row0 + t] = x;
      }
      __syncthreads();
      for (int i = tid; i < KD * VP; i += 512) {
        const int r = i / VP, col = i % VP;
        sD[i] = sAl[r] * fmaf(-sK[r], sDe[col], sD[i]);
      }
      __syncthreads();
    }
  }
}

template <int KD, int VP>
static hipError_t launch_kd_vp(const float* q, const float* k, const float* v, const float* z, const float* A_log,
                               const float* dt_bias, const float* beta, const float* state_in, float scale,
                               const float* d_o, const float* d_state_out, float* dq, float* dk, float* dv, float* dg,
                               float* dbeta, float* dstate_in, char* ws, int B, int H, int T, int K, int V,
                               hipStream_t s) {
  const int BH = B * H;
  const int nck = (T + C - 1) / C;
  const Layout lo = layout(KD, VP, BH, nck);
  hipError_t e;
  if (T > 0) {
    hipLaunchKernelGGL(prep_kernel<KD>, dim3(nck, BH), dim3(256), 0, s, q, k, z, A_log, dt_bias, beta, scale,
                       reinterpret_cast<float*>(ws + lo.rec), H, T, K, nck);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(seq_kernel<KD>, dim3(2 * (VP / 16) * BH), dim3(256), 0, s, q, k, v, z, A_log, dt_bias, beta,
                     state_in, scale, d_o, d_state_out, ws, dv, dstate_in, H, T, K, V, VP, nck, BH);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (T > 0) {
    hipLaunchKernelGGL((grad_kernel<KD, VP>), dim3(nck, BH), dim3(512), 0, s, d_o, ws, scale, dq, dk, dg, dbeta, T,
                       K, V, nck);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((grad_token_kernel<KD, VP>), dim3((nck + GTOK - 1) / GTOK, BH), dim3(512), 0, s, q, k, v, z,
                       A_log, dt_bias, beta, scale, d_o, ws, dq, dk, dg, dbeta, H, T, K, V, nck);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cb

static int cb_kd(int K) { return K <= 16 ? 16 : K <= 32 ? 32 : K <= 64 ? 64 : 128; }
static int cb_vp(int V) { return V <= 32 ? 32 : V <= 64 ? 64 : 128; }

size_t chunk_bwd_mfma_workspace_bytes(int B, int H, int T, int K, int V) {
  if (B < 1 || H < 1 || T < 0) return 0;
  const int nck = (T + cb::C - 1) / cb::C;
  return cb::layout(cb_kd(K), cb_vp(V), (long long)B * H, nck).bytes;
}

hipError_t launch_chunk_bwd_mfma(const float* q, const float* k, const float* v, const float* z, const float* A_log,
                                 const float* dt_bias, const float* beta, const float* state_in, float scale,
                                 const float* d_o, const float* d_state_out, float* dq, float* dk, float* dv,
                                 float* dg, float* dbeta, float* dstate_in, void* workspace, int B, int H, int T,
                                 int K, int V, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
#define CB_CASE(KD_, VP_)                                                                                          \
  if (cb_kd(K) == KD_ && cb_vp(V) == VP_)                                                                          \
    return cb::launch_kd_vp<KD_, VP_>(q, k, v, z, A_log, dt_bias, beta, state_in, scale, d_o, d_state_out, dq, dk, \
                                      dv, dg, dbeta, dstate_in, ws, B, H, T, K, V, s);
  CB_CASE(16, 32) CB_CASE(16, 64) CB_CASE(16, 128)
  CB_CASE(32, 32) CB_CASE(32, 64) CB_CASE(32, 128)
  CB_CASE(64, 32) CB_CASE(64, 64) CB_CASE(64, 128)
  CB_CASE(128, 32) CB_CASE(128, 64) CB_CASE(128, 128)
#undef CB_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
