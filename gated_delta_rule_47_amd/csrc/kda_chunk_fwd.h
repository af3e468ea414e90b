// Fused chunked KDA forward for gfx950.
//
// One workgroup (4 waves) owns one (batch, head, value tile) and walks the sequence
// chunk by chunk, keeping the K x VT fp32 state in MFMA accumulator registers.  Per
// chunk of C tokens it runs, all on chip:
//   E1  gate (g <= 0, log2 units) fused with the loads of q, k, z; block-local
//       decay scans; the decay-weighted operands KE = k*L, QE = q*L, KR = k*R
//   F   per-(16-token block, channel) decay factors
//   E2  W~^T = KE*Gamma0, KD^T = KR*D0 (channel-major), then QGamma = QE*Gamma0
//   AP  A (strictly lower, beta-scaled) and P (lower) = 16x16 tiles on MFMA
//   T   (I + A)^-1: 16x16 diagonal blocks by forward substitution, off-diagonal
//       blocks by block substitution on fp32 MFMA, then T*diag(beta)
//   W   w = T diag(beta) W~          U  U = T diag(beta) V - w S
//   O   o = scale * (QGamma S + P U)  S  S = diag(Gamma_C) S + KD^T U
// The chunk equations are those of the WY form: with G the inclusive cumsum of g,
// A_ij = beta_i <k_i e^(G_i-G_j), k_j>, P_ij = <q_i e^(G_i-G_j), k_j>, and the carry
// decays by e^(G_last - G_j) (the adjoint page, section 2).
//
// Decay factorisation.  Inside a 16-token block the reference point is the block's
// midpoint m (after token 7): L_i = e^(G_i - G_m), R_j = e^(G_m - G_j), so
// L_i R_j = e^(G_i - G_j) and |exponent| <= one half-block of decay.  Every
// exponent is formed as a sum of non-positive g's (no difference of two large
// cumulative sums).  Across blocks J < I the factor F_IJ = e^(G_mI - G_mJ) <= 1 is
// applied per channel to the row operand.  If some half-block decays by more than
// 2^thresh in some channel, L or R could overflow: that chunk is then evaluated
// token by token (exact, slower) instead.
//
// Gate layout: zc = 1 takes z (B,H,T,K) and dt_bias (H,K); zc = 0 is the scalar-decay
// case, z (B,H,T) and dt_bias (H), one gate value per token shared by every channel.
#pragma once

#include "kda_common.h"

namespace kda {

template <typename Tin, int KD_, int VT_, int C_>
struct FwdCfg {
  using Top = Tin;                                   // MFMA operand type
  static constexpr bool BF = sizeof(Tin) == 2;
  static constexpr int KS = Mfma<Top>::KS;
  static constexpr int KD = KD_;                     // padded key dim (multiple of 16 and KS)
  static constexpr int VT = VT_;                     // value columns per workgroup
  static constexpr int C = C_;
  static constexpr int VD = round_up(VT, 16);
  static constexpr int CD = round_up(C, cmax(16, KS));
  static constexpr int NB = C / 16;                  // 16-token blocks per chunk
  static constexpr int NBD = CD / 16;
  static constexpr int NPAIR = cmax(1, NB * (NB - 1) / 2);
  static constexpr int PAD = BF ? 8 : 4;             // row padding: rows start 16 B apart mod 256 B
  static constexpr int LD_TK = KD + PAD;             // [token][channel]
  static constexpr int LD_CT = CD + PAD;             // [channel|value|token][token]
  static constexpr int LD_ST = KD + PAD;             // S^T [value][channel]
  static constexpr int LD_A = CD + 4;                // fp32 [token][token]
  static constexpr int NMT = KD / 16, NNT = VD / 16, NS = NMT * NNT, NSW = (NS + 3) / 4;
  static constexpr int ES = (int)sizeof(Top);
  static constexpr int SZ_TK = CD * LD_TK * ES;
  static constexpr int SZ_KT = KD * LD_CT * ES;
  static constexpr int SZ_VT = VD * LD_CT * ES;
  static constexpr int SZ_TT = CD * LD_CT * ES;
  static constexpr int SZ_A = CD * LD_A * 4;
  static constexpr int SZ_ST = VD * LD_ST * ES;
  static constexpr int N_X = cmax(1024, 3 * KD + VD + NS * 16);
  static constexpr int OFF_KE = 0;                                   // KE, then -w
  static constexpr int OFF_QE = OFF_KE + SZ_TK;                      // QE, then QGamma
  static constexpr int OFF_KR = OFF_QE + SZ_TK;                      // KR, then T diag(beta)
  static constexpr int OFF_WT = OFF_KR + cmax(SZ_TK, SZ_TT);         // W~^T
  static constexpr int OFF_KDT = OFF_WT + SZ_KT;                     // KD^T
  static constexpr int OFF_VT = OFF_KDT + SZ_KT;                     // V^T
  static constexpr int OFF_A = OFF_VT + SZ_VT;                       // A -> T (fp32), then U^T
  static constexpr int OFF_P = OFF_A + cmax(SZ_A, SZ_VT);            // P
  static constexpr int OFF_ST = OFF_P + SZ_TT;                       // S^T
  static constexpr int OFF_X = OFF_ST + SZ_ST;                       // scratch (fp32)
  static constexpr int OFF_BETA = OFF_X + N_X * 4;
  static constexpr int OFF_H1 = OFF_BETA + CD * 4;
  static constexpr int OFF_H2 = OFF_H1 + NB * KD * 4;
  static constexpr int OFF_G0 = OFF_H2 + NB * KD * 4;
  static constexpr int OFF_D0 = OFF_G0 + NB * KD * 4;
  static constexpr int OFF_F = OFF_D0 + NB * KD * 4;
  static constexpr int OFF_GC = OFF_F + NPAIR * KD * 4;
  static constexpr int OFF_FLAG = OFF_GC + KD * 4;                  // per-wave flags
  static constexpr int TOTAL = OFF_FLAG + 16;
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
  static_assert(KD % KS == 0 && KD % 16 == 0 && C % 16 == 0, "tile shape");
  static_assert((SZ_TK | SZ_KT | SZ_VT | SZ_TT | SZ_A | SZ_ST) % 16 == 0, "16-byte alignment");
};

__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }  // J < I

// Store 4 consecutive values (one accumulator column segment) at dst[0..3].
template <typename Top>
__device__ __forceinline__ void store4(Top* dst, floatx4 v, float mul) {
  if constexpr (sizeof(Top) == 2) {
    short4 s;
    s[0] = (short)f2bf(v[0] * mul); s[1] = (short)f2bf(v[1] * mul);
    s[2] = (short)f2bf(v[2] * mul); s[3] = (short)f2bf(v[3] * mul);
    *reinterpret_cast<short4*>(dst) = s;
  } else {
    *reinterpret_cast<floatx4*>(dst) = v * mul;
  }
}

// Store 16 consecutive operand values.
template <typename Top>
__device__ __forceinline__ void store16(Top* dst, const float* v) {
  if constexpr (sizeof(Top) == 2) {
    short8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = (short)f2bf(v[e]); b[e] = (short)f2bf(v[8 + e]); }
    reinterpret_cast<short8*>(dst)[0] = a;
    reinterpret_cast<short8*>(dst)[1] = b;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      reinterpret_cast<floatx4*>(dst)[e] = floatx4{v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]};
  }
}

template <typename Tin, int KD, int VT, int C>
__global__ void __launch_bounds__(256)
chunk_fwd_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
                 const Tin* __restrict__ z, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                 const Tin* __restrict__ beta, const float* state_in, float scale, Tin* __restrict__ o,
                 float* state_out, float* __restrict__ ckpt, int H, int T, int K, int V, int n_vtiles, int total_wg,
                 float thresh, int zc) {
  using Cfg = FwdCfg<Tin, KD, VT, C>;
  using Top = Tin;
  using MM = Mfma<Top>;
  using MF = Mfma<float>;
  constexpr int KS = Cfg::KS, CD = Cfg::CD, VD = Cfg::VD, NB = Cfg::NB, NBD = Cfg::NBD;
  constexpr int LD_TK = Cfg::LD_TK, LD_CT = Cfg::LD_CT, LD_ST = Cfg::LD_ST, LD_A = Cfg::LD_A;
  constexpr int NNT = Cfg::NNT, NS = Cfg::NS, NSW = Cfg::NSW, NMT = Cfg::NMT;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
  Top* sKE = reinterpret_cast<Top*>(smem + Cfg::OFF_KE);
  Top* sW = sKE;
  Top* sQE = reinterpret_cast<Top*>(smem + Cfg::OFF_QE);
  Top* sKR = reinterpret_cast<Top*>(smem + Cfg::OFF_KR);
  Top* sTb = sKR;
  Top* sWT = reinterpret_cast<Top*>(smem + Cfg::OFF_WT);
  Top* sKDT = reinterpret_cast<Top*>(smem + Cfg::OFF_KDT);
  Top* sVT = reinterpret_cast<Top*>(smem + Cfg::OFF_VT);
  float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
  Top* sUT = reinterpret_cast<Top*>(smem + Cfg::OFF_A);
  Top* sP = reinterpret_cast<Top*>(smem + Cfg::OFF_P);
  Top* sST = reinterpret_cast<Top*>(smem + Cfg::OFF_ST);
  float* sX = reinterpret_cast<float*>(smem + Cfg::OFF_X);
  float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_BETA);
  float* sH1 = reinterpret_cast<float*>(smem + Cfg::OFF_H1);
  float* sH2 = reinterpret_cast<float*>(smem + Cfg::OFF_H2);
  float* sG0 = reinterpret_cast<float*>(smem + Cfg::OFF_G0);
  float* sD0 = reinterpret_cast<float*>(smem + Cfg::OFF_D0);
  float* sF = reinterpret_cast<float*>(smem + Cfg::OFF_F);
  float* sGC = reinterpret_cast<float*>(smem + Cfg::OFF_GC);
  int* sFlag = reinterpret_cast<int*>(smem + Cfg::OFF_FLAG);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // Workgroups are dispatched round-robin over the 8 XCDs: place the value tiles
  // of one head on one XCD so that their shared q/k/z reads meet in its L2.
  int p = blockIdx.x;
  if ((total_wg & 7) == 0) p = (blockIdx.x & 7) * (total_wg >> 3) + (blockIdx.x >> 3);
  const int bh = p / n_vtiles;
  const int v0 = (p % n_vtiles) * VT;
  const int h = bh % H;
  const int vcols = min(VT, V - v0);               // valid value columns in this tile

  for (int i = tid; i < Cfg::TOTAL / 16; i += 256) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  const float mult2 = gate_multiplier(A_log[h]) * kLog2e;   // g in log2 units: g2 = -mult2 * softplus
  const bool precise = !Cfg::BF || mult2 > 64.0f * kLog2e;

  // ---------------------------------------------------------------- initial state
  floatx4 sacc[NSW];
#pragma unroll
  for (int i = 0; i < NSW; ++i) {
    sacc[i] = zero4();
    const int tau = wave + 4 * i;
    if (tau < NS && state_in) {
      const int row0 = 16 * (tau / NNT) + 4 * lg, col = 16 * (tau % NNT) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row0 + r < K && col < vcols) sacc[i][r] = state_in[((size_t)bh * K + row0 + r) * V + v0 + col];
    }
  }
  lds_barrier();
  auto write_st = [&]() {
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int tau = wave + 4 * i;
      if (tau < NS) store4<Top>(sST + (16 * (tau % NNT) + l16) * LD_ST + 16 * (tau / NNT) + 4 * lg, sacc[i], 1.0f);
    }
  };
  write_st();
  lds_barrier();

  // Register prefetch of one chunk's raw activations: every load is unconditional
  // (token index clamped to T-1, masked after), so a chunk's loads issue as one batch.
  const int kpairs = K / 2;
  const bool has_k = tid < kpairs * NB;
  const int kc2 = tid % kpairs, kb = tid / kpairs;
  const bool has_v = tid < (VT / 2) * NB;
  const int vc2 = tid % (VT / 2), vb = tid / (VT / 2);
  const int vcol = min(2 * vc2, vcols - 2);     // in-bounds column for every lane
  Pair<Tin> rk[16], rq[16], rz[16], rv[16];
  float rbeta = 0.0f;
  auto prefetch = [&](int tn) {
    const size_t tb = (size_t)bh * T;
    if (has_k) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const size_t a = (tb + min(tn + 16 * kb + t, T - 1)) * K + 2 * kc2;
        rk[t] = Pair<Tin>::load(k + a);
        rq[t] = Pair<Tin>::load(q + a);
        rz[t] = zc ? Pair<Tin>::load(z + a) : Pair<Tin>::dup(z[tb + min(tn + 16 * kb + t, T - 1)]);
      }
    }
    if (has_v) {
#pragma unroll
      for (int t = 0; t < 16; ++t) rv[t] = Pair<Tin>::load(v + (tb + min(tn + 16 * vb + t, T - 1)) * V + v0 + vcol);
    }
    if (tid < C) rbeta = to_f<Tin>(beta[tb + min(tn + tid, T - 1)]);
  };
  if (T > 0) prefetch(0);

  const int nck = (T + C - 1) / C;
  for (int t0 = 0; t0 < T; t0 += C) {
    const int nval = min(C, T - t0);
    const size_t tokbase = (size_t)bh * T + t0;
    if (ckpt) {                                // state at the chunk start, for the adjoint's recompute
#pragma unroll
      for (int i = 0; i < NSW; ++i) {
        const int tau = wave + 4 * i;
        if (tau < NS) {
          const int row0 = 16 * (tau / NNT) + 4 * lg, col = 16 * (tau % NNT) + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row0 + r < K && col < vcols)
              ckpt[(((size_t)bh * nck + t0 / C) * K + row0 + r) * V + v0 + col] = sacc[i][r];
        }
      }
    }

    // ============================================================ E1
    // Thread = (pair of key channels, 16-token block): the gate, the block-local
    // decay scans and the decay-weighted operands, from the registers prefetched
    // during the previous chunk.  Tokens past T are identity tokens (all zero).
    bool bad = false;
    if (has_k) {
      const int c = 2 * kc2, b = kb;
      const float dtb0 = dt_bias ? dt_bias[zc ? h * K + c : h] : 0.0f;
      const float dtb1 = dt_bias ? dt_bias[zc ? h * K + c + 1 : h] : 0.0f;
      float g0[8], g1[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bool ok = 16 * b + t < nval;
        g0[t] = ok ? -mult2 * softplus_f(rz[t].x() + dtb0, precise) : 0.0f;
        g1[t] = ok ? -mult2 * softplus_f(rz[t].y() + dtb1, precise) : 0.0f;
      }
      float a0 = 0.0f, a1 = 0.0f;               // first half: L = e^-(sum_{t<m<=7} g) >= 1
#pragma unroll
      for (int t = 7; t >= 0; --t) {
        const int i = 16 * b + t;
        const bool ok = i < nval;
        const float kx = ok ? rk[t].x() : 0.0f, ky = ok ? rk[t].y() : 0.0f;
        const float qx = ok ? rq[t].x() : 0.0f, qy = ok ? rq[t].y() : 0.0f;
        const float L0 = fast_exp2(-a0), R0 = fast_exp2(a0), L1 = fast_exp2(-a1), R1 = fast_exp2(a1);
        store2<Top>(sKE + i * LD_TK + c, kx * L0, ky * L1);
        store2<Top>(sQE + i * LD_TK + c, qx * L0, qy * L1);
        store2<Top>(sKR + i * LD_TK + c, kx * R0, ky * R1);
        a0 += g0[t];
        a1 += g1[t];
      }
      const float h10 = a0, h11 = a1;
      a0 = 0.0f;
      a1 = 0.0f;                                // second half: L = e^(sum_{8<=m<=t} g) <= 1
#pragma unroll
      for (int t = 8; t < 16; ++t) {
        const int i = 16 * b + t;
        const bool ok = i < nval;
        a0 += ok ? -mult2 * softplus_f(rz[t].x() + dtb0, precise) : 0.0f;
        a1 += ok ? -mult2 * softplus_f(rz[t].y() + dtb1, precise) : 0.0f;
        const float kx = ok ? rk[t].x() : 0.0f, ky = ok ? rk[t].y() : 0.0f;
        const float qx = ok ? rq[t].x() : 0.0f, qy = ok ? rq[t].y() : 0.0f;
        const float L0 = fast_exp2(a0), R0 = fast_exp2(-a0), L1 = fast_exp2(a1), R1 = fast_exp2(-a1);
        store2<Top>(sKE + i * LD_TK + c, kx * L0, ky * L1);
        store2<Top>(sQE + i * LD_TK + c, qx * L0, qy * L1);
        store2<Top>(sKR + i * LD_TK + c, kx * R0, ky * R1);
      }
      sH1[b * KD + c] = h10;
      sH1[b * KD + c + 1] = h11;
      sH2[b * KD + c] = a0;
      sH2[b * KD + c + 1] = a1;
      bad = fminf(fminf(h10, h11), fminf(a0, a1)) < -thresh;
    }
    if (has_v) {                                // V^T rows for two value columns
      const int b = vb;
      float va[16], vb_[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const bool ok = 16 * b + t < nval && 2 * vc2 < vcols;
        va[t] = ok ? rv[t].x() : 0.0f;
        vb_[t] = ok ? rv[t].y() : 0.0f;
      }
      store16<Top>(sVT + (2 * vc2) * LD_CT + 16 * b, va);
      store16<Top>(sVT + (2 * vc2 + 1) * LD_CT + 16 * b, vb_);
    }
    if (tid < C) sBeta[tid] = tid < nval ? rbeta : 0.0f;
    if (t0 + C < T) prefetch(t0 + C);           // next chunk's loads overlap this chunk's work
    const unsigned long long ballot = __ballot(bad);
    if (lane == 0) sFlag[wave] = ballot != 0ull;
    lds_barrier();
    const int slow = sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3];

    if (slow) {
      // ========================================================== token-by-token chunk
      float* sAl = sX;
      float* sKk = sX + KD;
      float* sQq = sX + 2 * KD;
      float* sVv = sX + 3 * KD;
      float* sRed = sVv + VD;                 // [tile][16] partial column sums
      for (int i = 0; i < nval; ++i) {
        const size_t tok = tokbase + i;
        for (int c = tid; c < KD; c += 256) {
          if (c < K) {
            const float dtb = dt_bias ? dt_bias[zc ? h * K + c : h] : 0.0f;
            sAl[c] = fast_exp2(-mult2 * softplus_f(to_f<Tin>(z[zc ? tok * K + c : tok]) + dtb, true));
            sKk[c] = to_f<Tin>(k[tok * K + c]);
            sQq[c] = scale * to_f<Tin>(q[tok * K + c]);
          } else {
            sAl[c] = 0.0f; sKk[c] = 0.0f; sQq[c] = 0.0f;
          }
        }
        for (int vv = tid; vv < VD; vv += 256) sVv[vv] = vv < vcols ? to_f<Tin>(v[tok * V + v0 + vv]) : 0.0f;
        const float bt = to_f<Tin>(beta[tok]);
        lds_barrier();
#pragma unroll
        for (int j = 0; j < NSW; ++j) {        // S' = diag(alpha) S; partial S'^T k
          const int tau = wave + 4 * j;
          if (tau < NS) {
            const int row0 = 16 * (tau / NNT) + 4 * lg;
            float pr = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) { sacc[j][r] *= sAl[row0 + r]; pr += sacc[j][r] * sKk[row0 + r]; }
            pr += __shfl_xor(pr, 16);
            pr += __shfl_xor(pr, 32);
            if (lane < 16) sRed[tau * 16 + l16] = pr;
          }
        }
        lds_barrier();
        float po[NSW];
#pragma unroll
        for (int j = 0; j < NSW; ++j) {        // S += beta k (v - r)^T; partial S^T q_hat
          const int tau = wave + 4 * j;
          po[j] = 0.0f;
          if (tau < NS) {
            const int nt = tau % NNT, row0 = 16 * (tau / NNT) + 4 * lg;
            float rc = 0.0f;
            for (int mt = 0; mt < NMT; ++mt) rc += sRed[(mt * NNT + nt) * 16 + l16];
            const float e = sVv[16 * nt + l16] - rc;
            float pq = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) { sacc[j][r] += bt * sKk[row0 + r] * e; pq += sacc[j][r] * sQq[row0 + r]; }
            pq += __shfl_xor(pq, 16);
            pq += __shfl_xor(pq, 32);
            po[j] = pq;
          }
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
          const int tau = wave + 4 * j;
          if (tau < NS && lane < 16) sRed[tau * 16 + l16] = po[j];
        }
        lds_barrier();
        if (tid < vcols && o) {
          const int nt = tid / 16;
          float ov = 0.0f;
          for (int mt = 0; mt < NMT; ++mt) ov += sRed[(mt * NNT + nt) * 16 + (tid & 15)];
          o[tok * V + v0 + tid] = from_f<Tin>(ov);
        }
        lds_barrier();
      }
      write_st();
      lds_barrier();
      continue;
    }

    // ============================================================ F: block factors
    for (int c = tid; c < K; c += 256) {
      float h1v[NB], h2v[NB], tot[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        h1v[b] = sH1[b * KD + c];
        h2v[b] = sH2[b * KD + c];
        tot[b] = h1v[b] + h2v[b];
      }
      float pre = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) { sG0[b * KD + c] = fast_exp2(pre + h1v[b]); pre += tot[b]; }
      sGC[c] = fast_exp2(pre);
      float suf = 0.0f;
#pragma unroll
      for (int b = NB - 1; b >= 0; --b) { sD0[b * KD + c] = fast_exp2(h2v[b] + suf); suf += tot[b]; }
#pragma unroll
      for (int I = 1; I < NB; ++I)
#pragma unroll
        for (int J = 0; J < I; ++J) {
          float ex = h2v[J] + h1v[I];
#pragma unroll
          for (int m = J + 1; m < I; ++m) ex += tot[m];
          sF[pair_index(I, J) * KD + c] = fast_exp2(ex);
        }
    }
    lds_barrier();

    // ============================================================ E2a + AP
    for (int item = tid; item < K * NB; item += 256) {
      const int c = item % K, b = item / K;
      const float g0 = sG0[b * KD + c], d0 = sD0[b * KD + c];
      float wv[16], kdv[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int i = 16 * b + t;
        wv[t] = to_f<Top>(sKE[i * LD_TK + c]) * g0;
        kdv[t] = to_f<Top>(sKR[i * LD_TK + c]) * d0;
      }
      store16<Top>(sWT + c * LD_CT + 16 * b, wv);
      store16<Top>(sKDT + c * LD_CT + 16 * b, kdv);
    }
    {
      constexpr int NTA = NBD * NBD;
      constexpr int NTP = NB * (NB + 1) / 2;
      for (int task = wave; task < NTA + NTP; task += 4) {
        int I, J;
        const bool isA = task < NTA;
        if (isA) {
          I = task / NBD;
          J = task % NBD;
        } else {
          int pp = task - NTA;
          I = 0;
          while (pp > I) { pp -= I + 1; ++I; }
          J = pp;
        }
        floatx4 acc = zero4();
        const bool live = I < NB && J <= I;
        if (live) {
          const Top* src = isA ? sKE : sQE;
#pragma unroll
          for (int s = 0; s < KD / KS; ++s) {
            typename MM::frag a = MM::load(src, LD_TK, 16 * I, s * KS, lane);
            if (J < I) a = MM::scale(a, sF + pair_index(I, J) * KD, s * KS, lane);
            acc = MM::mma(a, MM::load(sKR, LD_TK, 16 * J, s * KS, lane), acc);
          }
        }
        const int j = 16 * J + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * lg + r;
          if (isA) sA[i * LD_A + j] = (live && j < i) ? sBeta[i] * acc[r] : 0.0f;
          else sP[i * LD_CT + j] = from_f<Top>(j <= i ? acc[r] : 0.0f);
        }
      }
    }
    lds_barrier();

    // ============================================================ E2b + diagonal inverses
    for (int item = tid; item < K * NB; item += 256) {
      const int c = item % K, b = item / K;
      const float g0 = sG0[b * KD + c];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        Top* e = sQE + (16 * b + t) * LD_TK + c;
        *e = from_f<Top>(to_f<Top>(*e) * g0);
      }
    }
    if (wave < NB && lane < 16) {
      const int I = wave, j = lane;
      float tcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* arow = sA + (16 * I + i) * LD_A + 16 * I;
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc += arow[m] * tcol[m];
        tcol[i] = (i == j) ? 1.0f : (i > j ? -acc : 0.0f);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sA[(16 * I + i) * LD_A + 16 * I + j] = tcol[i];
    }
    lds_barrier();

    // ============================================================ off-diagonal T blocks
#pragma unroll
    for (int I = 1; I < NB; ++I) {
      if (wave < I) {                          // X_J = sum_{M=J}^{I-1} A_IM T_MJ
        const int J = wave;
        floatx4 acc = zero4();
        for (int M = J; M < I; ++M)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = MF::mma(sA[(16 * I + l16) * LD_A + 16 * M + 4 * s + lg],
                          sA[(16 * M + 4 * s + lg) * LD_A + 16 * J + l16], acc);
        float* X = sX + wave * 256;
#pragma unroll
        for (int r = 0; r < 4; ++r) X[(4 * lg + r) * 16 + l16] = acc[r];
      }
      lds_barrier();
      if (wave < I) {                          // T_IJ = -T_II X_J
        const int J = wave;
        const float* X = sX + wave * 256;
        floatx4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = MF::mma(sA[(16 * I + l16) * LD_A + 16 * I + 4 * s + lg], X[(4 * s + lg) * 16 + l16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sA[(16 * I + 4 * lg + r) * LD_A + 16 * J + l16] = -acc[r];
      }
      lds_barrier();
    }
    for (int idx = tid; idx < CD * CD; idx += 256) {      // T diag(beta)
      const int i = idx / CD, j = idx % CD;
      sTb[i * LD_CT + j] = from_f<Top>(sA[i * LD_A + j] * sBeta[j]);
    }
    lds_barrier();

    // ============================================================ W: -w = -(T diag(beta)) W~
    {
      constexpr int NKT = KD / 16;
      for (int task = wave; task < NB * NKT; task += 4) {
        const int I = task / NKT, n = task % NKT;
        const int ns = (16 * (I + 1) + KS - 1) / KS;
        floatx4 acc = zero4();
        for (int s = 0; s < ns; ++s)
          acc = MM::mma(MM::load(sTb, LD_CT, 16 * I, s * KS, lane), MM::load(sWT, LD_CT, 16 * n, s * KS, lane), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) sW[(16 * I + 4 * lg + r) * LD_TK + 16 * n + l16] = from_f<Top>(-acc[r]);
      }
    }
    lds_barrier();

    // ============================================================ U = T diag(beta) V - w S   (stored as U^T)
    for (int task = wave; task < NBD * NNT; task += 4) {
      const int I = task / NNT, n = task % NNT;
      floatx4 acc = zero4();
      if (I < NB) {
        const int ns = (16 * (I + 1) + KS - 1) / KS;
        for (int s = 0; s < ns; ++s)
          acc = MM::mma(MM::load(sTb, LD_CT, 16 * I, s * KS, lane), MM::load(sVT, LD_CT, 16 * n, s * KS, lane), acc);
#pragma unroll
        for (int s = 0; s < KD / KS; ++s)
          acc = MM::mma(MM::load(sW, LD_TK, 16 * I, s * KS, lane), MM::load(sST, LD_ST, 16 * n, s * KS, lane), acc);
      }
      store4<Top>(sUT + (16 * n + l16) * LD_CT + 16 * I + 4 * lg, acc, 1.0f);
    }
    lds_barrier();

    // ============================================================ O and the state update
    for (int task = wave; task < NB * NNT; task += 4) {
      const int I = task / NNT, n = task % NNT;
      floatx4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KD / KS; ++s)
        acc = MM::mma(MM::load(sQE, LD_TK, 16 * I, s * KS, lane), MM::load(sST, LD_ST, 16 * n, s * KS, lane), acc);
      const int ns = (16 * (I + 1) + KS - 1) / KS;
      for (int s = 0; s < ns; ++s)
        acc = MM::mma(MM::load(sP, LD_CT, 16 * I, s * KS, lane), MM::load(sUT, LD_CT, 16 * n, s * KS, lane), acc);
      const int col = 16 * n + l16;
      if (col < vcols && o) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * lg + r;
          if (i < nval) o[(tokbase + i) * V + v0 + col] = from_f<Tin>(scale * acc[r]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int tau = wave + 4 * i;
      if (tau < NS) {
        const int mt = tau / NNT, nt = tau % NNT;
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[i][r] *= sGC[16 * mt + 4 * lg + r];
#pragma unroll
        for (int s = 0; s < CD / KS; ++s)
          sacc[i] = MM::mma(MM::load(sKDT, LD_CT, 16 * mt, s * KS, lane), MM::load(sUT, LD_CT, 16 * nt, s * KS, lane),
                            sacc[i]);
      }
    }
    lds_barrier();
    write_st();
    lds_barrier();
  }

  if (state_out) {
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int tau = wave + 4 * i;
      if (tau < NS) {
        const int row0 = 16 * (tau / NNT) + 4 * lg, col = 16 * (tau % NNT) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (row0 + r < K && col < vcols) state_out[((size_t)bh * K + row0 + r) * V + v0 + col] = sacc[i][r];
      }
    }
  }
}

template <typename Tin, int KD, int VT, int C>
hipError_t launch_chunk_fwd_inst(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                 const float* dt_bias, const void* beta, const float* state_in, float scale, void* o,
                                 float* state_out, float* ckpt, int B, int H, int T, int K, int V, int zc,
                                 hipStream_t s) {
  const int nvt = (V + VT - 1) / VT;
  const int total = B * H * nvt;
  const float thresh = sizeof(Tin) == 2 ? 64.0f : 24.0f;
  hipLaunchKernelGGL((chunk_fwd_kernel<Tin, KD, VT, C>), dim3(total), dim3(256), 0, s, (const Tin*)q,
                     (const Tin*)k, (const Tin*)v, (const Tin*)z, A_log, dt_bias, (const Tin*)beta, state_in, scale,
                     (Tin*)o, state_out, ckpt, H, T, K, V, nvt, total, thresh, zc);
  return hipGetLastError();
}

}  // namespace kda
