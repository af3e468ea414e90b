// Pipelined chunked KDA forward for bf16 activations on gfx950.
//
// One workgroup of 8 waves owns one (batch, head, value tile of <= 64 columns) and
// walks the sequence in blocks of C <= 32 tokens.  The work of a block splits into
//   K-side: the gate and block-local decay scans, the decay-weighted operands, the
//           strictly-lower A and the lower P (MFMA), T = (I + A)^-1;
//   V-side: Y = V - W~ S, U = T diag(beta) Y, o = scale (QGamma S + P U),
//           S = diag(Gamma_C) S + KD^T U.
// (U = T diag(beta) (V - W~ S) is the u - w S of the WY form with the product w = T
// diag(beta) W~ folded into the state-dependent side, which removes one token x
// channel product from the serial part of the walk.)  Only the V-side depends on the
// state.  Each step of the walk runs
//   phase 1: waves 0-3 compute the gate/scan/operands of block c+1 (VALU) while waves
//            4-7 run the V-side of block c (MFMA), each owning 16 value columns and all
//            K rows of the fp32 state in accumulator registers;
//   phase 2: the A/P tiles (7 waves), then T (wave 0), for block c+1.
// Operands written in phase 1 and read by the V-side are double-buffered in LDS.
//
// Activations reach LDS by buffer-to-LDS DMA (16 bytes per lane, 1 KB per instruction),
// issued by waves 0-3 two blocks ahead for q, k, z and one block ahead for v, into
// double-buffered staging areas; no activation passes through registers on its way in.
// q, k, z keep their [token][channel] rows, with the 16-byte chunks of each row
// permuted (XOR by the row's 8-token group) so that the K-side lanes -- one channel
// pair and 8 consecutive tokens each -- read them without bank conflicts.
//
// The V-side chains MFMA results into MFMAs without LDS: a 32-deep contraction over two
// 16-row accumulator tiles is fed with lane l supplying depth {4g..4g+3} of the first
// tile and {16+4g..16+4g+3} of the second (g = l/16) -- exactly the rows its
// accumulators hold -- and the LDS operand of the same product is read with the same
// depth order.  The sum over depth does not depend on its order.  The same registers
// serve as A or as B operand, so a product can be computed transposed when that makes
// its result layout the one the next step (or the global store) wants.
//
// Decay factors follow the block-midpoint factorisation of the single-wave-group kernel
// (kda_chunk_fwd.h): every L, R, Gamma0, D0 and F factor is 2^x with |x| bounded by one
// half-block of decay; a block whose half-block decay exceeds 2^thresh is evaluated
// token by token by the V-side waves instead.
#pragma once

#include <type_traits>

#include "kda_common.h"

namespace kda {

template <int KD_, int VT_, int C_>
struct PcCfg {
  static constexpr int KD = KD_, VT = VT_, C = C_;
  static constexpr int CD = 32;                       // token depth of every token contraction
  static constexpr int NB = C / 16;
  static constexpr int VD = round_up(VT, 16);
  static constexpr int NNT = VD / 16;                 // value-column tiles = active V-side waves
  static constexpr int NMT = KD / 16;                 // key-row tiles of the state
  static constexpr int LD_TK = KD + 8;                // [token][channel] bf16
  static constexpr int LD_CT = CD + 8;                // [channel|token][token] bf16
  static constexpr int LD_A = CD + 4;                 // [token][token] fp32
  static constexpr int SZ_TK = CD * LD_TK * 2;
  static constexpr int SZ_KT = KD * LD_CT * 2;
  static constexpr int SZ_TT = CD * LD_CT * 2;
  // staging of raw activations (DMA targets)
  static constexpr int RAW_T = CD * KD * 2;           // one tensor: 32 rows of KD channels
  static constexpr int RAW_BUF = 3 * RAW_T;           // k, q, z
  static constexpr int QKZ_DMA = C * KD / 512;        // 1 KB DMA instructions per tensor and block
  static constexpr int VRAW_BUF = NNT * 1024;         // per value tile: 32 rows x 16 columns
  // working buffers (written in phase 1 for block c+1, read in phase 2)
  static constexpr int OFF_KE = 0;
  static constexpr int OFF_QE = OFF_KE + SZ_TK;
  static constexpr int OFF_KR = OFF_QE + SZ_TK;
  static constexpr int OFF_KRF = OFF_KR + SZ_TK;      // F_10 * KR of tokens 0..15
  static constexpr int OFF_A = OFF_KRF + 16 * LD_TK * 2;   // A, then T (fp32)
  static constexpr int OFF_X = OFF_A + CD * LD_A * 4; // 16x16 fp32 scratch
  // phase-2 outputs, read by the V-side in the next phase 1
  static constexpr int OFF_P = OFF_X + 256 * 4;
  static constexpr int OFF_T = OFF_P + SZ_TT;
  // phase-1 outputs, double-buffered: -W~, QGamma, KD^T, Gamma_C, beta
  static constexpr int SET_WN = 0;
  static constexpr int SET_QG = SET_WN + SZ_TK;
  static constexpr int SET_KDT = SET_QG + SZ_TK;
  static constexpr int SET_GC = SET_KDT + SZ_KT;
  static constexpr int SET_BETA = SET_GC + KD * 4;
  static constexpr int SET_BYTES = SET_BETA + CD * 4;
  static constexpr int OFF_SET = OFF_T + SZ_TT;
  static constexpr int OFF_RAW = OFF_SET + 2 * SET_BYTES;
  static constexpr int OFF_VRAW = OFF_RAW + 2 * RAW_BUF;
  static constexpr int OFF_FLAG = OFF_VRAW + 2 * VRAW_BUF;
  static constexpr int TOTAL = OFF_FLAG + 64;
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
  static_assert(KD % 32 == 0 && (C == 16 || C == 32) && NNT <= 4, "tile shape");
  static_assert(OFF_SET % 16 == 0 && SET_BYTES % 16 == 0 && OFF_A % 16 == 0 && OFF_RAW % 16 == 0 &&
                    RAW_T % 1024 == 0 && OFF_VRAW % 16 == 0,
                "16-byte alignment");
  // position of the 16-byte channel chunk ch16 in staging row r
  static __device__ __forceinline__ int swz(int r) { return (4 * ((r >> 3) & 3)) & (KD / 8 - 1); }
};

// A operand rows [row0, row0+16) with the accumulator-compatible depth order over
// [d0, d0+32): lane slots 0..3 = depth d0+4g.., slots 4..7 = depth d0+16+4g..
__device__ __forceinline__ short8 lds_a_perm(const bf16_t* base, int ld, int row0, int d0, int lane) {
  const bf16_t* p = base + (row0 + (lane & 15)) * ld + d0 + 4 * (lane >> 4);
  const short4 a = *reinterpret_cast<const short4*>(p);
  const short4 b = *reinterpret_cast<const short4*>(p + 16);
  return short8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Operand built from two accumulator tiles (depth rows 0..15 and 16..31).
__device__ __forceinline__ short8 acc_perm(floatx4 x0, floatx4 x1) {
  const uint32_t a = pack_bf16x2(x0[0], x0[1]), b = pack_bf16x2(x0[2], x0[3]);
  const uint32_t c = pack_bf16x2(x1[0], x1[1]), d = pack_bf16x2(x1[2], x1[3]);
  return __builtin_bit_cast(short8, uint4{a, b, c, d});
}

__device__ __forceinline__ floatx4 mfma_bf16(short8 a, short8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ short8 lds_frag(const bf16_t* base, int ld, int rc0, int k0, int lane) {
  return *reinterpret_cast<const short8*>(base + (rc0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ void store4_bf16(bf16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// Keep the compiler from moving instructions across this point: used to issue a
// batch of LDS operand loads before the MFMAs that consume them.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// 16 bytes per lane from buffer offset `off` into LDS at lds + 16 * lane (lds must be
// the same for the whole wave).  Offsets past the buffer's range deliver zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (here: its DMAs and
// loads) have completed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Values of `a` held by the lanes 16*j + (lane % 16), j = 0..3, delivered to every lane
// (two permlane swaps, no LDS).
__device__ __forceinline__ void row_gather(float a, float* H) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  const auto p0 = __builtin_amdgcn_permlane32_swap(r16[0], r16[0], false, false);
  const auto p1 = __builtin_amdgcn_permlane32_swap(r16[1], r16[1], false, false);
  H[0] = __uint_as_float(p0[0]);
  H[1] = __uint_as_float(p1[0]);
  H[2] = __uint_as_float(p0[1]);
  H[3] = __uint_as_float(p1[1]);
}

template <int KD, int VT, int C>
__global__ void __launch_bounds__(512)
chunk_fwd_pc_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                    const bf16_t* __restrict__ z, const float* __restrict__ A_log,
                    const float* __restrict__ dt_bias, const bf16_t* __restrict__ beta,
                    const float* state_in, float scale, bf16_t* __restrict__ o, float* state_out, int H, int T,
                    int K, int V, int n_vtiles, int total_wg, float thresh) {
  using Cfg = PcCfg<KD, VT, C>;
  constexpr int CD = Cfg::CD, NB = Cfg::NB, NNT = Cfg::NNT, NMT = Cfg::NMT;
  constexpr int LD_TK = Cfg::LD_TK, LD_CT = Cfg::LD_CT, LD_A = Cfg::LD_A;
  constexpr int NS = KD / 32;                         // 32-deep channel slices

  __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
  bf16_t* sKE = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KE);
  bf16_t* sQE = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_QE);
  bf16_t* sKR = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KR);
  bf16_t* sKRF = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KRF);
  float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
  float* sX = reinterpret_cast<float*>(smem + Cfg::OFF_X);
  bf16_t* sP = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_P);
  bf16_t* sT = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_T);
  int* sFlag = reinterpret_cast<int*>(smem + Cfg::OFF_FLAG);   // [set][wave]
  auto set_base = [&](int set) __attribute__((always_inline)) { return smem + Cfg::OFF_SET + set * Cfg::SET_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

  int p = blockIdx.x;
  if ((total_wg & 7) == 0) p = (blockIdx.x & 7) * (total_wg >> 3) + (blockIdx.x >> 3);
  const int bh = p / n_vtiles;
  const int v0 = (p % n_vtiles) * VT;
  const int h = bh % H;
  const int vcols = min(VT, V - v0);
  const size_t tb = (size_t)bh * T;

  for (int i = tid; i < Cfg::TOTAL / 16; i += 512) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  const float mult2 = gate_multiplier(A_log[h]) * kLog2e;
  const bool precise = mult2 > 64.0f * kLog2e;

  const bool kwave = wave < 4;
  const int vw = wave - 4;
  const bool vact = !kwave && vw < NNT;

  // ------------------------------------------------------------------ K-side lane roles
  const int pair = 16 * (wave & 3) + l16;                  // key-channel pair (K-waves)
  const int hb = g;                                        // 8-token half-block
  const bool kact = kwave && 2 * pair < K;
  const float dtb0 = (kact && dt_bias) ? dt_bias[h * K + 2 * pair] : 0.0f;
  const float dtb1 = (kact && dt_bias) ? dt_bias[h * K + 2 * pair + 1] : 0.0f;
  // per-head buffer resources: offsets past the head's T tokens read as 0
  const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(k + tb * K, (unsigned)(T * K * 2));
  const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + tb * K, (unsigned)(T * K * 2));
  const __amdgpu_buffer_rsrc_t rs_z = make_rsrc(z + tb * K, (unsigned)(T * K * 2));
  const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(v + tb * V, (unsigned)(T * V * 2));
  const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(beta + tb, (unsigned)(T * 2));
  constexpr unsigned kOOB = 0xFFFFFFF0u;                   // an offset past any range: zeros

  // DMA of q, k, z rows [tn, tn + C) into staging buffer rb (K-waves; wave w issues
  // instructions j = w, w + 4, ... of each tensor).  Instruction j of a tensor fills rows
  // [j*512/KD, (j+1)*512/KD); lane l fills the chunk at position l % (KD/8) of row
  // j*512/KD + l/(KD/8) with channel chunk (position ^ swz(row)).
  auto dma_qkz = [&](int tn, int rb) __attribute__((always_inline)) {
    char* base = smem + Cfg::OFF_RAW + rb * Cfg::RAW_BUF;
    for (int j = wave; j < Cfg::QKZ_DMA; j += 4) {
      const int s = j * 64 + lane;
      const int r = s / (KD / 8), pos = s % (KD / 8);
      const int ch = 8 * (pos ^ Cfg::swz(r));
      const unsigned off = ch < K ? (unsigned)(((tn + r) * K + ch) * 2) : kOOB;
      dma16(rs_k, base + j * 1024, off);
      dma16(rs_q, base + Cfg::RAW_T + j * 1024, off);
      dma16(rs_z, base + 2 * Cfg::RAW_T + j * 1024, off);
    }
  };
  // DMA of the value tile of rows [tn, tn + C) into staging buffer rb: wave w < NNT
  // fills slot 2*row + half of tile w with columns v0 + 16w + 8*half .. + 8.
  auto dma_v = [&](int tn, int rb) __attribute__((always_inline)) {
    if (wave < NNT) {
      const int r = lane >> 1, c0 = 16 * wave + 8 * (lane & 1);
      const unsigned off = (r < C && c0 < vcols) ? (unsigned)(((tn + r) * V + v0 + c0) * 2) : kOOB;
      dma16(rs_v, smem + Cfg::OFF_VRAW + rb * Cfg::VRAW_BUF + wave * 1024, off);
    }
  };
  bf16_t rbeta = 0;
  auto load_beta = [&](int tn) __attribute__((always_inline)) {
    if (kwave && tid < C) rbeta = __builtin_amdgcn_raw_buffer_load_b16(rs_b, (unsigned)((tn + tid) * 2), 0, 0);
  };

  // ------------------------------------------------------------------ phase 1, K-side
  auto e1 = [&](auto precise_tag, int tn, int set) __attribute__((always_inline)) {
    constexpr bool PRECISE = decltype(precise_tag)::value;
    const int nval = min(C, T - tn);
    char* sb = set_base(set);
    bf16_t* sWN = reinterpret_cast<bf16_t*>(sb + Cfg::SET_WN);
    bf16_t* sQG = reinterpret_cast<bf16_t*>(sb + Cfg::SET_QG);
    bf16_t* sKDT = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KDT);
    float* sGC = reinterpret_cast<float*>(sb + Cfg::SET_GC);
    float* sBeta = reinterpret_cast<float*>(sb + Cfg::SET_BETA);
    // raw k, q, z of channel pair `pair`, tokens 8hb..8hb+7 (staging buffer of this block)
    Pair<bf16_t> rk[8], rq[8], rz[8];
    if (kact) {
      const char* rbase = smem + Cfg::OFF_RAW + ((tn / C) & 1) * Cfg::RAW_BUF + (8 * hb) * KD * 2 +
                          ((pair >> 2) ^ Cfg::swz(8 * hb)) * 16 + (pair & 3) * 4;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        rk[t].u = *reinterpret_cast<const uint32_t*>(rbase + t * KD * 2);
        rq[t].u = *reinterpret_cast<const uint32_t*>(rbase + Cfg::RAW_T + t * KD * 2);
        rz[t].u = *reinterpret_cast<const uint32_t*>(rbase + 2 * Cfg::RAW_T + t * KD * 2);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) rk[t].u = rq[t].u = rz[t].u = 0u;
    }
    // gate in log2 units, for every staged token (rows past T hold 0: finite)
    float gx[8], gy[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      gx[t] = -mult2 * softplus_f(rz[t].x() + dtb0, PRECISE);
      gy[t] = -mult2 * softplus_f(rz[t].y() + dtb1, PRECISE);
    }
    if (nval < CD) {                       // wave-uniform: a partial block, or C = 16
      const int lim = nval - 8 * hb;       // tokens at or past nval act as identity tokens
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bool ok = t < lim;
        gx[t] = ok ? gx[t] : 0.0f;
        gy[t] = ok ? gy[t] : 0.0f;
        rk[t].u = ok ? rk[t].u : 0u;
        rq[t].u = ok ? rq[t].u : 0u;
      }
    }
    // inclusive prefix over the lane's 8 tokens
    float px[8], py[8];
    float ax = 0.0f, ay = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      ax += gx[t];
      ay += gy[t];
      px[t] = ax;
      py[t] = ay;
    }
    // the four half-block sums of this channel pair (lanes l16 + 16*hb')
    float Hx[4], Hy[4];
    row_gather(ax, Hx);
    row_gather(ay, Hy);
    const int b = hb >> 1;
    const bool first = (hb & 1) == 0;
    const float G0x = fast_exp2(b ? Hx[0] + Hx[1] + Hx[2] : Hx[0]);   // chunk start -> block midpoint
    const float G0y = fast_exp2(b ? Hy[0] + Hy[1] + Hy[2] : Hy[0]);
    const float D0x = fast_exp2(b ? Hx[3] : Hx[1] + Hx[2] + Hx[3]);   // block midpoint -> chunk end
    const float D0y = fast_exp2(b ? Hy[3] : Hy[1] + Hy[2] + Hy[3]);
    const float F0x = fast_exp2(Hx[1] + Hx[2]), F0y = fast_exp2(Hy[1] + Hy[2]);   // midpoint 0 -> midpoint 1
    if (kact) {
      const int c = 2 * pair;
      float kdx[8], kdy[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float ex = first ? px[t] - ax : px[t], ey = first ? py[t] - ay : py[t];
        const float Lx = fast_exp2(ex), Ly = fast_exp2(ey), Rx = fast_exp2(-ex), Ry = fast_exp2(-ey);
        const float kx = rk[t].x(), ky = rk[t].y(), qx = rq[t].x(), qy = rq[t].y();
        const int j = 8 * hb + t;
        const float kex = kx * Lx, key = ky * Ly, qex = qx * Lx, qey = qy * Ly, krx = kx * Rx, kry = ky * Ry;
        store2<bf16_t>(sKE + j * LD_TK + c, kex, key);
        store2<bf16_t>(sQE + j * LD_TK + c, qex, qey);
        store2<bf16_t>(sKR + j * LD_TK + c, krx, kry);
        store2<bf16_t>(sQG + j * LD_TK + c, qex * G0x, qey * G0y);
        store2<bf16_t>(sWN + j * LD_TK + c, -kex * G0x, -key * G0y);
        if (NB == 2 && hb < 2) store2<bf16_t>(sKRF + j * LD_TK + c, krx * F0x, kry * F0y);
        kdx[t] = krx * D0x;
        kdy[t] = kry * D0y;
      }
      auto st8 = [](bf16_t* dst, const float* x) {
        *reinterpret_cast<uint4*>(dst) = uint4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                               pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      };
      st8(sKDT + c * LD_CT + 8 * hb, kdx);
      st8(sKDT + (c + 1) * LD_CT + 8 * hb, kdy);
      if (hb == 0) *reinterpret_cast<float2*>(sGC + c) = float2{fast_exp2(Hx[0] + Hx[1] + Hx[2] + Hx[3]),
                                                                fast_exp2(Hy[0] + Hy[1] + Hy[2] + Hy[3])};
    }
    if (kwave && tid < CD) sBeta[tid] = tid < nval ? bf2f(rbeta) : 0.0f;
    const bool bad = kact && fminf(ax, ay) < -thresh;
    const unsigned long long bal = __ballot(bad);
    if (lane == 0) sFlag[set * 8 + wave] = bal != 0ull;
  };

  // ------------------------------------------------------------------ phase 2 (all waves)
  // Ends before the workgroup barrier that closes the step.
  auto phase2 = [&](int set) __attribute__((always_inline)) {
    const float* sBeta = reinterpret_cast<const float*>(set_base(set) + Cfg::SET_BETA);
    // A (strictly lower, beta-scaled, fp32) and P (lower, bf16), one 16x16 tile per
    // wave, computed transposed: lane (g, l16) holds row i = 16I + l16, columns
    // 16J + 4g.., so each lane stores 4 consecutive columns of one row.
    if (wave < 7) {
      const bool isA = wave < 4;
      const int I = isA ? (wave >> 1) : (wave == 4 ? 0 : 1);
      const int J = isA ? (wave & 1) : (wave == 6 ? 1 : 0);
      const bool live = I < NB && J <= I;
      floatx4 acc = zero4();
      if (live) {
        const bf16_t* rows = (J < I) ? sKRF : sKR + 16 * J * LD_TK;   // column tokens j (F-scaled across blocks)
        const bf16_t* cols = isA ? sKE : sQE;
        short8 fa[NS], fb[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          fa[s] = lds_frag(rows, LD_TK, 0, 32 * s, lane);
          fb[s] = lds_frag(cols, LD_TK, 16 * I, 32 * s, lane);
        }
        sched_fence();
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = mfma_bf16(fa[s], fb[s], acc);
      }
      const int i = 16 * I + l16, j0 = 16 * J + 4 * g;
      float vals[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vals[r] = live && (isA ? j0 + r < i : j0 + r <= i) ? acc[r] : 0.0f;
      if (isA) {
        const float bi = sBeta[i];
        *reinterpret_cast<floatx4*>(sA + i * LD_A + j0) = floatx4{bi * vals[0], bi * vals[1], bi * vals[2], bi * vals[3]};
      } else if (live) {
        store4_bf16(sP + i * LD_CT + j0, vals[0], vals[1], vals[2], vals[3]);
      }
    }
    lds_barrier();
    if (wave == 0) {
      // diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution: lane (I, j)
      // holds column j of block I in registers; row i needs rows < i only.  The
      // strictly-lower rows are loaded up front so that the substitution waits on
      // LDS a few times rather than once per row.
      if (lane < 16 * NB) {
        const int I = lane >> 4, j = lane & 15;
        float* Ab = sA + 16 * I * LD_A + 16 * I;
        floatx4 ra[36];                                     // rows 1..15, columns < row, in float4 groups
#pragma unroll
        for (int i = 1, n = 0; i < 16; ++i)
#pragma unroll
          for (int qd = 0; qd < (i + 3) / 4; ++qd, ++n) ra[n] = *reinterpret_cast<const floatx4*>(Ab + i * LD_A + 4 * qd);
        float t[16];
        t[0] = j == 0 ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 1, n = 0; i < 16; ++i) {
          float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
          for (int m = 0; m < i; ++m) {
            const float a = ra[n + m / 4][m % 4];
            if (m & 1) a1 += a * t[m];
            else a0 += a * t[m];
          }
          n += (i + 3) / 4;
          t[i] = (i == j) ? 1.0f : (i > j ? -(a0 + a1) : 0.0f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          Ab[i * LD_A + j] = t[i];                          // fp32 T_II for the off-diagonal block
          sT[(16 * I + i) * LD_CT + 16 * I + j] = f2bf(t[i]);
        }
      }
      if (NB == 2) {                           // T_10 = -T_11 (A_10 T_00), fp32 MFMA
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        floatx4 x = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s)
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 + l16) * LD_A + 4 * s + g], sA[(4 * s + g) * LD_A + l16], x,
                                                   0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(4 * g + r) * 16 + l16] = x[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        floatx4 y = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s)
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 + l16) * LD_A + 16 + 4 * s + g], sX[(4 * s + g) * 16 + l16],
                                                   y, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 + 4 * g + r) * LD_CT + l16] = f2bf(-y[r]);
      }
    }
  };

  // ------------------------------------------------------------------ phase 1, V-side
  floatx4 sacc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) sacc[mt] = zero4();
  auto vside = [&](int set, int t0c) __attribute__((always_inline)) {
    const int nval = min(C, T - t0c);
    char* sb = set_base(set);
    const bf16_t* sWN = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_WN);
    const bf16_t* sQG = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_QG);
    const bf16_t* sKDT = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KDT);
    const float* sGC = reinterpret_cast<const float*>(sb + Cfg::SET_GC);
    const float* sBeta = reinterpret_cast<const float*>(sb + Cfg::SET_BETA);
    // staged values of this wave's 16 columns: slot 2*row + (column / 8)
    const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Cfg::OFF_VRAW + set * Cfg::VRAW_BUF + vw * 1024) +
                       (l16 >> 3) * 8 + (l16 & 7);
    const int col = 16 * vw + l16;
    const bool slow = sFlag[set * 8 + 0] | sFlag[set * 8 + 1] | sFlag[set * 8 + 2] | sFlag[set * 8 + 3];
    if (!slow) {
      // operands of Y = V - W~ S, loaded as one batch
      short8 fw[NB][NS];
      bf16_t vv[NB][4];
      floatx4 bt[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
#pragma unroll
        for (int s = 0; s < NS; ++s) fw[I][s] = lds_a_perm(sWN, LD_TK, 16 * I, 32 * s, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[I][r] = sV[(16 * I + 4 * g + r) * 16];
        bt[I] = *reinterpret_cast<const floatx4*>(sBeta + 16 * I + 4 * g);
      }
      short8 sp[NS];                           // the state as MFMA operand, per 32-row depth slice
#pragma unroll
      for (int s = 0; s < NS; ++s) sp[s] = acc_perm(sacc[2 * s], sacc[2 * s + 1]);
      sched_fence();
      floatx4 Y[2];
#pragma unroll
      for (int I = 0; I < NB; ++I) Y[I] = floatx4{bf2f(vv[I][0]), bf2f(vv[I][1]), bf2f(vv[I][2]), bf2f(vv[I][3])};
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int I = 0; I < NB; ++I) Y[I] = mfma_bf16(fw[I][s], sp[s], Y[I]);
      if (NB == 1) Y[1] = zero4();
      // operands of U = T diag(beta) Y and of o^T = S^T QG^T + U^T P^T
      short8 ft[NB], fp[NB], fq[NB][NS];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        ft[I] = lds_a_perm(sT, LD_CT, 16 * I, 0, lane);
        fp[I] = lds_a_perm(sP, LD_CT, 16 * I, 0, lane);
#pragma unroll
        for (int s = 0; s < NS; ++s) fq[I][s] = lds_a_perm(sQG, LD_TK, 16 * I, 32 * s, lane);
      }
      sched_fence();
      const short8 yb = acc_perm(Y[0] * bt[0], NB == 2 ? Y[1] * bt[NB - 1] : zero4());
      floatx4 U[2];
#pragma unroll
      for (int I = 0; I < NB; ++I) U[I] = mfma_bf16(ft[I], yb, zero4());
      if (NB == 1) U[1] = zero4();
      const short8 ub = acc_perm(U[0], U[1]);
      // o, computed transposed: lane holds token 16I + l16, value columns 16vw + 4g..+3
      floatx4 oT[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) oT[I] = mfma_bf16(ub, fp[I], zero4());
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int I = 0; I < NB; ++I) oT[I] = mfma_bf16(sp[s], fq[I][s], oT[I]);
      // operands of S = diag(Gamma_C) S + KD^T U
      short8 fk[NMT];
      floatx4 gc[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        fk[mt] = lds_a_perm(sKDT, LD_CT, 16 * mt, 0, lane);
        gc[mt] = *reinterpret_cast<const floatx4*>(sGC + 16 * mt + 4 * g);
      }
      sched_fence();
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) sacc[mt] = mfma_bf16(fk[mt], ub, sacc[mt] * gc[mt]);
      if (o) {
        const int c0 = 16 * vw + 4 * g;
#pragma unroll
        for (int I = 0; I < NB; ++I) {
          const int i = 16 * I + l16;
          if (i < nval && c0 < vcols)
            store4_bf16(o + (tb + t0c + i) * V + v0 + c0, scale * oT[I][0], scale * oT[I][1], scale * oT[I][2],
                        scale * oT[I][3]);
        }
      }
    } else {
      // token by token: this wave owns every key row of its 16 value columns, so both
      // reductions over K stay inside the wave
      for (int i = 0; i < nval; ++i) {
        const size_t tok = tb + t0c + i;
        const float vv = col < vcols ? bf2f(v[tok * V + v0 + col]) : 0.0f;
        const float bt = bf2f(beta[tok]);
        float rp = 0.0f;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {              // S' = diag(alpha) S, partial S'^T k
            const int c = 16 * mt + 4 * g + r;
            const bool ok = c < K;
            const float x = ok ? bf2f(z[tok * K + c]) + (dt_bias ? dt_bias[h * K + c] : 0.0f) : 0.0f;
            sacc[mt][r] *= ok ? fast_exp2(-mult2 * softplus_f(x, true)) : 0.0f;
            rp += sacc[mt][r] * (ok ? bf2f(k[tok * K + c]) : 0.0f);
          }
        rp += __shfl_xor(rp, 16);
        rp += __shfl_xor(rp, 32);
        const float e = bt * (vv - rp);
        float op = 0.0f;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {              // S += beta k e^T, partial S^T q_hat
            const int c = 16 * mt + 4 * g + r;
            const bool ok = c < K;
            sacc[mt][r] += (ok ? bf2f(k[tok * K + c]) : 0.0f) * e;
            op += sacc[mt][r] * (ok ? scale * bf2f(q[tok * K + c]) : 0.0f);
          }
        op += __shfl_xor(op, 16);
        op += __shfl_xor(op, 32);
        if (g == 0 && col < vcols && o) o[tok * V + v0 + col] = f2bf(op);
      }
    }
  };

  // ------------------------------------------------------------------ the walk
  // K-waves and V-waves run separate loops (a wave-uniform split) that execute the
  // same sequence of workgroup barriers: step c (c = -1 prepares block 0) is
  //   phase 1 | barrier | phase 2 (unless block c+1 goes token by token) | barrier.
  // The K-waves issue the DMAs of a step at its start and wait for them before its
  // closing barrier, so every staged row is in LDS for all waves after that barrier.
  const int nck = (T + C - 1) / C;
  lds_barrier();                               // LDS cleared before any DMA lands
  auto slow_of = [&](int set) __attribute__((always_inline)) {
    return sFlag[set * 8 + 0] | sFlag[set * 8 + 1] | sFlag[set * 8 + 2] | sFlag[set * 8 + 3];
  };
  auto e1_any = [&](int tn, int set) __attribute__((always_inline)) {
    if (precise) e1(std::true_type{}, tn, set);
    else e1(std::false_type{}, tn, set);
  };
  if (kwave) {
    if (nck > 0) {
      dma_qkz(0, 0);
      load_beta(0);
      wait_vm();
    }
    lds_barrier();                             // staged block 0 visible to all K-waves
    for (int c = -1; c < nck; ++c) {
      const int tn = (c + 1) * C;
      if (c + 2 < nck) dma_qkz(tn + C, (c + 2) & 1);
      if (c + 1 < nck) dma_v(tn, (c + 1) & 1);
      if (tn < T) {
        e1_any(tn, (c + 1) & 1);
        if (tn + C < T) load_beta(tn + C);
      }
      lds_barrier();
      if (tn < T && !slow_of((c + 1) & 1)) phase2((c + 1) & 1);
      wait_vm();
      lds_barrier();
    }
  } else {
    if (vact && state_in) {
      const int col = 16 * vw + l16;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * g + r;
          if (row < K && col < vcols) sacc[mt][r] = state_in[((size_t)bh * K + row) * V + v0 + col];
        }
    }
    lds_barrier();
    for (int c = -1; c < nck; ++c) {
      const int tn = (c + 1) * C;
      if (c >= 0 && vact) vside(c & 1, c * C);
      lds_barrier();
      if (tn < T && !slow_of((c + 1) & 1)) phase2((c + 1) & 1);
      lds_barrier();
    }
    if (vact && state_out) {
      const int col = 16 * vw + l16;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * g + r;
          if (row < K && col < vcols) state_out[((size_t)bh * K + row) * V + v0 + col] = sacc[mt][r];
        }
    }
  }
}

template <int KD, int VT, int C>
hipError_t launch_chunk_fwd_pc_inst(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                    const float* dt_bias, const void* beta, const float* state_in, float scale, void* o,
                                    float* state_out, int B, int H, int T, int K, int V, hipStream_t s) {
  const int nvt = (V + VT - 1) / VT;
  const int total = B * H * nvt;
  hipLaunchKernelGGL((chunk_fwd_pc_kernel<KD, VT, C>), dim3(total), dim3(512), 0, s, (const bf16_t*)q,
                     (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)z, A_log, dt_bias, (const bf16_t*)beta,
                     state_in, scale, (bf16_t*)o, state_out, H, T, K, V, nvt, total, 64.0f);
  return hipGetLastError();
}

}  // namespace kda
