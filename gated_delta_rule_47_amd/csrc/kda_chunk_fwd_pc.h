// Pipelined chunked KDA forward for bf16 activations on gfx950.
//
// One workgroup of 12 waves owns one (batch, head, value tile of <= 64 columns) and
// walks the sequence in blocks of C <= 32 tokens.  The work of a block b splits into
// three stages, each done by its own four waves:
//   E (waves 0-3):  the gate and block-local decay scans and the decay-weighted
//                   operands KE, QE, KR (and KR^T), from q, k, z staged in LDS;
//   W (waves 8-11): the strictly-lower A = diag(beta) KE KR^T and the lower
//                   P = QE KR^T (MFMA), and the inverses T_00, T_11 of the two 16x16
//                   diagonal blocks of I + A (column-sweep elimination);
//   V (waves 4-7):  the state-dependent part, each wave owning 16 value columns and all
//                   K rows of the fp32 state in accumulator registers: with
//                   S~ = diag(G0) S,  Y = V - KE S~,  U = (I + A)^-1 diag(beta) Y,
//                   o = scale (QE S~ + P U),  S = diag(D0) (S~ + KR^T U)  (the state is
//                   carried as S~ of the next block: one per-channel multiply a block).
// Step s of the walk runs E on block s+2, W on block s+1 and V on block s side by side
// and ends with the only workgroup barrier of the step; what a stage writes for block
// b is read by the next stage one step later, so E's outputs are triple-buffered and
// W's double-buffered in LDS.  Only V depends on the state.
//
// (U = (I + A)^-1 diag(beta) (V - W~ S) is the u - w S of the WY form with the product
// w = T diag(beta) W~ folded into the state-dependent side.  V applies the inverse
// blockwise, U_0 = T_00 Z_0 and U_1 = T_11 (Z_1 - A_10 U_0) with Z = diag(beta) Y, so the
// off-diagonal block of the inverse is never formed.)
//
// Activations reach LDS by buffer-to-LDS DMA (16 bytes per lane, 1 KB per instruction),
// issued by the E waves: each E wave stages the q, k, z rows of its own 32 channels one
// block ahead into a private area (it alone reads them, so its own wait on the DMA is
// the only synchronisation), and the v rows of block s+2 into a triple-buffered area
// that V reads after the step barriers in between.
//
// V chains MFMA results into MFMAs without LDS: a 32-deep contraction over two 16-row
// accumulator tiles is fed with lane l supplying depth {4g..4g+3} of the first tile and
// {16+4g..16+4g+3} of the second (g = l/16) -- exactly the rows its accumulators hold --
// and the LDS operand of the same product is read with the same depth order.  The sum
// over depth does not depend on its order.  The same registers serve as A or as B
// operand, so a product can be computed transposed when that makes its result layout
// the one the next step (or the global store) wants.
//
// Decays are taken relative to one reference per 32-token block, the cumulative
// log-decay m through its 16th token: KE = k 2^(G - m), QE = q 2^(G - m), KR = k 2^(m - G)
// (G the cumulative log2-decay of each token), so A = KE KR^T and P = QE KR^T hold the
// exact pairwise decays, and the chunk-level factors G0 = 2^m (block start to the
// reference) and D0 = 2^(G_last - m) (reference to block end) are per-channel scalings
// of the state: QGamma S = QE (G0 S), W~ S = KE (G0 S), and the carry
// diag(Gamma_C) S + KD^T U = diag(D0) (G0 S + KR^T U) since Gamma_C = G0 D0.  Every factor
// is 2^x with |x| at most one 16-token half of the block's decay; a block where that
// exceeds 2^thresh in some channel is evaluated token by token by the V waves.
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
  static constexpr int NNT = VD / 16;                 // value-column tiles = active V waves
  static constexpr int NMT = KD / 16;                 // key-row tiles of the state
  static constexpr int NWAVES = 12;
  // Row strides of the bf16 operand tiles, in elements: 2 (mod 32) banks of 4 bytes per
  // row, so that the 8-byte operand reads (16 consecutive rows per 128-byte LDS cycle)
  // and the 4-byte E writes (rows 8 apart) are free of bank conflicts.
  static constexpr int LD_TK = KD + 4;                // [token][channel] bf16
  static constexpr int LD_CT = CD + 4;                // [channel|token][token] bf16
  static constexpr int LD_A = CD + 4;                 // [token][token] fp32
  static constexpr int SZ_TK = CD * LD_TK * 2;
  static constexpr int SZ_KT = KD * LD_CT * 2;
  static constexpr int SZ_TT = CD * LD_CT * 2;
  // E outputs of one block (triple-buffered): KE, QE, KR, KR^T, G0, D0, beta, and
  // F = D0 * G0 of the next block (written with the next block)
  static constexpr int SET_KE = 0;
  static constexpr int SET_QE = SET_KE + SZ_TK;
  static constexpr int SET_KR = SET_QE + SZ_TK;
  static constexpr int SET_KRT = SET_KR + SZ_TK;
  static constexpr int SET_G0 = SET_KRT + SZ_KT;
  static constexpr int SET_D0 = SET_G0 + KD * 4;
  static constexpr int SET_F = SET_D0 + KD * 4;
  static constexpr int SET_BETA = SET_F + KD * 4;
  static constexpr int SET_BYTES = SET_BETA + CD * 4;
  // W outputs of one block (double-buffered): P, T (T_00 and T_11, zero elsewhere),
  // -A_10 (columns 0..15, zero in 16..31)
  static constexpr int WO_P = 0;
  static constexpr int WO_T = WO_P + SZ_TT;
  static constexpr int WO_A10 = WO_T + SZ_TT;
  static constexpr int WO_BYTES = WO_A10 + 16 * LD_CT * 2;
  // staging: per E wave, k, q, z rows of its 32 channels (4 chunks of 16 bytes per row)
  static constexpr int RAW_T = CD * 64;               // one tensor, 32 rows x 64 bytes
  static constexpr int RAW_WAVE = 3 * RAW_T;
  static constexpr int VRAW_BUF = NNT * 1024;         // per value tile: 32 rows x 16 columns
  static constexpr int OFF_SET = 0;
  static constexpr int OFF_WO = OFF_SET + 3 * SET_BYTES;
  static constexpr int OFF_A = OFF_WO + 2 * WO_BYTES;  // diagonal blocks of A (fp32), W scratch
  static constexpr int OFF_RAW = OFF_A + CD * LD_A * 4;
  static constexpr int OFF_VRAW = OFF_RAW + 4 * RAW_WAVE;
  static constexpr int OFF_FLAG = OFF_VRAW + 3 * VRAW_BUF;
  static constexpr int TOTAL = OFF_FLAG + 3 * 4 * 4;
  static constexpr int QKZ_DMA = C / 16;              // 1 KB DMA instructions per tensor, wave and block
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
  static_assert(KD % 32 == 0 && (C == 16 || C == 32) && NNT <= 4, "tile shape");
  static_assert(SET_BYTES % 16 == 0 && WO_BYTES % 16 == 0 && OFF_A % 16 == 0 && OFF_RAW % 16 == 0 &&
                    OFF_VRAW % 16 == 0 && SET_G0 % 16 == 0,
                "16-byte alignment");
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

__device__ __forceinline__ void store4_bf16(bf16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Keep the compiler from moving instructions across this point: used to issue a
// batch of LDS operand loads before the MFMAs that consume them.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// 16 bytes per lane from buffer offset `off` into LDS at lds + 16 * lane (lds must be
// the same for the whole wave).  Offsets past the buffer's range deliver zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (its DMAs, loads and
// stores) have completed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until this wave's outstanding LDS operations have completed.
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Make this wave's earlier LDS writes visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

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
__global__ void __launch_bounds__(768)
chunk_fwd_pc_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                    const bf16_t* __restrict__ z, const float* __restrict__ A_log,
                    const float* __restrict__ dt_bias, const bf16_t* __restrict__ beta,
                    const float* state_in, float scale, bf16_t* __restrict__ o, float* state_out, int H, int T,
                    int K, int V, int n_vtiles, int total_wg, float thresh) {
  using Cfg = PcCfg<KD, VT, C>;
  constexpr int CD = Cfg::CD, NB = Cfg::NB, NNT = Cfg::NNT, NMT = Cfg::NMT;
  constexpr int LD_TK = Cfg::LD_TK, LD_CT = Cfg::LD_CT, LD_A = Cfg::LD_A;
  constexpr int NS = KD / 32;                         // 32-deep channel slices
  constexpr int NTHR = Cfg::NWAVES * 64;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
  float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
  int* sFlag = reinterpret_cast<int*>(smem + Cfg::OFF_FLAG);   // [block % 3][E wave]
  auto set_base = [&](int b) __attribute__((always_inline)) { return smem + Cfg::OFF_SET + (b % 3) * Cfg::SET_BYTES; };
  auto wo_base = [&](int b) __attribute__((always_inline)) { return smem + Cfg::OFF_WO + (b & 1) * Cfg::WO_BYTES; };
  auto slow_of = [&](int b) __attribute__((always_inline)) {
    const int* f = sFlag + (b % 3) * 4;
    return (f[0] | f[1] | f[2] | f[3]) != 0;
  };

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
  const int nck = (T + C - 1) / C;

  for (int i = tid; i < Cfg::TOTAL / 16; i += NTHR) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  const float mult2 = gate_multiplier(A_log[h]) * kLog2e;
  lds_barrier();                               // LDS cleared before any DMA lands

  if (wave < 4) {
    // ================================================================ E waves
    const int pair = 16 * wave + l16;          // key-channel pair
    const int hb = g;                          // 8-token half-block
    const bool kact = 2 * pair < K;
    const bool precise = mult2 > 64.0f * kLog2e;
    const float dtb0 = (kact && dt_bias) ? dt_bias[h * K + 2 * pair] : 0.0f;
    const float dtb1 = (kact && dt_bias) ? dt_bias[h * K + 2 * pair + 1] : 0.0f;
    // per-head buffer resources: offsets past the head's T tokens read as 0
    const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(k + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_z = make_rsrc(z + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(v + tb * V, (unsigned)(T * V * 2));
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(beta + tb, (unsigned)(T * 2));
    constexpr unsigned kOOB = 0xFFFFFFF0u;     // an offset past any range: zeros
    char* raw = smem + Cfg::OFF_RAW + wave * Cfg::RAW_WAVE;

    // this wave's channels 32*wave .. +31 of rows [tn, tn + C): instruction j, lane l
    // fills row 16j + l/4 with channel chunk 4*wave + l%4 (chunks past K read as 0)
    auto dma_qkz = [&](int tn) __attribute__((always_inline)) {
      const int ch = 8 * (4 * wave + (lane & 3));
#pragma unroll
      for (int j = 0; j < Cfg::QKZ_DMA; ++j) {
        const int r = 16 * j + (lane >> 2);
        const unsigned off = ch < K ? (unsigned)(((tn + r) * K + ch) * 2) : kOOB;
        dma16(rs_k, raw + j * 1024, off);
        dma16(rs_q, raw + Cfg::RAW_T + j * 1024, off);
        dma16(rs_z, raw + 2 * Cfg::RAW_T + j * 1024, off);
      }
    };
    // value tile of block b (wave w < NNT: its 16 columns, slot 2*row + half)
    auto dma_v = [&](int b) __attribute__((always_inline)) {
      if (wave < NNT) {
        const int r = lane >> 1, c0 = 16 * wave + 8 * (lane & 1);
        const unsigned off = (r < C && c0 < vcols) ? (unsigned)(((b * C + r) * V + v0 + c0) * 2) : kOOB;
        dma16(rs_v, smem + Cfg::OFF_VRAW + (b % 3) * Cfg::VRAW_BUF + wave * 1024, off);
      }
    };
    bf16_t rbeta = 0, rbeta_next = 0;
    auto load_beta = [&](int tn) __attribute__((always_inline)) {
      if (tid < C) rbeta_next = __builtin_amdgcn_raw_buffer_load_b16(rs_b, (unsigned)((tn + tid) * 2), 0, 0);
    };

    auto e1 = [&](auto precise_tag, int b) __attribute__((always_inline)) {
      constexpr bool PRECISE = decltype(precise_tag)::value;
      const int tn = b * C;
      const int nval = min(C, T - tn);
      char* sb = set_base(b);
      bf16_t* sKE = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KE);
      bf16_t* sQE = reinterpret_cast<bf16_t*>(sb + Cfg::SET_QE);
      bf16_t* sKR = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KR);
      bf16_t* sKRT = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KRT);
      float* sG0 = reinterpret_cast<float*>(sb + Cfg::SET_G0);
      float* sD0 = reinterpret_cast<float*>(sb + Cfg::SET_D0);
      float* sBeta = reinterpret_cast<float*>(sb + Cfg::SET_BETA);
      // staged k, q, z of channel pair `pair`, tokens 8hb..8hb+7
      wait_vm();                               // this wave's DMA of block b (and beta)
      rbeta = rbeta_next;
      Pair<bf16_t> rk[8], rq[8], rz[8];
      {
        const char* rb = raw + (8 * hb) * 64 + (l16 >> 2) * 16 + (l16 & 3) * 4;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          rk[t].u = *reinterpret_cast<const uint32_t*>(rb + t * 64);
          rq[t].u = *reinterpret_cast<const uint32_t*>(rb + Cfg::RAW_T + t * 64);
          rz[t].u = *reinterpret_cast<const uint32_t*>(rb + 2 * Cfg::RAW_T + t * 64);
        }
      }
      wait_lgkm();                             // staging read: it may be refilled now
      if (b + 1 < nck) {
        dma_qkz(tn + C);
        load_beta(tn + C);
      }
      if (b < nck) dma_v(b);
      // Tokens at or past nval (a partial last block, or rows 16..31 when C = 16) are
      // identity tokens: their staged k and q are 0, and z = -inf makes their gate 0.
      if (nval < CD) {
        const int lim = nval - 8 * hb;
#pragma unroll
        for (int t = 0; t < 8; ++t) rz[t].u = t < lim ? rz[t].u : 0xFF80FF80u;
      }
      // gate in log2 units and its inclusive prefix over the lane's 8 tokens
      float px[8], py[8];
      float ax = 0.0f, ay = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        ax += -mult2 * softplus_f(rz[t].x() + dtb0, PRECISE);
        ay += -mult2 * softplus_f(rz[t].y() + dtb1, PRECISE);
        px[t] = ax;
        py[t] = ay;
      }
      // the four half-block sums of this channel pair (lanes l16 + 16*hb')
      float Hx[4], Hy[4];
      row_gather(ax, Hx);
      row_gather(ay, Hy);
      // exponent of token t relative to the reference m = H0 + H1: G_t - m
      const float offx = hb == 0 ? -(Hx[0] + Hx[1]) : hb == 1 ? -Hx[1] : hb == 2 ? 0.0f : Hx[2];
      const float offy = hb == 0 ? -(Hy[0] + Hy[1]) : hb == 1 ? -Hy[1] : hb == 2 ? 0.0f : Hy[2];
      if (kact) {
        const int c = 2 * pair;
        float krx[8], kry[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float ex = px[t] + offx, ey = py[t] + offy;
          const float Lx = fast_exp2(ex), Ly = fast_exp2(ey), Rx = fast_exp2(-ex), Ry = fast_exp2(-ey);
          const float kx = rk[t].x(), ky = rk[t].y(), qx = rq[t].x(), qy = rq[t].y();
          const int j = 8 * hb + t;
          krx[t] = kx * Rx;
          kry[t] = ky * Ry;
          store2<bf16_t>(sKE + j * LD_TK + c, kx * Lx, ky * Ly);
          store2<bf16_t>(sQE + j * LD_TK + c, qx * Lx, qy * Ly);
          store2<bf16_t>(sKR + j * LD_TK + c, krx[t], kry[t]);
        }
        auto st8 = [](bf16_t* dst, const float* x) {   // two 8-byte stores (rows are 8-byte aligned)
          *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          *reinterpret_cast<uint2*>(dst + 4) = uint2{pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        };
        st8(sKRT + c * LD_CT + 8 * hb, krx);
        st8(sKRT + (c + 1) * LD_CT + 8 * hb, kry);
        if (hb == 0) {
          const float2 g0v = float2{fast_exp2(Hx[0] + Hx[1]), fast_exp2(Hy[0] + Hy[1])};
          *reinterpret_cast<float2*>(sG0 + c) = g0v;
          *reinterpret_cast<float2*>(sD0 + c) = float2{fast_exp2(Hx[2] + Hx[3]), fast_exp2(Hy[2] + Hy[3])};
          if (b > 0) {                         // F of the previous block (this lane wrote its D0)
            char* sp = set_base(b - 1);
            const float2 dp = *reinterpret_cast<const float2*>(sp + Cfg::SET_D0 + 4 * c);
            *reinterpret_cast<float2*>(sp + Cfg::SET_F + 4 * c) = float2{dp.x * g0v.x, dp.y * g0v.y};
          }
        }
      }
      if (tid < CD) sBeta[tid] = tid < nval ? bf2f(rbeta) : 0.0f;
      const float worst = fminf(fminf(Hx[0] + Hx[1], Hx[2] + Hx[3]), fminf(Hy[0] + Hy[1], Hy[2] + Hy[3]));
      const unsigned long long bal = __ballot(kact && worst < -thresh);
      if (lane == 0) sFlag[(b % 3) * 4 + wave] = bal != 0ull;
    };

    if (nck > 0) {
      dma_qkz(0);
      load_beta(0);
    }
    for (int s = -2; s < nck; ++s) {
      if (s + 2 < nck) {
        if (precise) e1(std::true_type{}, s + 2);
        else e1(std::false_type{}, s + 2);
      }
      wait_vm();                               // v rows of block s+2 in LDS before the barrier
      lds_barrier();
    }
  } else if (wave >= 8) {
    // ================================================================ W waves
    const int ww = wave - 8;
    auto wstage = [&](int b) __attribute__((always_inline)) {
      char* sb = set_base(b);
      const float* sBeta = reinterpret_cast<const float*>(sb + Cfg::SET_BETA);
      const bf16_t* sKE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KE);
      const bf16_t* sQE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_QE);
      const bf16_t* sKR = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KR);
      char* wb = wo_base(b);
      bf16_t* sP = reinterpret_cast<bf16_t*>(wb + Cfg::WO_P);
      bf16_t* sT = reinterpret_cast<bf16_t*>(wb + Cfg::WO_T);
      bf16_t* sA10 = reinterpret_cast<bf16_t*>(wb + Cfg::WO_A10);
      // tiles of this wave: ww 0: A_00; 1: A_11; 2: A_10 and P_00; 3: P_10 and P_11.
      // Each tile is computed transposed: lane (g, l16) holds row i = 16I + l16,
      // columns 16J + 4g..+3.
#pragma unroll
      for (int tix = 0; tix < 2; ++tix) {
        const int kind = ww == 0 ? (tix == 0 ? 0 : -1) : ww == 1 ? (tix == 0 ? 3 : -1)
                       : ww == 2 ? (tix == 0 ? 1 : 4) : (tix == 0 ? 5 : 6);
        // kinds: 0 A_00, 1 A_10, 3 A_11, 4 P_00, 5 P_10, 6 P_11
        if (kind < 0) continue;
        const bool isA = kind < 4;
        const int I = (kind == 0 || kind == 4) ? 0 : 1;
        const int J = (kind == 3 || kind == 6) ? 1 : 0;
        if (I >= NB) continue;
        const bf16_t* cols = isA ? sKE : sQE;
        short8 fa[NS], fb[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          fa[s] = lds_a_perm(sKR, LD_TK, 16 * J, 32 * s, lane);   // same depth order on both sides
          fb[s] = lds_a_perm(cols, LD_TK, 16 * I, 32 * s, lane);
        }
        sched_fence();
        floatx4 acc = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = mfma_bf16(fa[s], fb[s], acc);
        const int i = 16 * I + l16, j0 = 16 * J + 4 * g;
        float vals[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vals[r] = (isA ? j0 + r < i : j0 + r <= i) ? acc[r] : 0.0f;
        if (isA && I == J) {                   // diagonal block: fp32 for the inverse
          const float bi = sBeta[i];
          *reinterpret_cast<floatx4*>(sA + i * LD_A + j0) =
              floatx4{bi * vals[0], bi * vals[1], bi * vals[2], bi * vals[3]};
        } else if (isA) {                      // A_10: bf16, negated, for V
          const float nb = -sBeta[i];
          store4_bf16(sA10 + l16 * LD_CT + j0, nb * vals[0], nb * vals[1], nb * vals[2], nb * vals[3]);
        } else {
          store4_bf16(sP + i * LD_CT + j0, vals[0], vals[1], vals[2], vals[3]);
        }
      }
      if (ww < NB) {
        // T_II = (I + A_II)^-1 for I = ww by forward substitution: lane j holds
        // column j; row i needs the strictly-lower part of row i and the entries of
        // rows < i.  Rows are loaded in three batches so that the substitution waits
        // on LDS a few times rather than once per row.
        wave_lds_fence();                      // this wave's A_II tile
        if (lane < 16) {
          const int I = ww, j = lane;
          const float* Ab = sA + 16 * I * LD_A + 16 * I;
          float t[16];
          t[0] = j == 0 ? 1.0f : 0.0f;
          auto rows = [&](auto lo_tag, auto hi_tag) __attribute__((always_inline)) {
            constexpr int LO = decltype(lo_tag)::value, HI = decltype(hi_tag)::value;
            floatx4 ra[HI - LO][4];
#pragma unroll
            for (int i = LO; i < HI; ++i)
#pragma unroll
              for (int qd = 0; qd < (i + 3) / 4; ++qd)
                ra[i - LO][qd] = *reinterpret_cast<const floatx4*>(Ab + i * LD_A + 4 * qd);
#pragma unroll
            for (int i = LO; i < HI; ++i) {
              float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
              for (int m = 0; m < i - 1; ++m) {
                if (m & 1) a1 = fmaf(ra[i - LO][m / 4][m % 4], t[m], a1);
                else a0 = fmaf(ra[i - LO][m / 4][m % 4], t[m], a0);
              }
              const float sum = fmaf(ra[i - LO][(i - 1) / 4][(i - 1) % 4], t[i - 1], a0 + a1);
              t[i] = i == j ? 1.0f : -sum;
            }
          };
          rows(std::integral_constant<int, 1>{}, std::integral_constant<int, 7>{});
          rows(std::integral_constant<int, 7>{}, std::integral_constant<int, 12>{});
          rows(std::integral_constant<int, 12>{}, std::integral_constant<int, 16>{});
#pragma unroll
          for (int i = 0; i < 16; ++i) sT[(16 * I + i) * LD_CT + 16 * I + j] = f2bf(t[i]);
        }
      }
    };
    for (int s = -2; s < nck; ++s) {
      const int b = s + 1;
      if (b >= 0 && b < nck && !slow_of(b)) wstage(b);
      lds_barrier();
    }
  } else {
    // ================================================================ V waves
    const int vw = wave - 4;
    const bool vact = vw < NNT;
    const int col = 16 * vw + l16;
    floatx4 sacc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) sacc[mt] = zero4();
    if (vact && state_in) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * g + r;
          if (row < K && col < vcols) sacc[mt][r] = state_in[((size_t)bh * K + row) * V + v0 + col];
        }
    }
    // Complete the state loads here: inside the walk the wave's only vector-memory
    // operations are its output stores, which must never hold up the next step.
    wait_vm();
    // Between blocks the state is kept as S~ = diag(G0) S of the next block when that
    // block takes the MFMA path (scaled = true), so a block costs one per-channel
    // multiply of the state (by F = D0 G0' or, before a token-path block or at the end,
    // by D0); a block entered unscaled is scaled by its own G0 first.
    bool scaled = false;
    // output rows of this head through a buffer resource: 32-bit offsets, no 64-bit
    // address arithmetic per store
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(o + tb * V, o ? (unsigned)(T * V * 2) : 0u);

    auto vside = [&](int b) __attribute__((always_inline)) {
      const int t0c = b * C;
      const int nval = min(C, T - t0c);
      char* sb = set_base(b);
      const bf16_t* sKE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KE);
      const bf16_t* sQE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_QE);
      const bf16_t* sKRT = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KRT);
      const float* sG0 = reinterpret_cast<const float*>(sb + Cfg::SET_G0);
      const bool next_fast = b + 1 < nck && !slow_of(b + 1);
      const float* sF = reinterpret_cast<const float*>(sb + (next_fast ? Cfg::SET_F : Cfg::SET_D0));
      const float* sBeta = reinterpret_cast<const float*>(sb + Cfg::SET_BETA);
      char* wb = wo_base(b);
      const bf16_t* sP = reinterpret_cast<const bf16_t*>(wb + Cfg::WO_P);
      const bf16_t* sT = reinterpret_cast<const bf16_t*>(wb + Cfg::WO_T);
      const bf16_t* sA10 = reinterpret_cast<const bf16_t*>(wb + Cfg::WO_A10);
      // staged values of this wave's 16 columns: slot 2*row + (column / 8)
      const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Cfg::OFF_VRAW + (b % 3) * Cfg::VRAW_BUF + vw * 1024) +
                         (l16 >> 3) * 8 + (l16 & 7);
      if (!slow_of(b)) {
        if (!scaled) {                         // first block, or after a token-path block
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) sacc[mt] *= *reinterpret_cast<const floatx4*>(sG0 + 16 * mt + 4 * g);
        }
        // operands of Yn = KE S~ - V (= -Y), loaded as one batch
        short8 fw[NB][NS];
        bf16_t vv[NB][4];
        floatx4 bt[NB];
#pragma unroll
        for (int I = 0; I < NB; ++I) {
#pragma unroll
          for (int s = 0; s < NS; ++s) fw[I][s] = lds_a_perm(sKE, LD_TK, 16 * I, 32 * s, lane);
#pragma unroll
          for (int r = 0; r < 4; ++r) vv[I][r] = sV[(16 * I + 4 * g + r) * 16];
          bt[I] = *reinterpret_cast<const floatx4*>(sBeta + 16 * I + 4 * g);
        }
        sched_fence();
        // S~ as MFMA operand per 32-row slice
        short8 sp[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) sp[s] = acc_perm(sacc[2 * s], sacc[2 * s + 1]);
        floatx4 Yn[2];
#pragma unroll
        for (int I = 0; I < NB; ++I)
          Yn[I] = floatx4{-bf2f(vv[I][0]), -bf2f(vv[I][1]), -bf2f(vv[I][2]), -bf2f(vv[I][3])};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int I = 0; I < NB; ++I) Yn[I] = mfma_bf16(fw[I][s], sp[s], Yn[I]);
        // operands of U = (I + A)^-1 diag(beta) Y and of o^T = S~^T QE^T + U^T P^T
        short8 ft[NB], fp[NB], fq[NB][NS], fa10;
#pragma unroll
        for (int I = 0; I < NB; ++I) {
          ft[I] = lds_a_perm(sT, LD_CT, 16 * I, 0, lane);
          fp[I] = lds_a_perm(sP, LD_CT, 16 * I, 0, lane);
#pragma unroll
          for (int s = 0; s < NS; ++s) fq[I][s] = lds_a_perm(sQE, LD_TK, 16 * I, 32 * s, lane);
        }
        if (NB == 2) fa10 = lds_a_perm(sA10, LD_CT, 0, 0, lane);
        sched_fence();
        // U_0 = T_00 Z_0, U_1 = T_11 (Z_1 - A_10 U_0), Z = diag(beta) Y = -diag(beta) Yn
        floatx4 U[2];
        U[0] = mfma_bf16(ft[0], acc_perm(Yn[0] * -bt[0], zero4()), zero4());
        if (NB == 2) {
          const floatx4 Z1 = mfma_bf16(fa10, acc_perm(U[0], zero4()), Yn[1] * -bt[NB - 1]);
          U[1] = mfma_bf16(ft[NB - 1], acc_perm(zero4(), Z1), zero4());
        } else {
          U[1] = zero4();
        }
        const short8 ub = acc_perm(U[0], U[1]);
        // o, computed transposed: lane holds token 16I + l16, value columns 16vw + 4g..+3
        floatx4 oT[NB];
#pragma unroll
        for (int I = 0; I < NB; ++I) oT[I] = mfma_bf16(ub, fp[I], zero4());
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int I = 0; I < NB; ++I) oT[I] = mfma_bf16(sp[s], fq[I][s], oT[I]);
        // operands of S' = diag(F) (S~ + KR^T U), F = D0 G0' (next block scaled) or D0
        short8 fk[NMT];
        floatx4 fs[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          fk[mt] = lds_a_perm(sKRT, LD_CT, 16 * mt, 0, lane);
          fs[mt] = *reinterpret_cast<const floatx4*>(sF + 16 * mt + 4 * g);
        }
        sched_fence();
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) sacc[mt] = fs[mt] * mfma_bf16(fk[mt], ub, sacc[mt]);
        scaled = next_fast;
        if (o) {
          const int c0 = 16 * vw + 4 * g;
#pragma unroll
          for (int I = 0; I < NB; ++I) {
            const int i = 16 * I + l16;
            const u32x2 d = {pack_bf16x2(scale * oT[I][0], scale * oT[I][1]),
                             pack_bf16x2(scale * oT[I][2], scale * oT[I][3])};
            if (i < nval && c0 < vcols)
              __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, (unsigned)(((t0c + i) * V + v0 + c0) * 2), 0, 0);
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
            for (int r = 0; r < 4; ++r) {            // S' = diag(alpha) S, partial S'^T k
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
            for (int r = 0; r < 4; ++r) {            // S += beta k e^T, partial S^T q_hat
              const int c = 16 * mt + 4 * g + r;
              const bool ok = c < K;
              sacc[mt][r] += (ok ? bf2f(k[tok * K + c]) : 0.0f) * e;
              op += sacc[mt][r] * (ok ? scale * bf2f(q[tok * K + c]) : 0.0f);
            }
          op += __shfl_xor(op, 16);
          op += __shfl_xor(op, 32);
          if (g == 0 && col < vcols && o) o[tok * V + v0 + col] = f2bf(op);
        }
        wait_vm();                             // the token path's loads
        scaled = false;
      }
    };
    for (int s = -2; s < nck; ++s) {
      if (s >= 0 && vact) vside(s);
      lds_barrier();
    }
    if (vact && state_out) {
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
  hipLaunchKernelGGL((chunk_fwd_pc_kernel<KD, VT, C>), dim3(total), dim3(PcCfg<KD, VT, C>::NWAVES * 64), 0, s,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)z, A_log, dt_bias,
                     (const bf16_t*)beta, state_in, scale, (bf16_t*)o, state_out, H, T, K, V, nvt, total, 96.0f);
  return hipGetLastError();
}

}  // namespace kda
