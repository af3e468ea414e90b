// Pipelined chunked KDA forward for bf16 activations on gfx950.
//
// One workgroup of 16 waves owns one (batch, head, value tile of <= 64 columns) and
// walks the sequence in blocks of C <= 32 tokens.  The work of a block b splits into
// three stages, each done by its own waves:
//   E (waves 0-7):   the gate and block-local decay scans and the decay-weighted
//                    operands KE, QE, KR (V reads KR^T from KR with transposing LDS
//                    reads); wave e covers one 16-token half of
//                    the block and 32 key channels, from q, k, z loaded straight into
//                    registers two blocks ahead (KD <= 64: two waves share a channel
//                    group, each taking the even or the odd channel of every pair);
//   V (waves 8-11):  the state-dependent part, each wave owning 16 value columns and all
//                    K rows of the fp32 state in accumulator registers: with
//                    S~ = diag(G0) S,  Y = V - KE S~,  U = (I + A)^-1 diag(beta) Y,
//                    o = scale (QE S~ + P U),  S = diag(D0) (S~ + KR^T U)  (the state is
//                    carried as S~ of the next block: one per-channel multiply a block);
//   W (waves 12-15): the strictly-lower A = diag(beta) KE KR^T and the lower
//                    P = QE KR^T (MFMA), and the inverses T_00, T_11 of the two 16x16
//                    diagonal blocks of I + A (in 8 x 8 blocks: two short substitutions,
//                    then the off-diagonal block from two small products); W also
//                    stages v and beta of the block after next.
// Step s of the walk runs E on block s+2, W on block s+1 and V on block s side by side
// and ends with the only workgroup barrier of the step; what a stage writes for block
// b is read by the next stage one step later, so E's outputs are triple-buffered and
// W's double-buffered in LDS.  Only V depends on the state; it runs at the highest
// wave priority, W next, E last.
//
// (U = (I + A)^-1 diag(beta) (V - W~ S) is the u - w S of the WY form with the product
// w = T diag(beta) W~ folded into the state-dependent side.  V applies the inverse
// blockwise, U_0 = T_00 Z_0 and U_1 = T_11 (Z_1 - A_10 U_0) with Z = diag(beta) Y, so the
// off-diagonal block of the inverse is never formed.  E stores KE negated, so that V
// needs no sign flip of v.)
//
// The v rows of each block reach LDS by buffer-to-LDS DMA (16 bytes per lane), issued by
// W waves two steps before V reads them.  The E waves' only memory operations are their
// register loads, so waiting for one block's loads never waits for anything younger.
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
//
// SG (scalar decay): z is (B,H,T) and dt_bias (H): one gate value per token and head
// shares every key channel.  The E waves then load one gate input per token, evaluate the
// gate and the decay scan once per token and use one pair of factors for both channels of
// a lane; everything else is the per-channel kernel unchanged.
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
  static constexpr int NE = 8, NV = 4, NW = 4;        // waves of the E, V and W stages
  static_assert(NE == 8, "the slow flags of a block are read as one 8-byte word");
  static constexpr int NWAVES = NE + NV + NW;
  // Row strides of the bf16 operand tiles, in elements.  Within each 32-wide slice of a
  // row, the contraction index is stored in the order of perm32(), so that an MFMA operand
  // fragment is one 16-byte read.  Measured on gfx950, 16-byte reads of 16 rows are free of
  // bank conflicts for row strides of 96 or 288 bytes but run at half rate for 80 or 272
  // bytes, while the 4-byte writes of the E stage (rows 4 apart) cost the same for all of
  // them: the [token][channel] tiles, read most, take KD + 16 (288 bytes when K = 128); the
  // 32-token rows keep CD + 8 (80 bytes: the larger stride would not fit in LDS, and their
  // 8-byte row stores conflict at 96).
  static constexpr int LD_TK = KD + 16;               // [token][channel] bf16
  static constexpr int LD_CT = CD + 8;                // [channel|token][token] bf16
  static constexpr int LD_A = CD + 4;                 // [token][token] fp32
  static constexpr int SZ_TK = CD * LD_TK * 2;
  static constexpr int SZ_TT = CD * LD_CT * 2;
  // E outputs of one block (triple-buffered): KE, QE, KR, G0, D0, beta, and F = D0 * G0 of
  // the next block (written with the next block).  A block that takes the token path
  // parks the state of the V waves in its set meanwhile, so a set holds at least that.
  static constexpr int SET_KE = 0;
  static constexpr int SET_QE = SET_KE + SZ_TK;
  static constexpr int SET_KR = SET_QE + SZ_TK;
  static constexpr int SET_G0 = SET_KR + SZ_TK;
  static constexpr int SET_D0 = SET_G0 + KD * 4;
  static constexpr int SET_F = SET_D0 + KD * 4;
  static constexpr int SET_BETA = SET_F + KD * 4;
  static constexpr int PARK_BYTES = NV * NMT * 256 * 4;
  static constexpr int SET_BYTES = round_up(SET_BETA + CD * 4 > PARK_BYTES ? SET_BETA + CD * 4 : PARK_BYTES, 16);
  // W outputs of one block (double-buffered): P, T (T_00 and T_11, zero elsewhere),
  // -A_10 (columns 0..15, zero in 16..31)
  static constexpr int WO_P = 0;
  static constexpr int WO_T = WO_P + SZ_TT;
  static constexpr int WO_A10 = WO_T + SZ_TT;
  static constexpr int WO_BYTES = WO_A10 + 16 * LD_CT * 2;
  static constexpr int VRAW_BUF = NNT * 1024;         // staged v, per value tile: 32 rows x 16 columns
  static constexpr int OFF_SET = 0;
  static constexpr int OFF_WO = OFF_SET + 3 * SET_BYTES;
  static constexpr int OFF_A = OFF_WO + 2 * WO_BYTES;  // diagonal blocks of A (fp32), W scratch
  // per inverse wave: D^T and D (16 x 20 fp32 each) and M^T (8 x 12 fp32) of the blocked inverse
  static constexpr int WS_LD = 20, WS_MLD = 12;
  static constexpr int WS_BYTES = (2 * 16 * WS_LD + 8 * WS_MLD) * 4;
  static constexpr int OFF_WS = OFF_A + CD * LD_A * 4;
  static constexpr int OFF_VRAW = OFF_WS + 2 * WS_BYTES;
  static constexpr int OFF_FLAG = OFF_VRAW + 3 * VRAW_BUF;
  static constexpr int TOTAL = OFF_FLAG + 3 * NE;     // slow flags: one byte per E wave and block slot
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
  static_assert(KD % 32 == 0 && KD <= 128 && (C == 16 || C == 32) && NNT <= NV, "tile shape");
  static_assert(SET_BYTES % 16 == 0 && WO_BYTES % 16 == 0 && OFF_A % 16 == 0 && OFF_WS % 16 == 0 && OFF_VRAW % 16 == 0 &&
                    SET_G0 % 16 == 0,
                "16-byte alignment");
};

// LDS of the fused output norm, after the walk's own regions.  The output of a block is
// held for D steps (until the other value tile's sums of squares of its tokens have
// arrived): per block slot, each V wave's 32 x 16 bf16 output tile in its lanes' order
// (16 bytes per lane) and, per token, 16 partial sums of squares (one per V wave and
// lane group of 4 columns, contiguous), the tile's per-token totals, and the other
// tile's words for the block (prefetched by DMA); plus the weight row of the tile.
template <int KD, int VT, int C>
struct PnCfg {
  using Cfg = PcCfg<KD, VT, C>;
  static constexpr int D = 4, NH = 5;                 // steps a block is held; slots (> D)
  static constexpr int NPS = 2;                       // partial-sum slots (folded a step later)
  static constexpr int HELD_SLOT = Cfg::NV * 1024;
  static constexpr int NPART = Cfg::NV * 4;           // partial sums per token
  static constexpr int PSUM_SLOT = 32 * NPART * 4;
  static constexpr int OFF_HELD = round_up(Cfg::TOTAL, 16);
  static constexpr int OFF_PSUM = OFF_HELD + NH * HELD_SLOT;
  static constexpr int OFF_NW = OFF_PSUM + NPS * PSUM_SLOT;
  static constexpr int OFF_WSUM = OFF_NW + Cfg::VD * 4;   // [slot][32] fp32 totals
  static constexpr int TOTAL = OFF_WSUM + NH * 32 * 4;
  // (the prefetched words, [slot][32] x 8 bytes, are an LDS object of their own: a DMA in
  // flight into them then holds up no other LDS access of the issuing wave)
  static constexpr int PW_WORDS = NH * 32;
  static_assert(NH > D, "norm slots");
  __device__ static int slot(int b) { return b % NH; }
};

// Workspace of the fused norm when a head has two value tiles: a header (word 0: status,
// word 1: call epoch), then per (head, tile, block, token) one 8-byte word {sum of
// squares of the tile's outputs (fp32 bits), epoch}.
constexpr int PN_HEADER = 256;
constexpr int PN_MAX_HEADS = 128;               // heads per launch: both tiles resident
constexpr unsigned PN_STATUS_TIMEOUT = 1;       // a wait for the other tile's sums ran out

// Storage position of contraction index x inside its 32-wide slice: the indices
// {4g..4g+3, 16+4g..16+4g+3} that lane group g supplies to an MFMA are made contiguous.
__device__ __forceinline__ constexpr int perm32(int x) {
  return (x & ~31) + ((x & 15) >> 2) * 8 + ((x & 16) >> 2) + (x & 3);
}

// MFMA operand rows [row0, row0+16) over the contraction slice [d0, d0+32) (d0 a multiple
// of 32) from a tile stored in perm32 order: lane (g, l16) gets row row0 + l16, slots 0..3
// = index d0+4g.., slots 4..7 = index d0+16+4g.. -- the accumulator-compatible order.
__device__ __forceinline__ short8 lds_frag(const bf16_t* base, int ld, int row0, int d0, int lane) {
  return *reinterpret_cast<const short8*>(base + (row0 + (lane & 15)) * ld + d0 + 8 * (lane >> 4));
}

// The same fragment for the transpose of a [contraction index][row] tile whose columns
// are stored in perm32 order (as the [token][channel] tiles are): rows [row0, row0+16)
// (row0 a multiple of 16) are columns of the tile, the 32 contraction indices d0.. its
// rows, in the natural order.  Two transposing reads: in each group of 16 lanes, lane
// 4r + m reads row (d0 + 4g + r) (then d0 + 16 + 4g + r) at the four columns of rows
// row0 + 4m..+3, which perm32 keeps adjacent, and lane j of the group receives the
// column of row row0 + j of the four rows.
__device__ __forceinline__ short8 lds_frag_tr(const bf16_t* base, int ld, int row0, int d0, int lane) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  const int g = lane >> 4, r = (lane >> 2) & 3, m = lane & 3;
  const bf16_t* p = base + (d0 + 4 * g + r) * ld + perm32(row0) + 8 * m;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(__attribute__((address_space(3))) const void*)p);
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(__attribute__((address_space(3))) const void*)(p + 16 * ld));
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 8 bytes at buffer offset `off`, device scope (sc1): misses the CU's vector cache and
// reads L2, so another workgroup's stores on the same XCD are seen.
__device__ __forceinline__ u32x2 load_b64_dev(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16);
}


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
// Two 4-byte LDS writes in one instruction, a at byte offset OFF0 from lds and b at OFF1
// (multiples of 4 below 1024).  Written as asm so that the pairing is exactly this one; the
// compiler does not count it among the wave's LDS operations, so the writer waits for
// them itself (s_waitcnt lgkmcnt(0) in asm) before its next barrier.
template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_write2_b32(const void* lds, uint32_t a, uint32_t b) {
  static_assert(OFF0 % 4 == 0 && OFF1 % 4 == 0 && OFF0 / 4 < 256 && OFF1 / 4 < 256, "ds_write2_b32 offsets");
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("ds_write2_b32 %0, %1, %2 offset0:%3 offset1:%4" ::"v"(addr), "v"(a), "v"(b), "i"(OFF0 / 4),
               "i"(OFF1 / 4)
               : "memory");
}
__device__ __forceinline__ void lds_wait_asm() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until this wave's outstanding LDS operations have completed.
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Make this wave's earlier LDS writes visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// For the values a_j of `a` held by the lanes 16j + (lane % 16), j = 0..3: their total
// (a_0 + a_1) + (a_2 + a_3) in every lane, and in lane 16g + (lane % 16) the sum of the
// a_j with j < g (two permlane swaps, no LDS).  The 16-lane swap of a with itself leaves
// (a_0, a_0, a_2, a_2) and (a_1, a_1, a_3, a_3) over the four rows of 16 lanes; the
// 32-lane swap of their sum leaves (a_0 + a_1) and (a_2 + a_3) in every row.
__device__ __forceinline__ void quarter_scan(float a, int g, float& total, float& excl) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  const float e = __uint_as_float(r16[0]);
  const float p = e + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  const float p01 = __uint_as_float(r32[0]), p23 = __uint_as_float(r32[1]);
  total = p01 + p23;
  excl = ((g & 1) ? e : 0.0f) + ((g & 2) ? p01 : 0.0f);
}

// One block of nval tokens starting at token t0 of a head, token by token, for a wave
// that owns every key row of 16 value columns (lane = 16g + l16 holds column v0 + col,
// rows 16*mt + 4g + r) and keeps them in LDS at stl (row tile mt at stl + 256 * mt):
//   S' = diag(alpha) S,  e = beta (v - S'^T k),  S = S' + k e^T,  o = S^T q_hat.
// Both reductions over K stay inside the wave.  Used for blocks whose decay is too
// strong for the factorised MFMA path; kept out of line so that the register budget of
// the walk is not shaped by this rare path.  Pointers are the head's rows; operands come
// through buffer resources, four key channels per load.
template <int NMT, bool SG>
__device__ __attribute__((noinline)) void token_block(float* stl, const bf16_t* q, const bf16_t* k,
                                                     const bf16_t* v, const bf16_t* z, const bf16_t* beta,
                                                     const float* dt_bias, bf16_t* o, int T, int K, int V, int v0,
                                                     int vcols, int t0, int nval, float mult2, float scale,
                                                     int lane, int col, bf16_t* held, float* psum) {
  constexpr unsigned kOOB = 0xFFFFFFF0u;
  const int g = lane >> 4;
  const __amdgpu_buffer_rsrc_t tz = make_rsrc(z, (unsigned)(T * (SG ? 1 : K) * 2));
  const __amdgpu_buffer_rsrc_t tk = make_rsrc(k, (unsigned)(T * K * 2));
  const __amdgpu_buffer_rsrc_t tq = make_rsrc(q, (unsigned)(T * K * 2));
  const __amdgpu_buffer_rsrc_t tv = make_rsrc(v, (unsigned)(T * V * 2));
  const __amdgpu_buffer_rsrc_t tbe = make_rsrc(beta, (unsigned)(T * 2));
  const __amdgpu_buffer_rsrc_t tdb = make_rsrc(dt_bias, dt_bias ? (SG ? 4u : K * 4) : 0u);
  const float dtbs = (SG && dt_bias) ? dt_bias[0] : 0.0f;   // the head's one bias (SG)
  const __amdgpu_buffer_rsrc_t to = make_rsrc(o, o ? (unsigned)(T * V * 2) : 0u);
  auto elem = [](u32x2 w, int r) __attribute__((always_inline)) {
    const uint32_t u = r < 2 ? w.x : w.y;
    return __uint_as_float((r & 1) ? (u & 0xffff0000u) : (u << 16));
  };
  for (int i = 0; i < nval; ++i) {
    const int tok = t0 + i;
    const float vv =
        col < vcols ? bf2f(__builtin_amdgcn_raw_buffer_load_b16(tv, (unsigned)((tok * V + v0 + col) * 2), 0, 0)) : 0.0f;
    const float bt = bf2f(__builtin_amdgcn_raw_buffer_load_b16(tbe, (unsigned)(tok * 2), 0, 0));
    const float zs = SG ? bf2f(__builtin_amdgcn_raw_buffer_load_b16(tz, (unsigned)(tok * 2), 0, 0)) : 0.0f;
    float rp = 0.0f;
    for (int mt = 0; mt < NMT; ++mt) {        // S' = diag(alpha) S, partial S'^T k
      const int c0 = 16 * mt + 4 * g;
      const bool ok = c0 < K;                 // K is a multiple of 4
      const unsigned off = ok ? (unsigned)((tok * K + c0) * 2) : kOOB;
      const u32x2 zz = SG ? u32x2{0u, 0u} : __builtin_amdgcn_raw_buffer_load_b64(tz, off, 0, 0);
      const u32x2 kk = __builtin_amdgcn_raw_buffer_load_b64(tk, off, 0, 0);
      const floatx4 db =
          SG ? floatx4{dtbs, dtbs, dtbs, dtbs}
             : __builtin_bit_cast(floatx4,
                                  __builtin_amdgcn_raw_buffer_load_b128(tdb, ok ? (unsigned)(c0 * 4) : kOOB, 0, 0));
      floatx4 st = *reinterpret_cast<const floatx4*>(stl + mt * 256);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[r] *= ok ? fast_exp2(-mult2 * softplus_f((SG ? zs : elem(zz, r)) + db[r], true)) : 0.0f;
        rp += st[r] * elem(kk, r);
      }
      *reinterpret_cast<floatx4*>(stl + mt * 256) = st;
    }
    rp += __shfl_xor(rp, 16);
    rp += __shfl_xor(rp, 32);
    const float e = bt * (vv - rp);
    float op = 0.0f;
    for (int mt = 0; mt < NMT; ++mt) {        // S += beta k e^T, partial S^T q_hat
      const int c0 = 16 * mt + 4 * g;
      const unsigned off = c0 < K ? (unsigned)((tok * K + c0) * 2) : kOOB;
      const u32x2 kk = __builtin_amdgcn_raw_buffer_load_b64(tk, off, 0, 0);
      const u32x2 qq = __builtin_amdgcn_raw_buffer_load_b64(tq, off, 0, 0);
      floatx4 st = *reinterpret_cast<const floatx4*>(stl + mt * 256);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[r] += elem(kk, r) * e;
        op += st[r] * (scale * elem(qq, r));
      }
      *reinterpret_cast<floatx4*>(stl + mt * 256) = st;
    }
    op += __shfl_xor(op, 16);
    op += __shfl_xor(op, 32);
    if (held) {
      // fused norm: into the held tile, in the lane order of the MFMA path (token i of
      // the block at lane (i % 16) + 16 * (column % 16 / 4), half i / 16, element column % 4),
      // and the token's sum of squares over this wave's 16 columns
      if (g == 0) held[((i & 15) + 16 * ((col & 15) >> 2)) * 8 + (i >> 4) * 4 + (col & 3)] = f2bf(op);
      float sq = col < vcols ? op * op : 0.0f;
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
      sq += __shfl_xor(sq, 4);
      sq += __shfl_xor(sq, 8);
      if (lane < 4) psum[i * 16 + lane] = lane == 0 ? sq : 0.0f;   // this wave's 4 partials
    } else if (g == 0 && col < vcols) {
      __builtin_amdgcn_raw_buffer_store_b16(f2bf(op), to, (unsigned)((tok * V + v0 + col) * 2), 0, 0);
    }
  }
}

template <int KD, int VT, int C, bool SG, bool NORM = false>
__global__ void __launch_bounds__(1024)
chunk_fwd_pc_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                    const bf16_t* __restrict__ z, const float* __restrict__ A_log,
                    const float* __restrict__ dt_bias, const bf16_t* __restrict__ beta,
                    const float* state_in, float scale, bf16_t* __restrict__ o, float* state_out, int H, int T,
                    int K, int V, int n_vtiles, int total_wg, float thresh, const float* __restrict__ norm_w,
                    float eps, unsigned char* __restrict__ work, unsigned long long spin_ticks, int head0,
                    int nlaunch) {
  using Cfg = PcCfg<KD, VT, C>;
  using Pn = PnCfg<KD, VT, C>;
  constexpr int SMEM = NORM ? Pn::TOTAL : Cfg::TOTAL;
  static_assert(!NORM || (C == 32 && Pn::TOTAL + Pn::PW_WORDS * 8 <= 160 * 1024), "norm: 32-token blocks, LDS budget");
  constexpr int CD = Cfg::CD, NB = Cfg::NB, NNT = Cfg::NNT, NMT = Cfg::NMT;
  constexpr int LD_TK = Cfg::LD_TK, LD_CT = Cfg::LD_CT, LD_A = Cfg::LD_A;
  constexpr int NS = KD / 32;                         // 32-deep channel slices
  // E waves split each channel pair between two waves when KD <= 64 (per-channel gate)
  constexpr bool PSPLIT = KD <= 64 && !SG;
  constexpr int NTHR = Cfg::NWAVES * 64;

  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ __attribute__((aligned(16))) u32x2 s_pw[NORM ? Pn::PW_WORDS : 1];
  float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
  unsigned char* sFlag = reinterpret_cast<unsigned char*>(smem + Cfg::OFF_FLAG);   // [block % 3][E wave]
  // Buffer offsets of block b, passed through an empty asm so that the compiler keeps them
  // as one uniform term and folds each tile's constant offset into its LDS instructions.
  auto set_at = [&](int slot) __attribute__((always_inline)) {
    int off = __builtin_amdgcn_readfirstlane(slot * Cfg::SET_BYTES);
    asm volatile("" : "+s"(off));
    return smem + Cfg::OFF_SET + off;
  };
  auto set_base = [&](int b) __attribute__((always_inline)) { return set_at(b % 3); };
  auto wo_base = [&](int b) __attribute__((always_inline)) {
    int off = __builtin_amdgcn_readfirstlane((b & 1) * Cfg::WO_BYTES);
    asm volatile("" : "+s"(off));
    return smem + Cfg::OFF_WO + off;
  };
  auto flags_raw = [&](int b) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x2*>(sFlag + (b % 3) * Cfg::NE);
  };
  auto any_flag = [](u32x2 f) __attribute__((always_inline)) { return (f.x | f.y) != 0u; };
  auto slow_of = [&](int b) __attribute__((always_inline)) { return any_flag(flags_raw(b)); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

  int bh, v0, role = 0;
  bool paired = false;                         // fused norm over two value tiles
  if constexpr (NORM) {
    // the two tiles of head head0 + 8g + j are workgroups 16g + j and 16g + j + 8, which
    // the hardware places on one XCD (workgroup i runs on XCD i % 8): they share its L2
    if (n_vtiles == 2) {
      const int pr = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
      if (pr >= nlaunch) return;
      role = (blockIdx.x >> 3) & 1;
      bh = head0 + pr;
      paired = true;
    } else {
      if ((int)blockIdx.x >= nlaunch) return;
      bh = head0 + blockIdx.x;
    }
    v0 = role * VT;
  } else {
    int p = blockIdx.x;
    if ((total_wg & 7) == 0) p = (blockIdx.x & 7) * (total_wg >> 3) + (blockIdx.x >> 3);
    bh = p / n_vtiles;
    v0 = (p % n_vtiles) * VT;
  }
  const int h = bh % H;
  const int vcols = min(VT, V - v0);
  const size_t tb = (size_t)bh * T;
  const int nck = (T + C - 1) / C;

  for (int i = tid; i < SMEM / 16; i += NTHR) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);

  const float gmul = gate_multiplier(A_log[h]);
  const float mult2 = gmul * kLog2e;
  constexpr unsigned kOOB = 0xFFFFFFF0u;       // a buffer offset past any range: reads zeros
  lds_barrier();                               // LDS cleared before any DMA lands

  if (wave < Cfg::NE) {
    // ================================================================ E waves
    // Wave e covers tokens 16*half .. 16*half+15 of each block (half = e / 4) and key
    // channels 32*(e % 4) .. +31.  The block's decay reference sits between its two
    // halves, so a half needs nothing from the other one: the first half's exponents
    // are minus the decay still to come before the reference, the second half's are
    // the decay since it.  With KD <= 64 (per-channel gate) the waves that would hold
    // no channels take half of the others' instead: waves 2j and 2j + 1 of a half share
    // the 32 channels of group j, each the even or the odd channel of every pair (par),
    // so that each E wave does half the work of the KD = 128 mapping.
    const int half = wave >> 2;
    const int cw = PSPLIT ? (wave & 3) >> 1 : wave & 3;
    const int par = PSPLIT ? wave & 1 : 0;     // the lane's channel of its pair (PSPLIT)
    const int pair = 16 * cw + l16;            // key-channel pair
    const int pos = g;                          // quarter of the half: tokens 16*half + tq .. +3
    const int tq = 4 * pos;
    const bool kact = KD == 128 || 2 * pair < K;  // (K = KD = 128: every pair is a channel pair)
    // the precise softplus for strong gates (its small values matter once multiplied) and
    // for a zero multiplier (softplus2_direct can be +inf)
    const bool precise = !(gmul > 0.0f) || gmul > 64.0f;
    // dt_bias in log2 units: the gate is taken as -gmul softplus2(z log2(e) + dt_bias log2(e))
    // (PSPLIT: dtb0 is the lane's own channel)
    const float dtb0 = (kact && dt_bias) ? dt_bias[SG ? h : h * K + 2 * pair + par] * kLog2e : 0.0f;
    const float dtb1 = (kact && dt_bias) ? dt_bias[SG ? h : h * K + 2 * pair + 1] * kLog2e : 0.0f;
    // per-head buffer resources: offsets past the head's T tokens read as 0
    const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(k + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_z = SG ? make_rsrc(z + tb, (unsigned)(T * 2)) : make_rsrc(z + tb * K, (unsigned)(T * K * 2));

    // k, q, z of this lane's channel pair and four tokens, loaded two blocks ahead into one
    // of three register sets: block b lives in set b % 3, so a load never targets registers
    // whose previous contents are still to be read, and each load has two steps to arrive
    // (one step is about an HBM round trip under this kernel's load; measured, a step-ahead
    // prefetch left the E waves waiting).  These 12 loads per block are the E waves' only
    // memory operations, so the wait for a set leaves the two younger ones in flight.
    // (SG: the gate inputs stay 16-bit until they are used one step later, so that nothing
    // consumes a load in the step that issues it)
    typedef typename std::conditional<SG, unsigned short, uint32_t>::type ZRaw;
    struct Raw {
      uint32_t k[4], q[4];
      ZRaw z[4];
    };
    // Byte offset of the lane's first row in block 0.  Lanes without a channel pair or
    // without token rows (the second half when C = 16) start at 2^31, past any head's range
    // (a head's rows, plus the two blocks past its end that the prefetch reaches, stay below
    // 2^31 bytes: the boundary checks T + 64 tokens): they read zeros.
    const int rowb = (KD >= 64 ? KD : K) * 2;  // bytes per token row (K = KD unless KD = 32)
    const unsigned vbase = (kact && 16 * half < C) ? (unsigned)((16 * half + tq) * rowb + 4 * pair) : 0x80000000u;
    // SG: byte offset of the lane's first gate value (one bf16 per token) in block 0
    const unsigned zbase = (kact && 16 * half < C) ? (unsigned)((16 * half + tq) * 2) : 0x80000000u;
    // this lane's channel pair (PSPLIT: its channel) in a per-channel fp32 array, bytes
    const int dpoff = kact ? (PSPLIT ? 4 * (2 * pair + par) : 8 * pair) : 0;
    // element offset of the lane's first token row and channel pair in a [token][channel] tile
    const int rowoff = (16 * half + tq) * LD_TK + perm32(2 * pair);
    auto load_qkz = [&](int b, Raw& r) __attribute__((always_inline)) {
      unsigned off = vbase + (unsigned)(b * C * rowb);
      asm volatile("" : "+v"(off));            // one register; the row steps become immediates
      unsigned zoff = zbase + (unsigned)(b * C * 2);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        r.k[t] = buf_load_b32(rs_k, off + t * rowb);
        r.q[t] = buf_load_b32(rs_q, off + t * rowb);
        if constexpr (SG) r.z[t] = __builtin_amdgcn_raw_buffer_load_b16(rs_z, zoff + t * 2, 0, 0);
        else r.z[t] = buf_load_b32(rs_z, off + t * rowb);
      }
    };

    // e1 handles block b, whose buffers sit in slot sl = b % 3 (slp = (b - 1) % 3), for the
    // wave's half HALF (= half, as a constant: each half has its own code)
    auto e1 = [&](auto precise_tag, auto half_tag, auto tail_tag, int b, int sl, int slp, const Raw& cur,
                  Raw& nxt) __attribute__((always_inline)) {
      constexpr bool PRECISE = decltype(precise_tag)::value;
      constexpr int HALF = decltype(half_tag)::value;
      constexpr bool TAIL = decltype(tail_tag)::value;   // the block may hold identity tokens
      const int tn = b * C;
      const int nval = min(C, T - tn);
      char* sb = set_at(sl);
      bf16_t* sKE = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KE);
      bf16_t* sQE = reinterpret_cast<bf16_t*>(sb + Cfg::SET_QE);
      bf16_t* sKR = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KR);
      float* sG0 = reinterpret_cast<float*>(sb + Cfg::SET_G0);
      float* sD0 = reinterpret_cast<float*>(sb + Cfg::SET_D0);
      (void)nxt;                               // (loaded by the step: see estep)
      // D0 of the previous block, for its F (first half only; written a step ago).  Read
      // first and used before this step's first LDS write, so that the wait for it is for
      // it alone.
      float2 dprev = float2{0.0f, 0.0f};
      if constexpr (HALF == 0) dprev = *reinterpret_cast<const float2*>(set_at(slp) + Cfg::SET_D0 + dpoff);
      Pair<bf16_t> rk[4], rq[4], rz[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        rk[t].u = cur.k[t];
        rq[t].u = cur.q[t];
        if constexpr (SG) rz[t] = Pair<bf16_t>::dup((bf16_t)cur.z[t]);
        else rz[t].u = cur.z[t];
      }
      // Tokens at or past nval (a partial last block, or rows 16..31 when C = 16) are
      // identity tokens: their k and q read as 0, and z = -inf makes their gate 0.  (Blocks
      // known to be full skip the test: its merge would cost register copies on every step.)
      if (TAIL && nval < 16 * HALF + 16) {
        const int lim = nval - (16 * HALF + tq);
#pragma unroll
        for (int t = 0; t < 4; ++t) rz[t].u = t < lim ? rz[t].u : 0xFF80FF80u;
      }
      // gate in log2 units and its inclusive prefix over the lane's 4 tokens
      float px[4], py[4];
      float ax = 0.0f, ay = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float spx = fmaf(rz[t].x(), kLog2e, dtb0), spy = fmaf(rz[t].y(), kLog2e, dtb1);
        ax = fmaf(-gmul, PRECISE ? softplus2_f(spx, true) : softplus2_direct(spx), ax);
        if constexpr (SG) ay = ax;             // one gate per token: both channels share it
        else ay = fmaf(-gmul, PRECISE ? softplus2_f(spy, true) : softplus2_direct(spy), ay);
        px[t] = ax;
        py[t] = ay;
      }
      // Quarter sums of this half for the lane's channel pair (lanes l16 + 16j, j = 0..3):
      // the sum over the half, and the sum over the quarters before the lane's own.
      float sumx, sumy, exx, exy;
      quarter_scan(ax, g, sumx, exx);
      if constexpr (SG) {
        sumy = sumx;
        exy = exx;
      } else {
        quarter_scan(ay, g, sumy, exy);
      }
      // exponent of token t relative to the reference: G_t - m = px[t] + off (the first
      // half counts back from the reference, the second forward from it)
      const float offx = HALF == 0 ? exx - sumx : exx;
      const float offy = HALF == 0 ? exy - sumy : exy;
      // first half: G0 = 2^m, and F = D0 G0 of the previous block
      float2 g0 = float2{0.0f, 0.0f}, fp = float2{0.0f, 0.0f};
      if constexpr (HALF == 0) {
        g0 = float2{fast_exp2(sumx), fast_exp2(sumy)};
        fp = float2{dprev.x * g0.x, dprev.y * g0.y};
      }
      const unsigned long long bal = __ballot(kact && fminf(sumx, sumy) < -thresh);
      if (lane == 0) sFlag[sl * Cfg::NE + wave] = bal != 0ull ? 1 : 0;
      const int c = 2 * pair;
      if (HALF == 0 && kact && g == 0) {
        *reinterpret_cast<float2*>(sG0 + c) = g0;
        if (b > 0) *reinterpret_cast<float2*>(set_at(slp) + Cfg::SET_F + 4 * c) = fp;
      }
      if (kact) {
        float lx3 = 0.0f, ly3 = 0.0f;
        uint32_t wke[4], wqe[4], wkr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float ex = px[t] + offx, ey = py[t] + offy;
          const float Lx = fast_exp2(ex), Rx = fast_exp2(-ex);
          const float Ly = SG ? Lx : fast_exp2(ey), Ry = SG ? Rx : fast_exp2(-ey);
          const float kx = rk[t].x(), ky = rk[t].y(), qx = rq[t].x(), qy = rq[t].y();
          wke[t] = pack_bf16x2(-kx * Lx, -ky * Ly);   // KE is stored negated (V then needs no sign flip of v)
          wqe[t] = pack_bf16x2(qx * Lx, qy * Ly);
          wkr[t] = pack_bf16x2(kx * Rx, ky * Ry);
          if (t == 3) {
            lx3 = Lx;
            ly3 = Ly;
          }
        }
        // Rows t and t+2 in one instruction: the 64 bytes a group of 16 lanes writes to each
        // of the two rows then fall on distinct LDS banks (rows t and t+1, 288 bytes apart,
        // would share 8 of their 16 banks), and the lanes of groups g and g+1 (rows 4 apart)
        // cover all 64 banks once.
        constexpr int R1 = LD_TK * 2, R2 = 2 * R1, R3 = 3 * R1;   // row offsets in bytes
        lds_write2_b32<0, R2>(sKE + rowoff, wke[0], wke[2]);
        lds_write2_b32<R1, R3>(sKE + rowoff, wke[1], wke[3]);
        lds_write2_b32<0, R2>(sQE + rowoff, wqe[0], wqe[2]);
        lds_write2_b32<R1, R3>(sQE + rowoff, wqe[1], wqe[3]);
        lds_write2_b32<0, R2>(sKR + rowoff, wkr[0], wkr[2]);
        lds_write2_b32<R1, R3>(sKR + rowoff, wkr[1], wkr[3]);
        // D0 = 2^(G_last - m): the second half's last token, whose L it is
        if (HALF == 1 && g == 3) *reinterpret_cast<float2*>(sD0 + c) = float2{lx3, ly3};
      }
      lds_wait_asm();                          // the asm writes above, before the barrier
    };

    // The same for a PSPLIT wave: one channel (2 pair + par) of the lane's pair, so one
    // gate, one scan and two exponentials per token; the bf16 results of tokens t and
    // t + 2 are packed into one register and stored as two 16-bit halves.
    auto e1p = [&](auto precise_tag, auto half_tag, auto tail_tag, int b, int sl, int slp, const Raw& cur)
                   __attribute__((always_inline)) {
      constexpr bool PRECISE = decltype(precise_tag)::value;
      constexpr int HALF = decltype(half_tag)::value;
      constexpr bool TAIL = decltype(tail_tag)::value;
      const int tn = b * C;
      const int nval = min(C, T - tn);
      char* sb = set_at(sl);
      bf16_t* sKE = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KE);
      bf16_t* sQE = reinterpret_cast<bf16_t*>(sb + Cfg::SET_QE);
      bf16_t* sKR = reinterpret_cast<bf16_t*>(sb + Cfg::SET_KR);
      float* sG0 = reinterpret_cast<float*>(sb + Cfg::SET_G0);
      float* sD0 = reinterpret_cast<float*>(sb + Cfg::SET_D0);
      // the lane's bf16 of a pair word as fp32 bits (a byte permute: the low or the high
      // half into the high half, zeros below)
      const unsigned sel = par ? 0x03020c0cu : 0x01000c0cu;
      auto own = [&](uint32_t w) __attribute__((always_inline)) {
        return __uint_as_float(__builtin_amdgcn_perm(w, w, sel));
      };
      float zv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) zv[t] = own(cur.z[t]);
      float dprev = 0.0f;
      if constexpr (HALF == 0) dprev = *reinterpret_cast<const float*>(set_at(slp) + Cfg::SET_D0 + dpoff);
      if (TAIL && nval < 16 * HALF + 16) {     // identity tokens: gate 0
        const int lim = nval - (16 * HALF + tq);
#pragma unroll
        for (int t = 0; t < 4; ++t) zv[t] = t < lim ? zv[t] : -INFINITY;
      }
      float px[4];
      float ax = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float sp = fmaf(zv[t], kLog2e, dtb0);
        ax = fmaf(-gmul, PRECISE ? softplus2_f(sp, true) : softplus2_direct(sp), ax);
        px[t] = ax;
      }
      float sumx, exx;
      quarter_scan(ax, g, sumx, exx);
      const float offx = HALF == 0 ? exx - sumx : exx;
      float g0 = 0.0f, fp = 0.0f;
      if constexpr (HALF == 0) {
        g0 = fast_exp2(sumx);
        fp = dprev * g0;
      }
      const unsigned long long bal = __ballot(kact && sumx < -thresh);
      if (lane == 0) sFlag[sl * Cfg::NE + wave] = bal != 0ull ? 1 : 0;
      const int c = 2 * pair + par;
      if (HALF == 0 && kact && g == 0) {
        sG0[c] = g0;
        if (b > 0) *reinterpret_cast<float*>(set_at(slp) + Cfg::SET_F + 4 * c) = fp;
      }
      if (kact) {
        float l3 = 0.0f;
        uint32_t wke[2], wqe[2], wkr[2];       // tokens t (low half) and t + 2 (high half)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float ke[2], qe[2], kr[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int tt = t + 2 * u;
            const float ex = px[tt] + offx;
            const float L = fast_exp2(ex), Rr = fast_exp2(-ex);
            const float kv = own(cur.k[tt]), qv = own(cur.q[tt]);
            ke[u] = -kv * L;                   // KE is stored negated (see e1)
            qe[u] = qv * L;
            kr[u] = kv * Rr;
            if (tt == 3) l3 = L;
          }
          wke[t] = pack_bf16x2(ke[0], ke[1]);
          wqe[t] = pack_bf16x2(qe[0], qe[1]);
          wkr[t] = pack_bf16x2(kr[0], kr[1]);
        }
        auto put2 = [&](bf16_t* tile, const uint32_t* w) __attribute__((always_inline)) {
          unsigned short* e = reinterpret_cast<unsigned short*>(tile + rowoff + par);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            e[t * LD_TK] = (unsigned short)w[t];
            e[(t + 2) * LD_TK] = (unsigned short)(w[t] >> 16);
          }
        };
        put2(sKE, wke);
        put2(sQE, wqe);
        put2(sKR, wkr);
        // D0 = 2^(G_last - m): the second half's last token, whose L it is
        if (HALF == 1 && g == 3) sD0[c] = l3;
      }
    };

    Raw ra, rb, rc;
    load_qkz(0, ra);                           // (blocks past the end read zeros)
    load_qkz(1, rb);
    auto estep = [&](auto tail_tag, int s, int sl, int slp, Raw& cur, Raw& nxt) __attribute__((always_inline)) {
      using TT = decltype(tail_tag);
      const int b = s + 2;
      // The loads of the block after next, issued by every step alike (the index is clamped;
      // blocks past the end read zeros), so that the compiler sees the same load count on
      // every path and waits for the oldest set only.
      load_qkz(min(b + 2, nck + 1), nxt);
      sched_fence();
      if (b < nck) {
        using H0 = std::integral_constant<int, 0>;
        using H1 = std::integral_constant<int, 1>;
        if constexpr (PSPLIT) {
          if (precise) {
            if (half) e1p(std::true_type{}, H1{}, TT{}, b, sl, slp, cur);
            else e1p(std::true_type{}, H0{}, TT{}, b, sl, slp, cur);
          } else {
            if (half) e1p(std::false_type{}, H1{}, TT{}, b, sl, slp, cur);
            else e1p(std::false_type{}, H0{}, TT{}, b, sl, slp, cur);
          }
        } else if (precise) {
          if (half) e1(std::true_type{}, H1{}, TT{}, b, sl, slp, cur, nxt);
          else e1(std::true_type{}, H0{}, TT{}, b, sl, slp, cur, nxt);
        } else {
          if (half) e1(std::false_type{}, H1{}, TT{}, b, sl, slp, cur, nxt);
          else e1(std::false_type{}, H0{}, TT{}, b, sl, slp, cur, nxt);
        }
      }
      lds_barrier();
    };
    // three steps per iteration, so that register sets and LDS slots are fixed per position:
    // step s handles block s + 2 (set and slot (s + 2) % 3) and loads block s + 4.  The loops
    // run whole iterations only (no conditional step inside them), the last one or two steps
    // follow them: nck + 2 steps in all, as for the other stages.  The first loop covers the
    // iterations whose three blocks hold 32 real tokens each (none when C = 16, where the
    // second half of every block is identity tokens).
    const std::true_type tail{};
    const std::false_type full{};
    const int nfull = C == 32 ? T / C : 0;
    int s = -2;
    for (; s + 4 < nfull; s += 3) {
      estep(full, s, 0, 2, ra, rc);
      estep(full, s + 1, 1, 0, rb, ra);
      estep(full, s + 2, 2, 1, rc, rb);
    }
    for (; s + 2 < nck; s += 3) {
      estep(tail, s, 0, 2, ra, rc);
      estep(tail, s + 1, 1, 0, rb, ra);
      estep(tail, s + 2, 2, 1, rc, rb);
    }
    if (s < nck) estep(tail, s, 0, 2, ra, rc);
    if (s + 1 < nck) estep(tail, s + 1, 1, 0, rb, ra);
  } else if (wave >= Cfg::NE + Cfg::NV) {
    // ================================================================ W waves
    __builtin_amdgcn_s_setprio(2);             // issue ahead of the E waves (see the V waves)
    const int ww = wave - (Cfg::NE + Cfg::NV);
    // The W waves also stage the next blocks' inputs that are not per channel pair: the v
    // tile (waves 0 .. NNT-1 of the stage, 16 columns each, slot 2*row + half) and beta.
    // Each W wave loads beta of the rows its tiles scale (tokens 16*I + l16); the last one
    // loads all of the block's tokens and writes them to LDS for the V waves.  Both are
    // issued after the wave's last LDS read of a step and waited for at the start of the
    // next one, so their latency hides behind the barrier (an LDS DMA in flight would make
    // every LDS read wait for it).  Tokens past the head's range read as 0.
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(v + tb * V, (unsigned)(T * V * 2));
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(beta + tb, (unsigned)(T * 2));
    const int btok = ww == Cfg::NW - 1 ? lane : (ww == 0 ? 0 : 16) + l16;
    auto load_beta = [&](int b) __attribute__((always_inline)) {
      const unsigned off = btok < C ? (unsigned)((b * C + btok) * 2) : kOOB;
      return __builtin_amdgcn_raw_buffer_load_b16(rs_b, off, 0, 0);
    };
    auto dma_v = [&](int b) __attribute__((always_inline)) {
      if (ww < NNT) {
        const int r = lane >> 1, c0 = 16 * ww + 8 * (lane & 1);
        const unsigned off = (r < C && c0 < vcols) ? (unsigned)(((b * C + r) * V + v0 + c0) * 2) : kOOB;
        dma16(rs_v, smem + Cfg::OFF_VRAW + (b % 3) * Cfg::VRAW_BUF + ww * 1024, off);
      }
    };
    auto wstage = [&](int b, float rbeta) __attribute__((always_inline)) {
      char* sb = set_base(b);
      const bf16_t* sKE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KE);
      const bf16_t* sQE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_QE);
      const bf16_t* sKR = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KR);
      char* wb = wo_base(b);
      bf16_t* sP = reinterpret_cast<bf16_t*>(wb + Cfg::WO_P);
      bf16_t* sT = reinterpret_cast<bf16_t*>(wb + Cfg::WO_T);
      bf16_t* sA10 = reinterpret_cast<bf16_t*>(wb + Cfg::WO_A10);
      // tiles of this wave: ww 0: A_00; 1: A_11; 2: A_10 and P_00; 3: P_10 and P_11.
      // Each tile is computed transposed: lane (g, l16) holds row i = 16I + l16,
      // columns 16J + 4g..+3.  The two tiles of a wave share one operand, loaded once.
      auto frags = [&](const bf16_t* src, int row0, short8* f) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NS; ++s) f[s] = lds_frag(src, LD_TK, row0, 32 * s, lane);  // same depth order on both sides
      };
      auto dot = [&](const short8* fa, const short8* fb) __attribute__((always_inline)) {
        floatx4 acc = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = mfma_bf16(fa[s], fb[s], acc);
        return acc;
      };
      // kinds: 0 A_00, 1 A_10, 3 A_11, 4 P_00, 5 P_10, 6 P_11
      auto put = [&](int kind, floatx4 acc) __attribute__((always_inline)) {
        const bool isA = kind < 4;
        const int I = (kind == 0 || kind == 4) ? 0 : 1;
        const int J = (kind == 3 || kind == 6) ? 1 : 0;
        const int i = 16 * I + l16, j0 = 16 * J + 4 * g;
        float vals[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vals[r] = (isA ? j0 + r < i : j0 + r <= i) ? acc[r] : 0.0f;
        if (isA && I == J) {                   // diagonal block: fp32 for the inverse
          const float bi = -rbeta;             // beta of row i (the tile is -A: KE is stored negated)
          *reinterpret_cast<floatx4*>(sA + i * LD_A + j0) =
              floatx4{bi * vals[0], bi * vals[1], bi * vals[2], bi * vals[3]};
        } else if (isA) {                      // A_10: bf16, negated, for V
          const float nb = rbeta;              // (the tile is -A_10)
          store4_bf16(sA10 + l16 * LD_CT + perm32(j0), nb * vals[0], nb * vals[1], nb * vals[2], nb * vals[3]);
        } else {
          store4_bf16(sP + i * LD_CT + perm32(j0), vals[0], vals[1], vals[2], vals[3]);
        }
      };
      if (ww == 0 || (ww == 1 && NB == 2)) {   // A_II
        short8 fa[NS], fb[NS];
        frags(sKR, 16 * ww, fa);
        frags(sKE, 16 * ww, fb);
        sched_fence();
        put(ww == 0 ? 0 : 3, dot(fa, fb));
      } else if (ww == 2) {                    // A_10 and P_00: KR_0 shared
        short8 fa[NS], fb[NS], fc[NS];
        frags(sKR, 0, fa);
        frags(sQE, 0, fc);
        if (NB == 2) frags(sKE, 16, fb);
        sched_fence();
        put(4, dot(fa, fc));
        if (NB == 2) put(1, dot(fa, fb));
      } else if (ww == 3 && NB == 2) {         // P_10 and P_11: QE_1 shared
        short8 fa[NS], fb[NS], fc[NS];
        frags(sKR, 0, fa);
        frags(sKR, 16, fb);
        frags(sQE, 16, fc);
        sched_fence();
        put(5, dot(fa, fc));
        put(6, dot(fb, fc));
      }
      if (ww < NB) {
        // T_II = (I + N)^-1 for I = ww, N = A_II, in 8 x 8 blocks: with D = diag(T_a, T_b) the
        // inverses of the diagonal blocks, T = [[T_a, 0], [-T_b N_ba T_a, T_b]].
        //   1. lanes 0..15: lane j = 8h + jj forward-substitutes column jj of T_a (h = 0) or
        //      T_b (h = 1) -- seven rows, 28 FMAs -- and writes it to D^T (row j) and D;
        //   2. all lanes (k, j): M[k][j] = sum_l N_ba[k][l] T_a[l][j]  (8 FMAs);
        //   3. all lanes (i, j): T_ba[i][j] = -sum_k T_b[i][k] M[k][j]  (8 FMAs).
        // Each step reads what the previous one wrote in LDS (same wave: in order).
        const int I = ww;
        constexpr int WL = Cfg::WS_LD, ML = Cfg::WS_MLD;
        float* wsDT = reinterpret_cast<float*>(smem + Cfg::OFF_WS + I * Cfg::WS_BYTES);
        float* wsD = wsDT + 16 * WL;
        float* wsMT = wsD + 16 * WL;
        const float* Ab = sA + 16 * I * LD_A + 16 * I;
        wave_lds_fence();                      // this wave's A_II tile
        if (lane < 16) {
          const int h = lane >> 3, jj = lane & 7;
          const float* Nb = Ab + 8 * h * LD_A + 8 * h;   // diagonal 8 x 8 block h of N
          floatx4 rlo[8], rhi[8];
#pragma unroll
          for (int i = 1; i < 8; ++i) {
            rlo[i] = *reinterpret_cast<const floatx4*>(Nb + i * LD_A);
            rhi[i] = *reinterpret_cast<const floatx4*>(Nb + i * LD_A + 4);
          }
          float t[8];
          t[0] = jj == 0 ? 1.0f : 0.0f;
#pragma unroll
          for (int i = 1; i < 8; ++i) {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int m = 0; m < i; ++m) {
              const float nim = m < 4 ? rlo[i][m] : rhi[i][m - 4];
              if (m & 1) a1 = fmaf(nim, t[m], a1);
              else a0 = fmaf(nim, t[m], a0);
            }
            t[i] = i == jj ? 1.0f : -(a0 + a1);
          }
          float* dt = wsDT + lane * WL + 8 * h;          // D^T row j: column j of D
          *reinterpret_cast<floatx4*>(dt) = floatx4{t[0], t[1], t[2], t[3]};
          *reinterpret_cast<floatx4*>(dt + 4) = floatx4{t[4], t[5], t[6], t[7]};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            wsD[(8 * h + i) * WL + lane] = t[i];
            sT[(16 * I + 8 * h + i) * LD_CT + perm32(16 * I + lane)] = f2bf(t[i]);
          }
        }
        const int ki = lane >> 3, j = lane & 7;
        {
          const floatx4 n0 = *reinterpret_cast<const floatx4*>(Ab + (8 + ki) * LD_A);
          const floatx4 n1 = *reinterpret_cast<const floatx4*>(Ab + (8 + ki) * LD_A + 4);
          const floatx4 t0 = *reinterpret_cast<const floatx4*>(wsDT + j * WL);
          const floatx4 t1 = *reinterpret_cast<const floatx4*>(wsDT + j * WL + 4);
          float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
          for (int l = 0; l < 4; ++l) {
            m0 = fmaf(n0[l], t0[l], m0);
            m1 = fmaf(n1[l], t1[l], m1);
          }
          wsMT[j * ML + ki] = m0 + m1;         // M^T[j][k]
        }
        {
          const floatx4 b0 = *reinterpret_cast<const floatx4*>(wsD + (8 + ki) * WL + 8);
          const floatx4 b1 = *reinterpret_cast<const floatx4*>(wsD + (8 + ki) * WL + 12);
          const floatx4 c0 = *reinterpret_cast<const floatx4*>(wsMT + j * ML);
          const floatx4 c1 = *reinterpret_cast<const floatx4*>(wsMT + j * ML + 4);
          float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            u0 = fmaf(b0[k4], c0[k4], u0);
            u1 = fmaf(b1[k4], c1[k4], u1);
          }
          sT[(16 * I + 8 + ki) * LD_CT + perm32(16 * I + j)] = f2bf(-(u0 + u1));
        }
      }
    };
    bf16_t wbeta = 0;                          // beta of block b, this lane's token
    if (nck > 0) wbeta = load_beta(0);
    for (int s = -2; s < nck; ++s) {
      const int b = s + 1;
      wait_vm();                               // beta of block b, v of block b+1
      if (b >= 0 && b < nck) {
        if (!slow_of(b)) wstage(b, bf2f(wbeta));
        if (ww == Cfg::NW - 1 && lane < CD)
          reinterpret_cast<float*>(set_base(b) + Cfg::SET_BETA)[lane] = bf2f(wbeta);
      }
      if (b + 1 < nck) wbeta = load_beta(b + 1);
      if (s + 2 < nck) dma_v(s + 2);
      lds_barrier();
    }
  } else {
    // ================================================================ V waves
    // The state chain is the walk's critical path and shares each SIMD with two E waves
    // that have slack: the highest issue priority lets it go first whenever it is ready.
    __builtin_amdgcn_s_setprio(3);
    const int vw = wave - Cfg::NE;
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
    // Fused norm: this wave's 16 weights into LDS (1 without a weight row, 0 past the
    // tile's columns), the call's epoch from the workspace header.
    float* const nwl = reinterpret_cast<float*>(smem + Pn::OFF_NW);
    float* const psum = reinterpret_cast<float*>(smem + Pn::OFF_PSUM);
    unsigned epoch = 0;
    bool dead = false;                         // a wait for the other tile gave up
    if constexpr (NORM) {
      if (vact && lane < 16) {
        const int c = 16 * vw + lane;
        nwl[c] = c < vcols ? (norm_w ? norm_w[(size_t)h * V + v0 + c] : 1.0f) : 0.0f;
      }
      if (paired)
        epoch = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(work, 8u), 4, 0, 0));
    }
    // Complete the state loads here: inside the walk the wave's only vector-memory
    // operations are its output stores, which must never hold up the next step.
    wait_vm();
    // Between blocks the state is kept as S~ = diag(G0) S of the next block when that
    // block takes the MFMA path, and unscaled before a token-path block or at the end:
    // a block ends with one per-channel multiply of the state, by F = D0 G0' or by D0
    // (a token-path block by G0' or by nothing), and block 0 is scaled before the walk.
    // output rows of this head through a buffer resource: 32-bit offsets, no 64-bit
    // address arithmetic per store
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(o + tb * V, o ? (unsigned)(T * V * 2) : 0u);

    // Fused norm.  Words of value tile `tile` of this head: one per (block, token).
    auto ring_rsrc = [&](int tile) __attribute__((always_inline)) {
      const size_t row = (size_t)nck * 256;
      return make_rsrc(work + PN_HEADER + ((size_t)bh * 2 + tile) * row, (unsigned)row);
    };
    float* const wsum = reinterpret_cast<float*>(smem + Pn::OFF_WSUM);
    u32x2* const pwd = s_pw;
    // per-token total of this tile's partial sums of block b
    auto tile_sum = [&](int b, int t) __attribute__((always_inline)) {
      const float* ps = psum + (b & (Pn::NPS - 1)) * (32 * Pn::NPART) + t * Pn::NPART;
      float x = 0.0f;
#pragma unroll
      for (int w = 0; w < Pn::NPART; w += 4) {
        const floatx4 y = *reinterpret_cast<const floatx4*>(ps + w);
        x += (y[0] + y[1]) + (y[2] + y[3]);
      }
      return x;
    };
    // Wave 0 at step b+1: the tile's per-token sums of squares of block b (the V waves wrote
    // their partial sums during step b) into LDS, and, with two tiles, to the workspace: one
    // 8-byte store per token, sum and epoch together.
    auto norm_export = [&](int b) __attribute__((always_inline)) {
      if (lane < 32) {
        const float t = tile_sum(b, lane);
        wsum[Pn::slot(b) * 32 + lane] = t;
        if (paired)
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(t), epoch}, ring_rsrc(role),
                                                (unsigned)((b * 32 + lane) * 8), 0, 0);
      }
    };
    // Wave 0 at the end of step b+2: the other tile's words of block b (published at the
    // start of its step b+1) into LDS (DMA, device scope); waited for at the end of step
    // b+3, before its barrier; read at the end of step b+4.
    auto norm_prefetch = [&](int b) __attribute__((always_inline)) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ring_rsrc(1 - role),
                                               (__attribute__((address_space(3))) void*)(pwd + Pn::slot(b) * 32),
                                               4, (unsigned)(b * 256 + lane * 4), 0, 0, 16);
    };
    // y = o / sqrt(mean(o^2) + eps) * w for the held block bn: the sums of this tile from
    // LDS, those of the other tile from its words (waiting, bounded, until both of the
    // lane's words carry this call's epoch), then the stores.
    // own: this tile's totals are in LDS (exported before a barrier); else summed here.
    // pre: the other tile's words were prefetched into LDS; else (or if they were not yet
    // there) they are read, and waited for, directly.
    auto norm_out = [&](int bn, bool own, bool pre) __attribute__((always_inline)) {
      const int slot = Pn::slot(bn);
      const int lg = lane >> 4, ll = lane & 15;
      float s0, s1;
      if (own) {
        s0 = wsum[slot * 32 + ll];
        s1 = wsum[slot * 32 + 16 + ll];
      } else {
        s0 = tile_sum(bn, ll);
        s1 = tile_sum(bn, 16 + ll);
      }
      if (paired) {
        const __amdgpu_buffer_rsrc_t rp = ring_rsrc(1 - role);
        const unsigned off0 = (unsigned)((bn * 32 + ll) * 8), off1 = off0 + 128;
        u32x2 a, c;
        if (pre) {
          // (through asm: the compiler would make these reads wait for the DMA into the
          // next slot, which is still in flight and which they do not touch)
          const unsigned pa =
              (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)(pwd + slot * 32 + ll);
          asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %2 offset:128\n\ts_waitcnt lgkmcnt(0)"
                       : "=&v"(a), "=&v"(c)
                       : "v"(pa)
                       : "memory");
        }
        if (!pre || (!dead && __ballot(a.y != epoch || c.y != epoch) != 0ull)) {
          a = load_b64_dev(rp, off0);
          c = load_b64_dev(rp, off1);
        }
        // (a zero bound gives up at once, whether or not the words are there yet)
        if (!dead && (spin_ticks == 0 || __ballot(a.y != epoch || c.y != epoch) != 0ull)) {
          dead = spin_ticks == 0;
          const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
          while (!dead) {
            __builtin_amdgcn_s_sleep(1);
            asm volatile("" ::: "memory");     // the loads below are repeated, not hoisted
            a = load_b64_dev(rp, off0);
            c = load_b64_dev(rp, off1);
            if (__ballot(a.y != epoch || c.y != epoch) == 0ull) break;
            dead = __builtin_amdgcn_s_memrealtime() - t0 > spin_ticks;
          }
          if (dead && lane == 0) __builtin_amdgcn_raw_buffer_store_b32(PN_STATUS_TIMEOUT, make_rsrc(work, 8u), 0, 0, 0);
        }
        s0 += __uint_as_float(a.x);
        s1 += __uint_as_float(c.x);
      }
      const float inv_v = 1.0f / (float)V;
      const float r0 = rsqrtf(fmaf(s0, inv_v, eps)), r1 = rsqrtf(fmaf(s1, inv_v, eps));
      const u32x4 hv = *reinterpret_cast<const u32x4*>(smem + Pn::OFF_HELD + slot * Pn::HELD_SLOT + vw * 1024 + lane * 16);
      const floatx4 wv = *reinterpret_cast<const floatx4*>(nwl + 16 * vw + 4 * lg);
      auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
      auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
      const u32x2 y0 = {pack_bf16x2(lo(hv.x) * r0 * wv[0], hi(hv.x) * r0 * wv[1]),
                        pack_bf16x2(lo(hv.y) * r0 * wv[2], hi(hv.y) * r0 * wv[3])};
      const u32x2 y1 = {pack_bf16x2(lo(hv.z) * r1 * wv[0], hi(hv.z) * r1 * wv[1]),
                        pack_bf16x2(lo(hv.w) * r1 * wv[2], hi(hv.w) * r1 * wv[3])};
      const int nvb = min(C, T - bn * C);
      const int c0 = 16 * vw + 4 * lg;
      if (c0 < vcols) {
        if (ll < nvb)
          __builtin_amdgcn_raw_buffer_store_b64(y0, rs_o, (unsigned)(((bn * C + ll) * V + v0 + c0) * 2), 0, 0);
        if (16 + ll < nvb)
          __builtin_amdgcn_raw_buffer_store_b64(y1, rs_o, (unsigned)(((bn * C + 16 + ll) * V + v0 + c0) * 2), 0, 0);
      }
    };
    // at the start of step s: publish block s-1, prefetch the other tile's words of block
    // s-2, finish block s-3
    // Step s: at its start wave 0 publishes block s-1 (partial sums written during step
    // s-1).  At its end (where the plain forward stores its output) wave 0 first waits for
    // the prefetch of block s-3 (issued a step earlier; its own stores of this step are
    // not issued yet, so the wait costs nothing), the V waves finish block s-4, and wave 0
    // starts the prefetch of block s-2.  The exchange so tolerates about two steps of
    // drift between the two workgroups.
    static_assert(!NORM || Pn::D == 4, "the step schedule assumes a 4-step hold");
    auto norm_step = [&](int s) __attribute__((always_inline)) {
      if (vw == 0 && s >= 1) norm_export(s - 1);
    };
    auto norm_end = [&](int s) __attribute__((always_inline)) {
      if (paired && vw == 0) wait_vm();
      if (vact && s >= Pn::D) norm_out(s - Pn::D, true, paired);
      if (paired && vw == 0 && s >= 2) norm_prefetch(s - 2);
    };

    // nf: the raw slow flags of block b+1, loaded at the top of the step and only examined
    // after phase C, so that their read never stalls the start of a step
    auto vside = [&](auto fast_tag, int b, u32x2 nf) __attribute__((always_inline)) {
      constexpr bool FAST = decltype(fast_tag)::value;   // the factorised MFMA path, else token by token
      // KD = 128: the per-lane parts of the LDS and store offsets stay in registers across
      // the walk (about 25 fewer address instructions per step than recomputing them each
      // block; that workload is bound by the socket's power, so fewer instructions win).
      // Smaller KD: the lane index passes through an empty asm, which makes the offsets be
      // recomputed each block (measured faster there, where the step's latency bounds).
      int ln = lane;
      if constexpr (KD < 128) asm volatile("" : "+v"(ln));
      ln &= 63;                                // a known range lets LDS offsets fold into the loads
      const int lg = ln >> 4, ll = ln & 15;
      const int t0c = b * C;
      const int nval = min(C, T - t0c);
      char* sb = set_base(b);
      const bf16_t* sKE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KE);
      const bf16_t* sQE = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_QE);
      const bf16_t* sKR = reinterpret_cast<const bf16_t*>(sb + Cfg::SET_KR);
      const float* sBeta = reinterpret_cast<const float*>(sb + Cfg::SET_BETA);
      char* wb = wo_base(b);
      const bf16_t* sP = reinterpret_cast<const bf16_t*>(wb + Cfg::WO_P);
      const bf16_t* sT = reinterpret_cast<const bf16_t*>(wb + Cfg::WO_T);
      const bf16_t* sA10 = reinterpret_cast<const bf16_t*>(wb + Cfg::WO_A10);
      // staged values of this wave's 16 columns: slot 2*row + (column / 8)
      // staged values of this wave's 16 columns: row-major, 16 columns (32 bytes) per token
      const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Cfg::OFF_VRAW + (b % 3) * Cfg::VRAW_BUF + vw * 1024);
      if constexpr (FAST) {
        // Four phases, each loading its LDS operands as one batch before its MFMAs (the
        // batches are sized so that the state and the live operands fit the register budget
        // of a 16-wave workgroup).
        // (A) Y = V - KE S~ (accumulated as V + (-KE) S~: KE is stored negated) and
        // o^T = S~^T QE^T (+ U^T P^T below; the read scale is applied at the store), over the key
        // depth in rounds of at most two 32-deep slices.  o is computed transposed: ln
        // holds token 16I + ll, value columns 16vw + 4g..+3.
        floatx4 Y[2], oT[NB];
        {
          // column ll of tokens 16I + 4lg .. +3, one transposing read per I
          typedef short short4v __attribute__((ext_vector_type(4)));
          const bf16_t* pv = sV + (4 * lg + ((ln >> 2) & 3)) * 16 + 4 * (ln & 3);
#pragma unroll
          for (int I = 0; I < NB; ++I) {
            const short4v vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v*)(__attribute__((address_space(3))) const void*)(pv + 256 * I));
            Y[I] = floatx4{bf2f((bf16_t)vv[0]), bf2f((bf16_t)vv[1]), bf2f((bf16_t)vv[2]), bf2f((bf16_t)vv[3])};
            oT[I] = zero4();
          }
        }
        constexpr int NR = NS > 1 ? 2 : 1;     // slices per round
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += NR) {
          short8 fw[NB][NR], fq[NB][NR], sp[NR];
#pragma unroll
          for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int j = 0; j < NR; ++j) {
              fw[I][j] = lds_frag(sKE, LD_TK, 16 * I, 32 * (s0 + j), ln);
              fq[I][j] = lds_frag(sQE, LD_TK, 16 * I, 32 * (s0 + j), ln);
            }
          sched_fence();
#pragma unroll
          for (int j = 0; j < NR; ++j) sp[j] = acc_perm(sacc[2 * (s0 + j)], sacc[2 * (s0 + j) + 1]);
#pragma unroll
          for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int I = 0; I < NB; ++I) {
              Y[I] = mfma_bf16(fw[I][j], sp[j], Y[I]);
              oT[I] = mfma_bf16(sp[j], fq[I][j], oT[I]);
            }
        }
        // (C) U_0 = T_00 Z_0, U_1 = T_11 (Z_1 - A_10 U_0), Z = diag(beta) Y (fa10 holds -beta A_10)
        short8 ub;
        {
          short8 ft[NB], fp[NB], fa10;
          floatx4 bt[NB];
#pragma unroll
          for (int I = 0; I < NB; ++I) {
            ft[I] = lds_frag(sT, LD_CT, 16 * I, 0, ln);
            fp[I] = lds_frag(sP, LD_CT, 16 * I, 0, ln);
            bt[I] = *reinterpret_cast<const floatx4*>(sBeta + 16 * I + 4 * lg);
          }
          if (NB == 2) fa10 = lds_frag(sA10, LD_CT, 0, 0, ln);
          sched_fence();
          floatx4 U[2];
          U[0] = mfma_bf16(ft[0], acc_perm(Y[0] * bt[0], zero4()), zero4());
          if (NB == 2) {
            const floatx4 Z1 = mfma_bf16(fa10, acc_perm(U[0], zero4()), Y[1] * bt[NB - 1]);
            U[1] = mfma_bf16(ft[NB - 1], acc_perm(zero4(), Z1), zero4());
          } else {
            U[1] = zero4();
          }
          ub = acc_perm(U[0], U[1]);
#pragma unroll
          for (int I = 0; I < NB; ++I) oT[I] = mfma_bf16(ub, fp[I], oT[I]);
        }
        // (D) S' = diag(F) (S~ + KR^T U), F = D0 G0' (next block scaled) or D0; KR^T
        // comes from the [token][channel] KR tile through transposing reads
        sched_fence();
        const bool next_fast = b + 1 < nck && !any_flag(nf);
        const float* sF = reinterpret_cast<const float*>(sb + (next_fast ? Cfg::SET_F : Cfg::SET_D0));
        constexpr int DH = NMT > 4 ? 2 : 1;    // in halves of four row tiles when K = 128
#pragma unroll
        for (int hd = 0; hd < DH; ++hd) {
          constexpr int NM = NMT / DH;
          short8 fk[NM];
          floatx4 fs[NM];
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            fk[m] = lds_frag_tr(sKR, LD_TK, 16 * (hd * NM + m), 0, ln);
            fs[m] = *reinterpret_cast<const floatx4*>(sF + 16 * (hd * NM + m) + 4 * lg);
          }
          sched_fence();
#pragma unroll
          for (int m = 0; m < NM; ++m) sacc[hd * NM + m] = fs[m] * mfma_bf16(fk[m], ub, sacc[hd * NM + m]);
        }
        if constexpr (NORM) {
          // held for the norm: the scaled outputs as bf16, and the per-token sums of
          // squares over this wave's 16 columns taken before rounding
          static_assert(!NORM || NB == 2, "norm blocks are 32 tokens");
          const int slot = Pn::slot(b);
          float a[2][4], sq[2];
#pragma unroll
          for (int I = 0; I < 2; ++I) {
#pragma unroll
            for (int r = 0; r < 4; ++r) a[I][r] = scale * oT[I][r];
            sq[I] = fmaf(a[I][0], a[I][0], fmaf(a[I][1], a[I][1], fmaf(a[I][2], a[I][2], a[I][3] * a[I][3])));
          }
          *reinterpret_cast<u32x4*>(smem + Pn::OFF_HELD + slot * Pn::HELD_SLOT + vw * 1024 + ln * 16) =
              u32x4{pack_bf16x2(a[0][0], a[0][1]), pack_bf16x2(a[0][2], a[0][3]), pack_bf16x2(a[1][0], a[1][1]),
                    pack_bf16x2(a[1][2], a[1][3])};
          float* pw = psum + (b & (Pn::NPS - 1)) * (32 * Pn::NPART) + ll * Pn::NPART + vw * 4 + lg;
          pw[0] = sq[0];
          pw[16 * Pn::NPART] = sq[1];
        } else if (o) {
          const int c0 = 16 * vw + 4 * lg;
#pragma unroll
          for (int I = 0; I < NB; ++I) {
            const int i = 16 * I + ll;
            const u32x2 d = {pack_bf16x2(scale * oT[I][0], scale * oT[I][1]),
                             pack_bf16x2(scale * oT[I][2], scale * oT[I][3])};
            if (i < nval && c0 < vcols)
              __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, (unsigned)(((t0c + i) * V + v0 + c0) * 2), 0, 0);
          }
        }
      } else {
        // token by token (see token_block): the state waits in LDS meanwhile, in the
        // operand area of this block's set, which no other stage touches during this step
        float* stl = reinterpret_cast<float*>(sb) + vw * (NMT * 256) + ln * 4;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) *reinterpret_cast<floatx4*>(stl + mt * 256) = sacc[mt];
        token_block<NMT, SG>(stl, q + tb * K, k + tb * K, v + tb * V, SG ? z + tb : z + tb * K, beta + tb,
                             dt_bias ? dt_bias + (SG ? h : h * K) : nullptr, o ? o + tb * V : nullptr, T, K, V, v0,
                             vcols, t0c, nval, mult2, scale, ln, 16 * vw + ll,
                             NORM ? reinterpret_cast<bf16_t*>(smem + Pn::OFF_HELD + Pn::slot(b) * Pn::HELD_SLOT +
                                                              vw * 1024)
                                  : nullptr,
                             NORM ? psum + (b & (Pn::NPS - 1)) * (32 * Pn::NPART) + vw * 4 : nullptr);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) sacc[mt] = *reinterpret_cast<const floatx4*>(stl + mt * 256);
        wait_vm();                             // the token path's loads
        if (b + 1 < nck && !any_flag(nf)) {
          const float* sG0n = reinterpret_cast<const float*>(set_base(b + 1) + Cfg::SET_G0);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) sacc[mt] *= *reinterpret_cast<const floatx4*>(sG0n + 16 * mt + 4 * lg);
        }
      }
    };
    lds_barrier();                             // steps -2 and -1: E and W fill the pipeline
    lds_barrier();
    if (vact && nck > 0 && !slow_of(0)) {   // (flags of block 0 were written at step -2)
      const float* sG00 = reinterpret_cast<const float*>(set_base(0) + Cfg::SET_G0);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) sacc[mt] *= *reinterpret_cast<const floatx4*>(sG00 + 16 * mt + 4 * g);
    }
    // Runs of MFMA-path blocks in an inner loop of their own, so that the rare token-path
    // block does not shape the register allocation of the common one.  One barrier per step.
    // The flag of block s+1 is read during step s (E wrote it a step earlier), so that no
    // step starts with an LDS round trip.
    int s = 0;
    bool slow = nck > 0 && slow_of(0);
    while (s < nck) {
      while (s < nck && !slow) {
        const u32x2 f = flags_raw(s + 1);      // flags of block s+1 (stale, and unused, past the end)
        if constexpr (NORM) norm_step(s);
        if (vact) vside(std::true_type{}, s, f);
        if constexpr (NORM) norm_end(s);
        lds_barrier();
        slow = s + 1 < nck && any_flag(f);
        ++s;
      }
      if (s < nck) {
        const u32x2 f = flags_raw(s + 1);
        if constexpr (NORM) norm_step(s);
        if (vact) vside(std::false_type{}, s, f);
        if constexpr (NORM) norm_end(s);
        lds_barrier();
        slow = s + 1 < nck && any_flag(f);
        ++s;
      }
    }
    if constexpr (NORM) {
      // the last D blocks (their partial sums were written before the walk's last barrier;
      // the other tile's waits never depend on this tile's later steps)
      if (vw == 0 && nck >= 1) norm_export(nck - 1);
      if (vact)
        for (int bn = max(0, nck - Pn::D); bn < nck; ++bn)
          norm_out(bn, bn + 1 < nck, paired && bn + 3 < nck);
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

template <int KD, int VT, int C, bool SG>
hipError_t launch_chunk_fwd_pc_inst(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                    const float* dt_bias, const void* beta, const float* state_in, float scale, void* o,
                                    float* state_out, int B, int H, int T, int K, int V, hipStream_t s) {
  const int nvt = (V + VT - 1) / VT;
  const int total = B * H * nvt;
  hipLaunchKernelGGL((chunk_fwd_pc_kernel<KD, VT, C, SG>), dim3(total), dim3(PcCfg<KD, VT, C>::NWAVES * 64), 0, s,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)z, A_log, dt_bias,
                     (const bf16_t*)beta, state_in, scale, (bf16_t*)o, state_out, H, T, K, V, nvt, total, 96.0f,
                     nullptr, 0.0f, nullptr, 0ull, 0, 0);
  return hipGetLastError();
}

// The forward with the fused output norm (blocks of 32 tokens, 64-column value tiles).
// With two tiles per head the workgroups of a launch must all be resident (each waits
// for its partner's sums), so heads go PN_MAX_HEADS per launch, 256 workgroups at most.
static __global__ void pn_prologue_kernel(unsigned* hdr) {
  hdr[0] = 0u;                                 // status
  hdr[1] = hdr[1] + 1u;                        // epoch: no word of an earlier call matches
}

template <int KD>
hipError_t launch_chunk_fwd_norm_inst(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                      const float* dt_bias, const void* beta, const float* state_in, float scale,
                                      const float* norm_w, float eps, void* o, float* state_out, int B, int H, int T,
                                      int K, int V, void* work, unsigned long long spin_ticks, hipStream_t s) {
  constexpr int VT = 64, C = 32;
  const int nvt = V > VT ? 2 : 1;
  const int nheads = B * H;
  if (nvt == 2) {
    hipLaunchKernelGGL(pn_prologue_kernel, dim3(1), dim3(1), 0, s, (unsigned*)work);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int per = nvt == 2 ? PN_MAX_HEADS : nheads;
  for (int head0 = 0; head0 < nheads; head0 += per) {
    const int nb = min(per, nheads - head0);
    const int grid = nvt == 2 ? (nb + 7) / 8 * 16 : nb;
    hipLaunchKernelGGL((chunk_fwd_pc_kernel<KD, VT, C, false, true>), dim3(grid),
                       dim3(PcCfg<KD, VT, C>::NWAVES * 64), 0, s, (const bf16_t*)q, (const bf16_t*)k,
                       (const bf16_t*)v, (const bf16_t*)z, A_log, dt_bias, (const bf16_t*)beta, state_in, scale,
                       (bf16_t*)o, state_out, H, T, K, V, nvt, grid, 96.0f, norm_w, eps, (unsigned char*)work,
                       spin_ticks, head0, nb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
