// Paired chunked KDA forward for bf16 activations with V = 128 on gfx950.
//
// The two value tiles of a head (64 columns each) run in two workgroups, a "pair",
// that split the state-independent work between them instead of both doing all of it.
// Blocks of 32 tokens alternate between the two: the workgroup of role r "owns" the
// blocks b with b % 2 == r, and for those alone computes
//   E: the gate, the block-local decay scans and the decay-weighted operands
//      KE, QE, KR, G0, D0 (and the block's "slow" flags),
//   W: A = diag(beta) KE KR^T (strictly lower), P = QE KR^T (lower), the inverses
//      T_00, T_11 of the two diagonal blocks of I + A, and -beta A_10,
// into one LDS image of the block.  It publishes the image to a ring in device memory
// (the caller's workspace), and both workgroups bring every block's image back into
// LDS by buffer-to-LDS DMA for their own state stage
//   V: S~ = diag(G0) S,  Y = V - KE S~,  U = (I + A)^-1 diag(beta) Y,
//      o = scale (QE S~ + P U),  S = diag(D0) (S~ + KR^T U)
// over their own 64 value columns.  So each head's E and W work is done once, and
// each workgroup does half of it.
//
// The ring is read back through L2.  The two workgroups of a pair are launched as
// workgroups 16g + j and 16g + j + 8 (j < 8): the hardware hands workgroup i to XCD
// i % 8, so the pair shares one XCD and its L2.  An exporting wave stores its part of
// the image, waits until its stores are acknowledged by L2, then stores a 64-bit flag
// (call epoch, launch, block).  The importer polls the flags with device-scope loads (they
// miss the CU's vector cache and read L2) and issues the DMA only once every flag of
// the block reads (epoch, block); the DMA reads with device scope too.  Every wait is
// bounded by a real-time limit; a wave that gives up records an error status in the
// workspace header and stops waiting for the rest of the launch (its outputs are then
// undefined; the host reads the status with kda_chunk_fwd_status).  Each workgroup
// also publishes its XCD id at start, and the importer checks that its partner's id
// equals its own before it trusts the first flags it sees.
//
// Step s of a workgroup (one barrier per step, s = -4 .. nblocks-1):
//   V waves:  block s from import slot s % 2 (imported during step s-1);
//   E-step (s % 2 == role): E waves compute own block s+4 into the own slot;
//            W waves wait for the partner's block s+1 and import it;
//   W-step (s % 2 != role): W waves compute W of own block s+3 in the own slot and
//            export their rows of it; E waves export the E rows of block s+3, import
//            own block s+1 (exported two steps earlier, no wait) and stage v of
//            blocks s+3 and s+4 and q, k, z of own block s+7.
// An own block's image is therefore complete in the ring at the end of step b-3 and
// read by the partner at step b-1, which leaves a step of slack; three ring slots per
// owner are enough because a workgroup at step t has seen its partner finish step t-3.
//
// The state is carried unscaled between blocks: a block starts with S~ = diag(G0) S
// and ends with S = diag(D0) (S~ + KR^T U), so that no block needs the next block's
// factors (which the other workgroup computes).
#pragma once

#include "kda_chunk_fwd_pc.h"

namespace kda {

template <int KD_>
struct PxCfg {
  static constexpr int KD = KD_, VT = 64, C = 32, CD = 32, NB = 2;
  static constexpr int NNT = VT / 16;                 // value-column tiles = V waves
  static constexpr int NMT = KD / 16;                 // key-row tiles of the state
  static constexpr int NE = 8, NV = 4, NW = 4;
  static constexpr int NWAVES = NE + NV + NW;
  static constexpr int LD_TK = KD + 16;               // [token][channel] bf16 rows (see PcCfg)
  static constexpr int LD_CT = CD + 8;                // [channel|token][token] bf16 rows
  static constexpr int LD_A = CD + 4;                 // [token][token] fp32 rows
  static constexpr int SZ_TK = CD * LD_TK * 2;
  static constexpr int SZ_TT = CD * LD_CT * 2;
  // One block's image: the E part, then the W part.  Offsets are 16-byte aligned.
  static constexpr int IM_KE = 0;
  static constexpr int IM_QE = IM_KE + SZ_TK;
  static constexpr int IM_KR = IM_QE + SZ_TK;
  static constexpr int IM_G0 = IM_KR + SZ_TK;         // KD fp32: block start -> reference
  static constexpr int IM_D0 = IM_G0 + KD * 4;        // KD fp32: reference -> block end
  static constexpr int IM_SLOW = IM_D0 + KD * 4;      // one word per E wave
  static constexpr int IM_EEND = IM_SLOW + 64;
  static constexpr int IM_BETA = IM_EEND;             // CD fp32
  static constexpr int IM_P = IM_BETA + CD * 4;       // P (lower, zero above the diagonal)
  static constexpr int IM_T = IM_P + SZ_TT;           // T_00, T_11 (zero elsewhere)
  static constexpr int IM_A10 = IM_T + SZ_TT;         // -beta A_10 (columns 0..15)
  static constexpr int IM_END = IM_A10 + 16 * LD_CT * 2;
  static constexpr int IM_BYTES = round_up(IM_END, 1024);   // imported in whole 1 KB DMAs
  static constexpr int N_DMA = IM_BYTES / 1024;
  static constexpr int N_ECHUNK = IM_EEND / 16;       // 16-byte chunks of the E part
  static constexpr int ROWS16 = 16 * LD_CT * 2;       // bytes of 16 rows of a P/T/A10 tile
  static constexpr int PARK_BYTES = NV * NMT * 256 * 4;
  // LDS: the own slot (E and W of own blocks), two import slots (V), W scratch, staged v.
  static constexpr int OFF_OWN = 0;
  static constexpr int OFF_IMP = IM_BYTES;
  static constexpr int OFF_A = OFF_IMP + 2 * IM_BYTES;
  static constexpr int WS_LD = 20, WS_MLD = 12;
  static constexpr int WS_BYTES = (2 * 16 * WS_LD + 8 * WS_MLD) * 4;
  static constexpr int OFF_WS = OFF_A + CD * LD_A * 4;
  static constexpr int OFF_VRAW = OFF_WS + 2 * WS_BYTES;
  static constexpr int VRAW_BUF = NNT * 1024;         // 32 rows x 64 columns bf16
  static constexpr int NVRAW = 4;                     // v of blocks s .. s+2 are live at step s
  static constexpr int TOTAL = OFF_VRAW + NVRAW * VRAW_BUF;
  // Ring of one pair: NSLOT images, their flags, the two XCD words.
  static constexpr int NSLOT = 6;                     // three per owner
  static constexpr int NFLAG = NE + NW;               // one flag per exporting wave
  static constexpr int RING_FLAGS = NSLOT * IM_BYTES;
  static constexpr int RING_XCC = RING_FLAGS + NSLOT * NFLAG * 8;
  static constexpr int PAIR_BYTES = round_up(RING_XCC + 16, 256);
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
  static_assert(PARK_BYTES <= IM_BYTES, "token path parks the state in an import slot");
  static_assert(IM_G0 % 16 == 0 && IM_BETA % 16 == 0 && IM_P % 16 == 0 && IM_T % 16 == 0 && IM_A10 % 16 == 0 &&
                    OFF_A % 16 == 0 && OFF_WS % 16 == 0 && OFF_VRAW % 16 == 0,
                "16-byte alignment");
  static_assert(KD % 32 == 0 && KD <= 128, "key dim");
};

// Bytes of the workspace header (word 0: status, word 1: call epoch) before the rings.
constexpr int PX_HEADER = 256;
// Pairs per launch: one workgroup per CU on a 256-CU device.
constexpr int PX_MAX_PAIRS = 128;

// Device-side status codes of the paired forward (workspace header word 0).
constexpr unsigned PX_STATUS_TIMEOUT = 1;   // a wait for the partner's block ran out
constexpr unsigned PX_STATUS_XCC = 2;       // the two workgroups of a pair are not on one XCD

__device__ __forceinline__ void store_b64(__amdgpu_buffer_rsrc_t r, unsigned off, unsigned long long x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, 0);
}

// 16 bytes per lane from buffer offset `off` into LDS at lds + 16 * lane, device scope.
__device__ __forceinline__ void dma16_dev(__amdgpu_buffer_rsrc_t r, void* lds, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 16);
}

template <int KD, bool SG>
__global__ void __launch_bounds__(1024)
chunk_fwd_px_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                    const bf16_t* __restrict__ z, const float* __restrict__ A_log,
                    const float* __restrict__ dt_bias, const bf16_t* __restrict__ beta,
                    const float* state_in, float scale, bf16_t* __restrict__ o, float* state_out, int H, int T,
                    int K, int head0, int npairs, unsigned char* __restrict__ work, unsigned batch,
                    unsigned long long spin_ticks, float thresh) {
  using Cfg = PxCfg<KD>;
  constexpr int CD = Cfg::CD, NNT = Cfg::NNT, NMT = Cfg::NMT;
  constexpr int LD_TK = Cfg::LD_TK, LD_CT = Cfg::LD_CT, LD_A = Cfg::LD_A;
  constexpr int NS = KD / 32;
  constexpr int NTHR = Cfg::NWAVES * 64;
  constexpr int C = 32, NB = 2, V = 128, VT = 64;
  constexpr unsigned kOOB = 0xFFFFFFF0u;

  // workgroups 16g + j and 16g + j + 8 form pair 8g + j
  const int pair = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
  const int role = (blockIdx.x >> 3) & 1;
  if (pair >= npairs) return;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::TOTAL];
  char* const own = smem + Cfg::OFF_OWN;
  float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
  auto imp = [&](int b) __attribute__((always_inline)) {
    int off = __builtin_amdgcn_readfirstlane((b & 1) * Cfg::IM_BYTES);
    asm volatile("" : "+s"(off));
    return smem + Cfg::OFF_IMP + off;
  };
  auto vraw = [&](int b) __attribute__((always_inline)) {
    int off = __builtin_amdgcn_readfirstlane((b & (Cfg::NVRAW - 1)) * Cfg::VRAW_BUF);
    asm volatile("" : "+s"(off));
    return smem + Cfg::OFF_VRAW + off;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

  const int bh = head0 + pair;                 // head index in the whole call
  const int h = bh % H;
  const int v0 = role * VT;
  const size_t tb = (size_t)bh * T;
  const int nck = (T + C - 1) / C;

  // ring of this pair, status word in the header
  const __amdgpu_buffer_rsrc_t rs_ring =
      make_rsrc(work + PX_HEADER + (size_t)pair * Cfg::PAIR_BYTES, (unsigned)Cfg::PAIR_BYTES);
  const __amdgpu_buffer_rsrc_t rs_stat = make_rsrc(work, 8u);
  // the call's epoch (header word 1, advanced by px_prologue_kernel before every call);
  // a flag is (epoch, launch of the call, block), so no flag of an earlier call matches
  const unsigned epoch = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(rs_stat, 4, 0, 0));
  const unsigned long long tag = ((unsigned long long)epoch << 32) | ((unsigned long long)batch << 20);
  auto ring_slot = [](int b) { return (b & 1) * 3 + (b >> 1) % 3; };
  auto flag_of = [&](int b) { return tag | (unsigned)b; };
  const unsigned my_xcc = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 15u;   // HW_REG_XCC_ID[3:0]

  for (int i = tid; i < Cfg::TOTAL / 16; i += NTHR) reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  if (wave == 0 && lane == 0) store_b64(rs_ring, Cfg::RING_XCC + role * 8, flag_of((int)my_xcc));
  wait_vm();                                   // the XCD word lands before any flag of this workgroup

  const float gmul = gate_multiplier(A_log[h]);
  const float mult2 = gmul * kLog2e;
  lds_barrier();

  if (wave < Cfg::NE) {
    // ================================================================ E waves
    const int half = wave >> 2;
    const int cw = wave & 3;
    const int cpair = 16 * cw + l16;           // key-channel pair
    const int tq = 4 * g;                       // tokens 16*half + tq .. +3
    const bool kact = KD == 128 || 2 * cpair < K;
    const bool precise = gmul > 64.0f;
    const float dtb0 = (kact && dt_bias) ? dt_bias[SG ? h : h * K + 2 * cpair] * kLog2e : 0.0f;
    const float dtb1 = (kact && dt_bias) ? dt_bias[SG ? h : h * K + 2 * cpair + 1] * kLog2e : 0.0f;
    const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(k + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_z =
        SG ? make_rsrc(z + tb, (unsigned)(T * 2)) : make_rsrc(z + tb * K, (unsigned)(T * K * 2));
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(v + tb * V, (unsigned)(T * V * 2));
    typedef typename std::conditional<SG, unsigned short, uint32_t>::type ZRaw;
    struct Raw {
      uint32_t k[4], q[4];
      ZRaw z[4];
    };
    const int rowb = (KD >= 64 ? KD : K) * 2;
    const unsigned vbase = kact ? (unsigned)((16 * half + tq) * rowb + 4 * cpair) : 0x80000000u;
    const unsigned zbase = kact ? (unsigned)((16 * half + tq) * 2) : 0x80000000u;
    const int rowoff = (16 * half + tq) * LD_TK + perm32(2 * cpair);
    // q, k, z of own block b into a register set; b is clamped to nck (past the end: zeros)
    auto load_qkz = [&](int b, Raw& r) __attribute__((always_inline)) {
      unsigned off = vbase + (unsigned)(b * C * rowb);
      asm volatile("" : "+v"(off));
      unsigned zoff = zbase + (unsigned)(b * C * 2);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        r.k[t] = buf_load_b32(rs_k, off + t * rowb);
        r.q[t] = buf_load_b32(rs_q, off + t * rowb);
        if constexpr (SG) r.z[t] = __builtin_amdgcn_raw_buffer_load_b16(rs_z, zoff + t * 2, 0, 0);
        else r.z[t] = buf_load_b32(rs_z, off + t * rowb);
      }
    };
    // E of own block b into the own slot (the wave's half and channel slice)
    auto e1 = [&](auto precise_tag, auto half_tag, int b, const Raw& cur) __attribute__((always_inline)) {
      constexpr bool PRECISE = decltype(precise_tag)::value;
      constexpr int HALF = decltype(half_tag)::value;
      const int nval = min(C, T - b * C);
      bf16_t* sKE = reinterpret_cast<bf16_t*>(own + Cfg::IM_KE);
      bf16_t* sQE = reinterpret_cast<bf16_t*>(own + Cfg::IM_QE);
      bf16_t* sKR = reinterpret_cast<bf16_t*>(own + Cfg::IM_KR);
      float* sG0 = reinterpret_cast<float*>(own + Cfg::IM_G0);
      float* sD0 = reinterpret_cast<float*>(own + Cfg::IM_D0);
      Pair<bf16_t> rk[4], rq[4], rz[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        rk[t].u = cur.k[t];
        rq[t].u = cur.q[t];
        if constexpr (SG) rz[t] = Pair<bf16_t>::dup((bf16_t)cur.z[t]);
        else rz[t].u = cur.z[t];
      }
      // tokens at or past nval are identity tokens: k, q read as 0, z = -inf gives g = 0
      if (nval < 16 * HALF + 16) {
        const int lim = nval - (16 * HALF + tq);
#pragma unroll
        for (int t = 0; t < 4; ++t) rz[t].u = t < lim ? rz[t].u : 0xFF80FF80u;
      }
      float px[4], py[4];
      float ax = 0.0f, ay = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ax = fmaf(-gmul, softplus2_f(fmaf(rz[t].x(), kLog2e, dtb0), PRECISE), ax);
        if constexpr (SG) ay = ax;
        else ay = fmaf(-gmul, softplus2_f(fmaf(rz[t].y(), kLog2e, dtb1), PRECISE), ay);
        px[t] = ax;
        py[t] = ay;
      }
      float sumx, sumy, exx, exy;
      quarter_scan(ax, g, sumx, exx);
      if constexpr (SG) {
        sumy = sumx;
        exy = exx;
      } else {
        quarter_scan(ay, g, sumy, exy);
      }
      const float offx = HALF == 0 ? exx - sumx : exx;
      const float offy = HALF == 0 ? exy - sumy : exy;
      const unsigned long long bal = __ballot(kact && fminf(sumx, sumy) < -thresh);
      if (lane == 0) reinterpret_cast<int*>(own + Cfg::IM_SLOW)[wave] = bal != 0ull;
      const int c = 2 * cpair;
      if (HALF == 0 && kact && g == 0)
        *reinterpret_cast<float2*>(sG0 + c) = float2{fast_exp2(sumx), fast_exp2(sumy)};
      if (kact) {
        float lx3 = 0.0f, ly3 = 0.0f;
        uint32_t wke[4], wqe[4], wkr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float ex = px[t] + offx, ey = py[t] + offy;
          const float Lx = fast_exp2(ex), Rx = fast_exp2(-ex);
          const float Ly = SG ? Lx : fast_exp2(ey), Ry = SG ? Rx : fast_exp2(-ey);
          const float kx = rk[t].x(), ky = rk[t].y(), qx = rq[t].x(), qy = rq[t].y();
          wke[t] = pack_bf16x2(-kx * Lx, -ky * Ly);
          wqe[t] = pack_bf16x2(qx * Lx, qy * Ly);
          wkr[t] = pack_bf16x2(kx * Rx, ky * Ry);
          if (t == 3) {
            lx3 = Lx;
            ly3 = Ly;
          }
        }
        constexpr int R1 = LD_TK * 2, R2 = 2 * R1, R3 = 3 * R1;
        lds_write2_b32<0, R2>(sKE + rowoff, wke[0], wke[2]);
        lds_write2_b32<R1, R3>(sKE + rowoff, wke[1], wke[3]);
        lds_write2_b32<0, R2>(sQE + rowoff, wqe[0], wqe[2]);
        lds_write2_b32<R1, R3>(sQE + rowoff, wqe[1], wqe[3]);
        lds_write2_b32<0, R2>(sKR + rowoff, wkr[0], wkr[2]);
        lds_write2_b32<R1, R3>(sKR + rowoff, wkr[1], wkr[3]);
        if (HALF == 1 && g == 3) *reinterpret_cast<float2*>(sD0 + c) = float2{lx3, ly3};
      }
      lds_wait_asm();
    };
    auto estep = [&](int s, const Raw& cur) __attribute__((always_inline)) {
      const int b = s + 4;
      if (b < nck) {
        using H0 = std::integral_constant<int, 0>;
        using H1 = std::integral_constant<int, 1>;
        if (precise) {
          if (half) e1(std::true_type{}, H1{}, b, cur);
          else e1(std::true_type{}, H0{}, b, cur);
        } else {
          if (half) e1(std::false_type{}, H1{}, b, cur);
          else e1(std::false_type{}, H0{}, b, cur);
        }
      }
      lds_barrier();
    };
    // W-step s: all of the E waves' memory traffic, issued together and waited for once at
    // the end of the step, so that an E-step has nothing in flight: q, k, z of own block
    // s+5 (the next E-step's) into the register set, v of blocks s+1 (waves 0..3) and s+2
    // (waves 4..7) into registers, the E part of own block s+3 to the ring, and the DMA of
    // own block s+1 (exported two steps earlier) into its import slot.  After the wait the
    // E flags of block s+3 are raised and v goes to LDS.
    auto xstep = [&](int s, Raw& r) __attribute__((always_inline)) {
      const int bx = s + 3, bi = s + 1;
      const bool xv = bx >= 0 && bx < nck;
      load_qkz(min(s + 5, nck), r);
      const int bv = s + 1 + (wave >> 2), vg = wave & 3;
      const bool vv = bv >= 0 && bv < nck;
      u32x4 vr = {0u, 0u, 0u, 0u};
      const int vrow = lane >> 1, vc0 = 16 * vg + 8 * (lane & 1);
      if (vv)
        vr = __builtin_amdgcn_raw_buffer_load_b128(rs_v, (unsigned)(((bv * C + vrow) * V + v0 + vc0) * 2), 0, 0);
      if (xv) {
        const unsigned sbase = (unsigned)(ring_slot(bx) * Cfg::IM_BYTES);
#pragma unroll
        for (int i = 0; i < (Cfg::N_ECHUNK + 511) / 512; ++i) {
          const int ch = i * 512 + wave * 64 + lane;
          if (ch < Cfg::N_ECHUNK) {
            const u32x4 d = *reinterpret_cast<const u32x4*>(own + ch * 16);
            __builtin_amdgcn_raw_buffer_store_b128(d, rs_ring, sbase + ch * 16, 0, 0);
          }
        }
      }
      if (bi >= 0 && bi < nck) {
        char* dst = imp(bi);
        const unsigned sbase = (unsigned)(ring_slot(bi) * Cfg::IM_BYTES);
        for (int c = wave; c < Cfg::N_DMA; c += Cfg::NE) dma16_dev(rs_ring, dst + c * 1024, sbase + c * 1024 + lane * 16);
      }
      wait_vm();
      if (xv && lane == 0)
        store_b64(rs_ring, Cfg::RING_FLAGS + (ring_slot(bx) * Cfg::NFLAG + wave) * 8, flag_of(bx));
      if (vv) *reinterpret_cast<u32x4*>(vraw(bv) + vg * 1024 + lane * 16) = vr;
      lds_barrier();
    };

    // One register set: an E-step consumes what the W-step before it loaded (role 0 loads
    // its first block here; role 1's first step is a W-step).
    Raw r;
    if (role == 0) load_qkz(0, r);
    for (int s = -4; s < nck; ++s) {
      if (((s - role) & 1) == 0) estep(s, r);
      else xstep(s, r);
    }
  } else if (wave >= Cfg::NE + Cfg::NV) {
    // ================================================================ W waves
    __builtin_amdgcn_s_setprio(2);
    const int ww = wave - (Cfg::NE + Cfg::NV);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(beta + tb, (unsigned)(T * 2));
    const int btok = ww == Cfg::NW - 1 ? lane : (ww == 0 ? 0 : 16) + l16;
    auto load_beta = [&](int b) __attribute__((always_inline)) {
      const unsigned off = btok < C ? (unsigned)((b * C + btok) * 2) : kOOB;
      return __builtin_amdgcn_raw_buffer_load_b16(rs_b, off, 0, 0);
    };
    bool dead = false, xcc_checked = false;
    auto give_up = [&](unsigned code) __attribute__((always_inline)) {
      dead = true;
      if (lane == 0) __builtin_amdgcn_raw_buffer_store_b32(code, rs_stat, 0, 0, 0);
    };
    // Wait until all flags of the partner's block b read (epoch, b).
    auto poll = [&](int b) __attribute__((always_inline)) {
      if (dead) return;
      if (spin_ticks == 0) {
        give_up(PX_STATUS_TIMEOUT);
        return;
      }
      const unsigned long long want = flag_of(b);
      const unsigned base = Cfg::RING_FLAGS + ring_slot(b) * Cfg::NFLAG * 8;
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        unsigned long long f = want;
        if (lane < Cfg::NFLAG) f = __builtin_bit_cast(unsigned long long, load_b64_dev(rs_ring, base + lane * 8));
        if (__ballot(f != want) == 0ull) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
          give_up(PX_STATUS_TIMEOUT);
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!xcc_checked) {
        xcc_checked = true;
        const unsigned long long x = __builtin_bit_cast(unsigned long long, load_b64_dev(rs_ring, Cfg::RING_XCC + (1 - role) * 8));
        if (x != flag_of((int)my_xcc)) give_up(PX_STATUS_XCC);
      }
    };
    auto wstage = [&](int b, float rbeta) __attribute__((always_inline)) {
      const bf16_t* sKE = reinterpret_cast<const bf16_t*>(own + Cfg::IM_KE);
      const bf16_t* sQE = reinterpret_cast<const bf16_t*>(own + Cfg::IM_QE);
      const bf16_t* sKR = reinterpret_cast<const bf16_t*>(own + Cfg::IM_KR);
      bf16_t* sP = reinterpret_cast<bf16_t*>(own + Cfg::IM_P);
      bf16_t* sT = reinterpret_cast<bf16_t*>(own + Cfg::IM_T);
      bf16_t* sA10 = reinterpret_cast<bf16_t*>(own + Cfg::IM_A10);
      (void)b;
      auto frags = [&](const bf16_t* src, int row0, short8* f) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NS; ++s) f[s] = lds_frag(src, LD_TK, row0, 32 * s, lane);
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
        if (isA && I == J) {
          const float bi = -rbeta;
          *reinterpret_cast<floatx4*>(sA + i * LD_A + j0) =
              floatx4{bi * vals[0], bi * vals[1], bi * vals[2], bi * vals[3]};
        } else if (isA) {
          const float nb = rbeta;
          store4_bf16(sA10 + l16 * LD_CT + perm32(j0), nb * vals[0], nb * vals[1], nb * vals[2], nb * vals[3]);
        } else {
          store4_bf16(sP + i * LD_CT + perm32(j0), vals[0], vals[1], vals[2], vals[3]);
        }
      };
      if (ww <= 1) {                           // A_II
        short8 fa[NS], fb[NS];
        frags(sKR, 16 * ww, fa);
        frags(sKE, 16 * ww, fb);
        sched_fence();
        put(ww == 0 ? 0 : 3, dot(fa, fb));
      } else if (ww == 2) {                    // A_10 and P_00: KR_0 shared
        short8 fa[NS], fb[NS], fc[NS];
        frags(sKR, 0, fa);
        frags(sQE, 0, fc);
        frags(sKE, 16, fb);
        sched_fence();
        put(4, dot(fa, fc));
        put(1, dot(fa, fb));
      } else {                                 // P_10 and P_11: QE_1 shared
        short8 fa[NS], fb[NS], fc[NS];
        frags(sKR, 0, fa);
        frags(sKR, 16, fb);
        frags(sQE, 16, fc);
        sched_fence();
        put(5, dot(fa, fc));
        put(6, dot(fb, fc));
      }
      if (ww < NB) {
        // T_II = (I + N)^-1 for I = ww, N = A_II, in 8 x 8 blocks (see chunk_fwd_pc_kernel)
        const int I = ww;
        constexpr int WL = Cfg::WS_LD, ML = Cfg::WS_MLD;
        float* wsDT = reinterpret_cast<float*>(smem + Cfg::OFF_WS + I * Cfg::WS_BYTES);
        float* wsD = wsDT + 16 * WL;
        float* wsMT = wsD + 16 * WL;
        const float* Ab = sA + 16 * I * LD_A + 16 * I;
        wave_lds_fence();
        if (lane < 16) {
          const int hh = lane >> 3, jj = lane & 7;
          const float* Nb = Ab + 8 * hh * LD_A + 8 * hh;
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
          float* dt = wsDT + lane * WL + 8 * hh;
          *reinterpret_cast<floatx4*>(dt) = floatx4{t[0], t[1], t[2], t[3]};
          *reinterpret_cast<floatx4*>(dt + 4) = floatx4{t[4], t[5], t[6], t[7]};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            wsD[(8 * hh + i) * WL + lane] = t[i];
            sT[(16 * I + 8 * hh + i) * LD_CT + perm32(16 * I + lane)] = f2bf(t[i]);
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
          wsMT[j * ML + ki] = m0 + m1;
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
      if (ww == Cfg::NW - 1 && lane < CD) reinterpret_cast<float*>(own + Cfg::IM_BETA)[lane] = rbeta;
    };
    // This wave's rows of the W part: W0, W1 the T rows 0..15, 16..31; W2 the P rows
    // 0..15 and -beta A_10; W3 the P rows 16..31 and beta.  Each range is whole 16-byte
    // chunks of rows only this wave writes (the zero blocks inside them are never written).
    auto wexport = [&](int b) __attribute__((always_inline)) {
      wave_lds_fence();
      const unsigned sbase = (unsigned)(ring_slot(b) * Cfg::IM_BYTES);
      constexpr int R16 = Cfg::ROWS16 / 16;    // chunks in 16 rows
      const int off0 = ww == 0 ? Cfg::IM_T : ww == 1 ? Cfg::IM_T + Cfg::ROWS16 : ww == 2 ? Cfg::IM_P : Cfg::IM_P + Cfg::ROWS16;
      const int off1 = ww == 2 ? Cfg::IM_A10 : Cfg::IM_BETA;
      const int n1 = ww == 2 ? R16 : ww == 3 ? CD * 4 / 16 : 0;
      for (int ch = lane; ch < R16 + n1; ch += 64) {
        const int off = ch < R16 ? off0 + ch * 16 : off1 + (ch - R16) * 16;
        const u32x4 d = *reinterpret_cast<const u32x4*>(own + off);
        __builtin_amdgcn_raw_buffer_store_b128(d, rs_ring, sbase + off, 0, 0);
      }
      wait_vm();
      if (lane == 0) store_b64(rs_ring, Cfg::RING_FLAGS + (ring_slot(b) * Cfg::NFLAG + Cfg::NE + ww) * 8, flag_of(b));
    };
    // beta of own blocks: wb0 for the next W-step's block, wb1 for the one after (loaded at
    // the end of an E-step, after its wait, so that no poll waits for it)
    bf16_t wb0 = 0, wb1 = 0;
    if (role < nck) wb0 = load_beta(role);
    for (int s = -4; s < nck; ++s) {
      if (((s - role) & 1) == 0) {
        // E-step: import the partner's block s+1
        const int bi = s + 1;
        if (bi >= 0 && bi < nck) {
          poll(bi);
          if (!dead) {
            char* dst = imp(bi);
            const unsigned sbase = (unsigned)(ring_slot(bi) * Cfg::IM_BYTES);
            for (int c = ww; c < Cfg::N_DMA; c += Cfg::NW) dma16_dev(rs_ring, dst + c * 1024, sbase + c * 1024 + lane * 16);
          }
        }
        wait_vm();
        if (s + 6 < nck) wb1 = load_beta(s + 6);   // own block of the W-step after next
      } else {
        // W-step: W of own block s+3, then its rows to the ring
        const int b = s + 3;
        if (b >= 0) {
          if (b < nck) {
            wstage(b, bf2f(wb0));
            wexport(b);
          }
          wb0 = wb1;
        }
      }
      lds_barrier();
    }
  } else {
    // ================================================================ V waves
    __builtin_amdgcn_s_setprio(3);
    const int vw = wave - Cfg::NE;
    const int col = 16 * vw + l16;
    floatx4 sacc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) sacc[mt] = zero4();
    if (state_in) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * g + r;
          if (row < K) sacc[mt][r] = state_in[((size_t)bh * K + row) * V + v0 + col];
        }
    }
    wait_vm();
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(o + tb * V, o ? (unsigned)(T * V * 2) : 0u);
    auto slow_of = [&](int b) __attribute__((always_inline)) {
      const int4* f = reinterpret_cast<const int4*>(imp(b) + Cfg::IM_SLOW);
      const int4 a = f[0], c = f[1];
      return ((a.x | a.y | a.z | a.w) | (c.x | c.y | c.z | c.w)) != 0;
    };
    auto vside = [&](auto fast_tag, int b) __attribute__((always_inline)) {
      constexpr bool FAST = decltype(fast_tag)::value;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      ln &= 63;
      const int lg = ln >> 4, ll = ln & 15;
      const int t0c = b * C;
      const int nval = min(C, T - t0c);
      char* sb = imp(b);
      const bf16_t* sKE = reinterpret_cast<const bf16_t*>(sb + Cfg::IM_KE);
      const bf16_t* sQE = reinterpret_cast<const bf16_t*>(sb + Cfg::IM_QE);
      const bf16_t* sKR = reinterpret_cast<const bf16_t*>(sb + Cfg::IM_KR);
      const float* sBeta = reinterpret_cast<const float*>(sb + Cfg::IM_BETA);
      const bf16_t* sP = reinterpret_cast<const bf16_t*>(sb + Cfg::IM_P);
      const bf16_t* sT = reinterpret_cast<const bf16_t*>(sb + Cfg::IM_T);
      const bf16_t* sA10 = reinterpret_cast<const bf16_t*>(sb + Cfg::IM_A10);
      const bf16_t* sV = reinterpret_cast<const bf16_t*>(vraw(b) + vw * 1024);
      if constexpr (FAST) {
        // S~ = diag(G0) S
        {
          const float* sG0 = reinterpret_cast<const float*>(sb + Cfg::IM_G0);
          floatx4 gs[NMT];
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) gs[mt] = *reinterpret_cast<const floatx4*>(sG0 + 16 * mt + 4 * lg);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) sacc[mt] *= gs[mt];
        }
        // (A) Y = V - KE S~ and o^T = S~^T QE^T (see chunk_fwd_pc_kernel)
        floatx4 Y[2], oT[NB];
        {
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
        constexpr int NR = NS > 1 ? 2 : 1;
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
        // (C) U_0 = T_00 Z_0, U_1 = T_11 (Z_1 - A_10 U_0), Z = diag(beta) Y
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
          fa10 = lds_frag(sA10, LD_CT, 0, 0, ln);
          sched_fence();
          floatx4 U[2];
          U[0] = mfma_bf16(ft[0], acc_perm(Y[0] * bt[0], zero4()), zero4());
          const floatx4 Z1 = mfma_bf16(fa10, acc_perm(U[0], zero4()), Y[1] * bt[1]);
          U[1] = mfma_bf16(ft[1], acc_perm(zero4(), Z1), zero4());
          ub = acc_perm(U[0], U[1]);
#pragma unroll
          for (int I = 0; I < NB; ++I) oT[I] = mfma_bf16(ub, fp[I], oT[I]);
        }
        // (D) S = diag(D0) (S~ + KR^T U)
        sched_fence();
        const float* sF = reinterpret_cast<const float*>(sb + Cfg::IM_D0);
        constexpr int DH = NMT > 4 ? 2 : 1;
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
        if (o) {
          const int c0 = 16 * vw + 4 * lg;
#pragma unroll
          for (int I = 0; I < NB; ++I) {
            const int i = 16 * I + ll;
            const u32x2 d = {pack_bf16x2(scale * oT[I][0], scale * oT[I][1]),
                             pack_bf16x2(scale * oT[I][2], scale * oT[I][3])};
            if (i < nval)
              __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, (unsigned)(((t0c + i) * V + v0 + c0) * 2), 0, 0);
          }
        }
      } else {
        // token by token, the state parked in this block's import slot meanwhile
        float* stl = reinterpret_cast<float*>(sb) + vw * (NMT * 256) + ln * 4;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) *reinterpret_cast<floatx4*>(stl + mt * 256) = sacc[mt];
        token_block<NMT, SG>(stl, q + tb * K, k + tb * K, v + tb * V, SG ? z + tb : z + tb * K, beta + tb,
                             dt_bias ? dt_bias + (SG ? h : h * K) : nullptr, o ? o + tb * V : nullptr, T, K, V, v0,
                             VT, t0c, nval, mult2, scale, ln, 16 * vw + ll, nullptr, nullptr);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) sacc[mt] = *reinterpret_cast<const floatx4*>(stl + mt * 256);
        wait_vm();
      }
    };
    for (int i = 0; i < 4; ++i) lds_barrier();   // steps -4 .. -1
    int s = 0;
    while (s < nck) {
      bool slow = slow_of(s);
      while (s < nck && !slow) {
        vside(std::true_type{}, s);
        lds_barrier();
        ++s;
        if (s < nck) slow = slow_of(s);
      }
      if (s < nck) {
        vside(std::false_type{}, s);
        lds_barrier();
        ++s;
      }
    }
    if (state_out) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * g + r;
          if (row < K) state_out[((size_t)bh * K + row) * V + v0 + col] = sacc[mt][r];
        }
    }
  }
}

// Before every call: clear the status word and advance the epoch (header words 0 and
// 1).  A kernel rather than a host write or memset, so that a captured graph advances
// the epoch on every replay.
static __global__ void px_prologue_kernel(unsigned* hdr) {
  hdr[0] = 0u;
  hdr[1] = hdr[1] + 1u;
}

// One launch per PX_MAX_PAIRS heads, in head order on the stream (they reuse the rings).
template <int KD, bool SG>
hipError_t launch_chunk_fwd_px_inst(const void* q, const void* k, const void* v, const void* z, const float* A_log,
                                    const float* dt_bias, const void* beta, const float* state_in, float scale,
                                    void* o, float* state_out, int B, int H, int T, int K, void* work,
                                    unsigned long long spin_ticks, hipStream_t s) {
  hipLaunchKernelGGL(px_prologue_kernel, dim3(1), dim3(1), 0, s, (unsigned*)work);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int nheads = B * H;
  for (int head0 = 0; head0 < nheads; head0 += PX_MAX_PAIRS) {
    const int np = min(PX_MAX_PAIRS, nheads - head0);
    const int grid = (np + 7) / 8 * 16;
    hipLaunchKernelGGL((chunk_fwd_px_kernel<KD, SG>), dim3(grid), dim3(PxCfg<KD>::NWAVES * 64), 0, s,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)z, A_log, dt_bias,
                       (const bf16_t*)beta, state_in, scale, (bf16_t*)o, state_out, H, T, K, head0, np,
                       (unsigned char*)work, (unsigned)(head0 / PX_MAX_PAIRS), spin_ticks, 96.0f);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
