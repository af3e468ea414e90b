// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef uint16_t bf16_t;   // bfloat16 bit pattern as stored in HBM and LDS

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef short short4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kALogMin = -10.0f;
constexpr float kALogMax = 20.0f;

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ bf16_t f2bf(float f) {   // round to nearest even (v_cvt_pk_bf16_f32)
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ------------------------------------------------------------------ gate
// Multiplier exp(clamp(A_log, -10, 20)) of the released KDA gate (the clamp stays,
// kdafix page "Fix 1 -- decay form").  Evaluated once per head with the precise expf.
__device__ __forceinline__ float gate_multiplier(float a_log) {
  return expf(fminf(fmaxf(a_log, kALogMin), kALogMax));
}

// softplus(x) = max(x,0) + log(1 + e^-|x|), natural units.  log1p is taken from the
// hardware log2 of u = 1 + y; with `precise`, the rounding of u is undone by the
// factor y / (u - 1) (Kahan's log1p identity), which keeps full relative accuracy
// when y = e^-|x| is tiny.  That matters once the multiplier exp(A) is large.
__device__ __forceinline__ float softplus_f(float x, bool precise) {
  float y = fast_exp2(-fabsf(x) * kLog2e);
  float u = 1.0f + y;
  float l = fast_log2(u) * kLn2;
  if (precise) {
    float d = u - 1.0f;
    l = (d == 0.0f) ? y : l * (y * fast_rcp(d));
  }
  return fmaxf(x, 0.0f) + l;
}

// The same in log2 units: for x2 = x log2(e), softplus(x) log2(e) = max(x2, 0) + log2(1 + 2^-|x2|).
__device__ __forceinline__ float softplus2_f(float x2, bool precise) {
  float y = fast_exp2(-fabsf(x2));
  float u = 1.0f + y;
  float l = fast_log2(u);
  if (precise) {
    float d = u - 1.0f;
    l = (d == 0.0f) ? y * kLog2e : l * (y * fast_rcp(d));
  }
  return fmaxf(x2, 0.0f) + l;
}

// log2(1 + 2^x2) evaluated directly: two transcendentals and one add.  Within fp32 rounding
// of softplus2_f for x2 < 128; from there on it is +inf.  A caller that multiplies it by a
// positive gate multiplier then sees a -inf decay, which sends the block to its exact
// token path; with a zero multiplier it would make a NaN, so such heads use softplus2_f.
__device__ __forceinline__ float softplus2_direct(float x2) { return fast_log2(1.0f + fast_exp2(x2)); }

// ------------------------------------------------------------------ MFMA fragments
// One wave computes a 16x16 fp32 tile C += A(16 x KS) * B(KS x 16) per instruction.
// Operands live in LDS "depth-contiguous": A as [row][depth], B as [col][depth].
// Lane l supplies row/col (l % 16) and depth elements starting at DPL*(l / 16).
// The accumulator holds C[4*(l/16) + r][l % 16], r = 0..3.
template <typename Top> struct Mfma;

template <> struct Mfma<float> {            // v_mfma_f32_16x16x4_f32
  static constexpr int KS = 4;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* base, int ld, int rc0, int k0, int lane) {
    return base[(rc0 + (lane & 15)) * ld + k0 + (lane >> 4)];
  }
  static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  // multiply the depth elements of a fragment by per-depth factors f[k0 + ...]
  static __device__ __forceinline__ frag scale(frag a, const float* f, int k0, int lane) {
    return a * f[k0 + (lane >> 4)];
  }
};

template <> struct Mfma<bf16_t> {           // v_mfma_f32_16x16x32_bf16
  static constexpr int KS = 32;
  typedef short8 frag;
  static __device__ __forceinline__ frag load(const bf16_t* base, int ld, int rc0, int k0, int lane) {
    return *reinterpret_cast<const short8*>(base + (rc0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
  }
  static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag scale(frag a, const float* f, int k0, int lane) {
    const float* fp = f + k0 + 8 * (lane >> 4);
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (short)f2bf(bf2f((bf16_t)a[e]) * fp[e]);
    return r;
  }
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier ordering LDS only.  The kernels never exchange data between
// threads through global memory, so the barrier need not wait for outstanding
// HBM loads and stores (a plain __syncthreads() fences global memory as well and
// would stall every barrier on in-flight output stores and prefetches).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two consecutive activation elements loaded with one 4-byte (bf16) or 8-byte
// (fp32) access.
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
  uint32_t u;
  static __device__ __forceinline__ Pair load(const bf16_t* p) {
    Pair r;
    r.u = *reinterpret_cast<const uint32_t*>(p);
    return r;
  }
  // one value for both elements (a scalar-decay gate input serves every channel)
  static __device__ __forceinline__ Pair dup(bf16_t x) {
    Pair r;
    r.u = ((uint32_t)x << 16) | (uint32_t)x;
    return r;
  }
  __device__ __forceinline__ float x() const { return __uint_as_float(u << 16); }
  __device__ __forceinline__ float y() const { return __uint_as_float(u & 0xffff0000u); }
};
template <> struct Pair<float> {
  float2 f;
  static __device__ __forceinline__ Pair load(const float* p) {
    Pair r;
    r.f = *reinterpret_cast<const float2*>(p);
    return r;
  }
  static __device__ __forceinline__ Pair dup(float x) {
    Pair r;
    r.f = float2{x, x};
    return r;
  }
  __device__ __forceinline__ float x() const { return f.x; }
  __device__ __forceinline__ float y() const { return f.y; }
};

// Buffer resource over [base, base + bytes): 32-bit byte offsets, and the hardware
// range check returns 0 for any load past the end (raw buffer, 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_load_b32(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
// Two floats rounded to bf16 and packed low/high in one register (one v_cvt_pk_bf16_f32:
// a two-element vector conversion, so the pair is never split into scalar conversions).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){a, b}, bf16x2_t));
}

// Store two consecutive operand values.
template <typename T> __device__ __forceinline__ void store2(T* dst, float a, float b);
template <> __device__ __forceinline__ void store2<float>(float* dst, float a, float b) {
  *reinterpret_cast<float2*>(dst) = float2{a, b};
}
template <> __device__ __forceinline__ void store2<bf16_t>(bf16_t* dst, float a, float b) {
  *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(a, b);
}

constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

}  // namespace kda
