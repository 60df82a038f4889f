// Device-side helpers shared by the gfx950 kernels: vector types for the MFMA
// operands, bf16 / e4m3 conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace rf {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over [p, p + nbytes): raw buffer loads through it take a
// 32-bit per-lane byte offset plus a scalar offset, and read 0 past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
// Cache policy for bytes that are read once (non-temporal, streaming). On
// MI355X it lifts a plain HBM read stream from about 6.2 to 7.0 TB/s. Data
// that other workgroups read again from L2 (attention K/V tiles, GEMM
// operands) keeps the default policy: there the hint measured slower.
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The scale of the scores, in the form the MFMA kernels use it: a positive
// factor c (exp2 units) and a transform of the bf16 query bits (w & q_and) ^
// q_xor. A negative scale flips the sign of every query value (exact), so
// the scaled scores are the same while c stays positive and the running
// maxima, the masking to -inf and the lazy reference keep their meaning; a
// zero scale zeroes the query, so every score is exactly 0.
struct ScoreScale {
  float c;
  uint32_t q_and, q_xor;
};
inline ScoreScale score_scale(float scale) {
  if (scale > 0.f) return {scale * kLog2e, ~0u, 0u};
  if (scale < 0.f) return {-scale * kLog2e, ~0u, 0x80008000u};
  return {kLog2e, 0u, 0u};
}
constexpr float kNegInf = -__builtin_inff();

// Workgroup barrier for handing LDS contents between waves. It waits for this
// wave's own LDS operations and then meets the other waves; unlike
// __syncthreads(), whose fence also drains every outstanding global and buffer
// load, loads issued for later pipeline stages stay in flight. Loads that write
// LDS directly are counted by vmcnt: wait for them explicitly before calling.
// The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so
// the body can use I in constant expressions (immediate offsets, register
// indices).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// ds_read_b64_tr_b16 (gfx950 transposing LDS read) through inline asm, at LDS
// byte address addr + OFF. Within each group of 16 lanes, lane j supplies the
// address of four consecutive bf16 values (8 bytes); lane i receives element
// 16 s + i (s = 0..3) of the group's 64 values taken in lane order, i.e. when
// lane j points at row r0 + j / 4, columns c0 + 4 (j % 4) .. +3 of a row-major
// tile, lane i receives rows r0 .. r0 + 3 of column c0 + i.
// The builtin form makes the compiler wait for every outstanding buffer-to-LDS
// load before the read (it cannot prove the two disjoint), which drains the
// prefetches of later tiles. The asm form is invisible to that analysis, and
// to the compiler's own LDS wait counting: the result may be used only after
// lds_wait_for() has covered it.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Wait until at most N LDS operations are outstanding (they complete in issue
// order), and make x depend on the wait so its uses stay behind it.
template <int N, class T>
__device__ __forceinline__ void lds_wait_for(T& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}

// bf16 <-> fp32. A bf16 value is the upper half of an fp32 bit pattern, so the
// widening is exact; the narrowing uses the hardware round-to-nearest-even
// convert (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r.x = (__bf16)lo;
  r.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Raw 2^x (v_exp_f32): exact enough for the softmax weights, no range fix-up;
// 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- wavefront reductions

// Sum and max over lanes l and l ^ 32 without LDS: v_permlane32_swap (gfx950)
// applied to (x, x) returns x[l % 32] and x[32 + l % 32] in every lane l, so
// both lanes of a pair combine the same two values in the same order.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same across the two 16-lane rows of each half-wave (v_permlane16_swap):
// lane l combines x[l & ~16] and x[l | 16].
__device__ __forceinline__ float row_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane exchanges within a 16-lane row by DPP (no LDS): quad permutations
// xor 1 and xor 2, then the half-row mirror (lane i <-> 7 - i in each 8) and
// the row mirror (i <-> 15 - i). After the four steps of a commutative
// operation every lane of the row holds the row's result.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfRowMirror = 0x141, kDppRowMirror = 0x140;

// Max and sum over the 64 lanes of a fully active wave: four DPP steps inside
// each row, then the row and half-wave swaps. Every lane gets the same value
// (each step combines the same two operands in the same order in both lanes
// of a pair).
__device__ __forceinline__ float wave_max(float v) {
  v = __builtin_fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppHalfRowMirror>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return half_swap_max(row_swap_max(v));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppHalfRowMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return half_swap_sum(row_swap_sum(v));
}

// Merge of two online-softmax statistics (m, l): both rescaled to the larger max.
// A side with m = -inf is the identity and contributes nothing (weight 0; a NaN
// in its l still reaches the result, as 0 * NaN).
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  const float a = (m == kNegInf) ? 0.f : fast_exp2((m - mn) * kLog2e);
  const float b = (m2 == kNegInf) ? 0.f : fast_exp2((m2 - mn) * kLog2e);
  l = l * a + l2 * b;
  m = mn;
}

// ---------------------------------------------------------------- e4m3 (OCP E4M3, no inf, max 448)

// Round-to-nearest-even encoding of a finite fp32 value to an e4m3 code, with
// the magnitude clamped to 448 first (saturation). Exact integer bit logic on
// the fp32 pattern: subnormal codes hold m * 2^-9, normal codes hold
// (1 + m/8) * 2^(e-7) with e in 1..15.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal grid of step 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.f);  // 0..8; 8 is the smallest normal code
  } else {
    const uint32_t ab = bits & 0x7fffffffu;
    const int e = (int)(ab >> 23) - 127;  // -6 .. 8
    uint32_t mant = ab & 0x7fffffu;
    uint32_t r = mant >> 20;
    const uint32_t rem = mant & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    int ee = e + 7;
    if (r == 8u) { r = 0; ++ee; }
    code = ((uint32_t)ee << 3) | r;
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  float v = (e == 0) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

}  // namespace rf
