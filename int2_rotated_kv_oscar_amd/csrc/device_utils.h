// Device helpers for gfx950 (CDNA4) kernels: MFMA operand types, exact
// bfloat16 three-way splits, f16/bf16 conversions, wave64 shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar_dev {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// D = A(16x32) B(32x16) + C.  Lane l holds A[l%16][8(l/16) .. +7],
// B[8(l/16) .. +7][l%16]; D[4(l/16) + r][l%16] in element r.
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// float32 -> bfloat16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// x = hi + mid + lo exactly (each a bfloat16): a float32 significand has 24
// bits, each part carries 8.
struct Split3 {
  uint32_t hi, mid, lo;
};
__device__ __forceinline__ Split3 split3(float x) {
  Split3 s;
  s.hi = bf16_rne(x);
  const float r1 = x - bf16_to_f32(s.hi);
  s.mid = bf16_rne(r1);
  const float r2 = r1 - bf16_to_f32(s.mid);
  s.lo = bf16_rne(r2);
  return s;
}
// x = hi + lo to 16 significant bits.
__device__ __forceinline__ void split2(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - bf16_to_f32(hi));
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xFFFFu) | (hi16 << 16); }

__device__ __forceinline__ uint32_t f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(unsigned short, h);
}
__device__ __forceinline__ float f16_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(b & 0xFFFFu));
}
// two floats -> packed f16x2 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) { return pack2(f16_bits(a), f16_bits(b)); }

// packed f16x2 multiply
// Two floats -> packed f16 pair, rounded toward zero (one instruction).
__device__ __forceinline__ uint32_t pack_f16x2_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ uint32_t hmul2(uint32_t a, uint32_t b) {
  f16x2 x = __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b);
  return __builtin_bit_cast(uint32_t, x);
}

// each 16-bit half shifted right by 8
__device__ __forceinline__ uint32_t shr8_halves(uint32_t x) {
  u16x2 v = __builtin_bit_cast(u16x2, x);
  v = v >> (unsigned short)8;
  return __builtin_bit_cast(uint32_t, v);
}

// r / 3: the product with 1/3 refined once with its exact residual, so that
// a quotient representable in float32 comes out exactly.  With coarse
// rotated values (a Hadamard or identity rotation of bf16 rows) the range is
// often three times an f16 rounding midpoint; the exact quotient then rounds
// to even on the way to f16, as the definition's real-number division does.
// The 16-level variant divides by 15 the same way.
template <int TOP = 3>
__device__ __forceinline__ float div3(float r) {
  constexpr float kInv = 1.0f / float(TOP);
  const float s0 = r * kInv;
  return __builtin_fmaf(__builtin_fmaf(-float(TOP), s0, r), kInv, s0);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
// Workgroup barrier that orders LDS accesses only: global loads still in
// flight (prefetched pages) are not waited for, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding), and no memory
// access moved across it: LDS written by global_load_lds (whose completion the
// compiler does not track) is read after it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's own LDS reads and writes completed
// (lgkmcnt(0)), with global_load_lds requests still in flight: a release
// fence on LDS would also wait for those (vmcnt(0)).  LDS written by such
// requests is covered by wait_vm, not by this barrier.
__device__ __forceinline__ void lds_barrier_keep_dma() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt 63, expcnt 7: not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Cross-row exchange without LDS: v_permlane16_swap / v_permlane32_swap on two
// copies of v leave, in every lane, the values of rows (r, r^1) or (r, r^2) of
// 16 lanes as the pair (first, second) in the same order for both rows, so a
// commutative reduction of the pair is identical in both partner lanes.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max16(float v) {  // over lanes with equal l%16
  float a, b;
  pair16(v, a, b);
  pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_min16(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(fminf(a, b), a, b);
  return fminf(a, b);
}
__device__ __forceinline__ float wave_sum16(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(a + b, a, b);
  return a + b;
}

}  // namespace oscar_dev
