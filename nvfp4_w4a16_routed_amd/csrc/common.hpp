// Device helpers shared by the Flint MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// ----------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> nearest bf16 value, kept in fp32.
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// ------------------------------------------------------------ NVFP4 parts

// E4M3 (OCP "fn": bias 7, subnormals, S.1111.111 = NaN) byte -> fp32.
// gfx950's v_cvt_f32_fp8 decodes the OCP E4M3 format exactly.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// The two E2M1 codes of byte SEL of `w` -> bf16 pair (low nibble in .x).
// The hardware scale operand only contributes its exponent, so it is 1.0
// here and the E4M3 block scale is applied to the fp32 partial sums.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, v);
}

// Eight E2M1 codes of one dword -> four packed bf16 pairs, K order kept.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, uint32_t out[4]) {
  out[0] = fp4x2_to_bf16x2<0>(w);
  out[1] = fp4x2_to_bf16x2<1>(w);
  out[2] = fp4x2_to_bf16x2<2>(w);
  out[3] = fp4x2_to_bf16x2<3>(w);
}

// acc + a.x * b.x + a.y * b.y on packed bf16 pairs (one rounding to fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ------------------------------------------------------------- SwiGLU

// silu(g) * u in fp32 with the sigmoid from the hardware exp2 and
// reciprocal approximations (the pages likewise use approximate exp2/rcp).
__device__ __forceinline__ float swiglu(float g, float u) {
  float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  float s = __builtin_amdgcn_rcpf(1.0f + e);
  return (g * s) * u;
}

// ------------------------------------------------------- wave reductions

// Sum over aligned groups of L lanes (L a power of two <= 64); every lane of
// a group ends with the group's sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// ------------------------------------------------------------ memory ops

__device__ __forceinline__ u32x4_t load16(const void *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

// Streaming (read-once) 16-byte load: non-temporal hint for weight bytes.
__device__ __forceinline__ u32x4_t load16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

__device__ __forceinline__ uint32_t load_u16(const void *p) {
  return *reinterpret_cast<const uint16_t *>(p);
}

}  // namespace flint
