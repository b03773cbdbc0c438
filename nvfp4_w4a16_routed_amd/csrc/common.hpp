// Device helpers shared by the Flint MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t v2u32_t;

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

// Two fp32 -> packed bf16 (a in the low half), round to nearest even, by
// gfx950's paired converter.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
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
//
// Reductions within aligned groups of L lanes (L a power of two <= 64) with
// DPP: quad permutes, half-row and row mirrors inside a 16-lane row (after
// which every lane of the row holds the row's result), then row_bcast15 /
// row_bcast31 across rows (after which the LAST lane of each 32- or 64-lane
// group holds the group's result).  Each step combines two partial results
// in a fixed order, so the result does not depend on timing.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v, float old = 0.0f) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, ROW_MASK == 0xF));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v, int old = 0) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, ROW_MASK == 0xF);
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16 lanes
constexpr int kDppBcast15 = 0x142;    // lane 15 of each row -> next row
constexpr int kDppBcast31 = 0x143;    // lane 31 -> rows 2 and 3

// Sum over groups of L lanes; valid in every lane for L <= 16, in the last
// lane of the group for L = 32 and 64.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "group size");
  if constexpr (L >= 2) v += dpp_f32<kDppXor1>(v);
  if constexpr (L >= 4) v += dpp_f32<kDppXor2>(v);
  if constexpr (L >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp_f32<kDppMirror>(v);
  if constexpr (L >= 32) v += dpp_f32<kDppBcast15, 0xA>(v);  // rows 1, 3 += rows 0, 2
  if constexpr (L >= 64) v += dpp_f32<kDppBcast31, 0xC>(v);  // rows 2, 3 += lane 31
  return v;
}

// Maximum over the wave, returned uniformly (from lane 63).
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_i32<kDppXor1>(v));
  v = max(v, dpp_i32<kDppXor2>(v));
  v = max(v, dpp_i32<kDppHalfMirror>(v));
  v = max(v, dpp_i32<kDppMirror>(v));
  v = max(v, dpp_i32<kDppBcast15, 0xA>(v, v));
  v = max(v, dpp_i32<kDppBcast31, 0xC>(v, v));
  return __builtin_amdgcn_readlane(v, 63);
}

// ------------------------------------------------- cross-wave signalling
//
// Data exchanged between waves of one grid (which may run on different
// XCDs, each with its own L2) is written and read with device-scope
// ("agent") relaxed atomic accesses: such stores are performed at the
// device's coherence point and such loads read from it, so no L2 writeback
// or invalidate is needed.  A producer publishes by waiting until its
// stores are performed (s_waitcnt vmcnt(0)) and then writing a flag word; a
// consumer polls the flag and then reads the data.

template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes (8-byte aligned) read at device scope.
__device__ __forceinline__ u32x4_t ld_dev16(const void *p) {
  const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
  const uint64_t a = ld_dev(q), b = ld_dev(q + 1);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}


// Waits until every store this wave issued has been performed.
__device__ __forceinline__ void stores_performed() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // keeps the compiler's order
  __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0) (expcnt, lgkmcnt: any)
}

// ------------------------------------------------------------ memory ops

// Buffer descriptor of `bytes` bytes at p (raw, untyped; word 3 as the
// gfx9-family raw buffer accesses expect).  At most 2^31 - 1 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, size_t bytes) {
  const int n = bytes > 0x7fffffffu ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}

// A byte offset past the end of every descriptor above (they hold fewer than
// 2^31 bytes), also after adding a few KB: buffer loads from it return zero
// without touching memory and buffer stores to it are dropped.  Used to keep
// the number of memory instructions on a path fixed.
constexpr uint32_t kOOB = 0x80000000u;

// Cache-policy operands of buffer accesses: streaming (non-temporal) reads,
// and stores performed at device scope (the SC1 bit).
constexpr int kPolicyStream = 2;
constexpr int kPolicyDevice = 16;

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
