// Selection keys of the router's top-k (gfx950, wave64).
//
// The order (page "vllm.models.flint.ops.moe": the "Numerics" paragraph and
// the router's top-k routine _topk_row): the larger bf16 logit first, equal
// logits by the smaller expert index.  A logit's bit pattern is mapped to a
// signed integer that sorts the way the logit does -- the sign-magnitude to
// two's-complement map: non-negative patterns keep their value, negative ones
// keep the sign and have their 15 magnitude bits inverted, so -0 lands just
// below +0 and NaNs beyond the infinities of their sign -- and the expert
// index is appended below it, inverted, so every key is unique and a larger
// key ranks higher.  Keys lie in [-2^23, 2^23).
#pragma once

#include <climits>

#include "common.hpp"

namespace flint {

constexpr int kNoKey = INT_MIN;  // below every key: an empty or used slot

__device__ __forceinline__ int rank_key(uint32_t bits, int e) {
  const int v = (int)(int16_t)(uint16_t)bits;  // the pattern, sign-extended
  const int mono = v < 0 ? v ^ 0x7fff : v;      // monotone in the logit
  return mono * 256 + (255 - e);
}

// Expert index and logit bits of a key.
__device__ __forceinline__ int key_expert(int key) { return 255 - (key & 0xff); }
__device__ __forceinline__ uint32_t key_logit_bits(int key) {
  const int mono = key >> 8;  // arithmetic shift: the integer part of key / 256
  const int v = mono < 0 ? mono ^ 0x7fff : mono;
  return (uint32_t)v & 0xffffu;
}

// The fp32 sigmoid score of a selected logit: RN32(1 / RN32(1 + RN32(exp(-l)))).
// exp is the device library's double exp, rounded once to fp32, which is the
// correctly rounded value for every bf16 input (checked over all 65 536
// patterns against the CPU oracle); the division and addition are IEEE fp32
// (the library is built with correctly rounded division).
__device__ __forceinline__ float router_score(int key) {
  const float l = bf16_to_f32(key_logit_bits(key));
  const float a = (float)exp(-(double)l);
  const float d = 1.0f + a;
  return 1.0f / d;
}

}  // namespace flint
