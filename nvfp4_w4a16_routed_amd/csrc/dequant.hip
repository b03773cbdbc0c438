// Exact NVFP4 dequantisation to bf16 (vLLM page "vllm.models.flint.ops.moe",
// _dequant8 / _dequant_rows: each weight is its E2M1 value times the E4M3
// scale of its 16-element block; the product has at most 6 significant bits,
// so it is exact in bf16).  Uses the same converters as the GEMV kernels.
#include "common.hpp"
#include "internal.hpp"

namespace flint {

namespace {

// One thread per 8 consecutive elements (one dword of codes).
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ s, int rows, int K,
               uint16_t *__restrict__ out) {
  const int words_per_row = K / 8;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long)rows * words_per_row) return;
  const int r = (int)(gid / words_per_row), wd = (int)(gid % words_per_row);
  const uint32_t code = *reinterpret_cast<const uint32_t *>(w + (size_t)r * (K / 2) + wd * 4);
  const float sc = e4m3_to_f32(s[(size_t)r * (K / 16) + wd / 2]);
  uint32_t pk[4];
  fp4x8_to_bf16(code, pk);
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t lo = f32_to_bf16(bf16_lo(pk[d]) * sc);
    uint32_t hi = f32_to_bf16(bf16_hi(pk[d]) * sc);
    o[d] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x4_t *>(out + (size_t)r * K + wd * 8) = o;
}

}  // namespace

hipError_t launch_dequant(const uint8_t *w, const uint8_t *s, int rows, int K, uint16_t *out,
                          hipStream_t st) {
  const long n = (long)rows * (K / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w, s,
                     rows, K, out);
  return hipGetLastError();
}

}  // namespace flint
