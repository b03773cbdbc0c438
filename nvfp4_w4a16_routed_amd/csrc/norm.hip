// Residual add and RMS norm in front of the MoE block, and the final add of
// a precomputed shared output.
//
// Residual add and RMS norm (page
// "vllm.models.flint.ops.moe", _add_rms_norm and flint_moe_ll):
//   s = fp32(a) + fp32(r)                       (one fp32 rounding)
//   residual' = bf16(s)
//   xn = bf16((s * rsqrt(mean(s^2) + eps)) * w)  (fp32)
// The pages do not print their rsqrt helper; it is read here as the
// correctly rounded 1 / sqrt (the library is built with correctly rounded
// fp32 division and square root).  One block per row; each thread keeps
// its s values (8 per 16-byte chunk, at most 4 chunks: H <= 8192) between
// the two passes.  The sum of squares is reduced in a fixed order (within
// a thread, DPP steps within a wave, then the four waves in order), so the
// result does not depend on timing.
#include "common.hpp"
#include "internal.hpp"

namespace flint {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormChunks = 4;  // 16-byte chunks per thread: H <= 256 * 8 * 4

__global__ void __launch_bounds__(kNormThreads) add_rmsnorm_kernel(const uint16_t *__restrict__ a,
                                                                   const uint16_t *__restrict__ r,
                                                                   const uint16_t *__restrict__ w, float eps,
                                                                   int H, uint16_t *__restrict__ res_out,
                                                                   uint16_t *__restrict__ xn_out) {
  __shared__ float wsum[kNormThreads / kWave];
  const size_t row = (size_t)blockIdx.x * H;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  float sv[kNormChunks][8];
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormChunks; ++j) {
    const int c = (j * kNormThreads + (int)threadIdx.x) * 8;
    if (c < H) {
      const u32x4_t av = load16(a + row + c), rv = load16(r + row + c);
      u32x4_t ov;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = bf16_lo(av[d]) + bf16_lo(rv[d]), hi = bf16_hi(av[d]) + bf16_hi(rv[d]);
        sv[j][2 * d] = lo;
        sv[j][2 * d + 1] = hi;
        acc += lo * lo;
        acc += hi * hi;
        ov[d] = pack_bf16x2(lo, hi);
      }
      *reinterpret_cast<u32x4_t *>(res_out + row + c) = ov;
    }
  }
  acc = __shfl(group_sum<kWave>(acc), kWave - 1, kWave);
  if (lane == 0) wsum[wv] = acc;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += wsum[i];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int j = 0; j < kNormChunks; ++j) {
    const int c = (j * kNormThreads + (int)threadIdx.x) * 8;
    if (c < H) {
      const u32x4_t wt = load16(w + c);
      u32x4_t ov;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        ov[d] = pack_bf16x2(sv[j][2 * d] * inv * bf16_lo(wt[d]), sv[j][2 * d + 1] * inv * bf16_hi(wt[d]));
      *reinterpret_cast<u32x4_t *>(xn_out + row + c) = ov;
    }
  }
}

}  // namespace

bool add_rmsnorm_supported(int H) { return H > 0 && H % 8 == 0 && H <= kNormThreads * 8 * kNormChunks; }

hipError_t launch_add_rmsnorm(const uint16_t *a, const uint16_t *r, const uint16_t *w, float eps, int M,
                              int H, uint16_t *res_out, uint16_t *xn_out, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(M), dim3(kNormThreads), 0, st, a, r, w, eps, H, res_out, xn_out);
  return hipGetLastError();
}

}  // namespace flint
