// Decode-path expert kernels: gate/up + SwiGLU, down projection, combine.
//
// Semantics (vLLM page "vllm.models.flint.ops.moe": module docstring
// "Numerics", _gate_up_gemv_kernel, _down_gemv_kernel, their BF16 variants
// and _combine_kernel):
//   g = fp32(x . W13[e, n]) * alpha13[e],  u = fp32(x . W13[e, I + n]) * alpha13[e]
//   act = bf16(silu(g) * u)
//   y   = bf16(fp32(act . W2[e, h]) * alpha2[e])
//   out = bf16(bf16(sum_j tw_j * y_j) + shared)
// BF16 weights (and the shared expert) have no alpha.  NVFP4 weights are
// dequantised exactly: E2M1 code -> bf16 by the hardware converter, E4M3
// block scale applied to the fp32 partial sum of its 16 elements.
//
// Work is expert-centric: a block handles one (expert slot, row block) and
// streams each weight row of a touched expert exactly once, applying it to
// every pair routed to that expert.  Untouched experts are never read.
//
// Lane mapping of one weight row of K elements split in 16-byte chunks (32
// NVFP4 codes or 8 bf16): LPR lanes share a row, lane q of a row owns chunks
// q + LPR * i (i < CPL), so every load instruction reads LPR * 16 contiguous
// bytes of a row; 64 / LPR rows are in flight per load instruction.
#include "common.hpp"
#include "internal.hpp"

namespace flint {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = 4;

constexpr int pow2_divisor(int n, int cap) {
  int p = 1;
  while (p * 2 <= cap && n % (p * 2) == 0) p *= 2;
  return p;
}

template <int FMT, int K>
struct RowMap {
  static constexpr int CE = FMT == kNvfp4 ? 32 : 8;        // elements per chunk
  static constexpr int NC = K / CE;                          // chunks per row
  static constexpr int LPR = pow2_divisor(NC, kWave);        // lanes per row
  static constexpr int CPL = NC / LPR;                       // chunks per lane
  static constexpr int RS = kWave / LPR;                     // rows per slice
  static constexpr int ROW_BYTES = FMT == kNvfp4 ? K / 2 : K * 2;
  static constexpr int VEC_U4 = CE / 8;                      // 16B vector loads per chunk
  static_assert(K % CE == 0, "row length");
};

// Weight registers of one row for one lane: raw chunks, and for NVFP4 the
// codes converted to bf16 pairs plus the two block scales of each chunk.
template <int FMT, int K>
struct RowRegs {
  using Map = RowMap<FMT, K>;
  u32x4_t raw[Map::CPL];
  uint32_t sc[Map::CPL];  // NVFP4: two E4M3 bytes of the chunk
};

template <int FMT, int K>
__device__ __forceinline__ void load_row(RowRegs<FMT, K> &r, const uint8_t *wrow,
                                         const uint8_t *srow, int q) {
  using Map = RowMap<FMT, K>;
#pragma unroll
  for (int i = 0; i < Map::CPL; ++i) {
    const int c = q + Map::LPR * i;
    r.raw[i] = load16_stream(wrow + (size_t)c * 16);
    if constexpr (FMT == kNvfp4) r.sc[i] = load_u16(srow + (size_t)c * 2);
  }
}

// Partial dot product of one lane's chunks of a row with the matching
// elements of a bf16 vector (row-major, K elements).
template <int FMT, int K>
__device__ __forceinline__ float row_dot(const RowRegs<FMT, K> &r, const uint16_t *vec, int q) {
  using Map = RowMap<FMT, K>;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < Map::CPL; ++i) {
    const int c = q + Map::LPR * i;
    const uint16_t *v = vec + (size_t)c * Map::CE;
    if constexpr (FMT == kNvfp4) {
      // 32 codes: elements 0..15 (dwords 0,1) under scale byte 0, 16..31
      // (dwords 2,3) under scale byte 1.
      float part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4_t va = load16(v + 16 * h);
        u32x4_t vb = load16(v + 16 * h + 8);
        uint32_t w0[4], w1[4];
        fp4x8_to_bf16(r.raw[i][2 * h], w0);
        fp4x8_to_bf16(r.raw[i][2 * h + 1], w1);
        float p = dot2_bf16(w0[0], va[0], 0.0f);
        p = dot2_bf16(w0[1], va[1], p);
        p = dot2_bf16(w0[2], va[2], p);
        p = dot2_bf16(w0[3], va[3], p);
        p = dot2_bf16(w1[0], vb[0], p);
        p = dot2_bf16(w1[1], vb[1], p);
        p = dot2_bf16(w1[2], vb[2], p);
        p = dot2_bf16(w1[3], vb[3], p);
        part[h] = p;
      }
      acc += part[0] * e4m3_to_f32(r.sc[i] & 0xffu);
      acc += part[1] * e4m3_to_f32((r.sc[i] >> 8) & 0xffu);
    } else {
      u32x4_t va = load16(v);
      acc = dot2_bf16(r.raw[i][0], va[0], acc);
      acc = dot2_bf16(r.raw[i][1], va[1], acc);
      acc = dot2_bf16(r.raw[i][2], va[2], acc);
      acc = dot2_bf16(r.raw[i][3], va[3], acc);
    }
  }
  return acc;
}

// Job of a block: expert slot (or the single shared/dense job) and row block.
struct Job {
  int expert;      // expert index into the weight arrays
  int p_begin;     // range into the pair list
  int p_end;
  bool valid;
};

__device__ __forceinline__ Job job_of(int routed, Plan plan, int slot, int M) {
  Job j;
  if (!routed) {  // dense job: expert 0, pairs 0..M-1 are the tokens
    j.expert = 0;
    j.p_begin = 0;
    j.p_end = M;
    j.valid = slot == 0;
    return j;
  }
  const int n = plan.n_active[0];
  j.valid = slot < n;
  if (!j.valid) return j;
  j.expert = plan.active[slot];
  j.p_begin = plan.offs[slot];
  j.p_end = plan.offs[slot + 1];
  return j;
}

// ------------------------------------------------------------- gate/up

// Row pairs per wave: at least 2, and a whole number of row slices.
template <int FMT, int H>
struct GateUpGeo {
  using Map = RowMap<FMT, H>;
  static constexpr int RP = Map::RS >= 2 ? Map::RS : 2;
  static constexpr int NSL = RP / Map::RS;
  static constexpr int ROWS_PER_BLOCK = RP * kWaves;
};

// Grid (I / ROWS_PER_BLOCK, slots).  For a routed job, pair p's token is
// p / top_k; for the dense job (routed == 0) the pair index is the token.
template <int FMT, int H>
__global__ void __launch_bounds__(kThreads)
gate_up_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ w13,
               const uint8_t *__restrict__ s13, const float *__restrict__ a13, int M, int I,
               int top_k, int routed, Plan plan, uint16_t *__restrict__ act) {
  using Map = RowMap<FMT, H>;
  using Geo = GateUpGeo<FMT, H>;
  const Job job = job_of(routed, plan, blockIdx.y, M);
  if (!job.valid) return;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  const int n_base = blockIdx.x * Geo::ROWS_PER_BLOCK + wv * Geo::RP;

  const size_t mat_rows = 2 * (size_t)I;
  const uint8_t *wexp = w13 + (size_t)job.expert * mat_rows * Map::ROW_BYTES;
  const uint8_t *sexp = FMT == kNvfp4 ? s13 + (size_t)job.expert * mat_rows * (H / 16) : nullptr;
  RowRegs<FMT, H> g[Geo::NSL], u[Geo::NSL];
#pragma unroll
  for (int s = 0; s < Geo::NSL; ++s) {
    const int n = n_base + s * Map::RS + r;
    load_row(g[s], wexp + (size_t)n * Map::ROW_BYTES,
             FMT == kNvfp4 ? sexp + (size_t)n * (H / 16) : nullptr, q);
    load_row(u[s], wexp + (size_t)(I + n) * Map::ROW_BYTES,
             FMT == kNvfp4 ? sexp + (size_t)(I + n) * (H / 16) : nullptr, q);
  }
  const float alpha = FMT == kNvfp4 ? a13[job.expert] : 1.0f;

  for (int pi = job.p_begin; pi < job.p_end; ++pi) {
    const int p = routed ? plan.pairs[pi] : pi;
    const int t = routed ? p / top_k : p;
    const uint16_t *xr = x + (size_t)t * H;
#pragma unroll
    for (int s = 0; s < Geo::NSL; ++s) {
      float gs = group_sum<Map::LPR>(row_dot(g[s], xr, q));
      float us = group_sum<Map::LPR>(row_dot(u[s], xr, q));
      if (q == 0) {
        if constexpr (FMT == kNvfp4) {
          gs = gs * alpha;
          us = us * alpha;
        }
        const int n = n_base + s * Map::RS + r;
        act[(size_t)p * I + n] = (uint16_t)f32_to_bf16(swiglu(gs, us));
      }
    }
  }
}

// ---------------------------------------------------------------- down

template <int FMT, int I>
struct DownGeo {
  using Map = RowMap<FMT, I>;
  static constexpr int RW = Map::RS >= 8 ? Map::RS : 8;  // rows per wave
  static constexpr int NSL = RW / Map::RS;
  static constexpr int ROWS_PER_BLOCK = RW * kWaves;
};

// Grid (H / ROWS_PER_BLOCK, slots).  y[p, h] for every pair of the job.
template <int FMT, int I>
__global__ void __launch_bounds__(kThreads)
down_kernel(const uint16_t *__restrict__ act, const uint8_t *__restrict__ w2,
            const uint8_t *__restrict__ s2, const float *__restrict__ a2, int M, int H,
            int routed, Plan plan, uint16_t *__restrict__ y) {
  using Map = RowMap<FMT, I>;
  using Geo = DownGeo<FMT, I>;
  const Job job = job_of(routed, plan, blockIdx.y, M);
  if (!job.valid) return;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  const int h_base = blockIdx.x * Geo::ROWS_PER_BLOCK + wv * Geo::RW;

  const uint8_t *wexp = w2 + (size_t)job.expert * H * Map::ROW_BYTES;
  const uint8_t *sexp = FMT == kNvfp4 ? s2 + (size_t)job.expert * H * (I / 16) : nullptr;
  RowRegs<FMT, I> w[Geo::NSL];
#pragma unroll
  for (int s = 0; s < Geo::NSL; ++s) {
    const int h = h_base + s * Map::RS + r;
    load_row(w[s], wexp + (size_t)h * Map::ROW_BYTES,
             FMT == kNvfp4 ? sexp + (size_t)h * (I / 16) : nullptr, q);
  }
  const float alpha = FMT == kNvfp4 ? a2[job.expert] : 1.0f;

  for (int pi = job.p_begin; pi < job.p_end; ++pi) {
    const int p = routed ? plan.pairs[pi] : pi;
    const uint16_t *ar = act + (size_t)p * I;
#pragma unroll
    for (int s = 0; s < Geo::NSL; ++s) {
      float v = group_sum<Map::LPR>(row_dot(w[s], ar, q));
      if (q == 0) {
        if constexpr (FMT == kNvfp4) v = v * alpha;
        const int h = h_base + s * Map::RS + r;
        y[(size_t)p * H + h] = (uint16_t)f32_to_bf16(v);
      }
    }
  }
}

// ------------------------------------------------------------- combine

// out[t, h] = bf16(bf16(R) + sh[t, h]) with R the fp32 rounding of
// sum_j tw[t, j] * y[t*k + j, h].  The k products are exact in fp32 (bf16 x
// bf16) and their sum is formed exactly in fp64 before the single fp32
// rounding, so R is the correctly rounded fp32 sum whatever the order.
// One thread per (token, 8 columns).
__global__ void __launch_bounds__(kThreads)
combine_kernel(const uint16_t *__restrict__ y, const float *__restrict__ tw,
               const uint16_t *__restrict__ sh, int M, int H, int top_k,
               uint16_t *__restrict__ out) {
  const int cols8 = H / 8;
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  if (gid >= M * cols8) return;
  const int t = gid / cols8, c = gid % cols8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < top_k; ++j) {
    const double wj = (double)tw[(size_t)t * top_k + j];
    u32x4_t v = load16(y + ((size_t)t * top_k + j) * H + c * 8);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      acc[2 * d] += wj * (double)bf16_lo(v[d]);
      acc[2 * d + 1] += wj * (double)bf16_hi(v[d]);
    }
  }
  u32x4_t s = sh ? load16(sh + (size_t)t * H + c * 8) : u32x4_t{0, 0, 0, 0};
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float r0 = round_bf16((float)acc[2 * d]);
    float r1 = round_bf16((float)acc[2 * d + 1]);
    uint32_t lo = f32_to_bf16(r0 + bf16_lo(s[d]));
    uint32_t hi = f32_to_bf16(r1 + bf16_hi(s[d]));
    o[d] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x4_t *>(out + (size_t)t * H + c * 8) = o;
}

template <int FMT, int H>
hipError_t gate_up_h(const uint16_t *x, const void *w13, const uint8_t *s13, const float *a13,
                     int M, int I, int top_k, int max_slots, const Plan *plan, uint16_t *act,
                     hipStream_t st) {
  using Geo = GateUpGeo<FMT, H>;
  if (I % Geo::ROWS_PER_BLOCK) return hipErrorInvalidValue;
  dim3 grid(I / Geo::ROWS_PER_BLOCK, plan ? max_slots : 1);
  Plan p = plan ? *plan : Plan{nullptr, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL((gate_up_kernel<FMT, H>), grid, dim3(kThreads), 0, st, x,
                     (const uint8_t *)w13, s13, a13, M, I, top_k, plan ? 1 : 0, p, act);
  return hipGetLastError();
}

template <int FMT, int I>
hipError_t down_i(const uint16_t *act, const void *w2, const uint8_t *s2, const float *a2,
                  int M, int H, int max_slots, const Plan *plan, uint16_t *y, hipStream_t st) {
  using Geo = DownGeo<FMT, I>;
  if (H % Geo::ROWS_PER_BLOCK) return hipErrorInvalidValue;
  dim3 grid(H / Geo::ROWS_PER_BLOCK, plan ? max_slots : 1);
  Plan p = plan ? *plan : Plan{nullptr, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL((down_kernel<FMT, I>), grid, dim3(kThreads), 0, st, act,
                     (const uint8_t *)w2, s2, a2, M, H, plan ? 1 : 0, p, y);
  return hipGetLastError();
}

}  // namespace

// Compiled (H, I) shapes: the Flint configuration (2048, 768) and smaller
// shapes for tests.
bool decode_shape_supported(int H, int I) {
  const bool h_ok = H == 256 || H == 512 || H == 2048;
  const bool i_ok = I == 128 || I == 256 || I == 768;
  return h_ok && i_ok;
}

hipError_t launch_gate_up(int fmt, const uint16_t *x, const void *w13, const uint8_t *s13,
                          const float *a13, int M, int H, int I, int top_k, int max_slots,
                          const Plan *plan, uint16_t *act, hipStream_t st) {
#define FLINT_GU(F, HH) \
  if (fmt == F && H == HH) return gate_up_h<F, HH>(x, w13, s13, a13, M, I, top_k, max_slots, plan, act, st);
  FLINT_GU(kNvfp4, 256) FLINT_GU(kNvfp4, 512) FLINT_GU(kNvfp4, 2048)
  FLINT_GU(kBf16, 256) FLINT_GU(kBf16, 512) FLINT_GU(kBf16, 2048)
#undef FLINT_GU
  return hipErrorInvalidValue;
}

hipError_t launch_down(int fmt, const uint16_t *act, const void *w2, const uint8_t *s2,
                       const float *a2, int M, int H, int I, int top_k, int max_slots,
                       const Plan *plan, uint16_t *y, hipStream_t st) {
  (void)top_k;
#define FLINT_DN(F, II) \
  if (fmt == F && I == II) return down_i<F, II>(act, w2, s2, a2, M, H, max_slots, plan, y, st);
  FLINT_DN(kNvfp4, 128) FLINT_DN(kNvfp4, 256) FLINT_DN(kNvfp4, 768)
  FLINT_DN(kBf16, 128) FLINT_DN(kBf16, 256) FLINT_DN(kBf16, 768)
#undef FLINT_DN
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const uint16_t *y, const float *tw, const uint16_t *sh, int M,
                          int H, int top_k, uint16_t *out, hipStream_t st) {
  const int n = M * (H / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     st, y, tw, sh, M, H, top_k, out);
  return hipGetLastError();
}

}  // namespace flint
