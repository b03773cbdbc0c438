// Router logits, top-k selection with renormalised sigmoid weights, and the
// per-expert routing plan of the decode path.
//
// Semantics (vLLM page "vllm.models.flint.ops.moe": module docstring
// "Numerics", the router kernel _router_kernel and the top-k routine
// _topk_row):
//   logits[t, e] = bf16(fp32 sum_h x[t, h] * router[e, h])
//   selection: the larger logit first, equal logits by the smaller expert
//              index (rank_key in topk.hpp); k rounds of "take the largest
//              remaining key", E <= 256
//   s_j  = RN32(1 / RN32(1 + RN32(exp(-l_j))))  (exact exp, RN division)
//   tw_j = bf16(RN32(s_j / RN32(S + 1e-20))), S = fp32 sum of the s_j in
//          selection order.
//
// Cross-workgroup completion follows the pages' "last program does the
// top-k" scheme: a per-token-group arrival counter, incremented after each
// workgroup's logits are globally visible; the workgroup that arrives last
// runs the selection.  Unlike the pages' never-reset counter, the last
// arriver resets its counter to zero, so any number of workgroups per group
// works and the workspace is clean after every call.
#include "common.hpp"
#include "internal.hpp"
#include "topk.hpp"

namespace flint {

namespace {

constexpr int kThreads = 256;  // 4 waves

// Top-k of one token's logits by one wave (top_k <= E <= 256).  Selection j
// is kept in a register of lane j % 64 (slot j / 64).  Writes the ids, tw
// and (if non-NULL) scores rows of the token.
// NS key slots per lane (E <= 64 NS): expert lane + 64 i in slot i.
template <int NS>
__device__ void topk_token_ns(const uint16_t *lrow, int E, int top_k, int32_t *ids, float *tw,
                              float *scores) {
  const int lane = threadIdx.x & (kWave - 1);
  int keys[NS], sel[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + kWave * i;
    keys[i] = (e < E) ? rank_key(lrow[e], e) : kNoKey;
    sel[i] = kNoKey;
  }
  for (int j = 0; j < top_k; ++j) {
    int m = keys[0];
#pragma unroll
    for (int i = 1; i < NS; ++i) m = max(m, keys[i]);
    const int best = wave_max_i32(m);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      keys[i] = keys[i] == best ? kNoKey : keys[i];
      if ((j >> 6) == i) sel[i] = lane == (j & (kWave - 1)) ? best : sel[i];
    }
  }
  // Sigmoid score of each selected logit, by the lane that holds it.
  float s[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) s[i] = kWave * i + lane < top_k ? router_score(sel[i]) : 0.0f;
  // Renormalisation: fp32 sum in selection order, then one RN division each.
  float S = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    const int i = j >> 6;
    float v = s[0];
#pragma unroll
    for (int ii = 1; ii < NS; ++ii) v = i == ii ? s[ii] : v;
    S = S + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v),
                                                                 j & (kWave - 1)));
  }
  const float D = S + 1e-20f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int j = kWave * i + lane;
    if (j < top_k) {
      ids[j] = key_expert(sel[i]);
      tw[j] = round_bf16(s[i] / D);
      if (scores) scores[j] = s[i];
    }
  }
}

__device__ void topk_token(const uint16_t *lrow, int E, int top_k, int32_t *ids, float *tw,
                           float *scores) {
  if (E <= kWave) topk_token_ns<1>(lrow, E, top_k, ids, tw, scores);
  else if (E <= 2 * kWave) topk_token_ns<2>(lrow, E, top_k, ids, tw, scores);
  else topk_token_ns<4>(lrow, E, top_k, ids, tw, scores);
}

__device__ int block_inclusive_scan(int v, int *lds4) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == kWave - 1) lds4[wv] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wv; ++w) add += lds4[w];
  __syncthreads();
  return v + add;
}

// Builds the routing plan of M*top_k pairs from ids (visible to this block).
// Needs kThreads threads; mask is LDS of E * ceil(P/32) words.
__device__ void build_plan(const int32_t *ids, int M, int E, int top_k, Plan plan,
                           uint32_t *mask, int *lds4) {
  const int P = M * top_k;
  const int W = (P + 31) / 32;
  for (int i = threadIdx.x; i < E * W; i += kThreads) mask[i] = 0u;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kThreads) {
    int e = ids[p];
    if ((unsigned)e < (unsigned)E)  // out-of-range ids are dropped
      atomicOr(&mask[e * W + (p >> 5)], 1u << (p & 31));
  }
  __syncthreads();
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E)
    for (int w = 0; w < W; ++w) cnt += __popc(mask[e * W + w]);
  const int flag = cnt > 0 ? 1 : 0;
  const int base = block_inclusive_scan(cnt, lds4) - cnt;
  const int slot = block_inclusive_scan(flag, lds4) - flag;
  if (flag) {
    plan.active[slot] = e;
    plan.offs[slot] = base;
    int pos = base;
    for (int w = 0; w < W; ++w) {
      uint32_t bits = mask[e * W + w];
      while (bits) {
        int b = __builtin_ctz(bits);
        bits &= bits - 1u;
        plan.pairs[pos++] = w * 32 + b;
      }
    }
  }
  if (e == kThreads - 1) {
    // the last thread holds the inclusive totals of both scans
    plan.n_active[0] = slot + flag;
    plan.offs[slot + flag] = base + cnt;
  }
}

// Router GEMV + top-k (+ plan).  Grid (ceil(E / 4), ceil(M / 8)); wave w of
// block (eb, tg) computes expert 4*eb + w for the 8 tokens of group tg.
template <int H>
__global__ void __launch_bounds__(kThreads)
route_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ router, int M,
             int E, int top_k, uint16_t *__restrict__ logits, int32_t *__restrict__ ids,
             float *__restrict__ tw, int32_t *__restrict__ counters, Plan plan,
             int with_plan) {
  constexpr int NC = H / 8;                       // 16-byte chunks per row
  constexpr int CPL = (NC + kWave - 1) / kWave;   // chunks per lane
  __shared__ uint32_t mask[kMaxExperts * (kMaxDecodePairs / 32)];
  __shared__ int lds4[4];
  __shared__ int is_last;

  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int eb = blockIdx.x, tg = blockIdx.y;
  const int e = eb * kRouteExperts + wv;
  const int t0 = tg * kRouteTokens;
  const int nt = min(kRouteTokens, M - t0);

  if (e < E) {
    u32x4_t w[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      int c = lane + kWave * i;
      w[i] = (c < NC) ? load16(router + (size_t)e * H + c * 8) : u32x4_t{0, 0, 0, 0};
    }
    for (int ti = 0; ti < nt; ++ti) {
      const uint16_t *xr = x + (size_t)(t0 + ti) * H;
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        int c = lane + kWave * i;
        if (c < NC) {
          u32x4_t v = load16(xr + c * 8);
          acc = dot2_bf16(w[i][0], v[0], acc);
          acc = dot2_bf16(w[i][1], v[1], acc);
          acc = dot2_bf16(w[i][2], v[2], acc);
          acc = dot2_bf16(w[i][3], v[3], acc);
        }
      }
      acc = group_sum<kWave>(acc);
      if (lane == kWave - 1) logits[(size_t)(t0 + ti) * E + e] = (uint16_t)f32_to_bf16(acc);
    }
  }
  // Publish this block's logits, then count arrivals of the token group.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = atomicAdd(&counters[tg], 1);
    int last = (prev == (int)gridDim.x - 1);
    if (last) atomicExch(&counters[tg], 0);
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();  // acquire the other blocks' logits

  for (int ti = wv; ti < nt; ti += 4) {
    const int t = t0 + ti;
    topk_token(logits + (size_t)t * E, E, top_k, ids + (size_t)t * top_k,
               tw + (size_t)t * top_k, nullptr);
  }
  if (!with_plan) return;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = atomicAdd(&counters[kCtrRouteAll], 1);
    int last = (prev == (int)gridDim.y - 1);
    if (last) atomicExch(&counters[kCtrRouteAll], 0);
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  build_plan(ids, M, E, top_k, plan, mask, lds4);
}

// Top-k of given logits: one wave per token, 4 tokens per block.
__global__ void __launch_bounds__(kThreads)
topk_kernel(const uint16_t *__restrict__ logits, int M, int E, int top_k,
            int32_t *__restrict__ ids, float *__restrict__ tw, float *__restrict__ scores) {
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * 4 + wv;
  if (t >= M) return;
  topk_token(logits + (size_t)t * E, E, top_k, ids + (size_t)t * top_k,
             tw + (size_t)t * top_k, scores ? scores + (size_t)t * top_k : nullptr);
}

__global__ void __launch_bounds__(kThreads)
plan_kernel(const int32_t *__restrict__ ids, int M, int E, int top_k, Plan plan) {
  __shared__ uint32_t mask[kMaxExperts * (kMaxDecodePairs / 32)];
  __shared__ int lds4[4];
  build_plan(ids, M, E, top_k, plan, mask, lds4);
}

}  // namespace

hipError_t launch_topk(const uint16_t *logits, int M, int E, int top_k, int32_t *ids,
                       float *tw, float *scores, hipStream_t st) {
  dim3 grid((M + 3) / 4);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(kThreads), 0, st, logits, M, E, top_k, ids,
                     tw, scores);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t *ids, int M, int E, int top_k, const Plan &plan,
                       hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, st, ids, M, E, top_k, plan);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t *x, const uint16_t *router, int M, int H, int E,
                        int top_k, uint16_t *logits, int32_t *ids, float *tw,
                        int32_t *counters, const Plan *plan, hipStream_t st) {
  dim3 grid((E + kRouteExperts - 1) / kRouteExperts, (M + kRouteTokens - 1) / kRouteTokens);
  Plan p = plan ? *plan : Plan{nullptr, nullptr, nullptr, nullptr};
  int wp = plan ? 1 : 0;
  switch (H) {
#define FLINT_ROUTE_CASE(HH)                                                              \
  case HH:                                                                                \
    hipLaunchKernelGGL(route_kernel<HH>, grid, dim3(kThreads), 0, st, x, router, M, E,    \
                       top_k, logits, ids, tw, counters, p, wp);                          \
    break;
    FLINT_ROUTE_CASE(256)
    FLINT_ROUTE_CASE(512)
    FLINT_ROUTE_CASE(1024)
    FLINT_ROUTE_CASE(2048)
    FLINT_ROUTE_CASE(4096)
#undef FLINT_ROUTE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace flint
