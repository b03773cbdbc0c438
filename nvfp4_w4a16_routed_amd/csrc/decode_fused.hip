// The decode-path MoE block (M <= 64 tokens) as one persistent kernel.
//
// Semantics (vLLM page "vllm.models.flint.ops.moe": module docstring
// "Numerics"; _router_kernel/_topk_row, _gate_up_gemv_kernel,
// _down_gemv_kernel, their BF16 variants and _combine_kernel):
//   logits = bf16(fp32 x . router[e]);  top-k by the order-preserving key
//   s_j = RN32(1 / RN32(1 + RN32(exp(-l_j)))), tw_j = bf16(s_j / (S + 1e-20))
//   g, u = fp32 (x . W13[e, n]) * alpha13[e], (x . W13[e, I+n]) * alpha13[e]
//   act = bf16(silu(g) * u);  y = bf16(fp32 (act . W2[e, h]) * alpha2[e])
//   out = bf16(bf16(sum_j tw_j y_j) + shared(x))
// The shared expert follows the same rule with bf16 weights and no alpha.
//
// Instead of the pages' three programmatically chained launches, every step
// runs in one cooperative launch whose waves walk a common list of wave-sized
// work items.  Item i belongs to wave i mod (number of waves); the list is
//   [routing: (token, 4 experts)] [shared gate/up: row pairs]
//   [routed gate/up: (touched expert, row pairs)] [shared down: rows]
//   [routed down: (touched expert, rows)]
// Dependencies are arrival counters in the workspace:
//   - the last routing item of a token runs that token's top-k and marks its
//     experts in a touched-expert bitmask; gate/up items wait until every
//     token is routed (the pages' "last program does the top-k" scheme);
//   - a down item waits for all gate/up items of its expert (it loads its
//     weights before waiting, so the wait overlaps the HBM latency);
//   - the last down item to finish a block of output rows runs the combine
//     for those rows (all touched experts and the shared expert arrived).
// A wave waits only for items that precede it in the list, and every wave
// of the grid is resident (cooperative launch), so every wait ends.  The
// last wave to finish resets the counters for the next call.
//
// Weights of only the touched experts are read, each row exactly once;
// tokens of an expert are found by a ballot over the ids.
#include "common.hpp"
#include "internal.hpp"
#include "rowdot.hpp"

namespace flint {

namespace {

constexpr int kThreads = 256;
constexpr int kRouteExpertsPerItem = 4;
// Register budget of the kernel: at least kWavesPerEU waves fit on a SIMD
// whatever the allocator does, so kWavesPerEU blocks of 4 waves per CU are
// always co-resident.  The grid never exceeds that (the cooperative wait
// scheme needs every block resident).
constexpr int kWavesPerEU = 3;
// Largest batch whose x is staged in LDS for the gate/up items.
constexpr int kXLdsBytes = 32768;

struct FusedParams {
  const uint16_t *x;
  const uint16_t *router;
  const uint8_t *w13;
  const uint8_t *s13;
  const float *a13;
  const uint8_t *w2;
  const uint8_t *s2;
  const float *a2;
  const uint8_t *sgu;    // shared [2I, H] bf16, NULL = no shared expert
  const uint8_t *sdown;  // shared [H, I] bf16
  const int32_t *ids_in; // forced routing (NULL = route)
  const float *tw_in;
  uint16_t *logits;
  int32_t *ids;
  float *tw;
  uint16_t *act;
  uint16_t *y;
  uint16_t *sact;
  uint16_t *sh;
  uint16_t *out;
  DecodeSync *sync;
  int M, E, top_k;
#ifdef FLINT_TRACE
  uint64_t *trace;  // [waves][32] timestamps (s_memrealtime), timing builds only
#endif
};

#ifdef FLINT_TRACE
#define FLINT_MARK(P, gw, slot)                                                   \
  do {                                                                            \
    if ((threadIdx.x & 63) == 0) (P).trace[(size_t)(gw) * 32 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define FLINT_MARK(P, gw, slot) do { } while (0)
#endif

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ int bcast0(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------ phase barriers
//
// A phase ends when its last arrival is counted; that wave then raises the
// per-block flag go[b] of every block (each on its own line), and one wave
// per block polls only its own flag, so no line is polled by many waves.

__device__ void broadcast_phase(DecodeSync *S, int phase) {
  stores_performed();
  for (int b = threadIdx.x & (kWave - 1); b < (int)gridDim.x; b += kWave) store_agent(&S->go[b][0], phase);
}

// One token's routing is complete; the M-th raises phase 1 (and resets
// the counter).
__device__ __forceinline__ void routed_token(DecodeSync *S, int M) {
  if (arrive(&S->topk_done[0]) == M - 1) {
    if ((threadIdx.x & (kWave - 1)) == 0) store_agent(&S->topk_done[0], 0);
    broadcast_phase(S, 1);
  }
}

// All waves of the block wait until the block's flag reaches `phase`.
__device__ __forceinline__ void block_wait_phase(DecodeSync *S, int phase) {
  __syncthreads();
  if (threadIdx.x < kWave) wait_flag(&S->go[blockIdx.x][0], phase);
  __syncthreads();
}

// End of the gate/up phase for this block: a two-level arrival tree (blocks
// -> kBarrierGroups group counters -> one top counter); the last arrival
// clears the touched-expert mask (every wave has read it) and raises phase 2.
__device__ void block_end_gate_up(DecodeSync *S) {
  stores_performed();
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int NB = gridDim.x, ng = NB < kBarrierGroups ? NB : kBarrierGroups;
    const int g = blockIdx.x % ng;
    const int gsize = (NB - g + ng - 1) / ng;
    if (arrive(&S->grp_cnt[g][0]) == gsize - 1) {
      if (threadIdx.x == 0) store_agent(&S->grp_cnt[g][0], 0);
      if (arrive(&S->top_cnt[0]) == ng - 1) {
        if (threadIdx.x == 0) store_agent(&S->top_cnt[0], 0);
        if (threadIdx.x < 8) store_agent((int *)&S->active[threadIdx.x], 0);
        broadcast_phase(S, 2);
      }
    }
    wait_flag(&S->go[blockIdx.x][0], 2);
  }
  __syncthreads();
  if (threadIdx.x == 0) store_agent(&S->go[blockIdx.x][0], 0);  // no one reads it again
}

// ---------------------------------------------------------------- top-k

__device__ __forceinline__ int topk_key(uint32_t bits, int e, int E) {
  int b = (int)(bits & 0xffffu);
  int ord = (b >= 0x8000) ? (b ^ 0xffff) : (b | 0x8000);
  return (ord << 8) | (E - 1 - e);
}

__device__ __forceinline__ uint32_t key_bits(int key) {
  int o = key >> 8;
  return (uint32_t)((o >= 0x8000) ? (o ^ 0x8000) : (o ^ 0xffff));
}

// Top-k of token t by one wave (top_k <= E <= 256); marks the selected
// experts in the touched bitmask.
__device__ void topk_token(const FusedParams &P, int t) {
  const int lane = lane_id();
  const int E = P.E, k = P.top_k;
  const uint16_t *lrow = P.logits + (size_t)t * E;
  int keys[4], sel[4] = {-1, -1, -1, -1};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + kWave * i;
    keys[i] = (e < E) ? topk_key(ld_dev(&lrow[e]), e, E) : -1;
  }
  for (int j = 0; j < k; ++j) {
    int best = wave_max_i32(max(max(keys[0], keys[1]), max(keys[2], keys[3])));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (keys[i] == best) keys[i] = -1;
      if ((j >> 6) == i && lane == (j & (kWave - 1))) sel[i] = best;
    }
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = 0.0f;
    if (kWave * i + lane < k) {
      float l = bf16_to_f32(key_bits(sel[i]));
      float a = (float)exp(-(double)l);  // correctly rounded for every bf16 l
      float d = 1.0f + a;
      s[i] = 1.0f / d;
    }
  }
  float S = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int i = j >> 6;
    float v = (i == 0) ? s[0] : (i == 1) ? s[1] : (i == 2) ? s[2] : s[3];
    S = S + __shfl(v, j & (kWave - 1), kWave);
  }
  const float D = S + 1e-20f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = kWave * i + lane;
    if (j < k) {
      const int e = E - 1 - (sel[i] & 0xff);
      st_dev(&P.ids[(size_t)t * k + j], e);
      st_dev(&P.tw[(size_t)t * k + j], round_bf16(s[i] / D));
      __hip_atomic_fetch_or(&P.sync->active[e >> 5], 1u << (e & 31), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// --------------------------------------------------------------- routing

// Logits of 4 experts for token t; the token's last item runs its top-k.
template <int H>
__device__ void route_item(const FusedParams &P, int item) {
  constexpr int NC = H / 8;
  constexpr int CPL = (NC + kWave - 1) / kWave;
  const int lane = lane_id();
  const int nRB = (P.E + kRouteExpertsPerItem - 1) / kRouteExpertsPerItem;
  const int t = item / nRB, eb = item % nRB;
  u32x4_t w[kRouteExpertsPerItem][CPL], xv[CPL];
#pragma unroll
  for (int r = 0; r < kRouteExpertsPerItem; ++r) {
    const int e = eb * kRouteExpertsPerItem + r;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + kWave * i;
      w[r][i] = (e < P.E && c < NC) ? load16(P.router + (size_t)e * H + c * 8) : u32x4_t{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + kWave * i;
    xv[i] = (c < NC) ? load16(P.x + (size_t)t * H + c * 8) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int r = 0; r < kRouteExpertsPerItem; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      acc = dot2_bf16(w[r][i][0], xv[i][0], acc);
      acc = dot2_bf16(w[r][i][1], xv[i][1], acc);
      acc = dot2_bf16(w[r][i][2], xv[i][2], acc);
      acc = dot2_bf16(w[r][i][3], xv[i][3], acc);
    }
    acc = group_sum<kWave>(acc);
    const int e = eb * kRouteExpertsPerItem + r;
    if (lane == kWave - 1 && e < P.E)
      st_dev(&P.logits[(size_t)t * P.E + e], (uint16_t)f32_to_bf16(acc));
  }
  if (arrive(&P.sync->route_cnt[t][0]) != nRB - 1) return;
  if (lane == 0) store_agent(&P.sync->route_cnt[t][0], 0);  // last arrival: reset
  topk_token(P, t);
  routed_token(P.sync, P.M);
}

// Forced routing: token t's given ids / tw mark the touched experts.
__device__ void forced_item(const FusedParams &P, int t) {
  const int lane = lane_id();
  for (int j = lane; j < P.top_k; j += kWave) {
    const size_t p = (size_t)t * P.top_k + j;
    const int e = P.ids_in[p];
    if (P.ids != P.ids_in) st_dev(&P.ids[p], e);
    if (P.tw != P.tw_in) st_dev(&P.tw[p], P.tw_in[p]);
    if ((unsigned)e < (unsigned)P.E)
      __hip_atomic_fetch_or(&P.sync->active[e >> 5], 1u << (e & 31), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
  }
  routed_token(P.sync, P.M);
}

// ------------------------------------------------------------- plan view

// The routing as seen by an expert item: the touched-expert bitmask and the
// ids, from which slot -> expert and expert -> pairs are derived.
struct Routing {
  uint32_t active[8];
  int n_active;
  const uint8_t *ids;  // this wave's LDS copy of the ids of all M * top_k pairs
};

// The touched-expert bitmask (uniform) and this wave's copy of the ids.
__device__ __forceinline__ Routing load_routing(const FusedParams &P, uint8_t *ids_lds) {
  Routing R;
  R.n_active = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    R.active[w] = (uint32_t)bcast0(load_agent((const int *)&P.sync->active[w]));
    R.n_active += __popc(R.active[w]);
  }
  const int npairs = P.M * P.top_k;
  const int32_t *ids = P.ids_in ? P.ids_in : P.ids;
  for (int p = lane_id(); p < npairs; p += kWave) ids_lds[p] = (uint8_t)ld_dev(&ids[p]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  R.ids = ids_lds;
  return R;
}

// Expert of slot s (the s-th touched expert in ascending order).
__device__ __forceinline__ int slot_expert(const Routing &R, int s) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int c = __popc(R.active[w]);
    if (s < c) {
      uint32_t m = R.active[w];
      for (int i = 0; i < s; ++i) m &= m - 1u;
      return w * 32 + __builtin_ctz(m);
    }
    s -= c;
  }
  return 0;
}

// Calls f(p) for every pair p routed to expert e, in ascending order.
template <typename F>
__device__ __forceinline__ void for_each_pair(const FusedParams &P, const Routing &R, int e,
                                              F &&f) {
  const int npairs = P.M * P.top_k;
  for (int c0 = 0; c0 < npairs; c0 += kWave) {
    const int p = c0 + lane_id();
    uint64_t m = __ballot(p < npairs && R.ids[p] == e);
    while (m) {
      const int b = __builtin_ctzll(m);
      m &= m - 1ull;
      f(c0 + b);
    }
  }
}

// Smallest pair routed to expert e (-1 if none), uniform over the wave.
__device__ __forceinline__ int first_pair(const FusedParams &P, const Routing &R, int e) {
  const int npairs = P.M * P.top_k;
  for (int c0 = 0; c0 < npairs; c0 += kWave) {
    const int p = c0 + lane_id();
    const uint64_t m = __ballot(p < npairs && R.ids[p] == e);
    if (m) return c0 + __builtin_ctzll(m);
  }
  return -1;
}

// Calls f(p) for every pair p > after routed to expert e, ascending.
template <typename F>
__device__ __forceinline__ void for_each_pair_after(const FusedParams &P, const Routing &R, int e,
                                                    int after, F &&f) {
  const int npairs = P.M * P.top_k;
  for (int c0 = (after + 1) & ~(kWave - 1); c0 < npairs; c0 += kWave) {
    const int p = c0 + lane_id();
    uint64_t m = __ballot(p > after && p < npairs && R.ids[p] == e);
    while (m) {
      const int b = __builtin_ctzll(m);
      m &= m - 1ull;
      f(c0 + b);
    }
  }
}

// --------------------------------------------------------- expert items
//
// Every expert item is split in a load step (its weight rows into
// registers, issued one item ahead so the HBM latency overlaps the previous
// item's arithmetic) and a compute step.

// Weights of a gate/up item: rows[s] = gate row of slice s, rows[NSL + s]
// its up row (RP row pairs n_base .. n_base + RP - 1).
template <int FMT, int H, int I>
struct GateUpW {
  RowRegs<FMT, H> rows[2 * GateUpGeo<FMT, H>::NSL];
};

template <int FMT, int H, int I>
__device__ __forceinline__ void gate_up_load(GateUpW<FMT, H, I> &W, const uint8_t *wexp,
                                             const uint8_t *sexp, int n_base) {
  using Map = RowMap<FMT, H>;
  using Geo = GateUpGeo<FMT, H>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
#pragma unroll
  for (int s = 0; s < Geo::NSL; ++s) {
    const int n = n_base + s * Map::RS + r;
    load_row(W.rows[s], wexp + (size_t)n * Map::ROW_BYTES,
             FMT == kNvfp4 ? sexp + (size_t)n * (H / 16) : nullptr, q);
    load_row(W.rows[Geo::NSL + s], wexp + (size_t)(I + n) * Map::ROW_BYTES,
             FMT == kNvfp4 ? sexp + (size_t)(I + n) * (H / 16) : nullptr, q);
  }
}

// act[p, n] = bf16(silu(g) * u) for the item's rows and every pair p of
// the job (ROUTED: pairs of `expert` from the ids, token p / top_k, output
// act; shared expert: pairs = tokens, output sact).  x is read from the
// block's LDS copy when x_lds is non-NULL (so waiting for it never waits for
// weight loads queued after the item's own), else from global memory.
template <int FMT, int H, int I, bool ROUTED>
__device__ void gate_up_compute(const FusedParams &P, const Routing &R,
                                const GateUpW<FMT, H, I> &W, float alpha, int n_base, int expert,
                                const uint16_t *x_lds) {
  using Map = RowMap<FMT, H>;
  using Geo = GateUpGeo<FMT, H>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  uint16_t *dst = ROUTED ? P.act : P.sact;
  auto one = [&](int p) {
    const int t = ROUTED ? p / P.top_k : p;
    float acc[2 * Geo::NSL];
    GateUpW<FMT, H, I> w = W;
#pragma unroll
    for (int j = 0; j < 2 * Geo::NSL; ++j) opaque(w.rows[j]);
    if (x_lds)
      rows_dot<FMT, H, kSrcLds>(w.rows, x_lds + (size_t)t * H, q, acc);
    else
      rows_dot<FMT, H, kSrcGlobal>(w.rows, P.x + (size_t)t * H, q, acc);
#pragma unroll
    for (int s = 0; s < Geo::NSL; ++s) {
      float gs = group_sum<Map::LPR>(acc[s]);
      float us = group_sum<Map::LPR>(acc[Geo::NSL + s]);
      if (q == Map::LPR - 1) {  // the group's sum is in its last lane
        if constexpr (FMT == kNvfp4) {
          gs = gs * alpha;
          us = us * alpha;
        }
        st_dev(&dst[(size_t)p * I + n_base + s * Map::RS + r], (uint16_t)f32_to_bf16(swiglu(gs, us)));
      }
    }
  };
  if constexpr (ROUTED) {
    for_each_pair_after(P, R, expert, -1, one);
  } else {
    for (int t = 0; t < P.M; ++t) one(t);
  }
}

// Weights of a down item: RW output rows h_base .. h_base + RW - 1.
template <int FMT, int I>
struct DownW {
  RowRegs<FMT, I> rows[DownGeo<FMT, I>::NSL];
};

template <int FMT, int I>
__device__ __forceinline__ void down_load(DownW<FMT, I> &W, const uint8_t *wexp,
                                          const uint8_t *sexp, int h_base) {
  using Map = RowMap<FMT, I>;
  using Geo = DownGeo<FMT, I>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
#pragma unroll
  for (int s = 0; s < Geo::NSL; ++s) {
    const int h = h_base + s * Map::RS + r;
    load_row(W.rows[s], wexp + (size_t)h * Map::ROW_BYTES,
             FMT == kNvfp4 ? sexp + (size_t)h * (I / 16) : nullptr, q);
  }
}

// A pipeline stage: one item's weights and the vector of its first pair,
// loaded together one item ahead of their use.  Loads complete in issue
// order, so computing stage k (issued earlier) never waits for the loads of
// stage k + 1; only the vectors of further pairs are loaded late.
template <int FMT, int H, int I>
struct GuStage {
  GateUpW<FMT, H, I> w;
  int e, n_base;
};

template <int FMT, int I>
struct DnStage {
  DownW<FMT, I> w;
  VecRegs<FMT, I> a0;
  int e, h_base, p0;
};

// y[p, h] = bf16(fp32(act[p] . W2[h]) * alpha) for the item's rows and every
// pair of the job (shared expert: pairs = tokens, sact -> sh).  The first
// pair's activations (p0, a0) were loaded before the next item's weights.
template <int FMT, int H, int I, bool ROUTED>
__device__ void down_compute(const FusedParams &P, const Routing &R, const DownW<FMT, I> &W,
                             float alpha, int h_base, int expert, int p0,
                             const VecRegs<FMT, I> &a0) {
  using Map = RowMap<FMT, I>;
  using Geo = DownGeo<FMT, I>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  const uint16_t *src = ROUTED ? P.act : P.sact;
  uint16_t *dst = ROUTED ? P.y : P.sh;
  auto finish = [&](int p, float (&acc)[Geo::NSL]) {
#pragma unroll
    for (int s = 0; s < Geo::NSL; ++s) {
      float v = group_sum<Map::LPR>(acc[s]);
      if (q == Map::LPR - 1) {  // the group's sum is in its last lane
        if constexpr (FMT == kNvfp4) v = v * alpha;
        st_dev(&dst[(size_t)p * H + h_base + s * Map::RS + r], (uint16_t)f32_to_bf16(v));
      }
    }
  };
  if (p0 < 0) return;
  {
    float acc[Geo::NSL];
    rows_dot_regs(W.rows, a0, acc);
    finish(p0, acc);
  }
  auto other = [&](int p) {
    float acc[Geo::NSL];
    DownW<FMT, I> w = W;
#pragma unroll
    for (int j = 0; j < Geo::NSL; ++j) opaque(w.rows[j]);
    rows_dot<FMT, I, kSrcDevice>(w.rows, src + (size_t)p * I, q, acc);
    finish(p, acc);
  };
  if constexpr (ROUTED) {
    for_each_pair_after(P, R, expert, p0, other);
  } else {
    for (int t = p0 + 1; t < P.M; ++t) other(t);
  }
}

// out[t, h] for the CB rows starting at h0: R = fp32 rounding of the exact
// sum_j tw[t, j] * y[t*k + j, h] (products exact in fp32, summed exactly in
// fp64), out = bf16(bf16(R) + sh[t, h]).
template <int H>
__device__ void combine_rows(const FusedParams &P, int h0, int CB) {
  const int lane = lane_id();
  const int k = P.top_k;
  const float *tw = P.tw_in ? P.tw_in : P.tw;
  for (int idx = lane; idx < P.M * CB; idx += kWave) {
    const int t = idx / CB, h = h0 + idx % CB;
    double acc = 0.0;
    for (int j = 0; j < k; ++j) {
      const size_t p = (size_t)t * k + j;
      acc += (double)ld_dev(&tw[p]) * (double)bf16_to_f32(ld_dev(&P.y[p * H + h]));
    }
    const float routed = round_bf16((float)acc);
    const float s = P.sgu ? bf16_to_f32(ld_dev(&P.sh[(size_t)t * H + h])) : 0.0f;
    P.out[(size_t)t * H + h] = (uint16_t)f32_to_bf16(routed + s);
  }
}

// Work list (item i belongs to wave i mod NW):
//   phase A: [routing (token, 4 experts)] [shared gate/up] [shared down]
//   then, once every token is routed:
//   [routed gate/up (slot, row pairs)] [routed down (slot, rows)]
// A wave streams its routed gate/up items with one-item-ahead weight loads
// and, after its last one, counts one arrival per item on that item's
// expert slot; down items of a slot wait for all its gate/up items.  Down
// items likewise count arrivals per block of output rows at the end, and
// block cb is combined by wave cb mod NW once every contributor arrived.
template <int FMT, int H, int I>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
decode_kernel(FusedParams P) {
  using GU = GateUpGeo<FMT, H>;
  using SGU = GateUpGeo<kBf16, H>;
  using DN = DownGeo<FMT, I>;
  using SDN = DownGeo<kBf16, I>;
  constexpr int nGU = I / GU::RP;    // routed gate/up items per expert
  constexpr int nSGU = I / SGU::RP;  // shared gate/up items
  constexpr int nDN = H / DN::RW;    // routed down items per expert
  constexpr int nSDN = H / SDN::RW;  // shared down items
  constexpr int CB = DN::RW > SDN::RW ? DN::RW : SDN::RW;  // combine block rows
  constexpr int GU_RSZ = FMT == kNvfp4 ? H / 2 : H * 2;    // routed row bytes (w13)
  constexpr int DN_RSZ = FMT == kNvfp4 ? I / 2 : I * 2;    // routed row bytes (w2)
  __shared__ uint8_t ids_lds[kThreads / kWave][kMaxDecodePairs];
  extern __shared__ __attribute__((aligned(16))) uint16_t x_lds[];  // [M, H] when staged

  DecodeSync *S = P.sync;
  const int lane = lane_id();
  const int NW = gridDim.x * (kThreads / kWave);
  const int gw = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  const bool shared = P.sgu != nullptr;
  const bool forced = P.ids_in != nullptr;
  const int nRB = (P.E + kRouteExpertsPerItem - 1) / kRouteExpertsPerItem;
  const int nR = forced ? P.M : P.M * nRB;
  const int nS = shared ? nSGU : 0;
  const int nSD = shared ? nSDN : 0;
  const int nA = nR + nS;

  FLINT_MARK(P, gw, 0);
  // Phase A: routing, and the shared expert's gate/up meanwhile.
  for (int i = gw; i < nA; i += NW) {
    if (i < nR) {
      if (forced)
        forced_item(P, i);
      else
        route_item<H>(P, i);
    } else {
      GateUpW<kBf16, H, I> W;
      const int n_base = (i - nR) * SGU::RP;
      gate_up_load(W, P.sgu, nullptr, n_base);
      gate_up_compute<kBf16, H, I, false>(P, Routing{}, W, 1.0f, n_base, 0, nullptr);
    }
  }
  stores_performed();
  FLINT_MARK(P, gw, 1);
  block_wait_phase(S, 1);  // every token routed
  FLINT_MARK(P, gw, 2);
  const Routing R = load_routing(P, ids_lds[threadIdx.x / kWave]);
  const int nB = R.n_active * nGU;
  const int nC = R.n_active * nDN;
  const int cb_target = R.n_active * (CB / DN::RW) + (shared ? CB / SDN::RW : 0);

  // Stage x in LDS for the gate/up items (small batches).
  const bool stage_x = P.M * H * 2 <= kXLdsBytes;
  if (stage_x) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(P.x);
    u32x4_t *dstl = reinterpret_cast<u32x4_t *>(x_lds);
    for (int v = threadIdx.x; v < P.M * H / 8; v += kThreads) dstl[v] = load16(src + v);
  }
  __syncthreads();
  const uint16_t *xl = stage_x ? x_lds : nullptr;

  // Routed gate/up: items b = gw, gw + NW, ... < nB, two-stage pipeline.
  {
    auto load = [&](GuStage<FMT, H, I> &st, int b) {
      st.e = slot_expert(R, b / nGU);
      st.n_base = (b % nGU) * GU::RP;
      gate_up_load(st.w, P.w13 + (size_t)st.e * 2 * I * GU_RSZ,
                   FMT == kNvfp4 ? P.s13 + (size_t)st.e * 2 * I * (H / 16) : nullptr, st.n_base);
    };
    auto run = [&](const GuStage<FMT, H, I> &st) {
      gate_up_compute<FMT, H, I, true>(P, R, st.w, FMT == kNvfp4 ? P.a13[st.e] : 1.0f, st.n_base,
                                       st.e, xl);
    };
    // Ping-pong between two stages (no register copies between items).
    GuStage<FMT, H, I> sa, sb;
    int b = gw;
    if (b < nB) load(sa, b);
    while (b < nB) {
      if (b + NW < nB) load(sb, b + NW);
      __builtin_amdgcn_sched_barrier(0);
      run(sa);
      b += NW;
      if (b >= nB) break;
      if (b + NW < nB) load(sa, b + NW);
      __builtin_amdgcn_sched_barrier(0);
      run(sb);
      b += NW;
    }
  }
  FLINT_MARK(P, gw, 3);
  // End of the gate/up phase: every act (and sact) row is written.
  block_end_gate_up(S);

  // Down: items c = gw, gw + NW, ... < nC + nSD (routed, then shared).
  {
    auto load = [&](DnStage<FMT, I> &st, int c) {
      st.e = slot_expert(R, c / nDN);
      st.h_base = (c % nDN) * DN::RW;
      st.p0 = first_pair(P, R, st.e);
      if (st.p0 >= 0)
        load_vec<FMT, I, kSrcDevice>(st.a0, P.act + (size_t)st.p0 * I, lane % RowMap<FMT, I>::LPR);
      down_load(st.w, P.w2 + (size_t)st.e * H * DN_RSZ,
                FMT == kNvfp4 ? P.s2 + (size_t)st.e * H * (I / 16) : nullptr, st.h_base);
    };
    auto run = [&](const DnStage<FMT, I> &st) {
      down_compute<FMT, H, I, true>(P, R, st.w, FMT == kNvfp4 ? P.a2[st.e] : 1.0f, st.h_base,
                                    st.e, st.p0, st.a0);
    };
    DnStage<FMT, I> sa, sb;
    int c = gw;
    if (c < nC) load(sa, c);
    while (c < nC) {
      if (c + NW < nC) load(sb, c + NW);
      __builtin_amdgcn_sched_barrier(0);
      run(sa);
      c += NW;
      if (c >= nC) break;
      if (c + NW < nC) load(sa, c + NW);
      __builtin_amdgcn_sched_barrier(0);
      run(sb);
      c += NW;
    }
    // c is now this wave's first index at or past nC.
    // The shared expert's down items follow the routed ones in the list.
    for (; c < nC + nSD; c += NW) {
      DownW<kBf16, I> W;
      VecRegs<kBf16, I> a0;
      const int hb = (c - nC) * SDN::RW;
      down_load(W, P.sdown, nullptr, hb);
      load_vec<kBf16, I, kSrcDevice>(a0, P.sact, lane % RowMap<kBf16, I>::LPR);
      down_compute<kBf16, H, I, false>(P, R, W, 1.0f, hb, 0, 0, a0);
    }
    // One arrival per down item on the combine block of its rows.
    stores_performed();
    if (lane == 0)
      for (int cc = gw; cc < nC + nSD; cc += NW) {
        const int hb = cc < nC ? (cc % nDN) * DN::RW : (cc - nC) * SDN::RW;
        __hip_atomic_fetch_add(&S->rb_cnt[hb / CB][0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  // Combine: block cb belongs to wave cb mod NW.
  for (int cb = gw; cb < H / CB; cb += NW) {
    wait_flag(&S->rb_cnt[cb][0], cb_target);
    if (lane == 0) store_agent(&S->rb_cnt[cb][0], 0);  // sole consumer: reset
    combine_rows<H>(P, cb * CB, CB);
  }
  FLINT_MARK(P, gw, 4);
}


struct LaunchInfo {
  int grid = 0;
};

template <int FMT, int H, int I>
hipError_t launch_fused(const FusedParams &P, hipStream_t st) {
  static thread_local LaunchInfo info[2][64];  // [x staged][device]
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const bool stage_x = P.M * H * 2 <= kXLdsBytes;
  const size_t lds = stage_x ? (size_t)kXLdsBytes : 0;
  LaunchInfo &li = info[stage_x][dev];
  if (li.grid == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<FMT, H, I>, kThreads, lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    // kWavesPerEU blocks per CU are guaranteed to fit (see kWavesPerEU).
    li.grid = cus * (per_cu < kWavesPerEU ? per_cu : kWavesPerEU);
    if (li.grid > kMaxDecodeBlocks) li.grid = kMaxDecodeBlocks;
  }
  FusedParams p = P;
  void *args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(decode_kernel<FMT, H, I>),
                                    dim3(li.grid), dim3(kThreads), args, (unsigned)lds, st);
}

}  // namespace

hipError_t launch_decode_fused(int fmt, const DecodeArgs &a, hipStream_t st) {
  FusedParams P{a.x,  a.router, a.w13, a.s13, a.a13, a.w2,  a.s2,   a.a2,  a.sgu,   a.sdown, a.ids_in,
                a.tw_in, a.logits, a.ids, a.tw, a.act, a.y, a.sact, a.sh, a.out, a.sync, a.M,
                a.E, a.top_k};
#define FLINT_FUSED(HH, II)                                                   \
  if (a.H == HH && a.I == II)                                                 \
    return fmt == kNvfp4 ? launch_fused<kNvfp4, HH, II>(P, st) : launch_fused<kBf16, HH, II>(P, st);
  FLINT_FUSED(2048, 768)
  FLINT_FUSED(256, 128)
  FLINT_FUSED(256, 256)
  FLINT_FUSED(512, 128)
  FLINT_FUSED(512, 256)
#undef FLINT_FUSED
  return hipErrorInvalidValue;
}

bool decode_shape_supported(int H, int I) {
  return (H == 2048 && I == 768) || (H == 256 && (I == 128 || I == 256)) ||
         (H == 512 && (I == 128 || I == 256));
}

}  // namespace flint
