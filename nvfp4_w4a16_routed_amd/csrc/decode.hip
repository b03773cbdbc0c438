// The decode-path MoE block (M <= 64 tokens) in one launch.
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
// Instead of the pages' three programmatically chained launches, one
// persistent launch (as many blocks as the GPU holds at once) runs every
// step.  The weight bytes of the touched experts are streamed exactly once,
// each wave owning a contiguous run of equal-sized work items and loading
// the next item while it computes the current one.
//
//   phase A  block-level items, no dependencies except as noted:
//            [routing: (8 tokens, 8 experts) per block]
//            [shared gate/up: 8 row pairs per block]
//            A routing block tells every block that its logits are written.
//   top-k    every block reads the logits and computes the top-k of every
//            token and the routing plan (touched experts in ascending order
//            and their pairs) in its own LDS: no plan is exchanged.
//   phase B  routed gate/up items (touched expert, row pairs), slot-major.
//   phase C  the first blocks: shared down (32 rows per block, after every
//            shared gate/up block); the other blocks' waves: routed down
//            items (touched expert, output rows), slot-major; a wave loads
//            its first items' weights, then waits only for the gate/up waves
//            of its own experts.
//   combine  32 output rows per item, after the down waves covering them.
//
// Completion is signalled with flags that hold the call's sequence number
// (unique per call), written after the flagged data is performed at device
// scope, so nothing has to be reset and no atomic read-modify-write is
// used (on one address they serialise at the memory side).  A wave
// waits only for work of an earlier phase, and every block of the grid is
// resident, so every wait ends; each wait also gives up after a bounded
// number of polls so a misused workspace cannot hang the GPU.
#include "common.hpp"
#include "internal.hpp"
#include "rowdot.hpp"

namespace flint {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;  // 8
constexpr int kRouteTokens8 = 8;          // tokens per routing block
constexpr int kXLdsBytes = 32768;         // x staged in LDS when M * H * 2 fits
// Cache-policy operand of a direct global->LDS load that reads at device
// scope (the SC1 bit, as the device-scope loads in common.hpp use).
constexpr int kCachePolicyDevice = 16;
// Register budget: at least this many waves per SIMD (two 8-wave blocks per
// CU), so enough weight bytes are in flight per CU.
constexpr int kWavesPerEU = 4;

struct Params {
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
  int seq;
  int M, E, top_k;
  int nb;             // blocks in the grid
  int n_route;        // routing blocks (0 with forced routing)
  int n_sgu, n_sdn;   // shared gate/up and shared down blocks (0 = none)
#ifdef FLINT_TRACE
  long long *trace;   // [waves][16] s_memrealtime stamps (timing builds only)
#endif
};

#ifdef FLINT_TRACE
#define TRACE(P, slot)                                                                       \
  do {                                                                                       \
    if (lane_id() == 0)                                                                      \
      (P).trace[((size_t)blockIdx.x * kWaves + wave_id()) * 16 + (slot)] =                   \
          __builtin_amdgcn_s_memrealtime();                                                  \
  } while (0)
#else
#define TRACE(P, slot) \
  do {                 \
  } while (0)
#endif

// Work geometry for one (format, H, I).
template <int FMT, int H, int I>
struct Geo {
  using GU = GateUpGeo<FMT, H>;     // routed gate/up rows per wave item
  using SGU = GateUpGeo<kBf16, H>;  // shared gate/up
  using DN = DownGeo<FMT, I>;       // routed down rows per wave item
  using SDN = DownGeo<kBf16, I>;    // shared down
  static constexpr int N_GU = I / GU::RP;  // wave items per expert
  static constexpr int N_DN = H / DN::RW;
  static constexpr int SGU_BLOCK = kWaves * SGU::RP;  // shared row pairs per block
  static constexpr int SDN_BLOCK = kWaves * SDN::RW;  // shared rows per block
  static constexpr int CB = SDN_BLOCK > DN::RW ? SDN_BLOCK : DN::RW;  // combine rows
  static_assert(I % GU::RP == 0 && I % SGU_BLOCK == 0, "gate/up items");
  static_assert(H % DN::RW == 0 && H % SDN_BLOCK == 0 && H % CB == 0, "down items");
  static_assert(CB % DN::RW == 0 && CB == SDN_BLOCK, "combine rows");
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Flag write: the wave's device-scope stores are performed first.
__device__ __forceinline__ void set_flag(int *f, int seq) {
  stores_performed();
  if (lane_id() == 0) st_dev(f, seq);
}

// One wave polls until flags[i] == seq for every i in [lo, hi) (all lanes
// read in parallel); gives up after a bounded number of polls.
__device__ void wave_wait_flags(const int *flags, int lo, int hi, int seq) {
  for (int it = 0, nap = 1; it < (1 << 20); ++it) {
    bool ok = true;
    for (int i = lo + lane_id(); i < hi; i += kWave) ok &= ld_dev(&flags[i]) == seq;
    if (__all(ok)) break;
    for (int s = 0; s < nap; ++s) __builtin_amdgcn_s_sleep(2);
    nap = nap < 4 ? nap * 2 : 4;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // keeps the compiler's order
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

// The block's routing of the call (LDS).
struct Route {
  int ids[kMaxDecodePairs];
  float tw[kMaxDecodePairs];
  unsigned long long tokmask[kMaxExperts];  // tokens that selected expert e
  int slot_of[kMaxExperts];
  int active[kMaxExperts];
  int offs[kMaxExperts + 1];
  int pairs[kMaxDecodePairs];
  int cum_gu[kMaxExperts + 1];  // cost before slot s of the gate/up items
  int cum_dn[kMaxExperts + 1];  // same for the down items
  int n_active;
};

// Work balance.  Item (s, j) of a phase (slot s, j < N items per slot)
// costs 2 + np_s units, np_s the pairs of slot s (weight bytes plus the
// arithmetic of every pair); each wave owns the items whose starting cost
// falls in its share [w Q, (w + 1) Q) of the total, so a hot expert's items
// are spread over more waves.
__device__ __forceinline__ int item_cost(const Route &R, int s) {
  return 2 + R.offs[s + 1] - R.offs[s];
}

// Smallest item (global index s * N + j) whose starting cost is >= x.
__device__ __forceinline__ int first_item(const Route &R, const int *cum, int N, int x) {
  const int U = R.n_active;
  if (x >= cum[U]) return U * N;
  int lo = 0, hi = U - 1;  // last slot with cum[slot] <= x
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  const int c = item_cost(R, lo);
  const int j = (x - cum[lo] + c - 1) / c;
  return j >= N ? (lo + 1) * N : lo * N + j;
}

// Wave that owns item (s, j).
__device__ __forceinline__ int owner(const Route &R, const int *cum, int s, int j, int Q) {
  return (cum[s] + j * item_cost(R, s)) / Q;
}

// Top-k of token t by one wave (top_k <= E <= 256) into LDS.
__device__ void topk_token(const Params &P, int t, Route &R) {
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
  float S = 0.0f;  // in selection order, one addition at a time
  for (int j = 0; j < k; ++j) {
    const int i = j >> 6;
    const float v = (i == 0) ? s[0] : (i == 1) ? s[1] : (i == 2) ? s[2] : s[3];
    S = S + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j & (kWave - 1)));
  }
  const float D = S + 1e-20f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = kWave * i + lane;
    if (j < k) {
      R.ids[t * k + j] = E - 1 - (sel[i] & 0xff);
      R.tw[t * k + j] = round_bf16(s[i] / D);
    }
  }
}

// Exclusive prefix sum over the wave (lane order).
__device__ __forceinline__ int wave_exclusive_scan(int v) {
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(x, o, kWave);
    if (lane_id() >= o) x += t;
  }
  return x - v;
}

// Routing plan from R.ids: touched experts ascending (slot order), pairs of
// each expert ascending (an expert has at most one pair per token), and the
// cumulative item costs of phases B and C (GU_ITEMS, DN_ITEMS items per
// slot).  Ends with the block synchronised.
template <int GU_ITEMS, int DN_ITEMS>
__device__ void build_plan(const Params &P, Route &R) {
  const int npairs = P.M * P.top_k, k = P.top_k;
  for (int e = threadIdx.x; e < kMaxExperts; e += kThreads) R.tokmask[e] = 0ull;
  __syncthreads();
  for (int p = threadIdx.x; p < npairs; p += kThreads) {
    const int e = R.ids[p];
    if ((unsigned)e < (unsigned)P.E) atomicOr(&R.tokmask[e], 1ull << (p / k));  // bad ids dropped
  }
  __syncthreads();
  if (wave_id() == 0) {
    // lane l holds experts 4l .. 4l + 3
    int cnt[4], flg[4], c = 0, f = 0, u = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane_id() + i;
      cnt[i] = e < P.E ? __popcll(R.tokmask[e]) : 0;
      flg[i] = cnt[i] > 0;
      c += cnt[i];
      f += flg[i];
      u += flg[i] ? 2 + cnt[i] : 0;
    }
    int base = wave_exclusive_scan(c), slot = wave_exclusive_scan(f);
    int cost = wave_exclusive_scan(u);  // in units of one item per slot
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane_id() + i;
      if (flg[i]) {
        R.slot_of[e] = slot;
        R.active[slot] = e;
        R.offs[slot] = base;
        R.cum_gu[slot] = cost * GU_ITEMS;
        R.cum_dn[slot] = cost * DN_ITEMS;
      }
      base += cnt[i];
      slot += flg[i];
      cost += flg[i] ? 2 + cnt[i] : 0;
    }
    if (lane_id() == kWave - 1) {
      R.n_active = slot;
      R.offs[slot] = base;
      R.cum_gu[slot] = cost * GU_ITEMS;
      R.cum_dn[slot] = cost * DN_ITEMS;
    }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < npairs; p += kThreads) {
    const int ee = R.ids[p];
    if ((unsigned)ee < (unsigned)P.E) {
      const int t = p / k;
      const int rank = __popcll(R.tokmask[ee] & ((1ull << t) - 1ull));
      R.pairs[R.offs[R.slot_of[ee]] + rank] = p;
    }
  }
  __syncthreads();
}

// --------------------------------------------------------- phase A items

// Copies n 16-byte chunks from global memory straight into LDS (direct
// loads: no registers, every load in flight at once), by waves
// wave, wave + nwaves, ... (each moves 1 KB blocks), then waits until the
// calling wave's copies have landed (this also waits for its other
// outstanding loads).  DEVICE: device-scope loads of data other blocks wrote.
template <bool DEVICE>
__device__ __forceinline__ void copy_to_lds(uint16_t *dst, const uint16_t *src, int n, int wave,
                                            int nwaves) {
  const int lane = lane_id();
  for (int b = wave; b * kWave < n; b += nwaves) {
    const int i = b * kWave + lane;
    if (i < n)
      __builtin_amdgcn_global_load_lds(src + (size_t)i * 8,
                                       (__attribute__((address_space(3))) void *)(dst + (size_t)b * 512),
                                       16, 0, DEVICE ? kCachePolicyDevice : 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies are in LDS
}

// Stages nr rows of a bf16 matrix with K columns into LDS (the whole block;
// the caller synchronises the block before reading them).
template <int K, bool DEVICE>
__device__ __forceinline__ void stage_rows(uint16_t *dst, const uint16_t *src, int nr) {
  copy_to_lds<DEVICE>(dst, src, nr * K / 8, wave_id(), kWaves);
}

// Routing block r: logits of experts 8 * (r % nEG) + wave for the 8 tokens
// of group r / nEG, then a flag to every block.  x (of the group, or all of
// it when it fits) is staged in LDS unless it already is.
template <int H>
__device__ void route_block(const Params &P, int r, uint16_t *xs, bool x_all, bool &staged) {
  constexpr int NC = H / 8;
  constexpr int CPL = (NC + kWave - 1) / kWave;
  const int lane = lane_id();
  const int nEG = (P.E + kWaves - 1) / kWaves;
  const int t0 = (r / nEG) * kRouteTokens8;
  const int nt = min(kRouteTokens8, P.M - t0);
  const int e = (r % nEG) * kWaves + wave_id();
  // router row first: its loads overlap the staging of x
  u32x4_t w[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + kWave * i;
    w[i] = (e < P.E && c < NC) ? load16(P.router + (size_t)e * H + c * 8) : u32x4_t{0, 0, 0, 0};
  }
  const int r0 = x_all ? 0 : t0;
  if (!(x_all && staged)) {
    __syncthreads();  // earlier readers of the staging area are done
    stage_rows<H, false>(xs, P.x + (size_t)r0 * H, x_all ? P.M : nt);
    staged = x_all;
  }
  __syncthreads();
  const uint16_t *xg = xs + (size_t)(t0 - r0) * H;
  if (e < P.E) {
    for (int ti = 0; ti < nt; ++ti) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + kWave * i;
        if (c < NC) {
          const u32x4_t v = load16(xg + (size_t)ti * H + c * 8);
          acc = dot2_bf16(w[i][0], v[0], acc);
          acc = dot2_bf16(w[i][1], v[1], acc);
          acc = dot2_bf16(w[i][2], v[2], acc);
          acc = dot2_bf16(w[i][3], v[3], acc);
        }
      }
      acc = group_sum<kWave>(acc);
      if (lane == kWave - 1) st_dev(&P.logits[(size_t)(t0 + ti) * P.E + e], (uint16_t)f32_to_bf16(acc));
    }
  }
  stores_performed();
  __syncthreads();
  for (int b = threadIdx.x; b < P.nb; b += kThreads) st_dev(&P.sync->go[b][r], P.seq);
}

// Gate/up of one wave on given weights: vector i (i < np) is x[tok(i)], its
// result goes to dst[pair(i) * I + n].  x is read from xl (LDS) when
// non-NULL, else from global memory.
template <int FMT, int H, int I, typename Tok, typename Pair>
__device__ __forceinline__ void gate_up_compute(const Params &P, const GateUpW<FMT, H, I> &W,
                                                float alpha, int n_base, int np, Tok tok,
                                                Pair pair, const uint16_t *xl, uint16_t *dst) {
  using Map = RowMap<FMT, H>;
  using G = GateUpGeo<FMT, H>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  for (int i = 0; i < np; ++i) {
    const int t = tok(i), p = pair(i);
    float acc[2 * G::NSL];
    if (xl)
      rows_dot<FMT, H, kSrcLds>(W.rows, xl + (size_t)t * H, q, acc);
    else
      rows_dot<FMT, H, kSrcGlobal>(W.rows, P.x + (size_t)t * H, q, acc);
#pragma unroll
    for (int s = 0; s < G::NSL; ++s) {
      float gs = group_sum<Map::LPR>(acc[s]);
      float us = group_sum<Map::LPR>(acc[G::NSL + s]);
      if (q == Map::LPR - 1) {  // the group's sum is in its last lane
        if constexpr (FMT == kNvfp4) {
          gs = gs * alpha;
          us = us * alpha;
        }
        st_dev(&dst[(size_t)p * I + n_base + s * Map::RS + r], (uint16_t)f32_to_bf16(swiglu(gs, us)));
      }
    }
  }
}

// Down of one wave on given weights for one vector (SRC: kSrcLds or
// kSrcDevice); the result row goes to dst_row.
template <int FMT, int H, int I, int SRC>
__device__ __forceinline__ void down_one(const DownW<FMT, I> &W, const uint16_t *vec, float alpha,
                                         int h_base, uint16_t *dst_row) {
  using Map = RowMap<FMT, I>;
  using G = DownGeo<FMT, I>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  float acc[G::NSL];
  rows_dot<FMT, I, SRC>(W.rows, vec, q, acc);
#pragma unroll
  for (int s = 0; s < G::NSL; ++s) {
    float val = group_sum<Map::LPR>(acc[s]);
    if (q == Map::LPR - 1) {
      if constexpr (FMT == kNvfp4) val = val * alpha;
      st_dev(&dst_row[h_base + s * Map::RS + r], (uint16_t)f32_to_bf16(val));
    }
  }
}

// ------------------------------------------------------------ the kernel

// Routed gate/up wave items of the call: U slots x N_GU items; wave gw
// owns [gw * C, (gw + 1) * C).
__device__ __forceinline__ int per_wave(int items, int nw) { return (items + nw - 1) / nw; }

template <int FMT, int H, int I>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
decode_kernel(Params P) {
  using Gm = Geo<FMT, H, I>;
  using GuMap = RowMap<FMT, H>;
  using DnMap = RowMap<FMT, I>;
  constexpr int GU_RSZ = FMT == kNvfp4 ? H / 2 : H * 2;  // routed row bytes (w13)
  constexpr int DN_RSZ = FMT == kNvfp4 ? I / 2 : I * 2;  // routed row bytes (w2)
  __shared__ Route R;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // x staging

  DecodeSync *S = P.sync;
  const int lane = lane_id(), wv = wave_id();
  const int NW = P.nb * kWaves;
  const int gw = blockIdx.x * kWaves + wv;
  const int k = P.top_k;
  const bool x_all = P.M * H * 2 <= kXLdsBytes;  // all of x fits the staging area
  TRACE(P, 0);

  // ---- phase A (block items b = blockIdx.x, blockIdx.x + nb, ...)
  const int nA = P.n_route + P.n_sgu;
  bool staged = false;  // all of x is in the staging area
  for (int b = blockIdx.x; b < nA; b += P.nb) {
    if (b < P.n_route) {
      route_block<H>(P, b, xs, x_all, staged);
    } else if (b < P.n_route + P.n_sgu) {
      // shared gate/up: 8 row pairs, every token (x staged in groups)
      const int sb = b - P.n_route;
      const int n_base = sb * Gm::SGU_BLOCK + wv * Gm::SGU::RP;
      GateUpW<kBf16, H, I> W;
      gate_up_load(W, P.sgu, nullptr, n_base);
      const int G = x_all ? P.M : kRouteTokens8;
      for (int g0 = 0; g0 < P.M; g0 += G) {
        if (!(x_all && staged)) {
          __syncthreads();
          stage_rows<H, false>(xs, P.x + (size_t)g0 * H, min(G, P.M - g0));
          staged = x_all;
        }
        __syncthreads();
        gate_up_compute<kBf16, H, I>(P, W, 1.0f, n_base, min(G, P.M - g0), [](int i) { return i; },
                                     [g0](int i) { return g0 + i; }, xs, P.sact);
      }
      stores_performed();
      __syncthreads();
      if (threadIdx.x == 0) st_dev(&S->sg[sb], P.seq);
    }
  }
  TRACE(P, 1);
  // Stage all of x for the gate/up items (small batches) while routing ends.
  if (x_all && !staged) {
    __syncthreads();
    stage_rows<H, false>(xs, P.x, P.M);
  }

  // ---- routing of every token, in this block's LDS
  if (P.ids_in) {
    for (int p = threadIdx.x; p < P.M * k; p += kThreads) {
      R.ids[p] = P.ids_in[p];
      R.tw[p] = P.tw_in[p];
    }
  } else {
    if (wv == 0) wave_wait_flags(S->go[blockIdx.x], 0, P.n_route, P.seq);
    __syncthreads();
    TRACE(P, 2);
    for (int t = wv; t < P.M; t += kWaves) topk_token(P, t, R);
  }
  __syncthreads();
  TRACE(P, 8);
  build_plan<Gm::N_GU, Gm::N_DN>(P, R);
  if (blockIdx.x == 0)
    for (int p = threadIdx.x; p < P.M * k; p += kThreads) {
      if (P.ids != P.ids_in) P.ids[p] = R.ids[p];
      if (P.tw != P.tw_in) P.tw[p] = R.tw[p];
    }
  TRACE(P, 3);
  const int U = R.n_active;
  const uint16_t *xl = x_all ? xs : nullptr;

  // ---- phase B: routed gate/up, wave gw owns items [b0, b1)
  const int QB = max(1, per_wave(R.cum_gu[U], NW));  // cost share of a wave
  {
    const int b0 = first_item(R, R.cum_gu, Gm::N_GU, gw * QB);
    const int b1 = first_item(R, R.cum_gu, Gm::N_GU, (gw + 1) * QB);
    struct St {
      GateUpW<FMT, H, I> w;
      float alpha;
    };
    auto load = [&](St &st, int i) {
      const int e = R.active[i / Gm::N_GU];
      const int n_base = (i % Gm::N_GU) * Gm::GU::RP;
      gate_up_load(st.w, P.w13 + (size_t)e * 2 * I * GU_RSZ,
                   FMT == kNvfp4 ? P.s13 + (size_t)e * 2 * I * (H / 16) : nullptr, n_base);
      st.alpha = FMT == kNvfp4 ? P.a13[e] : 1.0f;
    };
    auto run = [&](const St &st, int i) {
      const int s = i / Gm::N_GU;
      const int *pr = R.pairs + R.offs[s];
      gate_up_compute<FMT, H, I>(P, st.w, st.alpha, (i % Gm::N_GU) * Gm::GU::RP,
                                 R.offs[s + 1] - R.offs[s], [pr, k](int j) { return pr[j] / k; },
                                 [pr](int j) { return pr[j]; }, xl, P.act);
    };
    St sa, sb;
    int i = b0;
    if (i < b1) load(sa, i);
    while (i < b1) {
      if (i + 1 < b1) load(sb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      run(sa, i);
      if (++i >= b1) break;
      if (i + 1 < b1) load(sa, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      run(sb, i);
      ++i;
    }
    set_flag(&S->gw[gw], P.seq);
  }
  TRACE(P, 4);

  // ---- phase C: blocks [0, n_sdn) shared down; the waves of the other
  // blocks own routed down items [c0, c1) (wave index gc = gw - sdw; on a
  // grid too small to set those blocks apart, every wave takes both)
  const int sdw = 2 * P.n_sdn <= P.nb ? P.n_sdn * kWaves : 0;  // waves kept for shared down
  const int NWC = NW - sdw;
  const int gc = gw - sdw;
  const int QC = max(1, per_wave(R.cum_dn[U], NWC));
  {
    const int c0 = gc < 0 ? 0 : first_item(R, R.cum_dn, Gm::N_DN, gc * QC);
    const int c1 = gc < 0 ? 0 : first_item(R, R.cum_dn, Gm::N_DN, (gc + 1) * QC);
    struct St {
      DownW<FMT, I> w;
      float alpha;
    };
    auto load = [&](St &st, int i) {
      const int e = R.active[i / Gm::N_DN];
      down_load(st.w, P.w2 + (size_t)e * H * DN_RSZ,
                FMT == kNvfp4 ? P.s2 + (size_t)e * H * (I / 16) : nullptr,
                (i % Gm::N_DN) * Gm::DN::RW);
      st.alpha = FMT == kNvfp4 ? P.a2[e] : 1.0f;
    };
    St sa, sb;
    if (c0 < c1) load(sa, c0);
    if (c0 + 1 < c1) load(sb, c0 + 1);
    // The staging area is reused below: every wave of the block is done
    // with x (the first weights are already in flight).
    __syncthreads();
    for (int db = blockIdx.x; db < P.n_sdn; db += P.nb) {
      // shared down: 32 rows, every token (sact staged in groups)
      const int h_base = db * Gm::SDN_BLOCK + wv * Gm::SDN::RW;
      DownW<kBf16, I> W;
      down_load(W, P.sdown, nullptr, h_base);
      if (wv == 0) wave_wait_flags(S->sg, 0, P.n_sgu, P.seq);
      constexpr int G = kXLdsBytes / (2 * I) < kMaxDecodeM ? kXLdsBytes / (2 * I) : kMaxDecodeM;
      for (int g0 = 0; g0 < P.M; g0 += G) {
        __syncthreads();
        stage_rows<I, true>(xs, P.sact + (size_t)g0 * I, min(G, P.M - g0));
        __syncthreads();
        for (int t = g0; t < min(g0 + G, P.M); ++t)
          down_one<kBf16, H, I, kSrcLds>(W, xs + (size_t)(t - g0) * I, 1.0f, h_base,
                                         P.sh + (size_t)t * H);
      }
      stores_performed();
      __syncthreads();
      if (threadIdx.x == 0) st_dev(&S->sd[db], P.seq);
    }
    if (c0 < c1) {
      // gate/up waves that produced act of this wave's experts
      const int s_lo = c0 / Gm::N_DN, s_hi = (c1 - 1) / Gm::N_DN;
      const int w_lo = owner(R, R.cum_gu, s_lo, 0, QB);
      const int w_hi = owner(R, R.cum_gu, s_hi, Gm::N_GU - 1, QB);
      wave_wait_flags(S->gw, w_lo, w_hi + 1, P.seq);
    }
    TRACE(P, 5);
    // The activations of the current expert's first pairs are copied to a
    // slice of the staging area (x is no longer needed) when the expert
    // changes, so the item loop reads them from LDS and only weight loads
    // are in flight between items.
    constexpr int kCache = (kXLdsBytes / kWaves) / (2 * I);  // rows per wave
    static_assert(kCache >= 1, "activation cache");
    uint16_t *ac = xs + (size_t)wv * (kXLdsBytes / kWaves / 2);
    int cur = -1;
    auto run = [&](const St &st, int i) {
      const int s = i / Gm::N_DN;
      const int h_base = (i % Gm::N_DN) * Gm::DN::RW;
      const int *pr = R.pairs + R.offs[s];
      const int np = R.offs[s + 1] - R.offs[s];
      const int nc = np < kCache ? np : kCache;
      if (s != cur) {
        cur = s;
        for (int j = 0; j < nc; ++j)
          copy_to_lds<true>(ac + (size_t)j * I, P.act + (size_t)pr[j] * I, I / 8, 0, 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      for (int j = 0; j < nc; ++j)
        down_one<FMT, H, I, kSrcLds>(st.w, ac + (size_t)j * I, st.alpha, h_base,
                                     P.y + (size_t)pr[j] * H);
      for (int j = nc; j < np; ++j)
        down_one<FMT, H, I, kSrcDevice>(st.w, P.act + (size_t)pr[j] * I, st.alpha, h_base,
                                        P.y + (size_t)pr[j] * H);
    };
    int i = c0;
    while (i < c1) {
      __builtin_amdgcn_sched_barrier(0);
      run(sa, i);
      if (i + 2 < c1) load(sa, i + 2);
      if (++i >= c1) break;
      __builtin_amdgcn_sched_barrier(0);
      run(sb, i);
      if (i + 2 < c1) load(sb, i + 2);
      ++i;
    }
    if (gc >= 0) set_flag(&S->dw[gc], P.seq);
  }
  TRACE(P, 6);

  // ---- combine: item cb (CB output rows) on wave cb * stride
  constexpr int NCB = H / Gm::CB;
  const int stride = NW / NCB > 0 ? NW / NCB : 1;
  for (int cb = (NW >= NCB) ? (gw % stride == 0 ? gw / stride : NCB) : gw; cb < NCB;
       cb += (NW >= NCB) ? NCB : NW) {
    const int h0 = cb * Gm::CB;
    // routed down items of rows [h0, h0 + CB) for every slot
    constexpr int IPB = Gm::CB / Gm::DN::RW;  // down items per combine block
    for (int it = 0, nap = 1; it < (1 << 20); ++it) {
      bool ok = true;
      for (int s = lane; s < U; s += kWave) {
        const int j0 = h0 / Gm::DN::RW;
        const int w_hi = owner(R, R.cum_dn, s, j0 + IPB - 1, QC);
        for (int w = owner(R, R.cum_dn, s, j0, QC); w <= w_hi; ++w) ok &= ld_dev(&S->dw[w]) == P.seq;
      }
      if (P.sgu && lane == 0) ok &= ld_dev(&S->sd[cb]) == P.seq;
      if (__all(ok)) break;
      for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
      nap = nap < 4 ? nap * 2 : 4;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // y of the rows for a group of tokens is gathered into this wave's LDS
    // slice with direct loads (one round trip per group), then summed.
    uint16_t *yl = xs + (size_t)wv * (kXLdsBytes / kWaves / 2);
    constexpr int SLICE = kXLdsBytes / kWaves / 2;  // bf16 per slice
    // tokens per group: at most 4 outputs and 4 gathered chunks per lane
    const int G = min(4 * kWave / Gm::CB, SLICE / (k * Gm::CB));
    for (int t0 = 0; t0 < P.M; t0 += (G > 0 ? G : 1)) {
      const int nt = G > 0 ? min(G, P.M - t0) : 1;
      float shv[4] = {0.f, 0.f, 0.f, 0.f};
      if (G > 0) {
        const int n = nt * k * (Gm::CB / 8);  // 16-byte chunks, <= 4 per lane
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = u * kWave + lane;
          if (i < n) {
            const int p = t0 * k + i / (Gm::CB / 8), part = i % (Gm::CB / 8);
            __builtin_amdgcn_global_load_lds(
                P.y + (size_t)p * H + h0 + part * 8,
                (__attribute__((address_space(3))) void *)(yl + (size_t)u * kWave * 8), 16, 0,
                kCachePolicyDevice);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int o = u * kWave + lane;
          if (P.sgu && o < nt * Gm::CB)
            shv[u] = bf16_to_f32(ld_dev(&P.sh[(size_t)(t0 + o / Gm::CB) * H + h0 + o % Gm::CB]));
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): y is in LDS
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int o = u * kWave + lane;
          if (o < nt * Gm::CB) {
            const int tl = o / Gm::CB, hh = o % Gm::CB, t = t0 + tl;
            double acc = 0.0;  // exact: every product has 16 significant bits
            for (int j = 0; j < k; ++j)
              if ((unsigned)R.ids[t * k + j] < (unsigned)P.E)
                acc += (double)R.tw[t * k + j] * (double)bf16_to_f32(yl[(tl * k + j) * Gm::CB + hh]);
            const float routed = round_bf16((float)acc);
            P.out[(size_t)t * H + h0 + hh] = (uint16_t)f32_to_bf16(routed + shv[u]);
          }
        }
      } else {
        // more pairs per token than a slice holds: device-scope loads
        for (int hh = lane; hh < Gm::CB; hh += kWave) {
          double acc = 0.0;
          for (int j = 0; j < k; ++j) {
            const int p = t0 * k + j;
            if ((unsigned)R.ids[p] < (unsigned)P.E)
              acc += (double)R.tw[p] * (double)bf16_to_f32(ld_dev(&P.y[(size_t)p * H + h0 + hh]));
          }
          const float sv = P.sgu ? bf16_to_f32(ld_dev(&P.sh[(size_t)t0 * H + h0 + hh])) : 0.0f;
          P.out[(size_t)t0 * H + h0 + hh] = (uint16_t)f32_to_bf16(round_bf16((float)acc) + sv);
        }
      }
    }
  }
  TRACE(P, 7);
}

struct GridInfo {
  int nb = 0;
};

template <int FMT, int H, int I>
hipError_t launch(Params P, hipStream_t st) {
  using Gm = Geo<FMT, H, I>;
  static thread_local GridInfo info[64];  // [device]
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static_assert(kRouteTokens8 * H * 2 <= kXLdsBytes, "routing group staging");
  const bool x_all = P.M * H * 2 <= kXLdsBytes;
  // The staging area holds all of x (small batches) or one routing group,
  // and later the activations the down items read.
  const size_t lds = kXLdsBytes;
  GridInfo &gi = info[dev];
  if (gi.nb == 0) {
    // Blocks resident at once with the largest staging area: the grid.
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<FMT, H, I>, kThreads,
                                                     kXLdsBytes);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    gi.nb = cus * per_cu;
    if (gi.nb > kMaxDecodeBlocks) gi.nb = kMaxDecodeBlocks;
  }
  P.nb = gi.nb;
  const int nEG = (P.E + kWaves - 1) / kWaves;
  const int nTG = (P.M + kRouteTokens8 - 1) / kRouteTokens8;
  P.n_route = P.ids_in ? 0 : nEG * nTG;
  P.n_sgu = P.sgu ? I / Gm::SGU_BLOCK : 0;
  P.n_sdn = P.sgu ? H / Gm::SDN_BLOCK : 0;
  if (P.n_sgu > kMaxSharedBlocks || P.n_sdn > kMaxSharedBlocks || P.n_route > kMaxRouteBlocks)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_kernel<FMT, H, I>), dim3(P.nb), dim3(kThreads), lds, st, P);
  return hipGetLastError();
}

}  // namespace

#ifdef FLINT_TRACE
long long *g_flint_trace = nullptr;
#endif

hipError_t launch_decode(int fmt, const DecodeArgs &a, hipStream_t st) {
  Params P{};
  P.x = a.x;
  P.router = a.router;
  P.w13 = a.w13;
  P.s13 = a.s13;
  P.a13 = a.a13;
  P.w2 = a.w2;
  P.s2 = a.s2;
  P.a2 = a.a2;
  P.sgu = a.sgu;
  P.sdown = a.sdown;
  P.ids_in = a.ids_in;
  P.tw_in = a.tw_in;
  P.logits = a.logits;
  P.ids = a.ids;
  P.tw = a.tw;
  P.act = a.act;
  P.y = a.y;
  P.sact = a.sact;
  P.sh = a.sh;
  P.out = a.out;
  P.sync = a.sync;
  P.seq = a.seq;
  P.M = a.M;
  P.E = a.E;
  P.top_k = a.top_k;
#ifdef FLINT_TRACE
  P.trace = g_flint_trace;
#endif
#define FLINT_DECODE(HH, II)                                                \
  if (a.H == HH && a.I == II)                                               \
    return fmt == kNvfp4 ? launch<kNvfp4, HH, II>(P, st) : launch<kBf16, HH, II>(P, st);
  FLINT_DECODE(2048, 768)
  FLINT_DECODE(256, 128)
  FLINT_DECODE(256, 256)
  FLINT_DECODE(512, 128)
  FLINT_DECODE(512, 256)
#undef FLINT_DECODE
  return hipErrorInvalidValue;
}

bool decode_shape_supported(int H, int I) {
  return (H == 2048 && I == 768) || (H == 256 && (I == 128 || I == 256)) ||
         (H == 512 && (I == 128 || I == 256));
}

}  // namespace flint

#ifdef FLINT_TRACE
extern "C" void flint_set_trace(long long *p) { flint::g_flint_trace = p; }
#endif
