// The decode-path MoE block (M <= 64 tokens) in one launch.
//
// Semantics (vLLM page "vllm.models.flint.ops.moe": module docstring
// "Numerics"; _router_kernel/_topk_row, _gate_up_gemv_kernel,
// _down_gemv_kernel, their BF16 variants and _combine_kernel):
//   logits = bf16(fp32 x . router[e]);  top-k: larger logit, then smaller index
//   s_j = RN32(1 / RN32(1 + RN32(exp(-l_j)))), tw_j = bf16(s_j / (S + 1e-20))
//   g, u = fp32 (x . W13[e, n]) * alpha13[e], (x . W13[e, I+n]) * alpha13[e]
//   act = bf16(silu(g) * u);  y = bf16(fp32 (act . W2[e, h]) * alpha2[e])
//   out = bf16(bf16(sum_j tw_j y_j) + shared(x))
// The shared expert follows the same rule with bf16 weights and no alpha.
//
// Instead of the pages' three programmatically chained launches, one
// persistent launch (one 16-wave block per compute unit) runs every step.
// The weight bytes of the touched experts are streamed exactly once.
//
//   phase A  started at once, while routing is in progress:
//            [routing blocks: logits of (8 tokens, 16 experts) per block,
//             each written with the call's sequence number, then a flag]
//            [shared gate/up: one row pair per wave, spread over all blocks]
//            [shared down: a few rows per wave, spread over all blocks,
//             after every shared gate/up]
//   top-k    in every block, waves without shared work wait for the routing
//            flags, read the logits and compute the top-k of every token;
//            the wave that finishes the last token builds the routing plan
//            (touched experts in ascending order and their pairs) in the
//            block's LDS: no plan is exchanged and no block barrier is used.
//   phase B  routed gate/up items (touched expert, row pairs): each block
//            owns a contiguous share of equal cost, and its waves take the
//            share's items one at a time from a counter in LDS (waves of a
//            compute unit run at different speeds; taking work as they go
//            evens that out).  The last wave of the block to finish raises
//            the block's flag.
//   phase C  routed down items (touched expert, output rows), shared out the
//            same way; an item first waits for the flags of the blocks that
//            own its expert's gate/up items.
//   combine  32 output rows per item, after the down items covering them.
//
// Completion is signalled with values that carry the call's sequence
// number (unique per call), written after the data they cover is performed
// at device scope, so nothing has to be reset and no atomic read-modify-
// write touches global memory (on one address they serialise at the memory
// side).  A wave waits only for work of an earlier phase, and every block of
// the grid is resident, so every wait ends; each wait also gives up after a
// bounded number of polls so a misused workspace cannot hang the GPU.
#include "common.hpp"
#include "internal.hpp"
#include "rowdot.hpp"
#include "topk.hpp"

#include <hip/hip_ext.h>

#include <mutex>

namespace flint {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;  // 16
constexpr int kRouteTokens = 4;           // tokens per routing item (one load round trip)
constexpr int kXLdsBytes = kDecodeXStage;  // x staged in LDS when M * H * 2 fits
constexpr int kSliceBytes = 4096;         // per-wave LDS slice (results, act cache)
constexpr int kMaxRowGroups = 16;         // down row groups per block
constexpr int kShPreMax = kMaxRowGroups * 16 * 8;  // shared output values staged for the combine
constexpr int kCacheLdsBytes = kWaves * kSliceBytes;
// Cache-policy operand of a direct global->LDS load that reads at device
// scope (the SC1 bit, as the device-scope loads in common.hpp use).
constexpr int kCachePolicyDevice = 16;
// Register budget: at least this many waves per SIMD (one 16-wave block per
// CU), so enough weight bytes are in flight per CU.
constexpr int kWavesPerEU = 4;

// Kinds of bounded waits, recorded in DecodeSync::wait_err when one gives up.
enum WaitKind {
  kWaitLogits = 1,          // a token's tagged router logits
  kWaitSharedGateUp = 2,    // the shared gate/up blocks' flags
  kWaitGateUp = 4,          // the gate/up blocks of a routed expert
  kWaitCombineShared = 8,   // the shared down blocks of a combined row group
  kWaitCombineDown = 16,    // (reserved: each block combines its own rows)
  kWaitLds = 32,            // a wave of the same block (LDS counter)
  kWaitProbe = 64           // the test hook's wait
};

struct Params {
  const uint16_t *x;
  const uint16_t *router;
  const uint8_t *w13;
  const uint8_t *s13;
  const float *a13;
  const uint8_t *w2;
  const uint8_t *s2;
  const float *a2;
  const uint8_t *sgu;    // shared [2I, H] bf16 (or E2M1 codes), NULL = no shared expert
  const uint8_t *sdown;  // shared [H, I] bf16 (or E2M1 codes)
  const uint8_t *ssgu, *ssdown;  // NVFP4 shared expert: E4M3 block scales
  const float *asgu, *asdown;    // NVFP4 shared expert: global scales (device)
  const uint16_t *sh_ext;        // precomputed shared output [M, H], NULL = none
  // Residual add + RMS norm in front of the block (NULL ln_a: x is given):
  // every block forms xn = bf16((s * rsqrt(mean s^2 + eps)) * ln_w) with
  // s = ln_a + ln_r itself; block 0 writes res_out = bf16(s) and xn_out.
  const uint16_t *ln_a, *ln_r, *ln_w;
  float eps;
  uint16_t *res_out, *xn_out;
  const int32_t *ids_in; // forced routing (NULL = route)
  const float *tw_in;
  uint16_t *logits;
  unsigned long long *tlog;  // [kFlagCopies][M, E] (seq << 32) | bf16 bits of the logit
  int32_t *ids;
  float *tw;
  uint16_t *act;
  uint16_t *y;
  uint16_t *sact;
  uint16_t *sh;
  uint16_t *out;
  DecodeSync *sync;
  int seq;
  int polls;          // polls before a device-scope wait gives up
  int probe;          // non-zero: block 0 also waits for a word nobody sets
  int M, E, top_k;
  int nb;             // blocks in the grid
  int n_route;        // routing items (0 with forced routing)
  int n_sgu, n_sdn;   // shared gate/up items (row pairs) and shared down items (0 = none)
#ifdef FLINT_TRACE
  long long *trace;   // [waves][16] s_memrealtime stamps (timing builds only)
#endif
};

#ifdef FLINT_TRACE
// Timing builds: each wave stamps s_memrealtime into LDS (no global store
// that a later wait would include) and writes its stamps out at the end.
__shared__ long long g_trace_lds[kWaves * 16];
#define TRACE(P, slot)                                                        \
  do {                                                                        \
    if (lane_id() == 0) g_trace_lds[wave_id() * 16 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define TRACE_FIRST(P, slot)                                                  \
  do {                                                                        \
    if (lane_id() == 0 && g_trace_lds[wave_id() * 16 + (slot)] == 0)           \
      g_trace_lds[wave_id() * 16 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define TRACE_INIT()                                                          \
  do {                                                                        \
    if (lane_id() < 16) g_trace_lds[wave_id() * 16 + lane_id()] = 0;          \
  } while (0)
#define TRACE_FLUSH(P)                                                        \
  do {                                                                        \
    if (lane_id() < 16)                                                       \
      (P).trace[((size_t)blockIdx.x * kWaves + wave_id()) * 16 + lane_id()] = \
          g_trace_lds[wave_id() * 16 + lane_id()];                            \
  } while (0)
#else
#define TRACE(P, slot) \
  do {                 \
  } while (0)
#define TRACE_FIRST(P, slot) \
  do {                       \
  } while (0)
#define TRACE_INIT() \
  do {               \
  } while (0)
#define TRACE_FLUSH(P) \
  do {                 \
  } while (0)
#endif

// Work geometry for one (routed format, shared format, H, I).
template <int FMT, int SFMT, int H, int I>
struct Geo {
  using GU = GateUpGeo<FMT, H>;     // routed gate/up rows per wave item
  using SGU = GateUpGeo<SFMT, H>;   // shared gate/up
  using DN = DownGeo<FMT, I>;       // routed down rows per wave item
  using SDN = DownGeo<SFMT, I>;     // shared down
  static constexpr int N_GU = I / GU::RP;  // wave items per expert
  static constexpr int N_DN = H / DN::RW;
  static constexpr int CB = DN::RW > 32 ? DN::RW : 32;  // combine rows per item
  // results per vector of an item, the most of the four item kinds
  static constexpr int NV_MAX = GU::RP > DN::RW ? (GU::RP > SDN::RW ? GU::RP : SDN::RW)
                                                : (DN::RW > SDN::RW ? DN::RW : SDN::RW);
  static constexpr int OUT_BYTES = kWave * (NV_MAX > SGU::RP ? NV_MAX : SGU::RP) * 2;
  static_assert(OUT_BYTES <= kSliceBytes / 2, "output buffer");
  static_assert(I % GU::RP == 0 && I % SGU::RP == 0, "gate/up items");
  static_assert(H % DN::RW == 0 && H % SDN::RW == 0 && H % CB == 0, "down items");
  static_assert(CB % DN::RW == 0 && CB % SDN::RW == 0, "combine rows");
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Flag write: the wave's device-scope stores are performed first.
__device__ __forceinline__ void set_flag(int *f, int seq) {
  stores_performed();
  if (lane_id() == 0) st_dev(f, seq);
}

// A wait that gave up records its kind in the workspace's error word (one
// device-scope OR per wave): the call's results are then not valid, and the
// host reads the word with flint_moe_wait_errors.
__device__ __forceinline__ void wait_failed(DecodeSync *S, int kind) {
  if (lane_id() == 0)
    __hip_atomic_fetch_or(&S->wait_err, kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave polls until flags[i] == seq for every i in [lo, hi) (all lanes
// read in parallel); after `polls` polls it gives up and records `kind`.
__device__ void wave_wait_flags(const int *flags, int lo, int hi, int seq, int polls,
                                DecodeSync *S, int kind) {
  bool done = false;
  for (int it = 0, nap = 1; it < polls; ++it) {
    bool ok = true;
    for (int i = lo + lane_id(); i < hi; i += kWave) ok &= ld_dev(&flags[i]) == seq;
    if (__all(ok)) {
      done = true;
      break;
    }
    for (int s = 0; s < nap; ++s) __builtin_amdgcn_s_sleep(2);
    nap = nap < 4 ? nap * 2 : 4;
  }
  if (!done) wait_failed(S, kind);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // keeps the compiler's order
}

// ---------------------------------------------------------------- top-k

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
  int next_b, next_c;  // next item of the block's phase B / C share (relative)
  int done_b, done_c;  // waves of the block done with phase B / C
  int done_sg, done_sd;  // waves of the block done with shared gate/up / down
  int topk_done;         // tokens whose top-k is in ids / tw
  int plan_ready;        // the plan is built
  int x_staged;          // waves whose part of x is in LDS
  int sg_ready;          // every shared gate/up block is done
  int slot_ready[kMaxExperts];  // phase C: the slot's gate/up blocks are done
  int done_rg[kMaxRowGroups];   // phase C: items done per row group of the block
  int sums_ready;               // phase C: the fp64 sums are zeroed
  int sh_ready;                 // phase C: sh_pre holds the shared output of the block's rows
  uint16_t sh_pre[kShPreMax];   // [n_rg][M][RW] shared output rows of the combine
};

// Work balance.  Item (s, j) of a phase (slot s, j < N items per slot)
// costs kItemCost + kPairCost * np_s units, np_s the pairs of slot s: the
// item's weight bytes, then the arithmetic of each pair, which dominates
// (measured on MI355X: a pair of a gate/up item costs about three times the
// item's weight traffic).  Each block owns the items whose starting cost
// falls in its share [b Q, (b + 1) Q) of the total, so a hot expert's items
// are spread over more blocks.
constexpr int kItemCost = 1;
constexpr int kPairCost = 3;
// A top_k up to this is selected by repeated wave maxima, a larger one by
// a bit-by-bit threshold search.
constexpr int kTopkByMax = 16;
__device__ __forceinline__ int item_cost(const Route &R, int s) {
  return kItemCost + kPairCost * (R.offs[s + 1] - R.offs[s]);
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

// Top-k of token t by one wave (top_k <= E <= 256) into LDS.  The logits
// are polled until every one carries this call's sequence number (bounded:
// after P.polls polls it records the failure and goes on with what it read,
// so the kernel still ends).  Block 0 also writes the plain bf16 logits.  The token's selected
// experts are also OR-ed into R.tokmask.
//
// Selection: the keys (rank_key: the logit's order, then the smaller expert
// index) are unique, so the top_k largest are exactly those >= the top_k-th
// largest key.  A small top_k takes top_k rounds of a wave maximum; a larger
// one finds the threshold key by a radix search with ballot counts, and the
// selected keys are then ranked among themselves (descending key = the
// selection order), which fixes the order of ids, of the weights and of the
// fp32 sum of the scores.
// NS slots per lane (E <= 64 NS): expert lane + 64 i in slot i.
template <int NS>
__device__ void topk_token(const Params &P, int t, Route &R, int *scratch) {
  const int lane = lane_id();
  const int E = P.E, k = P.top_k;
  const unsigned long long *trow = P.tlog + ((size_t)(blockIdx.x % kFlagCopies) * P.M + t) * E;
  // slots past E read expert E - 1 and are masked, so every load is issued
  // at once and nothing branches
  int ee[NS];
  bool valid[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ee[i] = lane + kWave * i;
    valid[i] = ee[i] < E;
    ee[i] = valid[i] ? ee[i] : E - 1;
  }
  unsigned long long v[NS];
  bool done = false;
  for (int it = 0, nap = 1; it < P.polls; ++it) {
#pragma unroll
    for (int i = 0; i < NS; ++i) v[i] = ld_dev(&trow[ee[i]]);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NS; ++i) ok &= !valid[i] || (uint32_t)(v[i] >> 32) == (uint32_t)P.seq;
    if (__all(ok)) {
      done = true;
      break;
    }
    for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
    nap = nap < 8 ? nap * 2 : 8;
  }
  if (!done) wait_failed(P.sync, kWaitLogits);
  TRACE(P, 13);
  int keys[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const uint32_t bits = (uint32_t)v[i] & 0xffffu;
    keys[i] = valid[i] ? rank_key(bits, ee[i]) : kNoKey;
  }
  if (blockIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (valid[i]) P.logits[(size_t)t * E + ee[i]] = (uint16_t)(v[i] & 0xffffu);
  }
  // Lanes j < top_k (top_k <= 64 here) get the selected keys, lane j the
  // (j+1)-th largest (0 = largest = first in the pages' order).
  int key = kNoKey;
  if (k <= kTopkByMax) {
    // k rounds of a wave maximum (keys are unique): the short dependent
    // chain of a small top_k
    for (int r = 0; r < k; ++r) {
      int lm = keys[0];
#pragma unroll
      for (int i = 1; i < NS; ++i) lm = max(lm, keys[i]);
      const int m = wave_max_i32(lm);
#pragma unroll
      for (int i = 0; i < NS; ++i) keys[i] = keys[i] == m ? kNoKey : keys[i];
      key = lane == r ? m : key;
    }
  } else {
    // the top_k-th largest key, by a radix search from the top bit with
    // ballot counts over the keys offset to [0, 2^24) (no key: -1)
    int ukey[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) ukey[i] = keys[i] == kNoKey ? -1 : keys[i] + (1 << 23);
    int thr = 0;
#pragma unroll
    for (int bit = 23; bit >= 0; --bit) {
      const int cand = thr | (1 << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NS; ++i) cnt += __popcll(__ballot(ukey[i] >= cand));
      thr = cnt >= k ? cand : thr;
    }
    // compact the selected keys into scratch[0 .. k), then rank them
    int base = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const bool sel = ukey[i] >= thr;
      const unsigned long long m = __ballot(sel);
      if (sel) scratch[base + __popcll(m & ((1ull << lane) - 1ull))] = keys[i];
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int ck = lane < k ? scratch[lane] : kNoKey;
    int rank = 0;
    for (int j = 0; j < k; ++j) rank += __builtin_amdgcn_readlane(ck, j) > ck;
    // lane rank takes key ck
    key = __builtin_amdgcn_ds_permute(rank * 4, ck);
    key = lane < k ? key : kNoKey;
  }
  const float sc = lane < k ? router_score(key) : 0.0f;
  // the fp32 sum of the scores in selection order, one addition at a time
  float S = 0.0f;
  for (int r = 0; r < k; ++r)
    S = S + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), r));
  const float D = S + 1e-20f;
  if (lane < k) {
    const int e = key_expert(key);
    R.ids[t * k + lane] = e;
    R.tw[t * k + lane] = round_bf16(sc / D);
    atomicOr(&R.tokmask[e], 1ull << t);
  }
}

// The same selection for top_k > 64 (k rounds of "take the largest key").
__device__ void topk_token_long(const Params &P, int t, Route &R) {
  const int lane = lane_id();
  const int E = P.E, k = P.top_k;
  const unsigned long long *trow = P.tlog + ((size_t)(blockIdx.x % kFlagCopies) * P.M + t) * E;
  unsigned long long v[4] = {0ull, 0ull, 0ull, 0ull};
  bool done = false;
  for (int it = 0, nap = 1; it < P.polls; ++it) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + kWave * i;
      if (e < E) {
        v[i] = ld_dev(&trow[e]);
        ok &= (uint32_t)(v[i] >> 32) == (uint32_t)P.seq;
      }
    }
    if (__all(ok)) {
      done = true;
      break;
    }
    for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
    nap = nap < 8 ? nap * 2 : 8;
  }
  if (!done) wait_failed(P.sync, kWaitLogits);
  int keys[4], sel[4] = {kNoKey, kNoKey, kNoKey, kNoKey};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    const uint32_t bits = (uint32_t)v[i] & 0xffffu;
    keys[i] = (e < E) ? rank_key(bits, e) : kNoKey;
    if (blockIdx.x == 0 && e < E) P.logits[(size_t)t * E + e] = (uint16_t)bits;
  }
  for (int j = 0; j < k; ++j) {
    int best = wave_max_i32(max(max(keys[0], keys[1]), max(keys[2], keys[3])));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (keys[i] == best) keys[i] = kNoKey;
      if ((j >> 6) == i && lane == (j & (kWave - 1))) sel[i] = best;
    }
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = kWave * i + lane < k ? router_score(sel[i]) : 0.0f;
  float S = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int i = j >> 6;
    const float v2 = (i == 0) ? s[0] : (i == 1) ? s[1] : (i == 2) ? s[2] : s[3];
    S = S + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v2), j & (kWave - 1)));
  }
  const float D = S + 1e-20f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = kWave * i + lane;
    if (j < k) {
      const int e = key_expert(sel[i]);
      R.ids[t * k + j] = e;
      R.tw[t * k + j] = round_bf16(s[i] / D);
      atomicOr(&R.tokmask[e], 1ull << t);
    }
  }
}

// Exclusive prefix sum over the wave (lane order), with DPP: shifts by 1,
// 2, 4, 8 inside each 16-lane row, then the running totals of rows 0 and 0-1
// carried into the later rows.
__device__ __forceinline__ int wave_exclusive_scan(int v) {
  int x = v;
  x += dpp_i32<0x111>(x);  // row_shr:1 (lanes shifted in from outside the row read 0)
  x += dpp_i32<0x112>(x);  // row_shr:2
  x += dpp_i32<0x114>(x);  // row_shr:4
  x += dpp_i32<0x118>(x);  // row_shr:8
  x += dpp_i32<kDppBcast15, 0xA>(x, 0);  // rows 1, 3 += last lane of rows 0, 2
  x += dpp_i32<kDppBcast31, 0xC>(x, 0);  // rows 2, 3 += lane 31
  return x - v;
}

// Routing plan from R.ids and R.tokmask, built by one wave: touched experts ascending
// (slot order), pairs of each expert ascending (an expert has at most one
// pair per token), and the cumulative item costs of phases B and C
// (GU_ITEMS, DN_ITEMS items per slot).  Ends by raising R.plan_ready.
template <int GU_ITEMS, int DN_ITEMS>
__device__ void build_plan_wave(const Params &P, Route &R) {
  const int npairs = P.M * P.top_k, k = P.top_k, lane = lane_id();
  // R.tokmask (tokens that selected each expert) was filled with the ids
  // lane l holds experts 4l .. 4l + 3
  int cnt[4], flg[4], c = 0, f = 0, u = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    cnt[i] = e < P.E ? __popcll(R.tokmask[e]) : 0;
    flg[i] = cnt[i] > 0;
    c += cnt[i];
    f += flg[i];
    u += flg[i] ? kItemCost + kPairCost * cnt[i] : 0;
  }
  int base = wave_exclusive_scan(c), slot = wave_exclusive_scan(f);
  int cost = wave_exclusive_scan(u);  // in units of one item per slot
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (flg[i]) {
      R.slot_of[e] = slot;
      R.active[slot] = e;
      R.offs[slot] = base;
      R.cum_gu[slot] = cost * GU_ITEMS;
      R.cum_dn[slot] = cost * DN_ITEMS;
    }
    base += cnt[i];
    slot += flg[i];
    cost += flg[i] ? kItemCost + kPairCost * cnt[i] : 0;
  }
  if (lane == kWave - 1) {
    R.next_b = R.next_c = R.done_b = R.done_c = 0;
    R.n_active = slot;
    R.offs[slot] = base;
    R.cum_gu[slot] = cost * GU_ITEMS;
    R.cum_dn[slot] = cost * DN_ITEMS;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int p = lane; p < npairs; p += kWave) {
    const int ee = R.ids[p];
    if ((unsigned)ee < (unsigned)P.E) {
      const int t = p / k;
      const int rank = __popcll(R.tokmask[ee] & ((1ull << t) - 1ull));
      R.pairs[R.offs[R.slot_of[ee]] + rank] = p;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) __hip_atomic_store(&R.plan_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until an LDS counter of the block reaches n.  The waves it waits for
// belong to the same (resident) block and their own waits are bounded, so
// this ends; as a guard it gives up after 2^22 polls and records kWaitLds.
__device__ __forceinline__ void wait_lds_at_least(int *c, int n, DecodeSync *S) {
  bool done = false;
  for (int it = 0; it < (1 << 22); ++it) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= n) {
      done = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!done) wait_failed(S, kWaitLds);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Waits until the block's plan is built (as wait_lds_at_least).
__device__ __forceinline__ void wait_plan(Route &R, DecodeSync *S) {
  wait_lds_at_least(&R.plan_ready, 1, S);
}

// --------------------------------------------------------- phase A items

// Issues the copy of n 16-byte chunks from global memory straight into LDS
// (direct loads: no registers, every load in flight at once), by waves
// wave, wave + nwaves, ... (each moves 1 KB blocks).  DEVICE: device-scope
// loads of data other blocks wrote.  copy_to_lds then waits until the
// calling wave's copies have landed (this also waits for its other
// outstanding loads).
template <bool DEVICE>
__device__ __forceinline__ void issue_copy_to_lds(uint16_t *dst, const uint16_t *src, int n,
                                                  int wave, int nwaves) {
  const int lane = lane_id();
  for (int b = wave; b * kWave < n; b += nwaves) {
    const int i = b * kWave + lane;
    if (i < n)
      __builtin_amdgcn_global_load_lds(src + (size_t)i * 8,
                                       (__attribute__((address_space(3))) void *)(dst + (size_t)b * 512),
                                       16, 0, DEVICE ? kCachePolicyDevice : 0);
  }
}
template <bool DEVICE>
__device__ __forceinline__ void copy_to_lds(uint16_t *dst, const uint16_t *src, int n, int wave,
                                            int nwaves) {
  issue_copy_to_lds<DEVICE>(dst, src, n, wave, nwaves);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies are in LDS
}

// Stages nr rows of a bf16 matrix with K columns into LDS (the whole block;
// the caller synchronises the block before reading them).
template <int K, bool DEVICE>
__device__ __forceinline__ void stage_rows(uint16_t *dst, const uint16_t *src, int nr) {
  copy_to_lds<DEVICE>(dst, src, nr * K / 8, wave_id(), kWaves);
}

// Routing block r: logits of experts kWaves * (r % nEG) + wave for the 8
// tokens of group r / nEG, each stored with the call's sequence number in
// one 8-byte word, then the block's flag.  x (of the group, or all of it
// when it fits) is staged in LDS unless it already is.
// Routing item r (one wave): logits of expert r % E for the kRouteTokens
// tokens of group r / E, each stored with the call's sequence number in one 8-byte
// word (the value and its "written" mark arrive together).  x is read from
// global memory (it is an input), so the item needs no LDS and can start at
// once.
// The residual add and RMS norm of row t (page "vllm.models.flint.ops.moe",
// _add_rms_norm), by one wave: s = fp32(a + r) (one rounding), the fp32 sum
// of s^2 (each lane sums its chunks in order with fused multiply-adds, then
// the fixed DPP tree), inv = 1 / sqrt(sum / H + eps) (correctly rounded),
// xn = bf16((s * inv) * w).  Lane l holds 16-byte chunks l + 64 i of the
// row, as route_item reads x.  Every wave that forms a row's xn gets the
// same bits, so routing and the staged copy agree.
template <int H>
__device__ __forceinline__ void norm_row(const Params &P, int t,
                                         u32x4_t (&xn)[(H / 8 + kWave - 1) / kWave],
                                         u32x4_t (&res)[(H / 8 + kWave - 1) / kWave]) {
  constexpr int NC = H / 8, CPL = (NC + kWave - 1) / kWave;
  const int lane = lane_id();
  float sv[CPL][8];
  u32x4_t w[CPL];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + kWave * i;
    u32x4_t a{0, 0, 0, 0}, r{0, 0, 0, 0};
    w[i] = u32x4_t{0, 0, 0, 0};
    if (c < NC) {  // every load of the row in flight at once
      a = load16(P.ln_a + (size_t)t * H + c * 8);
      r = load16(P.ln_r + (size_t)t * H + c * 8);
      w[i] = load16(P.ln_w + c * 8);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      sv[i][2 * d] = bf16_lo(a[d]) + bf16_lo(r[d]);
      sv[i][2 * d + 1] = bf16_hi(a[d]) + bf16_hi(r[d]);
    }
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(sv[i][e], sv[i][e], ss);
  ss = group_sum<kWave>(ss);
  ss = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ss), kWave - 1));
  const float inv = 1.0f / sqrtf(ss / (float)H + P.eps);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      xn[i][d] = pack_bf16x2((sv[i][2 * d] * inv) * bf16_lo(w[i][d]),
                             (sv[i][2 * d + 1] * inv) * bf16_hi(w[i][d]));
      res[i][d] = pack_bf16x2(sv[i][2 * d], sv[i][2 * d + 1]);
    }
  }
}

// NORM: x is the block's staged normed rows in LDS (xl), formed in front of
// the routing; wait_x() waits for them (after the router row's loads are
// issued, so their round trip overlaps the staging).
template <int H, bool NORM, typename WaitX>
__device__ void route_item(const Params &P, int r, const uint16_t *xl, WaitX &&wait_x) {
  constexpr int NC = H / 8;
  constexpr int CPL = (NC + kWave - 1) / kWave;
  const int lane = lane_id();
  const int e = r % P.E;
  const int t0 = (r / P.E) * kRouteTokens;
  const int nt = min(kRouteTokens, P.M - t0);
  u32x4_t w[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + kWave * i;
    w[i] = c < NC ? load16(P.router + (size_t)e * H + c * 8) : u32x4_t{0, 0, 0, 0};
  }
  const unsigned long long tag = (unsigned long long)(uint32_t)P.seq << 32;
  if constexpr (NORM) wait_x();
  for (int g = 0; g < nt; g += 4) {
    u32x4_t xv[4][CPL];
    if constexpr (NORM) {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = lane + kWave * i;
          xv[ti][i] = (g + ti < nt && c < NC) ? load16(xl + (size_t)(t0 + g + ti) * H + c * 8)
                                              : u32x4_t{0, 0, 0, 0};
        }
    } else {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = lane + kWave * i;
          xv[ti][i] = (g + ti < nt && c < NC) ? load16(P.x + (size_t)(t0 + g + ti) * H + c * 8)
                                              : u32x4_t{0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        acc = dot2_bf16(w[i][0], xv[ti][i][0], acc);
        acc = dot2_bf16(w[i][1], xv[ti][i][1], acc);
        acc = dot2_bf16(w[i][2], xv[ti][i][2], acc);
        acc = dot2_bf16(w[i][3], xv[ti][i][3], acc);
      }
      acc = group_sum<kWave>(acc);
      // one copy per XCD (every block polls the logits)
      acc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc), kWave - 1));
      if (lane < kFlagCopies && g + ti < nt)
        st_dev(&P.tlog[((size_t)lane * P.M + t0 + g + ti) * P.E + e], tag | f32_to_bf16(acc));
    }
  }
}

// Gate/up of one wave on given weights for vectors i < np (np <= 64):
// vector i is x[tok(i)], read from xl (LDS) when non-NULL, else from global
// memory.  Results go to the wave's output buffer: ob[i * RP + row] (bf16)
// for the item's RP row pairs.
template <int FMT, int H, int I, typename Tok>
__device__ __forceinline__ void gate_up_compute(const Params &P, const GateUpW<FMT, H, I> &W,
                                                float alpha, int np, Tok tok, const uint16_t *xl,
                                                uint16_t *ob) {
  using Map = RowMap<FMT, H>;
  using G = GateUpGeo<FMT, H>;
  const int lane = lane_id();
  const int r = lane / Map::LPR, q = lane % Map::LPR;
  auto finish = [&](int i, float (&acc)[2 * G::NSL]) {
#pragma unroll
    for (int s = 0; s < G::NSL; ++s) {
      float gs = group_sum<Map::LPR>(acc[s]);
      float us = group_sum<Map::LPR>(acc[G::NSL + s]);
      if (q == Map::LPR - 1) {  // the group's sum is in its last lane
        if constexpr (FMT == kNvfp4) {
          gs = gs * alpha;
          us = us * alpha;
        }
        ob[i * G::RP + s * Map::RS + r] = (uint16_t)f32_to_bf16(swiglu(gs, us));
      }
    }
  };
  if (xl) {
    for (int i = 0; i < np; ++i) {
      float acc[2 * G::NSL];
      rows_dot<FMT, H, kSrcLds>(W.rows, xl + (size_t)tok(i) * H, q, acc);
      finish(i, acc);
    }
  } else if (np > 0) {
    // x from global memory: the next vector's part is loaded while this one
    // is used (one round trip per item instead of one per vector)
    VecRegs<FMT, H> xa, xb;
    load_vec<FMT, H, kSrcGlobal>(xa, P.x + (size_t)tok(0) * H, q);
    for (int i = 0; i < np; i += 2) {
      load_vec<FMT, H, kSrcGlobal>(xb, P.x + (size_t)tok(i + 1 < np ? i + 1 : i) * H, q);
      float acc[2 * G::NSL];
      rows_dot_regs<FMT, H>(W.rows, xa, acc);
      finish(i, acc);
      if (i + 1 >= np) break;
      load_vec<FMT, H, kSrcGlobal>(xa, P.x + (size_t)tok(i + 2 < np ? i + 2 : i + 1) * H, q);
      rows_dot_regs<FMT, H>(W.rows, xb, acc);
      finish(i + 1, acc);
    }
  }
}

// Down of one wave on given weights for vector j (SRC: kSrcLds or
// kSrcDevice); its RW results go to ob[j * RW + row].
template <int FMT, int H, int I, int SRC>
__device__ __forceinline__ void down_one(const DownW<FMT, I> &W, const uint16_t *vec, float alpha,
                                         int j, uint16_t *ob) {
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
      ob[j * G::RW + s * Map::RS + r] = (uint16_t)f32_to_bf16(val);
    }
  }
}

// Writes an item's results with one store instruction per 16 bytes: lane j
// stores the NV bf16 values ob[j * NV ...] at byte offset off of descriptor
// dst (kOOB for lanes without a vector: dropped), performed at device scope.
// The stores of an item are always issued, so their number never varies.
template <int NV>
__device__ __forceinline__ void store_results(__amdgpu_buffer_rsrc_t dst, uint32_t off,
                                              const uint16_t *ob) {
  static_assert(NV == 1 || NV == 2 || NV == 4 || NV % 8 == 0, "results per vector");
  // the item's results were written by other lanes of this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint16_t *src = ob + lane_id() * NV;
  if constexpr (NV == 1) {
    __builtin_amdgcn_raw_buffer_store_b16(src[0], dst, off, 0, kPolicyDevice);
  } else if constexpr (NV == 2) {
    __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t *>(src), dst, off, 0,
                                          kPolicyDevice);
  } else if constexpr (NV == 4) {
    const uint2 v = *reinterpret_cast<const uint2 *>(src);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32_t, v), dst, off, 0,
                                          kPolicyDevice);
  } else {
#pragma unroll
    for (int c = 0; c < NV / 8; ++c)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t *>(src + 8 * c), dst,
                                             off + 16 * c, 0, kPolicyDevice);
  }
}

// ------------------------------------------------------------ the kernel

__device__ __forceinline__ int per_wave(int items, int nw) { return (items + nw - 1) / nw; }

// Next item of the block's share of a phase: one LDS counter per phase,
// taken by lane 0 and broadcast (items come out in increasing order).
__device__ __forceinline__ int take_item(int *ctr, int base) {
  int v = 0;
  if (lane_id() == 0) v = atomicAdd(ctr, 1);
  return base + __builtin_amdgcn_readfirstlane(v);
}

// A wave is done with its phase: once the stores of all kWaves waves are
// performed, the last of them raises the block's flag.
__device__ __forceinline__ void block_done(int *ctr, int *flag, int seq) {
  stores_performed();
  if (lane_id() == 0) {
    if (atomicAdd(ctr, 1) == kWaves - 1) st_dev(flag, seq);
  }
}
// The same with the flag written to every copy flag[c * stride], c < kFlagCopies.
__device__ __forceinline__ void block_done_copies(int *ctr, int *flag, int stride, int seq) {
  stores_performed();
  if (lane_id() == 0) {
    if (atomicAdd(ctr, 1) == kWaves - 1)
      for (int c = 0; c < kFlagCopies; ++c) st_dev(flag + c * stride, seq);
  }
}

// Block that owns item (s, j) of a phase partitioned in shares of cost Q.
__device__ __forceinline__ int owner_block(const Route &R, const int *cum, int s, int j, int Q,
                                           int nb) {
  const int b = owner(R, cum, s, j, Q);
  return b < nb ? b : nb - 1;
}

// NORM: the residual add + RMS norm in front of the block is formed by every
// block into its x staging area (all of x fits), before the routing items.
template <int FMT, int SFMT, bool NORM, int H, int I>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
decode_kernel(Params P) {
  using Gm = Geo<FMT, SFMT, H, I>;
  using DnMap = RowMap<FMT, I>;
  constexpr int GU_RSZ = FMT == kNvfp4 ? H / 2 : H * 2;  // routed row bytes (w13)
  constexpr int DN_RSZ = FMT == kNvfp4 ? I / 2 : I * 2;  // routed row bytes (w2)
  __shared__ Route R;
  // Dynamic LDS: x staging (kXLdsBytes), then one slice per wave
  // (kSliceBytes each: the down items' activation cache, the combine's y).
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  uint16_t *slice = xs + kXLdsBytes / 2 + (size_t)wave_id() * (kSliceBytes / 2);
  uint16_t *ob = slice + (kSliceBytes - Gm::OUT_BYTES) / 2;  // an item's results

  DecodeSync *S = P.sync;
  const int lane = lane_id(), wv = wave_id();
  const int NW = P.nb * kWaves;
  const int gw = blockIdx.x * kWaves + wv;
  const int k = P.top_k;
  const bool x_all = P.M * H * 2 <= kXLdsBytes;  // all of x fits the staging area
  TRACE_INIT();
  TRACE(P, 0);

  if (threadIdx.x == 0) {
    R.done_sg = R.done_sd = R.topk_done = R.plan_ready = R.x_staged = R.sg_ready = R.sums_ready = 0;
    R.sh_ready = 0;
  }
  if (threadIdx.x < kMaxExperts) {
    R.tokmask[threadIdx.x] = 0ull;
    R.slot_ready[threadIdx.x] = 0;
  }
  if (threadIdx.x < kMaxRowGroups) R.done_rg[threadIdx.x] = 0;
  __syncthreads();  // publishes the counters
  // Test hook: one wave waits for a word that no block ever sets, so the
  // wait gives up and records kWaitProbe (the host asks for it).
  if (P.probe && blockIdx.x == 0 && wv == 0)
    wave_wait_flags(&S->probe, 0, 1, ~P.seq, P.polls, S, kWaitProbe);

  auto wait_x = [&]() {
    if (x_all) wait_lds_at_least(&R.x_staged, kWaves - 1, S);
  };
  if constexpr (NORM) {
    // The normed rows, formed by every wave but the last of this block
    // (block 0 also writes them and the residual sum out), before the
    // routing items that read them here.
    constexpr int NC = H / 8, CPL = (NC + kWave - 1) / kWave;
    if (wv < kWaves - 1) {
      for (int t = wv; t < P.M; t += kWaves - 1) {
        u32x4_t xn[CPL], rs[CPL];
        norm_row<H>(P, t, xn, rs);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = lane + kWave * i;
          if (c < NC) {
            *reinterpret_cast<u32x4_t *>(xs + (size_t)t * H + c * 8) = xn[i];
            if (blockIdx.x == 0) {
              *reinterpret_cast<u32x4_t *>(P.xn_out + (size_t)t * H + c * 8) = xn[i];
              *reinterpret_cast<u32x4_t *>(P.res_out + (size_t)t * H + c * 8) = rs[i];
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) atomicAdd(&R.x_staged, 1);
    }
  }

  // ---- phase A1: routing items, one per wave from the last wave of each
  // block down (item r: block r % nb); they read x from global memory (the
  // staged normed rows with NORM).
  for (int r = blockIdx.x + P.nb * (kWaves - 1 - wv); r < P.n_route; r += P.nb * kWaves) {
    __builtin_amdgcn_s_setprio(3);  // on the critical path
    route_item<H, NORM>(P, r, xs, wait_x);
    __builtin_amdgcn_s_setprio(0);
  }
  TRACE(P, 1);
  // All of x in LDS when it fits (shared gate/up and phase B read it
  // there), staged by every wave but the last; R.x_staged counts them.
  if (!NORM && x_all && wv < kWaves - 1) {
    copy_to_lds<false>(xs, P.x, P.M * H / 8, wv, kWaves - 1);
    if (lane == 0) atomicAdd(&R.x_staged, 1);
  }

  // Shared-expert items go to every block: shared gate/up items to its
  // first nsg waves, shared down items to the next nsd waves; the remaining
  // waves compute the top-k.
  const int sh0 = 0;  // first block with shared items
  const int nbs = P.nb - sh0;
  const int bs = (int)blockIdx.x - sh0;
  const int nsg = P.sgu ? min((P.n_sgu + nbs - 1) / nbs, kWaves / 2) : 0;
  const int nsd = P.sgu ? min((P.n_sdn + nbs - 1) / nbs, kWaves / 2) : 0;

  // ---- phase A2: shared gate/up, one row-pair item per wave (item j:
  // block sh0 + j % nbs, wave j / nbs), every token.
  // (an NVFP4 shared expert: E2M1 codes, E4M3 block scales and one global
  // scale per matrix, the routed experts' rule)
  constexpr bool kNvShared = SFMT == kNvfp4;
  constexpr size_t kSguBytes = kNvShared ? (size_t)2 * I * H / 2 : (size_t)2 * I * H * 2;
  constexpr size_t kSdnBytes = kNvShared ? (size_t)H * I / 2 : (size_t)H * I * 2;
  if (P.sgu) {
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(P.sgu, kSguBytes);
    const __amdgpu_buffer_rsrc_t rs_s =
        make_rsrc(kNvShared ? (const void *)P.ssgu : (const void *)P.sgu,
                  kNvShared ? (size_t)2 * I * (H / 16) : 0);
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(P.sact, (size_t)P.M * I * 2);
    const float alpha = kNvShared ? *P.asgu : 1.0f;
    for (int j = (bs >= 0 && wv < nsg) ? bs + nbs * wv : P.n_sgu; j < P.n_sgu; j += nbs * nsg) {
      const int n_base = j * Gm::SGU::RP;
      GateUpW<SFMT, H, I> W;
      gate_up_load(W, rs_w, 0u, rs_s, 0u, n_base);
      wait_x();
      TRACE(P, 9);
      for (int g0 = 0; g0 < P.M; g0 += kWave) {
        const int nt = min(kWave, P.M - g0);
        gate_up_compute<SFMT, H, I>(P, W, alpha, nt, [g0](int i) { return g0 + i; },
                                    x_all ? xs : nullptr, ob);
        store_results<Gm::SGU::RP>(
            rs_o, lane < nt ? (uint32_t)(((g0 + lane) * I + n_base) * 2) : kOOB, ob);
      }
      TRACE(P, 11);
    }
    block_done_copies(&R.done_sg, &S->sg[0][blockIdx.x], kMaxSharedBlocks, P.seq);
  }

  // ---- phase A3: shared down, one item (RW rows) per wave (item j: block
  // sh0 + j % nbs, wave nsg + j / nbs), after every shared gate/up block.
  // sact is staged in a part of the staging area that x does not use.
  if (P.sgu) {
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(P.sdown, kSdnBytes);
    const __amdgpu_buffer_rsrc_t rs_s =
        make_rsrc(kNvShared ? (const void *)P.ssdown : (const void *)P.sdown,
                  kNvShared ? (size_t)H * (I / 16) : 0);
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(P.sh, (size_t)P.M * H * 2);
    const float alpha = kNvShared ? *P.asdown : 1.0f;
    const int free_el = kXLdsBytes / 2 - (x_all ? P.M * H : 0);
    const int per = free_el / max(1, min(nsd, kWaves));  // bf16 per shared-down wave
    // the wave's slice when the free part of the staging area is too small
    constexpr int kSliceRows = (kSliceBytes - Gm::OUT_BYTES) / (2 * I);
    static_assert(kSliceRows >= 1, "shared activations staging");
    const int region = per >= I ? per / I * I : kSliceRows * I;
    const int G = min(kWave, region / I);  // tokens per staged group, >= 1
    bool waited = false;
    const int ws = wv - nsg;  // this wave's place among the shared down waves
    for (int j = (bs >= 0 && ws >= 0 && ws < nsd) ? bs + nbs * ws : P.n_sdn; j < P.n_sdn;
         j += nbs * nsd) {
      const int h_base = j * Gm::SDN::RW;
      DownW<SFMT, I> W;
      down_load(W, rs_w, 0u, rs_s, 0u, h_base);
      if (!waited) {
        // the block's first shared down wave polls the flags, the others
        // wait for its word in LDS
        if (ws == 0) {
          wave_wait_flags(S->sg[blockIdx.x % kFlagCopies], sh0, sh0 + min(nbs, P.n_sgu), P.seq, P.polls, S,
                          kWaitSharedGateUp);
          if (lane == 0) __hip_atomic_store(&R.sg_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
          wait_lds_at_least(&R.sg_ready, 1, S);
        }
        waited = true;
      }
      TRACE(P, 14);
      uint16_t *sl = per >= I ? xs + (x_all ? P.M * H : 0) + (size_t)ws * region : slice;
      for (int g0 = 0; g0 < P.M; g0 += G) {
        const int nt = min(G, P.M - g0);
        copy_to_lds<true>(sl, P.sact + (size_t)g0 * I, nt * I / 8, 0, 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int t = 0; t < nt; ++t)
          down_one<SFMT, H, I, kSrcLds>(W, sl + (size_t)t * I, alpha, t, ob);
        store_results<Gm::SDN::RW>(
            rs_o, lane < nt ? (uint32_t)(((g0 + lane) * H + h_base) * 2) : kOOB, ob);
      }
      TRACE(P, 15);
    }
    block_done(&R.done_sd, &S->sd[blockIdx.x], P.seq);
  }
  TRACE(P, 2);

  // ---- routing of every token (waves without shared-expert items), in this
  // block's LDS; the wave that completes the last token builds the plan.
  {
    // top-k waves: those with no shared-expert item (first waves: shared
    // gate/up, last waves: shared down), token t on wave w0 + t % nfree
    const int nfree = kWaves - nsg - nsd >= 1 ? kWaves - nsg - nsd : kWaves;
    const int w0 = kWaves - nsg - nsd >= 1 ? nsg + nsd : 0;
    const int slot = wv - w0;
    __builtin_amdgcn_s_setprio(3);  // on the critical path: ahead of other waves' work
    int mine = 0;
    for (int t = (slot >= 0 && slot < nfree) ? slot : P.M; t < P.M; t += nfree) {
      if (P.ids_in) {
        for (int j = lane; j < k; j += kWave) {
          const int e = P.ids_in[t * k + j];
          R.ids[t * k + j] = e;
          R.tw[t * k + j] = P.tw_in[t * k + j];
          if ((unsigned)e < (unsigned)P.E) atomicOr(&R.tokmask[e], 1ull << t);  // bad ids dropped
        }
      } else if (k <= kWave) {
        if (P.E <= kWave) topk_token<1>(P, t, R, reinterpret_cast<int *>(slice));
        else if (P.E <= 2 * kWave) topk_token<2>(P, t, R, reinterpret_cast<int *>(slice));
        else topk_token<4>(P, t, R, reinterpret_cast<int *>(slice));
      } else {
        topk_token_long(P, t, R);
      }
      ++mine;
    }
    TRACE(P, 8);
    int before = 0;
    if (mine > 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) before = atomicAdd(&R.topk_done, mine);
      before = __builtin_amdgcn_readfirstlane(before);
    }
    if (mine > 0 && before + mine == P.M) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      build_plan_wave<Gm::N_GU, Gm::N_DN>(P, R);
    } else {
      wait_plan(R, S);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if (blockIdx.x == 0)
    for (int p = threadIdx.x; p < P.M * k; p += kThreads) {
      if (P.ids != P.ids_in) P.ids[p] = R.ids[p];
      if (P.tw != P.tw_in) P.tw[p] = R.tw[p];
    }
  TRACE(P, 3);
  wait_x();
  const int U = R.n_active;
  const uint16_t *xl = x_all ? xs : nullptr;
  // phase C: this block's down row groups (RW output rows each): b, b + nb, ...
  const int n_rg = (int)blockIdx.x < Gm::N_DN ? (Gm::N_DN - 1 - (int)blockIdx.x) / P.nb + 1 : 0;

  // ---- phase B: routed gate/up; block share [b0, b1) of equal cost
  //
  // Memory instructions per item are fixed (every load issued, items past
  // the share read out of range; one store per 16 result bytes), so the
  // wait for an item's weights never waits for a store.
  //
  // One item in flight per wave: the 16 waves of a CU already keep about
  // 72 KB of weights in flight per CU (18 MB on the chip), enough for the
  // HBM rate, and a deeper queue only lengthens every round trip the
  // phases after it wait on (measured on MI355X: two items per wave were
  // slower end to end).
  const int QB = max(1, per_wave(R.cum_gu[U], P.nb));
  {
    const int b0 = first_item(R, R.cum_gu, Gm::N_GU, blockIdx.x * QB);
    const int b1 = first_item(R, R.cum_gu, Gm::N_GU, (blockIdx.x + 1) * QB);
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(P.w13, (size_t)P.E * 2 * I * GU_RSZ);
    const __amdgpu_buffer_rsrc_t rs_s =
        make_rsrc(FMT == kNvfp4 ? (const void *)P.s13 : (const void *)P.w13,
                  FMT == kNvfp4 ? (size_t)P.E * 2 * I * (H / 16) : 0);
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(P.act, (size_t)P.M * k * I * 2);
    struct St {
      GateUpW<FMT, H, I> w;
      float alpha;
    };
    auto load = [&](St &st, int i) {
      const bool ok = i < b1;
      const int e = __builtin_amdgcn_readfirstlane(ok ? R.active[i / Gm::N_GU] : 0);
      const int n_base = ok ? (i % Gm::N_GU) * Gm::GU::RP : 0;
      gate_up_load(st.w, rs_w, ok ? (uint32_t)e * 2 * I * GU_RSZ : kOOB, rs_s,
                   ok ? (uint32_t)e * 2 * I * (H / 16) : kOOB, n_base);
      st.alpha = FMT == kNvfp4 ? P.a13[e] : 1.0f;
    };
    auto run = [&](const St &st, int i) {
      const int s = i / Gm::N_GU;
      const int n_base = (i % Gm::N_GU) * Gm::GU::RP;
      const int *pr = R.pairs + R.offs[s];
      const int np = R.offs[s + 1] - R.offs[s];
      gate_up_compute<FMT, H, I>(P, st.w, st.alpha, np, [pr, k](int j) { return pr[j] / k; }, xl,
                                 ob);
      store_results<Gm::GU::RP>(
          rs_o, lane < np ? (uint32_t)((pr[lane] * I + n_base) * 2) : kOOB, ob);
    };
    // Items come out of the counter in increasing order: the first past the
    // share ends the wave's part.
    St sa;
    int ia = take_item(&R.next_b, b0);
    load(sa, ia);
    while (ia < b1) {
      __builtin_amdgcn_sched_barrier(0);
      run(sa, ia);
      ia = take_item(&R.next_b, b0);
      load(sa, ia);
    }
    // The block's last wave past its gate/up items raises the block's flag
    // (once the stores of all its waves are performed) and zeroes phase C's
    // fp64 sums, which live in the x staging area that no wave reads any more.
    stores_performed();
    int last = 0;
    if (lane == 0) last = atomicAdd(&R.done_b, 1) == kWaves - 1;
    if (__builtin_amdgcn_readfirstlane(last)) {
      if (lane < kFlagCopies) st_dev(&S->gb[lane][blockIdx.x], P.seq);
      double *sums = reinterpret_cast<double *>(xs);
      const int nsum = n_rg * P.M * Gm::DN::RW;
      for (int i = lane; i < nsum; i += kWave) sums[i] = 0.0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __hip_atomic_store(&R.sums_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // The shared output of the block's rows, staged for the combines now
      // (the shared expert is done long before the routed down items), so a
      // combine waits for no round trip of its own.
      if (P.sgu || P.sh_ext) {
        constexpr int RWC = Gm::DN::RW;
        for (int lr = 0; lr < n_rg; ++lr) {
          const int h_base = ((int)blockIdx.x + lr * P.nb) * RWC;
          if (P.sgu) {
            // the blocks holding the shared down items of these rows
            bool done = false;
            const int j0 = h_base / Gm::SDN::RW, j1 = (h_base + RWC - 1) / Gm::SDN::RW;
            for (int it = 0, nap = 1; it < P.polls; ++it) {
              bool ok = true;
              for (int j = j0 + lane; j <= j1; j += kWave) ok &= ld_dev(&S->sd[sh0 + j % nbs]) == P.seq;
              if (__all(ok)) {
                done = true;
                break;
              }
              for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
              nap = nap < 4 ? nap * 2 : 4;
            }
            if (!done) wait_failed(S, kWaitCombineShared);
          }
          for (int l = lane; l < P.M * RWC; l += kWave) {
            const size_t o = (size_t)(l / RWC) * H + h_base + l % RWC;
            R.sh_pre[lr * P.M * RWC + l] = P.sgu ? ld_dev(&P.sh[o]) : P.sh_ext[o];
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_store(&R.sh_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  TRACE(P, 4);

  // ---- phase C: routed down by row group, with the combine
  //
  // Block b owns the row groups g = b, b + nb, ... (RW output rows each) and
  // computes every slot's down item of them, so the combine of its rows
  // needs no other block's routed results.  An item adds tw * y of its pairs
  // into the row group's fp64 sums in LDS (each product of two bf16 values
  // has 16 significant bits, and their sums are exact, so the order of the
  // additions does not change them), and the wave that completes a row
  // group's last item rounds the sums, adds the shared output and stores the
  // rows.  A block's items start at the slot of its own first gate/up item
  // (done when the block is) and go round the slots; each slot's gate/up
  // blocks are polled once per block, and a slot known done has its
  // activations copied with the item's weights (one round trip).
  {
    constexpr int RW = Gm::DN::RW;
    const int n_items = n_rg * U;
    const int g0 = first_item(R, R.cum_gu, Gm::N_GU, blockIdx.x * QB);
    const int s_start = U > 0 && g0 < U * Gm::N_GU ? g0 / Gm::N_GU : 0;
    double *sums = reinterpret_cast<double *>(xs);  // [n_rg][M][RW]
    const int sum_bytes = (n_rg * P.M * RW * 8 + 15) & ~15;
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(P.w2, (size_t)P.E * H * DN_RSZ);
    const __amdgpu_buffer_rsrc_t rs_s =
        make_rsrc(FMT == kNvfp4 ? (const void *)P.s2 : (const void *)P.w2,
                  FMT == kNvfp4 ? (size_t)P.E * H * (I / 16) : 0);
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(P.y, (size_t)P.M * k * H * 2);
    // activation rows of an item: the first kCache in the wave's slice, the
    // next kCacheX in its part of the staging area after the sums, any
    // further ones read from global memory per use
    constexpr int kCache = (kSliceBytes - Gm::OUT_BYTES) / (2 * I);
    static_assert(kCache >= 1, "activation cache");
    const int per_wave_el = (kXLdsBytes - sum_bytes) / kWaves / 2 / 8 * 8;
    const int kCacheX = per_wave_el / I;
    uint16_t *xpart = xs + sum_bytes / 2 + (size_t)wv * per_wave_el;
    bool sums_seen = false;
    struct St {
      DownW<FMT, I> w;
      float alpha;
      bool act;  // the activations were requested with the weights
    };
    auto item_of = [&](int f, int &s, int &h_base, int &lr) {
      lr = f / U;
      s = s_start + (f - lr * U);
      if (s >= U) s -= U;
      h_base = ((int)blockIdx.x + lr * P.nb) * RW;
    };
    auto issue_act = [&](int s) {
      const int *pr = R.pairs + R.offs[s];
      const int np = R.offs[s + 1] - R.offs[s];
      const int nc = np < kCache ? np : kCache;
      const int nx = np - nc < kCacheX ? np - nc : kCacheX;
      for (int j = 0; j < nc + nx; ++j)
        issue_copy_to_lds<true>(j < nc ? slice + (size_t)j * I : xpart + (size_t)(j - nc) * I,
                                P.act + (size_t)pr[j] * I, I / 8, 0, 1);
    };
    // The combine of row group lr (rows h_base ..): the rounded sums plus the
    // shared output, for every token.
    auto combine = [&](int lr, int h_base) {
      const double *gs = sums + (size_t)lr * P.M * RW;
      TRACE(P, 6);
      const bool has_sh = P.sgu || P.sh_ext;
      if (has_sh) wait_lds_at_least(&R.sh_ready, 1, S);
      const uint16_t *shp = R.sh_pre + (size_t)lr * P.M * RW;
      for (int l = lane; l < P.M * RW; l += kWave) {
        const int t = l / RW, r = l % RW;
        const float routed = round_bf16((float)gs[t * RW + r]);
        const size_t o = (size_t)t * H + h_base + r;
        const float sv = has_sh ? bf16_to_f32(shp[l]) : 0.0f;
        P.out[o] = (uint16_t)f32_to_bf16(routed + sv);
      }
    };
    auto load = [&](St &st, int f) {
      const bool ok = f < n_items;
      int s = 0, h_base = 0, lr = 0;
      if (ok) item_of(f, s, h_base, lr);
      const int e = __builtin_amdgcn_readfirstlane(ok ? R.active[s] : 0);
      down_load(st.w, rs_w, ok ? (uint32_t)e * H * DN_RSZ : kOOB, rs_s,
                ok ? (uint32_t)e * H * (I / 16) : kOOB, h_base);
      st.alpha = FMT == kNvfp4 ? P.a2[e] : 1.0f;
      // the staging area holds the sums and act rows once every wave of the
      // block is past its gate/up items
      if (ok && !sums_seen) {
        wait_lds_at_least(&R.sums_ready, 1, S);
        sums_seen = true;
      }
      st.act = ok && __hip_atomic_load(&R.slot_ready[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
      if (st.act) issue_act(s);
    };
    auto run = [&](const St &st, int f) {
      int s, h_base, lr;
      item_of(f, s, h_base, lr);
      const int *pr = R.pairs + R.offs[s];
      const int np = R.offs[s + 1] - R.offs[s];
      const int nc = np < kCache ? np : kCache;
      const int nx = np - nc < kCacheX ? np - nc : kCacheX;
      if (!st.act) {
        if (__hip_atomic_load(&R.slot_ready[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
          wave_wait_flags(S->gb[blockIdx.x % kFlagCopies], owner_block(R, R.cum_gu, s, 0, QB, P.nb),
                          owner_block(R, R.cum_gu, s, Gm::N_GU - 1, QB, P.nb) + 1, P.seq, P.polls, S,
                          kWaitGateUp);
          if (lane == 0)
            __hip_atomic_store(&R.slot_ready[s], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        issue_act(s);
      }
      TRACE_FIRST(P, 10);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows are in LDS
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int j = 0; j < nc; ++j)
        down_one<FMT, H, I, kSrcLds>(st.w, slice + (size_t)j * I, st.alpha, j, ob);
      for (int j = 0; j < nx; ++j)
        down_one<FMT, H, I, kSrcLds>(st.w, xpart + (size_t)j * I, st.alpha, nc + j, ob);
      for (int j = nc + nx; j < np; ++j)
        down_one<FMT, H, I, kSrcDevice>(st.w, P.act + (size_t)pr[j] * I, st.alpha, j, ob);
      // y (an output of the call) and the item's share of the sums
      store_results<RW>(rs_o, lane < np ? (uint32_t)((pr[lane] * H + h_base) * 2) : kOOB, ob);
      double *gs = sums + (size_t)lr * P.M * RW;
      for (int l = lane; l < np * RW; l += kWave) {
        const int j = l / RW, r = l % RW, p = pr[j];
        atomicAdd(&gs[(p / k) * RW + r], (double)R.tw[p] * (double)bf16_to_f32(ob[j * RW + r]));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      int c = 0;
      if (lane == 0) c = atomicAdd(&R.done_rg[lr], 1);
      if (__builtin_amdgcn_readfirstlane(c) != U - 1) return;
      // the row group's last item: the combine of its rows for every token
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      combine(lr, h_base);
    };
    St sa;
    int ia = take_item(&R.next_c, 0);
    load(sa, ia);
    TRACE(P, 5);
    while (ia < n_items) {
      __builtin_amdgcn_sched_barrier(0);
      run(sa, ia);
      ia = take_item(&R.next_c, 0);
      load(sa, ia);
    }
    // no routed pairs at all: the rows are the shared output alone
    if (U == 0)
      for (int lr = wv; lr < n_rg; lr += kWaves) {
        wait_lds_at_least(&R.sums_ready, 1, S);
        combine(lr, ((int)blockIdx.x + lr * P.nb) * RW);
      }
  }
  TRACE(P, 7);
  TRACE_FLUSH(P);
}

struct GridInfo {
  int nb = 0;
};

// Decode launches are chained per device: every block of the grid must be
// resident at once (the blocks wait on each other), so two decode grids on
// different streams must not run together.  Each launch carries a stop
// event in its own dispatch (hipExtLaunchKernel: no separate marker between
// back-to-back launches); a launch on a stream other than the previous
// launch's first waits for that event.  Launches on one stream are ordered
// by the stream.
struct LaunchChain {
  std::mutex mu;
  hipEvent_t done = nullptr;
  hipStream_t last = nullptr;
  bool any = false;
};
LaunchChain g_chain[64];  // [device]

// launch_fn(stop_event) queues the kernel with the given stop event.
template <typename F>
hipError_t chained_launch(int dev, hipStream_t st, F &&launch_fn) {
  LaunchChain &c = g_chain[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  hipError_t e;
  if (!c.done && (e = hipEventCreate(&c.done)) != hipSuccess) {
    c.done = nullptr;
    return e;
  }
  if (c.any && c.last != st && (e = hipStreamWaitEvent(st, c.done, 0)) != hipSuccess) return e;
  if ((e = launch_fn(c.done)) != hipSuccess) return e;
  c.last = st;
  c.any = true;
  return hipSuccess;
}

template <int FMT, int SFMT, bool NORM, int H, int I>
hipError_t launch(Params P, hipStream_t st) {
  using Gm = Geo<FMT, SFMT, H, I>;
  static thread_local GridInfo info[64];  // [device]
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  // The staging area holds all of x (small batches), one routing group or a
  // group of shared activations; the per-wave slices follow it.
  const size_t lds = kXLdsBytes + kCacheLdsBytes;
  GridInfo &gi = info[dev];
  if (gi.nb == 0) {
    // Blocks resident at once: the grid (one block per compute unit).
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<FMT, SFMT, NORM, H, I>, kThreads,
                                                     lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    gi.nb = cus * per_cu;
    if (gi.nb > kMaxDecodeBlocks) gi.nb = kMaxDecodeBlocks;
  }
  P.nb = gi.nb;
  // the down row groups of a block and their fp64 sums (in the staging area)
  const int n_rg = (Gm::N_DN + P.nb - 1) / P.nb;
  if (n_rg > kMaxRowGroups || (size_t)n_rg * P.M * Gm::DN::RW * 8 > kXLdsBytes / 2 ||
      n_rg * P.M * Gm::DN::RW > kShPreMax)
    return hipErrorInvalidValue;
  const int nTG = (P.M + kRouteTokens - 1) / kRouteTokens;
  P.n_route = P.ids_in ? 0 : P.E * nTG;  // routing items (expert, token group)
  P.n_sgu = P.sgu ? I / Gm::SGU::RP : 0;  // shared gate/up items (row pairs)
  P.n_sdn = P.sgu ? H / Gm::SDN::RW : 0;  // shared down items
  if (P.nb > kMaxSharedBlocks) return hipErrorInvalidValue;
  return chained_launch(dev, st, [&](hipEvent_t stop) {
    void *args[] = {&P};
    return hipExtLaunchKernel(reinterpret_cast<const void *>(&decode_kernel<FMT, SFMT, NORM, H, I>), dim3(P.nb),
                              dim3(kThreads), args, lds, st, nullptr, stop, 0);
  });
}

__global__ void take_wait_errors_kernel(DecodeSync *sync, int32_t *out) {
  *out = sync->wait_err;
  sync->wait_err = 0;
}

}  // namespace

hipError_t launch_take_wait_errors(DecodeSync *sync, int32_t *out, hipStream_t st) {
  hipLaunchKernelGGL(take_wait_errors_kernel, dim3(1), dim3(1), 0, st, sync, out);
  return hipGetLastError();
}

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
  P.ssgu = a.ssgu;
  P.ssdown = a.ssdown;
  P.asgu = a.asgu;
  P.asdown = a.asdown;
  P.sh_ext = a.sh_ext;
  P.ln_a = a.ln_a;
  P.ln_r = a.ln_r;
  P.ln_w = a.ln_w;
  P.eps = a.eps;
  P.res_out = a.res_out;
  P.xn_out = a.xn_out;
  P.ids_in = a.ids_in;
  P.tw_in = a.tw_in;
  P.logits = a.logits;
  P.tlog = a.tlog;
  P.ids = a.ids;
  P.tw = a.tw;
  P.act = a.act;
  P.y = a.y;
  P.sact = a.sact;
  P.sh = a.sh;
  P.out = a.out;
  P.sync = a.sync;
  P.seq = a.seq;
  P.polls = a.polls > 0 ? a.polls : (1 << 20);
  P.probe = a.probe;
  P.M = a.M;
  P.E = a.E;
  P.top_k = a.top_k;
#ifdef FLINT_TRACE
  P.trace = g_flint_trace;
#endif
#define FLINT_DECODE(HH, II)                                                \
  if (a.H == HH && a.I == II)                                               \
    return fmt == kBf16 ? launch<kBf16, kBf16, false, HH, II>(P, st)                       \
           : a.ln_a    ? (a.ssgu ? launch<kNvfp4, kNvfp4, true, HH, II>(P, st)                \
                                 : launch<kNvfp4, kBf16, true, HH, II>(P, st))                \
           : a.ssgu    ? launch<kNvfp4, kNvfp4, false, HH, II>(P, st)                         \
                       : launch<kNvfp4, kBf16, false, HH, II>(P, st);
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
