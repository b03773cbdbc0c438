// Host-side internals of libflint_moe: workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flint {

enum WeightFmt { kNvfp4 = 0, kBf16 = 1 };

// Route kernel geometry: 8 tokens per token group, 4 experts per workgroup.
constexpr int kRouteTokens = 8;
constexpr int kRouteExperts = 4;
// Decode plan limits: pairs (M * top_k) per call and experts.
constexpr int kMaxDecodePairs = 512;
constexpr int kMaxExperts = 256;
constexpr int kMaxDecodeM = 64;
// Largest grid of the fused decode kernel (blocks).
constexpr int kMaxDecodeBlocks = 2048;
// Fan-in of the first level of the decode kernel's phase barrier.
constexpr int kBarrierGroups = 32;
// Synchronisation words of the fused decode kernel, each counter on its own
// 128-byte line.  They are zero between calls: every counter is reset by
// its last arrival or its single consumer.
constexpr int kLine = 32;  // ints per 128-byte line
struct DecodeSync {
  int route_cnt[kMaxDecodeM][kLine];  // routing items done, per token
  int topk_done[kLine];               // tokens whose top-k is done
  uint32_t active[kLine];             // touched-expert bitmask (words 0..7)
  int rb_cnt[512][kLine];             // down items done, per combine row block
  int grp_cnt[kBarrierGroups][kLine]; // blocks done with the gate/up phase, per group
  int top_cnt[kLine];                 // groups done with the gate/up phase
  int go[kMaxDecodeBlocks][kLine];    // per-block phase flag (1: routed, 2: gate/up done)
};

// The route kernel's arrival counters follow the decode block: token groups
// use indices 0 .. kCtrRouteAll - 1, kCtrRouteAll counts finished groups.
constexpr int kRouteCounterWords = 2048;
constexpr int kCtrRouteAll = kRouteCounterWords - 1;
constexpr size_t kCounterBytes = sizeof(DecodeSync) + sizeof(int) * kRouteCounterWords;

// Arguments of the fused decode kernel (device pointers).
struct DecodeArgs {
  const uint16_t *x, *router;
  const uint8_t *w13, *s13;
  const float *a13;
  const uint8_t *w2, *s2;
  const float *a2;
  const uint8_t *sgu, *sdown;   // shared expert (bf16), NULL = none
  const int32_t *ids_in;        // forced routing, NULL = route
  const float *tw_in;
  uint16_t *logits;
  int32_t *ids;
  float *tw;
  uint16_t *act, *y, *sact, *sh, *out;
  DecodeSync *sync;
  int M, H, E, I, top_k;
};

// Routing plan of one call (device pointers into the workspace):
//   n_active    number of experts used by at least one pair
//   active[s]   expert id of slot s (ascending), s < n_active
//   offs[s]     first index in `pairs` of slot s; offs[n_active] = M * top_k
//   pairs[...]  pair indices p = t * top_k + j, ascending within a slot
struct Plan {
  int32_t *n_active;
  int32_t *active;
  int32_t *offs;
  int32_t *pairs;
};

// Device buffers a call needs, carved out of the caller's workspace.
struct Workspace {
  DecodeSync *sync;         // zero between calls
  int32_t *route_counters;  // [kRouteCounterWords], zero between calls
  uint16_t *logits;    // [M, E]
  int32_t *ids;        // [M, k]
  float *tw;           // [M, k]
  Plan plan;
  uint16_t *act;       // [M*k, I]
  uint16_t *y;         // [M*k, H]
  uint16_t *sact;      // [M, SI]
  uint16_t *sh;        // [M, H]
  size_t bytes;        // total bytes used
};

// Lays the workspace out for the given sizes; base may be NULL to size it.
Workspace carve_workspace(void *base, int M, int H, int E, int I, int SI, int top_k);

// ---- launchers (each returns the hipError_t of its launch) ----

hipError_t launch_dequant(const uint8_t *w, const uint8_t *s, int rows, int K,
                          uint16_t *out, hipStream_t st);

hipError_t launch_topk(const uint16_t *logits, int M, int E, int top_k, int32_t *ids,
                       float *tw, float *scores, hipStream_t st);

// Router logits + top-k (+ routing plan when `plan` is non-NULL).
hipError_t launch_route(const uint16_t *x, const uint16_t *router, int M, int H, int E,
                        int top_k, uint16_t *logits, int32_t *ids, float *tw,
                        int32_t *counters, const Plan *plan, hipStream_t st);

// Routing plan from given ids (forced routing).
hipError_t launch_plan(const int32_t *ids, int M, int E, int top_k, const Plan &plan,
                       hipStream_t st);

// The whole decode block in one cooperative launch (fmt of the routed
// experts; the shared expert, if any, is bf16 with SI == I).
hipError_t launch_decode_fused(int fmt, const DecodeArgs &a, hipStream_t st);

// Whether the decode kernel is compiled for this (H, I) (both formats).
bool decode_shape_supported(int H, int I);

}  // namespace flint
