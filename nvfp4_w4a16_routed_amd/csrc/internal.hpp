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
constexpr int kMaxDecodePairs = 1024;
constexpr int kMaxExperts = 256;
constexpr int kMaxDecodeM = 64;
// Counter words at the start of the workspace.
constexpr int kCounterWords = 4096;
// Counter index of the route kernel's all-groups counter.
constexpr int kCtrRouteAll = kCounterWords - 1;

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
  int32_t *counters;   // [kCounterWords], zero between calls
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

// Gate/up + SwiGLU of every routed pair (decode), or of the shared expert
// (plan == NULL: one job covering tokens 0..M-1, weights w13 of one expert).
hipError_t launch_gate_up(int fmt, const uint16_t *x, const void *w13, const uint8_t *s13,
                          const float *a13, int M, int H, int I, int top_k, int max_slots,
                          const Plan *plan, uint16_t *act, hipStream_t st);

hipError_t launch_down(int fmt, const uint16_t *act, const void *w2, const uint8_t *s2,
                       const float *a2, int M, int H, int I, int top_k, int max_slots,
                       const Plan *plan, uint16_t *y, hipStream_t st);

hipError_t launch_combine(const uint16_t *y, const float *tw, const uint16_t *sh, int M,
                          int H, int top_k, uint16_t *out, hipStream_t st);

// Whether the decode kernels are compiled for this (H, I).
bool decode_shape_supported(int H, int I);

}  // namespace flint
