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
// Bytes of x the decode kernel stages in each block's LDS (all of x when
// M * H * 2 fits; the fused residual add + RMS norm needs that).
constexpr int kDecodeXStage = 65536;
// Decode kernel grid limits: blocks, routing blocks, and the blocks of its
// shared gate/up and shared down segments.
constexpr int kMaxDecodeBlocks = 1024;
constexpr int kMaxRouteBlocks = 256;
constexpr int kMaxSharedBlocks = 1024;
// Completion flags of the decode kernel.  A flag holds the sequence number
// of the call that set it (every call gets a new one), so flags never need
// resetting.
// Copies of a flag that many blocks poll: a reader polls the copy of its
// own XCD (block id mod 8), so each copy's lines are polled by an eighth of
// the grid instead of all of it.
constexpr int kFlagCopies = 8;

struct DecodeSync {
  int sg[kFlagCopies][kMaxSharedBlocks];  // shared gate/up block done (one copy per XCD)
  int sd[kMaxSharedBlocks];  // shared down block done
  int gb[kFlagCopies][kMaxDecodeBlocks];  // the block's routed gate/up items done (one copy per XCD)
  int db[kMaxDecodeBlocks];  // (unused: kept so the workspace layout does not change)
  int wait_err;              // OR of the kinds of waits that gave up (0 = none)
  int probe;                 // never written: the target of the test hook's wait
};

// The route kernel's arrival counters follow the decode block: token groups
// use indices 0 .. kCtrRouteAll - 1, kCtrRouteAll counts finished groups.
constexpr int kRouteCounterWords = 2048;
constexpr int kCtrRouteAll = kRouteCounterWords - 1;
constexpr size_t kCounterBytes = sizeof(DecodeSync) + sizeof(int) * kRouteCounterWords;

// Arguments of the decode kernel (device pointers).
struct DecodeArgs {
  const uint16_t *x, *router;
  const uint8_t *w13, *s13;
  const float *a13;
  const uint8_t *w2, *s2;
  const float *a2;
  const uint8_t *sgu, *sdown;   // shared expert (bf16, or E2M1 codes), NULL = none
  const uint8_t *ssgu, *ssdown; // NVFP4 shared expert: block scales (NULL: bf16 shared)
  const float *asgu, *asdown;   // NVFP4 shared expert: device global scales
  const uint16_t *sh_ext;       // precomputed shared output [M, H] (then sgu is NULL)
  // residual add + RMS norm formed inside the kernel (NULL ln_a: x given);
  // needs M * H * 2 <= kDecodeXStage
  const uint16_t *ln_a, *ln_r, *ln_w;
  float eps;
  uint16_t *res_out, *xn_out;
  const int32_t *ids_in;        // forced routing, NULL = route
  const float *tw_in;
  uint16_t *logits;
  unsigned long long *tlog;     // [kFlagCopies][M, E] logits tagged with the call's sequence number
  int32_t *ids;
  float *tw;
  uint16_t *act, *y, *sact, *sh, *out;
  DecodeSync *sync;
  int seq;    // call sequence number (never 0; unique per call)
  int polls;  // polls before a device-scope wait gives up (0 = default)
  int probe;  // test hook: non-zero makes one wait give up
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
  unsigned long long *tlog;  // [kFlagCopies][M, E] decode: tagged logits (one copy per XCD)
  int32_t *ids;        // [M, k]
  float *tw;           // [M, k]
  Plan plan;
  uint16_t *act;       // [M*k, I]
  uint16_t *y;         // [M*k, H]
  uint16_t *sact;      // [M, SI]
  uint16_t *sh;        // [M, H]
  int32_t *lists;      // [E, M] grouped pair lists
  int32_t *counts;     // [E]
  int32_t *sh_lists;   // [M] rows 0..M-1: the NVFP4 shared expert's list (E = 1)
  int32_t *sh_counts;  // [1]
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

// The whole decode block in one launch (fmt of the routed experts; the
// shared expert, if any, has SI == I and is bf16, or NVFP4 when a.ssgu is
// set and the routed experts are NVFP4).
hipError_t launch_decode(int fmt, const DecodeArgs &a, hipStream_t st);

// Whether the decode kernel is compiled for this (H, I) (both formats).
bool decode_shape_supported(int H, int I);

// Queues: *out = sync->wait_err, then sync->wait_err = 0.
hipError_t launch_take_wait_errors(DecodeSync *sync, int32_t *out, hipStream_t st);

// Arguments of the grouped (prefill) path: device pointers, caller-owned.
struct GroupedArgs {
  const uint16_t *x, *router;
  const uint8_t *w13, *s13;     // NVFP4 routed experts (NULL with BF16 experts)
  const float *a13;
  const uint8_t *w2, *s2;
  const float *a2;
  const uint16_t *bw13, *bw2;   // BF16 routed experts [E, 2I, H], [E, H, I] (else NULL)
  const uint16_t *sgu, *sdown;  // shared expert (bf16), NULL = none
  const uint16_t *sh_ext;       // precomputed shared output [M, H] (then sgu is NULL), or NULL
  void *sh_ready;               // hipEvent_t completing sh_ext, or NULL
  // NVFP4 shared expert (then sgu / sdown hold E2M1 codes), else NULL
  const uint8_t *s_gu, *s_down;
  const float *a_gu, *a_down;
  int32_t *sh_lists, *sh_counts;  // identity list of the M rows, for the routed kernel with E = 1
  const int32_t *ids_in;        // forced routing, NULL = route
  uint16_t *logits;             // [M, E]
  int32_t *ids;                 // [M, k] (ids_in when forced)
  float *tw;                    // [M, k]
  int32_t *lists;               // [E, M] pair lists
  int32_t *counts;              // [E]
  uint16_t *act, *y, *sact, *sh, *out;
  void **events;                // NULL, or 8 hipEvent_t: recorded before each stage and at the end
  bool inline_shared;           // the shared expert on the caller's stream (no side stream)
  int M, H, E, I, SI, top_k;
};

// Batches up to this many tokens run the expert GEMMs on the skinny kernels.
constexpr int kSkinnyMaxM = 64;

// Expert GEMMs with few rows per expert (skinny.hip): what one launch
// computes (device pointers).
struct SkinnyArgs {
  const uint16_t *a;      // A rows [a_rows, K] bf16
  const uint8_t *w;       // weights [E][wrows][K] bf16, or E2M1 codes [E][wrows][K / 2]
  const uint8_t *ws;      // E4M3 block scales [E][wrows][K / 16] (NVFP4), else NULL
  const float *alpha;     // per-expert global scales [E] (NVFP4), else NULL
  uint16_t *c;            // output rows [c_rows, ldc]
  const int32_t *ids;     // routed: expert ids [nrows * top_k] (pair p = t * top_k + j); NULL:
                          // one expert whose rows are 0 .. nrows - 1
  int top_k;
  int nrows;              // tokens
  int a_rows, c_rows;     // extents of A and C (rows)
  int K, wrows;           // reduction length; weight rows per expert
  int ncols, ldc, I;      // output columns; output row length; gate/up: offset of the up rows
  int E;
};

// gate_up: c[row, n] = bf16(swiglu(alpha a . W[n], alpha a . W[I + n])), n < ncols;
// else c[row, h] = bf16(alpha a . W[h]).  Routed: the rows of expert e are
// its pairs p, with A row p / top_k (gate/up) or p (down) and output row p;
// nrows * top_k <= 512.  One launch computes the routed GEMM r (weights in
// format wfmt_r: kNvfp4 or kBf16) and, if sh is non-NULL, the dense GEMM sh
// (the shared expert: ids NULL, format wfmt_s) with it.
hipError_t launch_skinny(const SkinnyArgs &r, int wfmt_r, const SkinnyArgs *sh, int wfmt_s, bool gate_up,
                         hipStream_t st);
bool skinny_shape_supported(int K, int ncols, bool gate_up);

// The MoE block with grouped MFMA GEMMs (any M >= 1).
hipError_t launch_grouped(const GroupedArgs &a, hipStream_t st);

// Whether the grouped kernels handle these sizes.
bool grouped_shape_supported(int H, int I, int SI);

// Residual add + RMS norm rows (norm.hip): res_out = bf16(a + r), xn_out =
// bf16((s * rsqrt(mean(s^2) + eps)) * w) for M rows of H.
bool add_rmsnorm_supported(int H);
hipError_t launch_add_rmsnorm(const uint16_t *a, const uint16_t *r, const uint16_t *w, float eps, int M,
                              int H, uint16_t *res_out, uint16_t *xn_out, hipStream_t st);

}  // namespace flint
