// C ABI of libflint_moe: argument validation, workspace layout, dispatch.
// Everything here runs on the host; kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/flint_moe.h"
#include "internal.hpp"

namespace flint {

static thread_local int g_last_hip_error = 0;

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return FLINT_OK;
  g_last_hip_error = (int)e;
  return FLINT_ERR_HIP;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Sequence numbers of decode calls: unique per call (1 .. 2^31 - 1, then
// around again), so completion flags left by earlier calls never match.
static std::atomic<uint32_t> g_seq{0};
static int next_seq() {
  for (;;) {
    const uint32_t v = (g_seq.fetch_add(1, std::memory_order_relaxed) + 1u) & 0x7fffffffu;
    if (v != 0) return (int)v;
  }
}

Workspace carve_workspace(void *base, int M, int H, int E, int I, int SI, int top_k) {
  Workspace w{};
  size_t off = 0;
  char *b = static_cast<char *>(base);
  auto take = [&](size_t bytes) -> void * {
    void *p = b ? b + off : nullptr;
    off = align_up(off + bytes, 256);
    return p;
  };
  const size_t P = (size_t)M * top_k;
  w.sync = static_cast<DecodeSync *>(take(sizeof(DecodeSync)));
  w.route_counters = static_cast<int32_t *>(take(sizeof(int32_t) * kRouteCounterWords));
  w.logits = static_cast<uint16_t *>(take(2 * (size_t)M * E));
  w.tlog = static_cast<unsigned long long *>(take(8 * (size_t)kFlagCopies * M * E));
  w.ids = static_cast<int32_t *>(take(4 * P));
  w.tw = static_cast<float *>(take(4 * P));
  w.plan.n_active = static_cast<int32_t *>(take(16));
  w.plan.active = static_cast<int32_t *>(take(4 * (size_t)E));
  w.plan.offs = static_cast<int32_t *>(take(4 * ((size_t)E + 1)));
  w.plan.pairs = static_cast<int32_t *>(take(4 * P));
  w.act = static_cast<uint16_t *>(take(2 * P * I));
  w.y = static_cast<uint16_t *>(take(2 * P * H));
  w.sact = static_cast<uint16_t *>(take(2 * (size_t)M * (SI > 0 ? SI : 0)));
  w.sh = static_cast<uint16_t *>(take(2 * (size_t)M * H));
  w.lists = static_cast<int32_t *>(take(4 * (size_t)E * M));
  w.counts = static_cast<int32_t *>(take(4 * (size_t)E));
  w.sh_lists = static_cast<int32_t *>(take(4 * (size_t)M));
  w.sh_counts = static_cast<int32_t *>(take(16));
  w.bytes = off;
  return w;
}

// ---- The library's own scratch for flint_moe_decode_noalloc.
//
// A file-scope device array: each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels.  kScratchBytes covers the largest decode workspace the
// decode entry points accept (M <= 64, M * top_k <= 512, E <= 256, H <= 2048,
// I = SI <= 768: 4.28 MiB at M = 64, top_k = 8, E = 256, of which y is
// 2 MiB and the eight copies of the tagged logits 1 MiB).
constexpr size_t kScratchBytes = size_t(5) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
static void *g_scratch_ptr[kMaxScratchDevices];
static std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on first use).
static hipError_t scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace flint

using namespace flint;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool route_h_ok(int H) { return H == 256 || H == 512 || H == 1024 || H == 2048 || H == 4096; }

int check_common(int M, int H, int E, int I, int top_k) {
  if (M < 0 || H <= 0 || E <= 0 || I <= 0) return FLINT_ERR_SHAPE;
  if (top_k < 1 || top_k > E || E > kMaxExperts) return FLINT_ERR_SHAPE;
  if ((long)M * top_k > (long)kMaxDecodePairs) return FLINT_ERR_SHAPE;
  if (M > kMaxDecodeM) return FLINT_ERR_SHAPE;
  if (!decode_shape_supported(H, I)) return FLINT_ERR_SHAPE;
  return FLINT_OK;
}

// The decode entry points' shared expert: none, a precomputed output, a
// bf16 expert, or (allow_nvfp4: NVFP4 routed experts) an NVFP4 expert.
int check_shared(const flint_shared_expert *sh, int H, int I, bool allow_nvfp4) {
  if (sh && sh->sh_in) return aligned16(sh->sh_in) ? FLINT_OK : FLINT_ERR_ALIGN;
  if (!sh || !sh->w_gu) return FLINT_OK;
  if (sh->s_gu && !allow_nvfp4) return FLINT_ERR_SHAPE;
  if (!sh->w_down) return FLINT_ERR_NULL;
  if (sh->s_gu && (!sh->s_down || !sh->a_gu || !sh->a_down)) return FLINT_ERR_NULL;
  if (!aligned16(sh->w_gu) || !aligned16(sh->w_down)) return FLINT_ERR_ALIGN;
  if (sh->s_gu && (!aligned16(sh->s_gu) || !aligned16(sh->s_down) ||
                   (reinterpret_cast<uintptr_t>(sh->a_gu) & 3u) ||
                   (reinterpret_cast<uintptr_t>(sh->a_down) & 3u)))
    return FLINT_ERR_ALIGN;
  if (!decode_shape_supported(H, sh->SI)) return FLINT_ERR_SHAPE;
  if (sh->SI != I) return FLINT_ERR_SHAPE;  // the decode kernel's shared expert is I wide
  return FLINT_OK;
}

// Inputs and outputs of the residual add + RMS norm formed inside the
// decode kernel (flint_moe_ll).
struct NormIn {
  const uint16_t *a, *r, *w;
  float eps;
  uint16_t *res, *xn;
};

int run_grouped(GroupedArgs a, bool have_w, const uint16_t *x, const uint16_t *router,
                const flint_shared_expert *shared, int M, int H, int E, int I, int top_k,
                uint16_t *out, const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                void *stream);

// The decode kernel runs batches up to this many tokens; larger ones run
// the chain of the grouped path with its skinny expert GEMMs (at that size
// each expert's weights serve many tokens, which the decode kernel's
// per-token dot products cannot reuse).
constexpr int kDecodeKernelMaxM = 16;

// The decode pipeline shared by the NVFP4 and BF16 experts (norm: the
// residual add + RMS norm in front, formed inside the kernel; x is then
// norm->xn, written by the kernel).
int run_decode(int fmt, const uint16_t *x, const uint16_t *router, const void *w13,
               const uint8_t *s13, const float *a13, const void *w2, const uint8_t *s2,
               const float *a2, const flint_shared_expert *shared, int M, int H, int E, int I,
               int top_k, uint16_t *out, const flint_moe_debug *dbg, void *ws,
               size_t ws_bytes, hipStream_t st, const NormIn *norm = nullptr,
               bool no_side_stream = false) {
  const bool ext_sh = shared && shared->sh_in;  // precomputed shared output
  const bool has_shared = !ext_sh && shared && shared->w_gu;
  const int SI = has_shared ? shared->SI : 0;
  Workspace W = carve_workspace(ws, M, H, E, I, SI, top_k);
  if (W.bytes > ws_bytes) return FLINT_ERR_WORKSPACE;
  if (M == 0) return FLINT_OK;
  if (M > kDecodeKernelMaxM && !norm && grouped_shape_supported(H, I, SI)) {
    GroupedArgs ga{};
    if (fmt == kNvfp4) {
      ga.w13 = static_cast<const uint8_t *>(w13);
      ga.s13 = s13;
      ga.a13 = a13;
      ga.w2 = static_cast<const uint8_t *>(w2);
      ga.s2 = s2;
      ga.a2 = a2;
    } else {
      ga.bw13 = static_cast<const uint16_t *>(w13);
      ga.bw2 = static_cast<const uint16_t *>(w2);
    }
    ga.inline_shared = no_side_stream;
    return run_grouped(ga, true, x, router, shared, M, H, E, I, top_k, out, dbg, ws, ws_bytes, st);
  }

  const bool forced = dbg && dbg->ids_in;
  uint16_t *logits = (dbg && dbg->logits_out) ? dbg->logits_out : W.logits;
  int32_t *ids = (dbg && dbg->ids_out) ? dbg->ids_out : W.ids;
  float *tw = (dbg && dbg->tw_out) ? dbg->tw_out : W.tw;
  uint16_t *act = (dbg && dbg->act_out) ? dbg->act_out : W.act;
  uint16_t *y = (dbg && dbg->y_out) ? dbg->y_out : W.y;
  uint16_t *sact = (dbg && dbg->sact_out) ? dbg->sact_out : W.sact;
  uint16_t *sh = (dbg && dbg->sh_out) ? dbg->sh_out : W.sh;
  void **ev = dbg ? dbg->stage_events : nullptr;
  auto mark = [&](int i) -> hipError_t {
    return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
  };
  DecodeArgs a{};
  a.x = x;
  a.router = router;
  a.w13 = static_cast<const uint8_t *>(w13);
  a.s13 = s13;
  a.a13 = a13;
  a.w2 = static_cast<const uint8_t *>(w2);
  a.s2 = s2;
  a.a2 = a2;
  a.sgu = has_shared ? reinterpret_cast<const uint8_t *>(shared->w_gu) : nullptr;
  a.sdown = has_shared ? reinterpret_cast<const uint8_t *>(shared->w_down) : nullptr;
  const bool nv_sh = has_shared && shared->s_gu;
  a.ssgu = nv_sh ? shared->s_gu : nullptr;
  a.ssdown = nv_sh ? shared->s_down : nullptr;
  a.asgu = nv_sh ? shared->a_gu : nullptr;
  a.asdown = nv_sh ? shared->a_down : nullptr;
  a.sh_ext = ext_sh ? shared->sh_in : nullptr;
  if (norm) {
    a.ln_a = norm->a;
    a.ln_r = norm->r;
    a.ln_w = norm->w;
    a.eps = norm->eps;
    a.res_out = norm->res;
    a.xn_out = norm->xn;
  }
  a.ids_in = forced ? dbg->ids_in : nullptr;
  a.tw_in = forced ? dbg->tw_in : nullptr;
  a.logits = logits;
  a.tlog = W.tlog;
  a.ids = forced && !(dbg->ids_out) ? const_cast<int32_t *>(dbg->ids_in) : ids;
  a.tw = forced && !(dbg->tw_out) ? const_cast<float *>(dbg->tw_in) : tw;
  a.act = act;
  a.y = y;
  a.sact = sact;
  a.sh = sh;
  a.out = out;
  a.sync = W.sync;
  a.seq = next_seq();
  a.polls = dbg ? dbg->wait_polls : 0;
  a.probe = dbg ? dbg->wait_probe : 0;
  a.M = M;
  a.H = H;
  a.E = E;
  a.I = I;
  a.top_k = top_k;
  // A precomputed shared output is read by the kernel's combine: the stream
  // waits for its event before the launch (every block of the decode grid
  // must be resident, so the kernel could not overlap its producer anyway).
  hipError_t e = hipSuccess;
  if (ext_sh && shared->sh_ready) e = hipStreamWaitEvent(st, (hipEvent_t)shared->sh_ready, 0);
  // One kernel runs every stage: the stage events bracket the whole of it.
  if (e == hipSuccess) e = mark(0);
  if (e == hipSuccess) e = launch_decode(fmt, a, st);
  for (int i = 1; i < FLINT_STAGE_EVENTS && e == hipSuccess; ++i) e = mark(i);
  return hip_status(e);
}

// The grouped pipeline shared by the NVFP4 and BF16 experts: a holds the
// expert weights (checked by the caller); everything else is checked here.
int run_grouped(GroupedArgs a, bool have_w, const uint16_t *x, const uint16_t *router,
                const flint_shared_expert *shared, int M, int H, int E, int I, int top_k,
                uint16_t *out, const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                void *stream) {
  const bool forced = dbg && dbg->ids_in;
  const bool ext_sh = shared && shared->sh_in;  // precomputed shared output
  const bool has_shared = !ext_sh && shared && shared->w_gu;
  const int SI = has_shared ? shared->SI : 0;
  if (M < 0 || top_k < 1 || E < 1 || top_k > E || E > kMaxExperts) return FLINT_ERR_SHAPE;
  if (!grouped_shape_supported(H, I, SI)) return FLINT_ERR_SHAPE;
  if (has_shared && SI < 64) return FLINT_ERR_SHAPE;  // a shared expert has a width
  // x, act and sact are read through buffer descriptors (byte offsets below
  // 2^31)
  const long long kDesc = 1ll << 31;
  if ((long long)M * H * 2 >= kDesc || (long long)M * top_k * I * 2 >= kDesc ||
      (long long)M * SI * 2 >= kDesc)
    return FLINT_ERR_SHAPE;
  if (M == 0) return FLINT_OK;  // nothing to compute; no pointer is used
  if (!x || !have_w || !out || (!forced && !router)) return FLINT_ERR_NULL;
  if (forced && !dbg->tw_in) return FLINT_ERR_NULL;
  if (has_shared && !shared->w_down) return FLINT_ERR_NULL;
  const bool nv_sh = has_shared && shared->s_gu;
  if (nv_sh && (!shared->s_down || !shared->a_gu || !shared->a_down)) return FLINT_ERR_NULL;
  if (nv_sh && (!aligned16(shared->s_gu) || !aligned16(shared->s_down) || !aligned16(shared->a_gu) ||
                !aligned16(shared->a_down)))
    return FLINT_ERR_ALIGN;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if (!aligned16(x) || (router && !aligned16(router)) || !aligned16(out) || !aligned16(ws) ||
      (has_shared && (!aligned16(shared->w_gu) || !aligned16(shared->w_down))) ||
      (ext_sh && !aligned16(shared->sh_in)))
    return FLINT_ERR_ALIGN;
  Workspace W = carve_workspace(ws, M, H, E, I, SI, top_k);
  if (W.bytes > ws_bytes) return FLINT_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  a.x = x;
  a.router = router;
  a.sgu = has_shared ? shared->w_gu : nullptr;
  a.sdown = has_shared ? shared->w_down : nullptr;
  a.sh_ext = ext_sh ? shared->sh_in : nullptr;
  a.sh_ready = ext_sh ? shared->sh_ready : nullptr;
  a.s_gu = nv_sh ? shared->s_gu : nullptr;
  a.s_down = nv_sh ? shared->s_down : nullptr;
  a.a_gu = nv_sh ? shared->a_gu : nullptr;
  a.a_down = nv_sh ? shared->a_down : nullptr;
  a.sh_lists = W.sh_lists;
  a.sh_counts = W.sh_counts;
  a.ids_in = forced ? dbg->ids_in : nullptr;
  a.logits = (dbg && dbg->logits_out) ? dbg->logits_out : W.logits;
  int32_t *ids = (dbg && dbg->ids_out) ? dbg->ids_out : W.ids;
  float *tw = (dbg && dbg->tw_out) ? dbg->tw_out : W.tw;
  if (forced) {
    // the given routing, copied where the outputs were asked for
    const size_t P = (size_t)M * top_k;
    if (dbg->ids_out) {
      hipError_t e = hipMemcpyAsync(ids, dbg->ids_in, 4 * P, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_status(e);
    } else {
      ids = const_cast<int32_t *>(dbg->ids_in);
    }
    if (dbg->tw_out) {
      hipError_t e = hipMemcpyAsync(tw, dbg->tw_in, 4 * P, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_status(e);
    } else {
      tw = const_cast<float *>(dbg->tw_in);
    }
  }
  a.ids = ids;
  a.tw = tw;
  a.lists = W.lists;
  a.counts = W.counts;
  a.act = (dbg && dbg->act_out) ? dbg->act_out : W.act;
  a.y = (dbg && dbg->y_out) ? dbg->y_out : W.y;
  a.sact = (dbg && dbg->sact_out) ? dbg->sact_out : W.sact;
  a.sh = (dbg && dbg->sh_out) ? dbg->sh_out : W.sh;
  a.out = out;
  a.events = dbg ? dbg->stage_events : nullptr;
  a.M = M;
  a.H = H;
  a.E = E;
  a.I = I;
  a.SI = SI;
  a.top_k = top_k;
  return hip_status(launch_grouped(a, st));
}

}  // namespace

extern "C" {

const char *flint_status_str(int status) {
  switch (status) {
    case FLINT_OK: return "ok";
    case FLINT_ERR_NULL: return "a required pointer is NULL";
    case FLINT_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case FLINT_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case FLINT_ERR_WORKSPACE: return "workspace missing or too small";
    case FLINT_ERR_HIP: return "a HIP call failed";
    default: return "unknown status";
  }
}

int flint_last_hip_error(void) { return g_last_hip_error; }

int flint_moe_workspace_bytes(int max_M, int H, int E, int I, int SI, int top_k, size_t *bytes) {
  if (!bytes) return FLINT_ERR_NULL;
  if (max_M < 0 || H <= 0 || E <= 0 || I <= 0 || SI < 0 || top_k < 1 || top_k > E ||
      E > kMaxExperts)
    return FLINT_ERR_SHAPE;
  *bytes = carve_workspace(nullptr, max_M, H, E, I, SI, top_k).bytes;
  return FLINT_OK;
}

int flint_moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws) return FLINT_ERR_NULL;
  if (!aligned16(ws)) return FLINT_ERR_ALIGN;
  if (ws_bytes < kCounterBytes) return FLINT_ERR_WORKSPACE;
  return hip_status(hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream));
}

int flint_moe_wait_errors(void *ws, size_t ws_bytes, int32_t *errors, void *stream) {
  if (!errors) return FLINT_ERR_NULL;
  if (!ws) {  // the library's own scratch (flint_moe_decode_noalloc)
    if (reinterpret_cast<uintptr_t>(errors) & 3u) return FLINT_ERR_ALIGN;
    void *p = nullptr;
    if (hipError_t e = scratch_ptr(&p); e != hipSuccess) return hip_status(e);
    return hip_status(launch_take_wait_errors(static_cast<DecodeSync *>(p), errors,
                                              (hipStream_t)stream));
  }
  if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(errors) & 3u)) return FLINT_ERR_ALIGN;
  if (ws_bytes < sizeof(DecodeSync)) return FLINT_ERR_WORKSPACE;
  return hip_status(launch_take_wait_errors(static_cast<DecodeSync *>(ws), errors,
                                            (hipStream_t)stream));
}

int flint_nvfp4_dequant(const uint8_t *w, const uint8_t *s, int rows, int K, uint16_t *out,
                        void *stream) {
  if (rows < 0 || K <= 0 || K % 32) return FLINT_ERR_SHAPE;
  if (rows == 0) return FLINT_OK;
  if (!w || !s || !out) return FLINT_ERR_NULL;
  if (!aligned16(w) || !aligned16(s) || !aligned16(out)) return FLINT_ERR_ALIGN;
  return hip_status(launch_dequant(w, s, rows, K, out, (hipStream_t)stream));
}

int flint_moe_topk(const uint16_t *logits, int M, int E, int top_k, int32_t *ids, float *tw,
                   float *scores, void *stream) {
  if (M < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > E) return FLINT_ERR_SHAPE;
  if (M == 0) return FLINT_OK;
  if (!logits || !ids || !tw) return FLINT_ERR_NULL;
  if (!aligned16(logits) || !aligned16(ids) || !aligned16(tw) || (scores && !aligned16(scores)))
    return FLINT_ERR_ALIGN;
  return hip_status(launch_topk(logits, M, E, top_k, ids, tw, scores, (hipStream_t)stream));
}

int flint_moe_route(const uint16_t *x, const uint16_t *router, int M, int H, int E, int top_k,
                    uint16_t *logits, int32_t *ids, float *tw, void *ws, size_t ws_bytes,
                    void *stream) {
  if (M < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > E || !route_h_ok(H) ||
      M > kCtrRouteAll * kRouteTokens)
    return FLINT_ERR_SHAPE;
  if (M == 0) return FLINT_OK;
  if (!x || !router || !ids || !tw) return FLINT_ERR_NULL;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(router) || !aligned16(ids) || !aligned16(tw) ||
      (logits && !aligned16(logits)) || !aligned16(ws))
    return FLINT_ERR_ALIGN;
  Workspace W = carve_workspace(ws, M, H, E, 1, 0, top_k);
  if (W.bytes > ws_bytes) return FLINT_ERR_WORKSPACE;
  if (M == 0) return FLINT_OK;
  return hip_status(launch_route(x, router, M, H, E, top_k, logits ? logits : W.logits, ids, tw,
                                 W.route_counters, nullptr, (hipStream_t)stream));
}

int flint_moe_decode(const uint16_t *x, const uint16_t *router, const flint_nvfp4_experts *w,
                     const flint_shared_expert *shared, int M, int H, int E, int I, int top_k,
                     uint16_t *out, const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                     void *stream) {
  const bool forced = dbg && dbg->ids_in;
  int st = check_common(M, H, E, I, top_k);
  if (st) return st;
  if (M == 0) return FLINT_OK;  // nothing to compute; no pointer is used
  if (!x || !w || !out || (!forced && !router)) return FLINT_ERR_NULL;
  if (!w->w13 || !w->s13 || !w->a13 || !w->w2 || !w->s2 || !w->a2) return FLINT_ERR_NULL;
  if (forced && !dbg->tw_in) return FLINT_ERR_NULL;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if ((st = check_shared(shared, H, I, true))) return st;
  if (!aligned16(x) || (router && !aligned16(router)) || !aligned16(out) || !aligned16(ws) ||
      !aligned16(w->w13) || !aligned16(w->s13) || !aligned16(w->a13) || !aligned16(w->w2) ||
      !aligned16(w->s2) || !aligned16(w->a2))
    return FLINT_ERR_ALIGN;
  return run_decode(kNvfp4, x, router, w->w13, w->s13, w->a13, w->w2, w->s2, w->a2, shared, M,
                    H, E, I, top_k, out, dbg, ws, ws_bytes, (hipStream_t)stream);
}

int flint_moe_decode_noalloc(const uint16_t *x, const uint16_t *router,
                             const flint_nvfp4_experts *w, const flint_shared_expert *shared,
                             int M, int H, int E, int I, int top_k, uint16_t *out,
                             const flint_moe_debug *dbg, void *stream) {
  // Every argument check of flint_moe_decode, then the library's scratch in
  // place of a caller workspace (too small for these sizes: FLINT_ERR_WORKSPACE).
  const bool forced = dbg && dbg->ids_in;
  int st = check_common(M, H, E, I, top_k);
  if (st) return st;
  if (M == 0) return FLINT_OK;
  if (!x || !w || !out || (!forced && !router)) return FLINT_ERR_NULL;
  if (!w->w13 || !w->s13 || !w->a13 || !w->w2 || !w->s2 || !w->a2) return FLINT_ERR_NULL;
  if (forced && !dbg->tw_in) return FLINT_ERR_NULL;
  if ((st = check_shared(shared, H, I, true))) return st;
  if (!aligned16(x) || (router && !aligned16(router)) || !aligned16(out) || !aligned16(w->w13) ||
      !aligned16(w->s13) || !aligned16(w->a13) || !aligned16(w->w2) || !aligned16(w->s2) ||
      !aligned16(w->a2))
    return FLINT_ERR_ALIGN;
  const bool has_shared = shared && !shared->sh_in && shared->w_gu;
  if (carve_workspace(nullptr, M, H, E, I, has_shared ? shared->SI : 0, top_k).bytes > kScratchBytes)
    return FLINT_ERR_WORKSPACE;
  void *ws = nullptr;
  if (hipError_t e = scratch_ptr(&ws); e != hipSuccess) return hip_status(e);
  return run_decode(kNvfp4, x, router, w->w13, w->s13, w->a13, w->w2, w->s2, w->a2, shared, M,
                    H, E, I, top_k, out, dbg, ws, kScratchBytes, (hipStream_t)stream, nullptr,
                    /*no_side_stream=*/true);
}

int flint_moe_ll(const uint16_t *attn_out, const uint16_t *residual, const uint16_t *ln_weight,
                 float eps, const uint16_t *router, const flint_nvfp4_experts *w,
                 const flint_shared_expert *shared, int M, int H, int E, int I, int top_k,
                 uint16_t *out, uint16_t *residual_out, uint16_t *xn_out,
                 const flint_moe_debug *dbg, void *ws, size_t ws_bytes, void *stream) {
  int st = check_common(M, H, E, I, top_k);
  if (st) return st;
  if (!add_rmsnorm_supported(H) || !(eps >= 0.0f) || eps > 3.0e38f) return FLINT_ERR_SHAPE;
  if (M == 0) return FLINT_OK;  // nothing to compute; no pointer is used
  if (!attn_out || !residual || !ln_weight || !residual_out || !xn_out) return FLINT_ERR_NULL;
  if (!aligned16(attn_out) || !aligned16(residual) || !aligned16(ln_weight) ||
      !aligned16(residual_out) || !aligned16(xn_out))
    return FLINT_ERR_ALIGN;
  // flint_moe_decode's own checks, before anything is queued
  const bool forced = dbg && dbg->ids_in;
  if (!w || !out || (!forced && !router)) return FLINT_ERR_NULL;
  if (!w->w13 || !w->s13 || !w->a13 || !w->w2 || !w->s2 || !w->a2) return FLINT_ERR_NULL;
  if (forced && !dbg->tw_in) return FLINT_ERR_NULL;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if ((st = check_shared(shared, H, I, true))) return st;
  if (carve_workspace(nullptr, M, H, E, I, shared && shared->w_gu ? shared->SI : 0, top_k).bytes > ws_bytes)
    return FLINT_ERR_WORKSPACE;
  if ((router && !aligned16(router)) || !aligned16(out) || !aligned16(ws) || !aligned16(w->w13) ||
      !aligned16(w->s13) || !aligned16(w->a13) || !aligned16(w->w2) || !aligned16(w->s2) ||
      !aligned16(w->a2))
    return FLINT_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if ((long)M * H * 2 <= kDecodeXStage && M <= kDecodeKernelMaxM) {
    // every block of the decode kernel forms the normed rows itself (they
    // fit its LDS): one launch
    const NormIn norm{attn_out, residual, ln_weight, eps, residual_out, xn_out};
    return run_decode(kNvfp4, xn_out, router, w->w13, w->s13, w->a13, w->w2, w->s2, w->a2, shared,
                      M, H, E, I, top_k, out, dbg, ws, ws_bytes, s, &norm);
  }
  if (hipError_t e = launch_add_rmsnorm(attn_out, residual, ln_weight, eps, M, H, residual_out, xn_out, s);
      e != hipSuccess)
    return hip_status(e);
  return flint_moe_decode(xn_out, router, w, shared, M, H, E, I, top_k, out, dbg, ws, ws_bytes, stream);
}

int flint_moe_bf16_decode(const uint16_t *x, const uint16_t *router, const flint_bf16_experts *w,
                          const flint_shared_expert *shared, int M, int H, int E, int I,
                          int top_k, uint16_t *out, const flint_moe_debug *dbg, void *ws,
                          size_t ws_bytes, void *stream) {
  const bool forced = dbg && dbg->ids_in;
  int st = check_common(M, H, E, I, top_k);
  if (st) return st;
  if (M == 0) return FLINT_OK;  // nothing to compute; no pointer is used
  if (!x || !w || !out || (!forced && !router)) return FLINT_ERR_NULL;
  if (!w->w13 || !w->w2) return FLINT_ERR_NULL;
  if (forced && !dbg->tw_in) return FLINT_ERR_NULL;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if ((st = check_shared(shared, H, I, false))) return st;  // NVFP4 shared: NVFP4 experts only
  if (!aligned16(x) || (router && !aligned16(router)) || !aligned16(out) || !aligned16(ws) ||
      !aligned16(w->w13) || !aligned16(w->w2))
    return FLINT_ERR_ALIGN;
  return run_decode(kBf16, x, router, w->w13, nullptr, nullptr, w->w2, nullptr, nullptr, shared,
                    M, H, E, I, top_k, out, dbg, ws, ws_bytes, (hipStream_t)stream);
}

int flint_moe_grouped(const uint16_t *x, const uint16_t *router, const flint_nvfp4_experts *w,
                      const flint_shared_expert *shared, int M, int H, int E, int I, int top_k,
                      uint16_t *out, const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                      void *stream) {
  if (M > 0 && w && (!w->w13 || !w->s13 || !w->a13 || !w->w2 || !w->s2 || !w->a2))
    return FLINT_ERR_NULL;
  if (M > 0 && w && (!aligned16(w->w13) || !aligned16(w->s13) || !aligned16(w->a13) ||
                     !aligned16(w->w2) || !aligned16(w->s2) || !aligned16(w->a2)))
    return FLINT_ERR_ALIGN;
  GroupedArgs a{};
  if (w) {
    a.w13 = w->w13;
    a.s13 = w->s13;
    a.a13 = w->a13;
    a.w2 = w->w2;
    a.s2 = w->s2;
    a.a2 = w->a2;
  }
  return run_grouped(a, w != nullptr, x, router, shared, M, H, E, I, top_k, out, dbg, ws, ws_bytes,
                     stream);
}

int flint_moe_bf16_grouped(const uint16_t *x, const uint16_t *router, const flint_bf16_experts *w,
                           const flint_shared_expert *shared, int M, int H, int E, int I, int top_k,
                           uint16_t *out, const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                           void *stream) {
  if (M > 0 && w && (!w->w13 || !w->w2)) return FLINT_ERR_NULL;
  if (M > 0 && w && (!aligned16(w->w13) || !aligned16(w->w2))) return FLINT_ERR_ALIGN;
  GroupedArgs a{};
  if (w) {
    a.bw13 = w->w13;
    a.bw2 = w->w2;
  }
  return run_grouped(a, w != nullptr, x, router, shared, M, H, E, I, top_k, out, dbg, ws, ws_bytes,
                     stream);
}

}  // extern "C"
