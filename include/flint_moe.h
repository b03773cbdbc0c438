/*
 * flint_moe.h - C ABI of the MI355X (gfx950) Flint routed-expert MoE block.
 *
 * The block (vLLM page "vllm.models.flint.ops.moe", module docstring,
 * "Numerics"; page "vllm.models.flint.model", FlintSparseMoeBlock):
 *   logits = bf16(x @ router^T)                       (fp32 accumulation)
 *   ids    = the top_k experts by logit, equal logits to the smaller index
 *   s_j    = fp32 sigmoid of the selected logits (exact exp, RN division)
 *   tw_j   = bf16(s_j / (sum_j s_j + 1e-20)), held in fp32
 *   per pair (t, j), expert e = ids[t, j]:
 *     g, u = fp32 (x[t] . W13[e, n]) * alpha13[e], (x[t] . W13[e, I + n]) * ...
 *     act  = bf16(silu(g) * u)
 *     y    = bf16((act . W2[e, h]) * alpha2[e])
 *   routed = bf16(sum_j tw_j * y_j)                   (fp32 accumulation)
 *   out    = bf16(routed + shared(x))                 (ungated shared SwiGLU)
 * NVFP4 weights are E2M1 codes times one E4M3 scale per 16 consecutive K
 * elements, dequantised exactly.  The shared expert and the BF16-expert
 * variant use the same rounding points with bf16 weights and no alpha.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to row-major, densely packed arrays
 *    owned by the caller.  bf16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is queued
 *    asynchronously; results are valid once the stream is synchronised.
 *  - No entry point allocates or frees device memory, synchronises the
 *    device, or keeps a pointer after its queued work completes.
 *  - Inputs are never modified.  Outputs are fully overwritten.
 *  - Arguments are validated on the host before anything is queued; a
 *    non-zero status means nothing was queued (FLINT_ERR_HIP: a HIP launch
 *    failed; flint_last_hip_error() gives its hipError_t).
 *  - Device pointers must be 16-byte aligned (FLINT_ERR_ALIGN otherwise).
 *  - Shapes (FLINT_ERR_SHAPE otherwise): 1 <= top_k <= E <= 256, and
 *      decode entry points: M <= 64, M * top_k <= 512, (H, I) one of
 *        (2048, 768), (256, 128), (256, 256), (512, 128), (512, 256),
 *        shared width SI == I (or no shared expert);
 *      flint_moe_grouped, flint_moe_bf16_grouped: H % 128 == 0,
 *        128 <= H <= 8192; I % 64 == 0,
 *        64 <= I <= 8192; a shared expert has SI % 64 == 0, 64 <= SI <=
 *        8192; M * H * 2, M * top_k * I * 2 and M * SI * 2 bytes each
 *        below 2^31 (the GEMMs address x, act and sact through 32-bit
 *        buffer offsets);
 *      flint_moe_route: H in {256, 512, 1024, 2048, 4096}, M <= 16376.
 *  - A workspace is used by one stream at a time: its counters are reset by
 *    the kernels themselves, so launches using one workspace must be
 *    serialised on one stream (as the pages require of their route counter).
 *  - The decode kernel needs all of its blocks resident at once (one per
 *    compute unit).  The library orders its own decode launches on a device
 *    one after another, also across streams; a caller must not run other
 *    long kernels concurrently with a decode call on the same GPU (its waits
 *    then give up: see flint_moe_wait_errors).
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum flint_status {
  FLINT_OK = 0,
  FLINT_ERR_NULL = -1,      /* a required pointer is NULL */
  FLINT_ERR_SHAPE = -2,     /* unsupported or inconsistent sizes */
  FLINT_ERR_ALIGN = -3,     /* a device pointer is not 16-byte aligned */
  FLINT_ERR_WORKSPACE = -4, /* workspace missing or too small */
  FLINT_ERR_HIP = -5        /* a HIP call failed */
};

/* NVFP4 routed experts in the ModelOpt checkpoint layout (page
 * "vllm.models.flint.ops.moe", FlintMoEWeights.from_modelopt and
 * FlintNvfp4Experts: w13 [E, 2I, H/2] with gate rows first, scales
 * [E, 2I, H/16] float8_e4m3fn, one fp32 global scale per expert shared by
 * gate and up; w2 [E, H, I/2], scales [E, H, I/16], fp32 [E]).
 * Byte c of a row packs K elements 2c (low nibble) and 2c + 1 (high nibble). */
typedef struct {
  const uint8_t *w13; /* [E, 2I, H/2] E2M1 codes, rows 0..I-1 gate, I..2I-1 up */
  const uint8_t *s13; /* [E, 2I, H/16] E4M3 block scales */
  const float *a13;   /* [E] global scale of gate and up */
  const uint8_t *w2;  /* [E, H, I/2] E2M1 codes */
  const uint8_t *s2;  /* [E, H, I/16] E4M3 block scales */
  const float *a2;    /* [E] global scale of down */
} flint_nvfp4_experts;

/* BF16 routed experts, plain row-major (the pages' BF16 decode path reads
 * the same logical matrices through a TRTLLM block layout; page
 * "vllm.models.flint.ops.moe", flint_moe_bf16_decode). */
typedef struct {
  const uint16_t *w13; /* [E, 2I, H] bf16, rows 0..I-1 gate, I..2I-1 up */
  const uint16_t *w2;  /* [E, H, I] bf16 */
} flint_bf16_experts;

/* Ungated shared SwiGLU expert (page "vllm.models.flint.model": Flint has
 * an ungated shared expert added to the routed sum).  w_gu == NULL means no
 * shared expert (its output is taken as 0).
 * Precomputed shared output (page "vllm.models.flint.ops.moe", flint_moe's
 * shared_output / shared_ready): when sh_in != NULL the block computes no
 * shared expert (w_gu, w_down and SI are ignored) and adds sh_in [M, H]
 * bf16 (16-byte aligned) in its place, out = bf16(bf16(routed) + sh_in);
 * sh_ready, a hipEvent_t or NULL, is waited on by the call's stream before
 * sh_in is read (decode entry points up to 16 tokens: before the block's one
 * kernel starts, whose combine reads it; flint_moe_grouped and the decode
 * entry points past 16 tokens: before the combine kernel), so the producer
 * may still be running when the call is made. */
typedef struct {
  const uint16_t *w_gu;   /* [2*SI, H] bf16, rows 0..SI-1 gate, SI..2SI-1 up */
  const uint16_t *w_down; /* [H, SI] bf16 */
  int SI;
  const uint16_t *sh_in;  /* NULL, or the precomputed shared output [M, H] */
  void *sh_ready;         /* NULL, or a hipEvent_t completing sh_in */
  /* NVFP4 shared expert (page "vllm.models.flint.ops.moe": E4M3 block scales
   * and one fp32 global scale per matrix; computed as a routed expert with
   * E = 1, the same rule as the routed experts).  When s_gu != NULL, w_gu
   * holds E2M1 codes [2*SI, H/2] (bytes), s_gu [2*SI, H/16], a_gu -> the
   * device fp32 global scale, w_down codes [H, SI/2], s_down [H, SI/16],
   * a_down.  Accepted by flint_moe_grouped and by the NVFP4 decode entry
   * points (flint_moe_decode, flint_moe_decode_noalloc, flint_moe_ll);
   * flint_moe_bf16_decode rejects it (FLINT_ERR_SHAPE). */
  const uint8_t *s_gu, *s_down;
  const float *a_gu, *a_down;
} flint_shared_expert;

/* Optional inputs and outputs of the MoE entry points; NULL = unused.
 * Intermediates use pair-major order p = t * top_k + j. */
typedef struct {
  const int32_t *ids_in; /* [M, top_k] forced routing (with tw_in): skips the router */
  const float *tw_in;    /* [M, top_k] */
  uint16_t *logits_out;  /* [M, E] bf16 router logits */
  int32_t *ids_out;      /* [M, top_k] */
  float *tw_out;         /* [M, top_k] */
  uint16_t *act_out;     /* [M*top_k, I] bf16 */
  uint16_t *y_out;       /* [M*top_k, H] bf16 */
  uint16_t *sact_out;    /* [M, SI] bf16 shared-expert activations */
  uint16_t *sh_out;      /* [M, H] bf16 shared-expert output */
  /* Stage timing: NULL, or an array of FLINT_STAGE_EVENTS hipEvent_t
   * (caller-created).  events[i] is recorded on `stream` just before stage i
   * is queued and events[FLINT_STAGE_EVENTS - 1] after the last stage, so
   * hipEventElapsedTime(events[i], events[i + 1]) times stage i.  Stages of
   * flint_moe_grouped: 0 router GEMM and top-k, 1 expert pair lists,
   * 2 shared gate/up, 3 routed gate/up, 4 routed down, 5 shared down,
   * 6 combine.  The decode entry points run one kernel up to 16 tokens (it
   * is stage 0 and the other stages take no time) and these stages past 16
   * tokens. */
  void **stage_events;
  /* Decode entry points only (test hooks of the bounded waits; 0 = off):
   * wait_polls > 0 caps every cross-block wait of the decode kernel at that
   * many polls (default 2^20); wait_probe != 0 adds one wait on a word that
   * nothing sets, which gives up and is reported by flint_moe_wait_errors
   * (FLINT_WAIT_PROBE).  A call whose wait gave up still ends, but its
   * results are not valid. */
  int wait_polls;
  int wait_probe;
} flint_moe_debug;

#define FLINT_STAGE_EVENTS 8

/* Kinds of bounded waits of the decode kernel, as bits of the word that
 * flint_moe_wait_errors returns.  The decode kernel runs one block per
 * compute unit and its blocks wait for each other's results; each wait is
 * bounded so the kernel always ends, and a wait that gives up sets its bit.
 * A set bit means a call's results are not valid: the grid was not fully
 * resident (another kernel held compute units for the whole wait), or the
 * workspace was used by two streams at once. */
#define FLINT_WAIT_LOGITS 1         /* a token's router logits */
#define FLINT_WAIT_SHARED_GATE_UP 2 /* the shared expert's gate/up blocks */
#define FLINT_WAIT_GATE_UP 4        /* a routed expert's gate/up blocks */
#define FLINT_WAIT_COMBINE_SHARED 8 /* the shared down blocks of a combined row group */
#define FLINT_WAIT_COMBINE_DOWN 16  /* reserved (no longer set: each block combines its own rows) */
#define FLINT_WAIT_LDS 32           /* a wave of the same block */
#define FLINT_WAIT_PROBE 64         /* the test hook (flint_moe_debug.wait_probe) */

/* Status code -> static string. */
const char *flint_status_str(int status);

/* hipError_t of the last FLINT_ERR_HIP returned on the calling thread. */
int flint_last_hip_error(void);

/* Bytes of device workspace the MoE entry points need for these sizes
 * (max_M tokens at most).  SI = 0 when there is no shared expert. */
int flint_moe_workspace_bytes(int max_M, int H, int E, int I, int SI, int top_k,
                              size_t *bytes);

/* Zeroes a workspace (its counters must start at zero).  Call once after
 * allocating it, on the stream that will use it. */
int flint_moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Exact NVFP4 dequantisation (page "vllm.models.flint.ops.moe", _dequant8 /
 * _dequant_rows: E2M1 value times E4M3 scale, exact in bf16): out[r, k] =
 * bf16(e2m1(code(r, k)) * e4m3(s[r, k / 16])), no global scale.
 * w [rows, K/2], s [rows, K/16], out [rows, K]; K % 32 == 0. */
int flint_nvfp4_dequant(const uint8_t *w, const uint8_t *s, int rows, int K,
                        uint16_t *out, void *stream);

/* Top-k of bf16 logits (page "vllm.models.flint.ops.moe", _topk_kernel /
 * _topk_row): ids [M, top_k] int32 in selection order, tw [M, top_k] fp32
 * holding bf16 values; scores (may be NULL) [M, top_k] receives the fp32
 * sigmoid scores s_j before renormalisation. */
int flint_moe_topk(const uint16_t *logits, int M, int E, int top_k, int32_t *ids,
                   float *tw, float *scores, void *stream);

/* Router (page "vllm.models.flint.ops.moe", route / _router_kernel): bf16
 * logits of x [M, H] against router [E, H], then top-k as flint_moe_topk.
 * logits (may be NULL) [M, E].  0 <= M <= 16376 (M = 0 queues nothing). */
int flint_moe_route(const uint16_t *x, const uint16_t *router, int M, int H, int E,
                    int top_k, uint16_t *logits, int32_t *ids, float *tw,
                    void *ws, size_t ws_bytes, void *stream);

/* Wait errors of the decode calls that used workspace ws: queues on
 * `stream` a copy of the workspace's wait-error word (an OR of FLINT_WAIT_*
 * bits, 0 = every wait ended normally) into *errors, a device int32, and
 * clears the word.  Read *errors after synchronising the stream.  ws = NULL
 * reads the library's own scratch on the current device (the calls of
 * flint_moe_decode_noalloc); ws_bytes is then ignored. */
int flint_moe_wait_errors(void *ws, size_t ws_bytes, int32_t *errors, void *stream);

/* The MoE block on NVFP4 experts for decode-size batches, 1 <= M <= 64
 * (page "vllm.models.flint.ops.moe", flint_moe, decode branch):
 * out [M, H] bf16.  Up to 16 tokens the whole block is one kernel (per-token
 * dot products over the touched experts' weights); past 16 tokens, where
 * each expert's weights serve several tokens, it runs the chain of
 * flint_moe_grouped with matrix-core GEMMs that stream each touched
 * expert's weights once (the same rounding rule either way). */
int flint_moe_decode(const uint16_t *x, const uint16_t *router,
                     const flint_nvfp4_experts *w, const flint_shared_expert *shared,
                     int M, int H, int E, int I, int top_k, uint16_t *out,
                     const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                     void *stream);

/* flint_moe_decode without a workspace, for callers that cannot allocate
 * device memory (serving loops that must not call hipMalloc, harnesses that
 * forbid it).  Same arguments (minus ws), rule, limits and errors as
 * flint_moe_decode; no memory is allocated or freed.  Its scratch is a
 * 5 MiB array inside the library, one per GPU, kept until the process
 * ends; sizes whose workspace would exceed it (flint_moe_workspace_bytes)
 * return FLINT_ERR_WORKSPACE (every size the decode entry points accept
 * fits).  Past 16 tokens the shared expert runs on `stream` itself (no
 * second stream).  Every call on a GPU shares that GPU's scratch: calls are ordered
 * by the library's per-device launch chain, but two calls must not be
 * queued concurrently from different host threads with debug outputs that
 * alias.  Nothing in the scratch needs clearing between calls (its flags
 * hold per-call sequence numbers).  Sequence numbers are taken when the call
 * is queued, so a graph that captured the call must not be replayed. */
int flint_moe_decode_noalloc(const uint16_t *x, const uint16_t *router,
                             const flint_nvfp4_experts *w, const flint_shared_expert *shared,
                             int M, int H, int E, int I, int top_k, uint16_t *out,
                             const flint_moe_debug *dbg, void *stream);

/* The decode MoE block behind a residual add and RMS norm (page
 * "vllm.models.flint.ops.moe", flint_moe_ll with _add_rms_norm):
 *   s = fp32(attn_out) + fp32(residual)          (one fp32 rounding)
 *   residual_out = bf16(s)
 *   xn_out = bf16((s * rsqrt(mean_h(s^2) + eps)) * ln_weight)   (fp32)
 *   out = flint_moe_decode(xn_out, ...)
 * attn_out, residual, residual_out, xn_out [M, H] bf16 (caller-owned, 16-byte
 * aligned; xn_out is both a result and the block's input); ln_weight [H]
 * bf16; eps >= 0; H % 8 == 0.  The other arguments, limits and errors are
 * those of flint_moe_decode; nothing is written when an argument is
 * rejected.  Inputs are not modified. */
int flint_moe_ll(const uint16_t *attn_out, const uint16_t *residual,
                 const uint16_t *ln_weight, float eps, const uint16_t *router,
                 const flint_nvfp4_experts *w, const flint_shared_expert *shared,
                 int M, int H, int E, int I, int top_k, uint16_t *out,
                 uint16_t *residual_out, uint16_t *xn_out,
                 const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                 void *stream);

/* The MoE block on NVFP4 experts for any M >= 1 with grouped MFMA GEMMs
 * (page "vllm.models.flint.ops.moe", flint_moe, grouped branch). */
int flint_moe_grouped(const uint16_t *x, const uint16_t *router,
                      const flint_nvfp4_experts *w, const flint_shared_expert *shared,
                      int M, int H, int E, int I, int top_k, uint16_t *out,
                      const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                      void *stream);

/* The MoE block on BF16 experts for decode-size batches, 1 <= M <= 64
 * (page "vllm.models.flint.ops.moe", flint_moe_bf16_decode). */
int flint_moe_bf16_decode(const uint16_t *x, const uint16_t *router,
                          const flint_bf16_experts *w, const flint_shared_expert *shared,
                          int M, int H, int E, int I, int top_k, uint16_t *out,
                          const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                          void *stream);

/* The MoE block on BF16 experts for any M >= 1 with grouped MFMA GEMMs (page
 * "vllm.models.flint.model", FlintSparseMoeBlock: BF16 experts use the decode
 * kernels for small batches and a grouped MoE GEMM otherwise; the rule is
 * flint_moe_bf16_decode's).  Shapes, limits, shared expert and errors as
 * flint_moe_grouped. */
int flint_moe_bf16_grouped(const uint16_t *x, const uint16_t *router,
                           const flint_bf16_experts *w, const flint_shared_expert *shared,
                           int M, int H, int E, int I, int top_k, uint16_t *out,
                           const flint_moe_debug *dbg, void *ws, size_t ws_bytes,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_MOE_H */
