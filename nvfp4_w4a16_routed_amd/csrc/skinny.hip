// Expert GEMMs with few rows per expert (decode-size batches): C = A . W^T
// on the matrix cores, each wave streaming its own weight rows.
//
// Semantics (vLLM page "vllm.models.flint.ops.moe": module docstring
// "Numerics", _gate_up_gemv_kernel, _down_gemv_kernel, _dequant8):
//   gate/up: g, u = fp32 (a . W13[e, n]) * alpha13[e], (a . W13[e, I + n]) * alpha13[e]
//            c[row, n] = bf16(silu(g) * u)
//   down:    c[row, h] = bf16(fp32 (a . W2[e, h]) * alpha2[e])
// with NVFP4 weights (E2M1 codes times their E4M3 block scale, exact) or
// bf16 weights (no global scale); the shared expert is the same product with
// one expert whose rows are all tokens.
//
// Shape of the work.  With a few rows per expert the product is bound by
// the weight stream.  A block of eight waves serves one expert: each wave
// owns 16 weight rows (gate/up: 8 output columns, their gate and up rows
// interleaved; down: 16 output rows) and walks K in steps of 128 with the
// next steps' weights in flight in registers, multiplying each step on
// v_mfma_f32_16x16x32_bf16 against one group of 16 A rows (an expert with
// more rows has one block per group and column tile):
//   A operand (16 x 32): lane l holds weight row l % 16, K slots 8 (l / 16)..
//   B operand (32 x 16): lane l holds A row l % 16 of the group, same K slots
//   D (16 x 16): lane l holds weight rows 4 (l / 16) .. + 3 of A row l % 16.
// Within a step, lane group q = l / 16 covers the K range [32 q, 32 q + 32),
// four MFMAs of eight K each, in the same order on both operands (the sum's
// order is free: fp32 accumulation), so a lane's weights of a step are 16
// contiguous bytes (NVFP4) and every weight row is read once per call.
//
// Routed rows: a block finds its group's pairs itself from the routing ids
// (a histogram of the ids over the experts, then the ranks of its expert's
// pairs in ascending pair order), so no pair-list pass runs before it.
//
// The A rows (the rows of those pairs) are shared by the block's
// waves: they pass through LDS in chunks of 256 K, two buffers, filled with
// coalesced 16-byte loads one chunk ahead and swapped at a barrier.  Loading
// A per wave in the MFMA layout instead (16 rows per instruction, four per
// step) costs the L1 several times the weight stream.
//
// E4M3 scales: a lane's two scale bytes of a step sit 8 bytes after those of
// the previous step, and two-byte loads per step cost the L1 as much as the
// codes.  Instead every lane loads 16 bytes per eight steps (lane group g:
// its row's scale bytes of steps 2 g and 2 g + 1 of the eight) and the lanes
// trade them with ds_bpermute (no LDS storage).
//
// NVFP4 codes are converted exactly: E2M1 pair to fp32 (hardware
// converter), times the block's E4M3 scale (the product has at most 6
// significant bits), to bf16 (exact).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace flint {

namespace {

constexpr int kSkWaves = 8;      // waves per block
constexpr int kSkXcds = 8;       // XCDs the blocks of a launch are dealt to in turn
constexpr int kSkK = 128;        // K per step
constexpr int kSkCK = 256;       // K per A chunk (two steps)
constexpr int kSkRowB = kSkCK * 2 + 16;  // bytes of one A row in LDS (16 pad: rows 4 banks apart)
constexpr int kSkBuf = 16 * kSkRowB;     // bytes of one A chunk buffer
static_assert(kSkCK == 2 * kSkK, "two steps per A chunk");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// Two E2M1 codes (byte SEL of w) times an E4M3 block scale -> bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_scaled(uint32_t w, float s) {
  const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return pack_bf16x2(v.x * s, v.y * s);
}

// One step's weights for the lane: NVFP4, 16 bytes of codes (32 codes);
// bf16, 64 bytes (32 values).
template <int WFMT>
struct SkW;
template <>
struct SkW<kNvfp4> {
  u32x4_t codes;
};
template <>
struct SkW<kBf16> {
  u32x4_t v[4];
};

// GATE_UP: output column n from weight rows n (gate) and I + n (up), 8 per
// wave; else output column h from weight row h, 16 per wave.
// NW waves per block; U = 4 chunks per loop pass (the weight ring: NVFP4 4
// steps in flight, 16 bytes per lane each; bf16 2 steps, 64 bytes).
//
// Block b computes unit b: a unit is (expert, group of 16 of its rows, NW
// column tiles), numbered densely over the experts that have rows
// (expert-major, then group, then column tile), so the launch's blocks
// with work come first in dispatch order, spread evenly over the CUs, and
// the blocks past the last unit (the grid is a bound on the units) exit at
// once.  (A shared work counter instead costs every block an atomic round
// trip before its first weight load.)
// LDS of a block.
struct SkLds {
  __attribute__((aligned(16))) uint8_t a[2 * kSkBuf];  // A chunk buffers
  int first[kMaxExperts + 1];  // first unit-group of each expert, then the total
  int wsum[4];
  int cnt[kMaxExperts];        // routed: pairs of each expert
  int bsum[16];
  int rows[16];                // routed: pair of each row of the group, or -1
};

// Unit `unit` of the GEMM g (the whole block takes part).
template <bool GATE_UP, int WFMT, int NW, int U>
__device__ __forceinline__ void sk_unit(const SkinnyArgs &g, const int unit, SkLds &L) {
  constexpr int CW = GATE_UP ? 8 : 16;  // output columns per wave
  constexpr bool NV = WFMT == kNvfp4;
  constexpr int NT = NW * kWave;
  constexpr int WD = NV ? 4 : 2;
  constexpr int SPT = 16 * (kSkCK / 8) / NT;  // A pieces (16 bytes) per thread per chunk
  static_assert(SPT * NT == 16 * (kSkCK / 8) && U == 4 && NW <= 16, "block shape");
  static_assert(kMaxExperts <= 4 * kWave && NT >= kMaxExperts, "one thread per expert in the prefix");
  uint8_t *const lds = L.a;
  int *const s_first = L.first;
  int *const s_wsum = L.wsum;
  int *const s_cnt = L.cnt;
  int *const s_bsum = L.bsum;
  int *const s_rows = L.rows;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int m = lane & 15, grp = lane >> 4;
  const int C = g.K / kSkCK;  // chunks
  const int KS = 2 * C;       // steps
  const bool routed = g.ids != nullptr;
  const int nE = routed ? g.E : 1;
  const int tiles = (g.ncols / CW + NW - 1) / NW;  // column-tile units per group

  // routed: the pairs of each expert, from the routing ids (one pair per
  // thread: nrows * top_k <= NT); an out-of-range id belongs to no expert
  int my_id = -1;
  if (routed) {
    for (int e = tid; e < nE; e += NT) s_cnt[e] = 0;
    if (tid < 16) s_rows[tid] = -1;
    __syncthreads();
    if (tid < g.nrows * g.top_k) {
      const int v = g.ids[tid];
      if ((unsigned)v < (unsigned)nE) {
        my_id = v;
        atomicAdd(&s_cnt[v], 1);
      }
    }
    __syncthreads();
  }
  // groups of 16 rows of each expert, prefix over the experts
  {
    int ng = 0;
    if (tid < nE) ng = ((routed ? s_cnt[tid] : g.nrows) + 15) >> 4;
    int incl = ng;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    if (wv < 4 && lane == kWave - 1) s_wsum[wv] = incl;
    __syncthreads();
    if (tid < nE) {
      int off = incl - ng;
      for (int w = 0; w < wv; ++w) off += s_wsum[w];
      s_first[tid] = off;
    }
    if (tid == 0) s_first[nE] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
  }
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(g.w, (size_t)g.E * g.wrows * g.K * (NV ? 1 : 4) / 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(NV ? (const void *)g.ws : (const void *)g.w,
                                              NV ? (size_t)g.E * g.wrows * (g.K / 16) : 0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, (size_t)g.a_rows * g.K * 2);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.c, (size_t)g.c_rows * g.ldc * 2);
  // this lane's MFMA operand at step half 0, t = 0
  const uint32_t rd_off = m * kSkRowB + grp * 64;
  const int half_sh = (grp & 1) * 16;

  __syncthreads();  // publishes s_first
  {
    int gidx, tile;
    if (routed) {
      if (unit >= s_first[nE] * tiles) return;  // the whole block
      gidx = unit / tiles;
      tile = unit - gidx * tiles;
    } else {
      // Dense (every row, one expert): the groups of a column tile read the
      // same weights, so they take block ids kSkXcds apart (blocks are
      // dealt to the XCDs in turn): the same XCD, hence its L2, at about
      // the same time.  Tiles are padded to a multiple of kSkXcds.
      const int ng = s_first[1];
      const int slot = unit % kSkXcds, round = unit / kSkXcds;
      gidx = round % ng;
      tile = (round / ng) * kSkXcds + slot;
      if (tile >= tiles) return;  // the whole block
    }
    // expert of group gidx: the last e with s_first[e] <= gidx (experts
    // without rows share their successor's first group)
    int lo = 0, hi = nE - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_first[mid] <= gidx) lo = mid;
      else hi = mid - 1;
    }
    const int e = lo;
    const int nb = 16 * (gidx - s_first[e]);  // first row of the group
    const int np = routed ? s_cnt[e] : g.nrows;
    // routed: rows nb .. nb + 15 of expert e are its pairs of those ranks in
    // ascending pair order (rank: matching pairs of smaller index)
    if (routed) {
      const bool match = my_id == e;
      const unsigned long long bal = __ballot(match);
      if (lane == 0) s_bsum[wv] = __popcll(bal);
      __syncthreads();
      int rank = __popcll(bal & ((1ull << lane) - 1ull));
      for (int w = 0; w < wv; ++w) rank += s_bsum[w];
      if (match && rank >= nb && rank < nb + 16) s_rows[rank - nb] = tid;
      __syncthreads();
    }

    // waves past the last column tile stream the last tile again (uniform
    // work for the barriers) and store nothing
    const int c0_raw = (tile * NW + wv) * CW;
    const bool store = c0_raw < g.ncols;
    const int c0 = store ? c0_raw : g.ncols - CW;

    // this lane's weight row
    const int wr = GATE_UP ? ((m & 1) ? g.I : 0) + c0 + (m >> 1) : c0 + m;
    const size_t wrow = (size_t)e * g.wrows + wr;
    const uint32_t wbase = (uint32_t)(wrow * (NV ? g.K / 2 : g.K * 2));
    const uint32_t sbase = (uint32_t)(wrow * (g.K / 16));
    const float alpha = g.alpha ? g.alpha[e] : 1.0f;

    auto load_w = [&](SkW<WFMT> &w, int ks) {
      const bool ok = ks < KS;
      if constexpr (NV) {
        w.codes = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rw, ok ? wbase + ks * (kSkK / 2) + grp * 16 : kOOB, 0, kPolicyStream));
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w.v[t] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                           rw, ok ? wbase + (ks * kSkK + grp * 32 + t * 8) * 2 : kOOB, 0,
                           kPolicyStream));
      }
    };
    // scale bytes of steps ks .. ks + 7: lane group grp loads its row's 16
    // bytes of steps ks + 2 grp, ks + 2 grp + 1 (each step's 8 bytes: two
    // per lane group of that step)
    u32x4_t sblk = {0u, 0u, 0u, 0u};
    auto load_s = [&](int ks) {
      if constexpr (NV)
        sblk = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, ks + 2 * grp < KS ? sbase + (ks + 2 * grp) * (kSkK / 16) : kOOB, 0,
                         kPolicyStream));
    };
    // -> sc[j]: this lane's two scale bytes (low half) of step i0 + j of the
    // eight whose bytes sblk holds
    uint32_t sc[4];
    auto take_s = [&](const int i0) {
      if constexpr (NV) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + j;
          const int src = ((i >> 1) * 16 + m) * 4;
          const uint32_t d0 = __builtin_amdgcn_ds_bpermute(src, (int)sblk[(i & 1) * 2]);
          const uint32_t d1 = __builtin_amdgcn_ds_bpermute(src, (int)sblk[(i & 1) * 2 + 1]);
          sc[j] = ((grp >> 1) ? d1 : d0) >> half_sh;
        }
      }
    };

    // A staging: piece q = tid + i NT (i < SPT) of a chunk is the 16 bytes
    // q % 32 of row q / 32 (row addresses set below)
    uint32_t st_off[SPT], abase[SPT];
    u32x4_t stage[SPT];
    auto load_a = [&](int c) {
#pragma unroll
      for (int i = 0; i < SPT; ++i)
        stage[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         ra, c < C && abase[i] != kOOB ? abase[i] + c * (kSkCK * 2) : kOOB, 0, 0));
    };
    auto write_a = [&](int buf) {
#pragma unroll
      for (int i = 0; i < SPT; ++i)
        *reinterpret_cast<u32x4_t *>(lds + buf * kSkBuf + st_off[i]) = stage[i];
    };

    SkW<WFMT> wq[WD];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // The first scales and weight steps go out before the row lookups that
    // the A rows wait for; then chunk 0 into buffer 0, chunk 1 on its way
    // and the last weight steps of the ring.  After the scales and after
    // chunk 1 at least as many loads follow as in the loop (per chunk its
    // A load and its two steps' weight loads, the scales of eight steps in
    // every fourth chunk), so the loop's waits are the same from its first
    // pass on (sched_barrier: the scheduler keeps this order).
    load_s(0);
#pragma unroll
    for (int d = 0; d < WD - 2; ++d) load_w(wq[d], d);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int q = tid + i * NT, srow = q >> 5, spiece = q & 31;
      st_off[i] = srow * kSkRowB + spiece * 16;
      abase[i] = kOOB;
      const int n = nb + srow;
      if (n < np) {
        const int p = routed ? s_rows[srow] : n;
        abase[i] = (uint32_t)(routed && GATE_UP ? p / g.top_k : p) * g.K * 2 + spiece * 16;
      }
    }
    load_a(0);
    write_a(0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(wq[WD - 2], WD - 2);
    load_w(wq[WD - 1], WD - 1);
    __syncthreads();

    // one step: weights of slot w (step ks), scales sc[i], A half h of buffer `buf`
    auto step = [&](int ks, SkW<WFMT> &w, int i, int buf, int h) {
      u32x4_t op[4];
      if constexpr (NV) {
        const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 0);
        const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t cw = w.codes[t];  // 8 codes: K 32 grp + 8 t ..
          const float s = t < 2 ? s0 : s1;
          op[t] = u32x4_t{fp4x2_scaled<0>(cw, s), fp4x2_scaled<1>(cw, s), fp4x2_scaled<2>(cw, s),
                          fp4x2_scaled<3>(cw, s)};
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) op[t] = w.v[t];
      }
      const uint8_t *ab = lds + buf * kSkBuf + rd_off + h * (kSkK * 2);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t *>(ab + t * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, op[t]),
                                                      __builtin_bit_cast(bf16x8_t, av), acc, 0, 0, 0);
      }
      load_w(w, ks + WD);
    };

    // Chunk c: chunk c + 1 (loaded during chunk c - 1) goes to the other
    // buffer and chunk c + 2 is requested before the two steps of chunk c,
    // so a wait for the A loads never waits for the weights of the steps
    // ahead.  Every chunk issues the same loads (past the end: out of
    // range, zeros), and the loop runs U = 4 chunks per pass with fixed
    // ring slots, which keeps the compiler's waits exact; the last C % 4
    // chunks run after it, straight-line.  P: c % 4.  The scales of eight
    // steps are traded among the lanes four steps at a time (P = 0, 2); the
    // next eight steps' are requested after the second trade.
    auto chunk = [&](int c, auto par) {
      constexpr int P = decltype(par)::value;
      if (P == 0) take_s(0);
      if (P == 2) {
        take_s(4);
        __builtin_amdgcn_sched_barrier(0);
        load_s(2 * c + 4);
      }
      write_a((P & 1) ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      load_a(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      step(2 * c, wq[(2 * P) % WD], 2 * (P & 1), P & 1, 0);
      step(2 * c + 1, wq[(2 * P + 1) % WD], 2 * (P & 1) + 1, P & 1, 1);
      __syncthreads();
    };
    int c = 0;
    for (; c + 3 < C; c += 4) {
      chunk(c, std::integral_constant<int, 0>{});
      chunk(c + 1, std::integral_constant<int, 1>{});
      chunk(c + 2, std::integral_constant<int, 2>{});
      chunk(c + 3, std::integral_constant<int, 3>{});
    }
    if (c < C) chunk(c, std::integral_constant<int, 0>{});
    if (c + 1 < C) chunk(c + 1, std::integral_constant<int, 1>{});
    if (c + 2 < C) chunk(c + 2, std::integral_constant<int, 2>{});

    // epilogue: lane holds weight rows 4 grp .. + 3 of row m of the group
    const int n = nb + m;
    if (store && n < np) {
      const int crow = routed ? s_rows[m] : n;
      if constexpr (GATE_UP) {
        // rows 4 grp + (0, 1, 2, 3) = gate / up of column c0 + 2 grp, then of c0 + 2 grp + 1
        const float g0 = acc[0] * alpha, u0 = acc[1] * alpha;
        const float g1 = acc[2] * alpha, u1 = acc[3] * alpha;
        const uint32_t v = f32_to_bf16(swiglu(g0, u0)) | (f32_to_bf16(swiglu(g1, u1)) << 16);
        __builtin_amdgcn_raw_buffer_store_b32(
            v, rc, (uint32_t)((size_t)crow * g.ldc + c0 + 2 * grp) * 2, 0, 0);
      } else {
        const uint32_t v0 = f32_to_bf16(acc[0] * alpha) | (f32_to_bf16(acc[1] * alpha) << 16);
        const uint32_t v1 = f32_to_bf16(acc[2] * alpha) | (f32_to_bf16(acc[3] * alpha) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(
            v2u32_t{v0, v1}, rc, (uint32_t)((size_t)crow * g.ldc + c0 + 4 * grp) * 2, 0, 0);
      }
    }
  }
}

// Blocks [0, sh_units) compute the units of sh (the shared expert: every
// token, first in dispatch order since its units stream more bytes), the
// others those of r (the routed experts).
template <bool GATE_UP, int WR, int WS, int NW, int U>
__global__ void __launch_bounds__(NW * kWave, 6) skinny_kernel(SkinnyArgs r, SkinnyArgs sh, int sh_units) {
  __shared__ SkLds L;
  if ((int)blockIdx.x < sh_units)
    sk_unit<GATE_UP, WS, NW, U>(sh, blockIdx.x, L);
  else
    sk_unit<GATE_UP, WR, NW, U>(r, blockIdx.x - sh_units, L);
}

template <bool GU, int WR, int WS>
hipError_t sk_launch(const SkinnyArgs &r, const SkinnyArgs &sh, long long sh_units, long long units,
                     hipStream_t st) {
  if (units <= 0) return hipSuccess;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((skinny_kernel<GU, WR, WS, kSkWaves, 4>), dim3((unsigned)units), dim3(kSkWaves * kWave),
                     0, st, r, sh, (int)sh_units);
  return hipGetLastError();
}

// Units of g: without routing ceil(nrows / 16) groups (exact); routed at
// most one group per expert with pairs plus one per 16 pairs (a bound).
long long sk_units(const SkinnyArgs &g, bool gate_up) {
  const int cw = gate_up ? 8 : 16;
  const long long tiles = (g.ncols / cw + kSkWaves - 1) / kSkWaves;
  const long long pairs = (long long)g.nrows * (g.ids ? g.top_k : 1);
  const long long groups =
      g.ids ? (pairs + 15) / 16 + (pairs < g.E ? pairs : g.E) : ((long long)g.nrows + 15) / 16;
  return g.ids ? groups * tiles : groups * ((tiles + kSkXcds - 1) / kSkXcds * kSkXcds);
}

}  // namespace

bool skinny_shape_supported(int K, int ncols, bool gate_up) {
  return K > 0 && K % kSkCK == 0 && ncols > 0 && ncols % (gate_up ? 8 : 16) == 0;
}

hipError_t launch_skinny(const SkinnyArgs &r, int wfmt_r, const SkinnyArgs *sh, int wfmt_s, bool gate_up,
                         hipStream_t st) {
  auto ok = [&](const SkinnyArgs &g) {
    return skinny_shape_supported(g.K, g.ncols, gate_up) &&
           (!g.ids || (g.E >= 1 && g.E <= kMaxExperts && (long)g.nrows * g.top_k <= kSkWaves * kWave));
  };
  if (!ok(r) || (sh && (!ok(*sh) || sh->ids))) return hipErrorInvalidValue;
  const long long su = sh ? sk_units(*sh, gate_up) : 0;
  const long long units = su + sk_units(r, gate_up);
  const SkinnyArgs &s = sh ? *sh : r;
  const bool nr = wfmt_r == kNvfp4, ns = sh ? wfmt_s == kNvfp4 : nr;
  if (gate_up) {
    if (nr) return ns ? sk_launch<true, kNvfp4, kNvfp4>(r, s, su, units, st)
                      : sk_launch<true, kNvfp4, kBf16>(r, s, su, units, st);
    return ns ? sk_launch<true, kBf16, kNvfp4>(r, s, su, units, st)
              : sk_launch<true, kBf16, kBf16>(r, s, su, units, st);
  }
  if (nr) return ns ? sk_launch<false, kNvfp4, kNvfp4>(r, s, su, units, st)
                    : sk_launch<false, kNvfp4, kBf16>(r, s, su, units, st);
  return ns ? sk_launch<false, kBf16, kNvfp4>(r, s, su, units, st)
            : sk_launch<false, kBf16, kBf16>(r, s, su, units, st);
}

}  // namespace flint
