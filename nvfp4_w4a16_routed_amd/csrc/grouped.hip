// The MoE block for prefill-size batches: grouped GEMMs on the matrix cores.
//
// Semantics (vLLM page "vllm.models.flint.ops.moe": module docstring
// "Numerics", the grouped branch of flint_moe and _combine_kernel):
//   logits = bf16(fp32 x . router^T);  top-k and weights as in decode
//   per expert e, for its pairs p = t * top_k + j (ascending):
//     g, u = fp32 (x[t] . W13[e, n]) * alpha13[e], (x[t] . W13[e, I + n]) * ...
//     act[p, n] = bf16(silu(g) * u)
//     y[p, h]   = bf16(fp32 (act[p] . W2[e, h]) * alpha2[e])
//   shared: sact = bf16(silu(xWg) * xWu), sh = bf16(sact . Wd)   (fp32 sums)
//   out[t, h] = bf16(bf16(sum_j tw[t, j] y[t*k + j, h]) + sh[t, h])
//
// Every product is C[rows, cols] = A[rows, K] . B[cols, K]^T on bf16 MFMAs
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation:
//  - router_kernel: the router logits (then topk_kernel);
//  - routed_gemm_kernel: the routed experts' gate/up and down, A rows
//    gathered through each expert's pair list, NVFP4 B tiles dequantised
//    exactly (E2M1 value times its E4M3 block scale, in fp32, then bf16) into
//    LDS;
//  - gemm_kernel: the shared expert's gate/up and down (bf16 B).
// Epilogues apply the rule: global scale, SwiGLU, bf16 rounding; a
// memory-bound kernel then forms the weighted combine and the shared add.
//
// gemm_kernel's tile: 256 rows x 128 columns, K steps of 32; 4 waves, wave w
// owns rows [64 w, 64 w + 64) and all 128 columns (2 x 4 MFMA tiles of
// 32 x 32).  Tiles go global -> registers (two K steps ahead) -> LDS (two
// stages), with the 16-byte chunks of each 64-byte LDS row XOR-swizzled so
// the accesses are spread over the LDS banks.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace flint {

namespace {

constexpr int kGThreads = 256;
constexpr int kBM = 256;  // tile rows (tokens)
constexpr int kBN = 128;  // tile columns (B rows)
constexpr int kBK = 32;   // K per step (4 chunks of 8 bf16)
constexpr int kStages = 2;  // LDS stages; register loads run two K steps ahead

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

enum GemmMode {
  kSharedGateUp = 1, // sact[t, n] = bf16(swiglu(x[t] . Wg[n], x[t] . Wu[n]))
  kSharedDown = 2,   // sh[t, h] = bf16(sact[t] . Wd[h])
  kRoutedGateUp = 3, // act[p, n] = bf16(swiglu(a13 x[t(p)] . W13[n], a13 x[t(p)] . W13[I+n]))
  kRoutedDown = 4,   // y[p, h] = bf16(a2 * act[p] . W2[h])
  // BF16 routed experts (no global scale), on gemm_kernel with gathered rows
  kBf16GateUp = 5,   // act[p, n] = bf16(swiglu(x[t(p)] . W13[e, n], x[t(p)] . W13[e, I+n]))
  kBf16Down = 6      // y[p, h] = bf16(act[p] . W2[e, h])
};

struct GemmArgs {
  const uint16_t *a;     // A source rows (x, sact or act), row length K
  const uint8_t *b;      // B: bf16 rows (shared), or NVFP4 codes (routed)
  const uint8_t *bs;     // NVFP4 scales (routed)
  const float *alpha;    // NVFP4 global scales [E] (routed)
  uint16_t *c;           // output rows
  int rows;              // shared expert: number of A rows (tokens)
  int a_rows;            // rows of the A matrix (its extent for the loads)
  int K;                 // reduction length
  int ncols;             // output columns (B rows; for gate/up: act columns)
  int ldc;               // output row length
  int I;                 // gate/up: offset of the up rows in B
  int top_k;
  // routed modes: expert pair lists
  const int32_t *lists;  // [E][list_stride] pair indices, ascending
  const int32_t *counts; // [E]
  int list_stride, E;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// (read from the first lane, so the compiler knows it is uniform in the wave)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// LDS position (in 16-byte chunks) of chunk c of tile row r.  The XOR
// pattern keeps the MFMA operand reads free of bank conflicts (16 lanes a
// cycle: 16 consecutive rows, one chunk each, a 256-byte bank window); the
// stores of loaded chunks are 1 KB contiguous per wave.
__device__ __forceinline__ int swz_x(int r) { return ((r >> 2) & 3) ^ ((r >> 1) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * 4 + (c ^ swz_x(r)); }

// E2M1 codes (8 per dword) times one E4M3 scale -> 8 exact bf16 values.
// The hardware converter applies only the exponent of its scale operand, so
// it converts with scale 1 and the fp32 product with the scale is formed
// explicitly; it has at most 6 significant bits, so truncating it to bf16
// is exact.
template <int SEL>
__device__ __forceinline__ uint32_t dequant2(uint32_t codes, float scale) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  const f2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
  const uint32_t lo = __float_as_uint(v[0] * scale), hi = __float_as_uint(v[1] * scale);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // high halves: {lo.bf16, hi.bf16}
}
__device__ __forceinline__ u32x4_t dequant8(uint32_t codes, float scale) {
  return u32x4_t{dequant2<0>(codes, scale), dequant2<1>(codes, scale), dequant2<2>(codes, scale),
                 dequant2<3>(codes, scale)};
}

// Products with bf16 B rows: the shared expert's (MODE kSharedGateUp,
// kSharedDown: every token, one B matrix) and the BF16 routed experts'
// (kBf16GateUp, kBf16Down: the rows of one expert's pair list, that
// expert's B matrix).
template <int MODE>
__global__ void __launch_bounds__(kGThreads, 2) gemm_kernel(GemmArgs g) {
  constexpr bool kGateUp = MODE == kSharedGateUp || MODE == kBf16GateUp;
  constexpr bool kRouted = MODE == kBf16GateUp || MODE == kBf16Down;
  __shared__ __attribute__((aligned(16))) uint16_t As[kStages][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kStages][kBN * kBK];
  __shared__ int rowidx[kBM];  // A row (token or pair) of each tile row, -1 = none
  __shared__ int outrow[kBM];  // output row of each tile row
  __shared__ int tile_info[4];

  const int lane = lane_id(), wv = wave_id();
  const int ntn = kGateUp ? g.ncols / (kBN / 2) : (g.ncols + kBN - 1) / kBN;  // column tiles
  // Tile of this block.  Blocks are dealt to the XCDs round-robin; the
  // column tiles of one row tile are given to consecutive blocks of one XCD
  // so its A rows are reused from that XCD's L2.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x % 8, per = nblk / 8;
  const int b = blockIdx.x < per * 8 ? xcd * per + blockIdx.x / 8 : blockIdx.x;
  const int mt = b / ntn, nt = b % ntn;
  int m0 = mt * kBM, nrows, expert = 0;
  if constexpr (kRouted) {
    // Row tile mt of the routed experts: expert e has ceil(count_e / 256)
    // row tiles, in expert order; tiles past the last one have no rows.
    if (wv == 0) {
      int c4[4], n4[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ee = 4 * lane + i;
        c4[i] = ee < g.E ? g.counts[ee] : 0;
        n4[i] = (c4[i] + kBM - 1) / kBM;
        tot += n4[i];
      }
      int incl = tot;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      int before = incl - tot;
      if (lane == 0) tile_info[0] = -1;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mt >= before && mt < before + n4[i]) {
          const int q = mt - before;
          tile_info[0] = 4 * lane + i;
          tile_info[1] = q * kBM;
          tile_info[2] = min(kBM, c4[i] - q * kBM);
        }
        before += n4[i];
      }
    }
    __syncthreads();
    expert = tile_info[0];
    if (expert < 0) return;
    m0 = tile_info[1];
    nrows = tile_info[2];
  } else {
    nrows = min(kBM, g.rows - m0);
    if (nrows <= 0) return;
  }
  const int n0 = nt * (kGateUp ? kBN / 2 : kBN);

  // Row indices of the tile; rows past the end repeat the first row (their
  // loads stay in bounds and their results are dropped).
  for (int i = threadIdx.x; i < kBM; i += kGThreads) {
    if constexpr (kRouted) {
      const int p = g.lists[(size_t)expert * g.list_stride + m0 + (i < nrows ? i : 0)];
      rowidx[i] = kGateUp ? p / g.top_k : p;
      outrow[i] = i < nrows ? p : -1;
    } else {
      const int src = m0 + (i < nrows ? i : 0);
      rowidx[i] = src;
      outrow[i] = i < nrows ? src : -1;
    }
  }
  __syncthreads();

  const int K = g.K;
  const int nk = K / kBK;
  // B row of tile column r
  auto brow = [&](int r) -> int {
    if constexpr (kGateUp) return r < kBN / 2 ? n0 + r : g.I + n0 + (r - kBN / 2);
    else return n0 + r;
  };
  const int ncols_b = kGateUp ? 2 * g.I : g.ncols;  // valid B rows

  // ---- loaders.  Each K step moves 256 x 32 A values and 128 x 32 B
  // values (as 16-byte chunks) global -> registers -> LDS.  Thread slot
  // s = (u * 4 + wave) * 64 + lane (u < 4 for A, u < 2 for B) owns LDS chunk
  // s, i.e. row s / 4 and stored chunk s % 4, which holds logical chunk
  // (s % 4) ^ swz_x(row): a wave's LDS stores are 1 KB contiguous and its
  // global loads read whole 64-byte row segments.  The rows a thread loads
  // never change, so their addresses are formed once.
  // Loads are buffer loads: a descriptor per operand (uniform), a fixed
  // per-thread byte offset (one VGPR) and the K step's offset in a scalar
  // register, so no vector register is spent forming addresses; reads past
  // a descriptor's size return zero instead of touching other memory.
  uint32_t a_off[4];
  int a_slot[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int sl = (u * 4 + wv) * kWave + lane;
    const int r = sl >> 2, c = (sl & 3) ^ swz_x(r);
    a_off[u] = (uint32_t)(((size_t)rowidx[r] * K + c * 8) * 2);
    a_slot[u] = sl;
  }
  uint32_t b_off[2];
  int b_slot[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = (u * 4 + wv) * kWave + lane;
    const int r = sl >> 2, c = (sl & 3) ^ swz_x(r);
    const int br = brow(r) < ncols_b ? brow(r) : 0;  // columns past the end: dropped
    b_off[u] = (uint32_t)(((size_t)br * K + c * 8) * 2);
    b_slot[u] = sl;
  }
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(g.a, (size_t)g.a_rows * K * 2);
  const __amdgpu_buffer_rsrc_t rs_b =
      make_rsrc(g.b + (size_t)expert * ncols_b * K * 2, (size_t)ncols_b * K * 2);

  struct Regs {
    u32x4_t a[4];
    u32x4_t b[2];
  };
  auto load = [&](Regs &R, int kb) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      R.a[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_off[u], kb * kBK * 2, 0));
#pragma unroll
    for (int u = 0; u < 2; ++u)
      R.b[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_b, b_off[u], kb * kBK * 2, 0));
  };
  auto store = [&](int stage, const Regs &R) {
    u32x4_t *as = reinterpret_cast<u32x4_t *>(&As[stage][0]);
    u32x4_t *bs = reinterpret_cast<u32x4_t *>(&Bs[stage][0]);
#pragma unroll
    for (int u = 0; u < 4; ++u) as[a_slot[u]] = R.a[u];
#pragma unroll
    for (int u = 0; u < 2; ++u) bs[b_slot[u]] = R.b[u];
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
  const bool mact0 = 64 * wv < nrows, mact1 = 64 * wv + 32 < nrows;

  // One K step kb on LDS stage kb % 2: loads of step kb + 2 into `next`
  // (their latency spans two steps), MFMAs, then step kb + 1's registers
  // (`held`, loaded one step ago) into the other stage, and a barrier.
  auto step = [&](int kb, Regs &next, Regs &held) {
    const int cur = kb & 1;
    // Always issued (past the end: a repeat of the last step, never used),
    // so the wait for `held` is "all but the loads just issued" on every path.
    load(next, min(kb + 2, nk - 1));
    const u32x4_t *Ac = reinterpret_cast<const u32x4_t *>(&As[cur][0]);
    const u32x4_t *Bc = reinterpret_cast<const u32x4_t *>(&Bs[cur][0]);
    // Every operand of the step is read first (one LDS round trip per step,
    // not one per K half), then the two K halves of 16 run back to back.
    u32x4_t av[2][2], bv[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ch = 2 * sub + (lane >> 5);
#pragma unroll
      for (int m = 0; m < 2; ++m) av[sub][m] = Ac[swz(64 * wv + 32 * m + (lane & 31), ch)];
#pragma unroll
      for (int n = 0; n < 4; ++n) bv[sub][n] = Bc[swz(32 * n + (lane & 31), ch)];
    }
    // (rows past the tile's end are computed too: the waves of a block run
    // in step, and a branch per wave would only break up the schedule)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[sub][m]),
                                                              __builtin_bit_cast(bf16x8_t, bv[sub][n]),
                                                              acc[m][n], 0, 0, 0);
      }
    }
    // Past the end this stores a repeat of the last step into the stage
    // nobody reads again; unconditional, so the loop body has no branch.
    store(cur ^ 1, held);
    __syncthreads();
  };

  // ---- prologue: step 0 in LDS, step 1 in registers
  Regs ra, rb;
  if (nk > 0) {
    load(ra, 0);
    load(rb, min(1, nk - 1));
    store(0, ra);
  }
  __syncthreads();
  // nk is even: every K here (H, I, SI) is a multiple of 64.
  for (int kb = 0; kb < nk; kb += 2) {
    step(kb, ra, rb);      // loads step kb + 2 into ra, stores step kb + 1 from rb
    step(kb + 1, rb, ra);  // loads step kb + 3 into rb, stores step kb + 2 from ra
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // the repeated loads of the last steps

  // ---- epilogue: acc[m][n][r] is C[row, col], row = 64 wv + 32 m + 8 (r / 4)
  // + 4 (lane / 32) + r % 4, col = 32 n + lane % 32.
  const int cl = lane & 31;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (!(m == 0 ? mact0 : mact1)) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 64 * wv + 32 * m + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= nrows) continue;
      const int orow = outrow[row];
      if constexpr (kGateUp) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = n0 + 32 * n + cl;
          g.c[(size_t)orow * g.ldc + col] = (uint16_t)f32_to_bf16(swiglu(acc[m][n][r], acc[m][n + 2][r]));
        }
      } else {  // kSharedDown, kBf16Down
#pragma unroll
        for (int n = 0; n < 4; ++n)
          g.c[(size_t)orow * g.ldc + n0 + 32 * n + cl] = (uint16_t)f32_to_bf16(acc[m][n][r]);
      }
    }
  }
}

// ---- The routed experts' GEMMs: one wave per SIMD, a 256 x 256 tile.
//
// Tile: 256 rows (pairs of one expert) x 256 columns (B rows), K stages of
// 64.  The block's 256 rows are eight 32-row slices; wave w owns slices w and
// w + 4 (so a short tile still spreads over every wave) and all 256 columns:
// 2 x 8 MFMA tiles of 32 x 32, 256 accumulator registers, which is why the
// kernel runs a single wave per SIMD (the accumulators sit in the AGPRs).
//  - A (activation rows) is not shared between waves: each lane loads its
//    rows' 64-byte K slices straight into registers, two stages ahead.
//  - B (NVFP4) is dequantised by every thread (one column: the stage's 64
//    values) into LDS, three buffers deep: codes are loaded four stages
//    ahead and dequantised two stages ahead, one barrier per stage, so the
//    MFMA operand reads never wait for the barrier.
//  - Operand lane l (row l % 32) holds k = 16 sub + 8 (l / 32) + 0..7 of
//    the stage for sub-step sub (the MFMA's own layout): each A load moves
//    32 contiguous bytes of each of 32 rows.
//  - The MFMA forms C^T (B is the first operand): a lane then holds four
//    consecutive output columns of one row, stored as 8 bytes.
// Slices past the tile's end are skipped: per wave 0, 1 or 2 live slices,
// each a separately compiled loop.
constexpr int kRBM = 256;   // tile rows
constexpr int kRBN = 256;   // tile columns (B rows)
constexpr int kRBK = 64;    // K per stage
constexpr int kRStages = 3; // LDS buffers of dequantised B
constexpr int kMaxTiles = 64; // tiles per block (the grid is sized for it)

// 16-byte chunk c (0..7, k = 8c .. 8c + 7 of the stage) of tile column r.
// Conflict-free for the MFMA reads (16 lanes: 16 consecutive columns, one
// chunk) and the dequant stores (16 lanes: 16 consecutive columns).
__device__ __forceinline__ int rswz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int N>
using IC = std::integral_constant<int, N>;

template <int MODE>
__global__ void __launch_bounds__(kGThreads, 1) routed_gemm_kernel(GemmArgs g) {
  constexpr bool kGU = MODE == kRoutedGateUp;
  constexpr int BN = kRBN, NN = BN / 32;  // tile columns, MFMA column tiles
  __shared__ u32x4_t Bs[kRStages][BN * 8];
  __shared__ int rows_s[2][kRBM];      // A row (token or pair) of each tile row, by tile parity
  __shared__ int outs_s[2][kRBM];      // output row of each tile row, -1 = none
  __shared__ int4 tiles_s[kMaxTiles];  // (expert, first pair, rows, column tile)
  __shared__ int ntiles_s;

  const int lane = lane_id(), wv = wave_id();
  const int colw = kGU ? BN / 2 : BN;  // output columns per tile
  const int ntn = (g.ncols + colw - 1) / colw;

  // This block's tiles.  Expert e has ceil(count_e / 256) row tiles, all
  // full but its last.  Row tiles are ordered by cost: every full tile, then
  // the partial ones of more than 128 rows (two slices on some wave: a full
  // tile's time), then those of at most 128 rows (half that), each class in
  // expert order.  Row tile rt belongs to XCD rt % 8 (blocks are dealt to
  // the XCDs round-robin); an XCD's tiles, row tile by row tile with its
  // column tiles consecutive (they share the XCD's L2), are dealt to its
  // blocks costliest first.
  for (int i = threadIdx.x; i < g.E; i += kGThreads) rows_s[0][i] = g.counts[i];
  __syncthreads();
  if (wv == 0) {
    int c4[4], nf[4], nl[4], ns[4], tf = 0, tl = 0, ts = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = 4 * lane + i;
      c4[i] = ee < g.E ? rows_s[0][ee] : 0;
      const int rem = c4[i] % kRBM;
      nf[i] = c4[i] / kRBM;
      nl[i] = rem > kRBM / 2;
      ns[i] = rem > 0 && rem <= kRBM / 2;
      tf += nf[i];
      tl += nl[i];
      ts += ns[i];
    }
    int pf = tf, pl = tl, ps = ts;  // inclusive prefixes over lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int xf = __shfl_up(pf, o, kWave), xl = __shfl_up(pl, o, kWave), xs = __shfl_up(ps, o, kWave);
      if (lane >= o) {
        pf += xf;
        pl += xl;
        ps += xs;
      }
    }
    const int TF = __shfl(pf, kWave - 1, kWave), TL = __shfl(pl, kWave - 1, kWave),
              TS = __shfl(ps, kWave - 1, kWave);
    const int x = blockIdx.x % 8, S = gridDim.x / 8, T = TF + TL + TS;
    const int L = (T > x ? (T - x + 7) / 8 : 0) * ntn;  // this XCD's tiles
    // round r of the deal gives block j the XCD's tile r S + j (r even) or
    // r S + S - 1 - j (r odd), which evens out the cost-ordered list
    const int jb = blockIdx.x / 8;
    int n = 0;
    for (int r = 0; r * S < L && n < kMaxTiles; ++r) {
      const int i = r * S + ((r & 1) ? S - 1 - jb : jb);
      if (i >= L) continue;
      const int rt = x + 8 * (i / ntn);
      const int cls = rt < TF ? 0 : (rt < TF + TL ? 1 : 2);
      const int j = cls == 0 ? rt : (cls == 1 ? rt - TF : rt - TF - TL);
      int acc = cls == 0 ? pf - tf : (cls == 1 ? pl - tl : ps - ts);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int cnt = cls == 0 ? nf[q4] : (cls == 1 ? nl[q4] : ns[q4]);
        if (j >= acc && j < acc + cnt) {
          const int q = cls == 0 ? j - acc : nf[q4];
          tiles_s[n] = make_int4(4 * lane + q4, q * kRBM, min(kRBM, c4[q4] - q * kRBM), i % ntn);
        }
        acc += cnt;
      }
      ++n;
    }
    if (lane == 0) ntiles_s = n;
  }
  __syncthreads();
  const int ntiles = ntiles_s;
  if (ntiles == 0) return;
  // Row lists: this thread's entry (tile row threadIdx.x) of tile k; rows
  // past the tile's end repeat its first (loaded by no live slice).
  auto fetch_row = [&](int k) -> int {
    const int4 t = tiles_s[k];
    return g.lists[(size_t)t.x * g.list_stride + t.y + ((int)threadIdx.x < t.z ? threadIdx.x : 0)];
  };
  auto store_row = [&](int slot, int k, int p) {
    rows_s[slot][threadIdx.x] = kGU ? p / g.top_k : p;
    outs_s[slot][threadIdx.x] = (int)threadIdx.x < tiles_s[k].z ? p : -1;
  };
  store_row(0, 0, fetch_row(0));  // (rows_s[0] held the counts: read above)
  __syncthreads();

  for (int k = 0; k < ntiles; ++k) {
    // the next tile's row list, in flight during this one (past the last
    // tile: a repeat of it, unused)
    const int pnext = fetch_row(min(k + 1, ntiles - 1));
    const int e = __builtin_amdgcn_readfirstlane(tiles_s[k].x);
    const int nrows = __builtin_amdgcn_readfirstlane(tiles_s[k].z);
    const int nt = __builtin_amdgcn_readfirstlane(tiles_s[k].w);
    const int *rowidx = rows_s[k & 1];
    const int *outrow = outs_s[k & 1];
    const int K = g.K, nk = K / kRBK;
    const int n0 = nt * colw;
    // B row of this thread's tile column (gate/up: columns 0..127 gate rows
    // n0 + c, 128..255 the matching up rows I + n0 + c); past the end: row 0.
    const int tc = threadIdx.x;
    int brow;
    if constexpr (kGU) {
      const int c = n0 + (tc & (BN / 2 - 1));
      brow = c < g.ncols ? (tc < BN / 2 ? c : g.I + c) : 0;
    } else {
      const int c = n0 + tc;
      brow = c < g.ncols ? c : 0;
    }
    const int ncols_b = kGU ? 2 * g.I : g.ncols;
    const size_t bexp = (size_t)e * ncols_b;
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(g.a, (size_t)g.a_rows * K * 2);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(g.b + bexp * (K / 2), (size_t)ncols_b * (K / 2));
    const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(g.bs + bexp * (K / 16), (size_t)ncols_b * (K / 16));
    const uint32_t bc_off = (uint32_t)brow * (K / 2), bs_off = (uint32_t)brow * (K / 16);

    // live 32-row slices of this wave: w (m = 0) and w + 4 (m = 1)
    const int nh = (nrows + 31) / 32;
    const int nm = (nh > wv) + (nh > wv + 4);
    const int h = lane >> 5;
    uint32_t a_off[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
      a_off[m] = (uint32_t)rowidx[32 * (wv + 4 * m) + (lane & 31)] * (uint32_t)(K * 2) + h * 16;

    struct Codes {
      u32x4_t c[2];  // 64 E2M1 codes: k = 32 i + 0..31
      uint32_t s;    // 4 E4M3 scales, one per 16 k
    };
    auto load_codes = [&](Codes &C, int s) {
      C.c[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_b, bc_off, s * 32, 0));
      C.c[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_b, bc_off, s * 32 + 16, 0));
      C.s = __builtin_amdgcn_raw_buffer_load_b32(rs_s, bs_off, s * 4, 0);
    };
    // Chunks 2 q and 2 q + 1 (k = 16 q .. 16 q + 15, scale byte q) of this
    // thread's column into an LDS buffer.
    auto dequant_pair = [&](u32x4_t *buf, const Codes &C, auto q_c) {
      constexpr int q = decltype(q_c)::value;
      const float sc = __builtin_amdgcn_cvt_f32_fp8((int)C.s, q);
      const u32x4_t &cw = C.c[q >> 1];
      buf[rswz(tc, 2 * q)] = dequant8(cw[2 * (q & 1)], sc);
      buf[rswz(tc, 2 * q + 1)] = dequant8(cw[2 * (q & 1) + 1], sc);
    };
    auto dequant_store = [&](u32x4_t *buf, const Codes &C) {
      dequant_pair(buf, C, IC<0>{});
      dequant_pair(buf, C, IC<1>{});
      dequant_pair(buf, C, IC<2>{});
      dequant_pair(buf, C, IC<3>{});
    };
    const float alpha = g.alpha[e];

    auto run = [&](auto nm_c) {
      constexpr int NM = decltype(nm_c)::value;
      constexpr int NA = NM > 0 ? NM : 1;
      f32x16_t acc[NA][NN];
#pragma unroll
      for (int m = 0; m < NA; ++m)
#pragma unroll
        for (int n = 0; n < NN; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
      u32x4_t A[3][NA][4];
      Codes C[3];
      auto load_a_m = [&](u32x4_t (&dst)[4], int m, int s) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[q] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_off[m], s * (kRBK * 2) + q * 32, 0));
      };
      auto load_a = [&](u32x4_t (&dst)[NA][4], int s) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[m][q] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_off[m], s * (kRBK * 2) + q * 32, 0));
      };
      // Stage s (J = s % 3) computes from LDS buffer J and registers A[J]; the
      // B tile of s + 1 is already in buffer J + 1 and s + 2's is dequantised
      // into buffer J + 2 during the stage, so the operand reads run ahead
      // across the stage's barrier (which only orders the dequant stores of
      // the next stage after this stage's reads of the buffer they reuse).
      // Requests: codes of s + 4 and A of s + 2, in the order they are
      // consumed, so each wait covers only what it needs.  Sub-step q reads
      // the B operands of the next sub-step (for q = 3: sub-step 0 of s + 1),
      // runs the MFMAs of q and dequantises a quarter of the codes of s + 2;
      // scheduling barriers keep each sub-step's work together.  Past the last
      // stage the loads repeat it and the stores fill a buffer never read.
      u32x4_t bf[2][NN];
      auto read_b = [&](u32x4_t (&dst)[NN], const u32x4_t *buf, int sub) {
        if constexpr (NM > 0) {
#pragma unroll
          for (int n = 0; n < NN; ++n) dst[n] = buf[rswz(32 * n + (lane & 31), 2 * sub + h)];
        }
      };
      auto stage = [&](auto j_c, int s) {
        constexpr int J = decltype(j_c)::value, J1 = (J + 1) % 3, J2 = (J + 2) % 3;
        auto sub_step = [&](auto q_c) {
          constexpr int q = decltype(q_c)::value;
          // the stage's requests, spread over the first sub-steps
          if constexpr (q == 0) load_codes(C[J1], min(s + 4, nk - 1));
          if constexpr (q == 1 && NM > 0) load_a_m(A[J2][0], 0, min(s + 2, nk - 1));
          if constexpr (q == 2 && NM > 1) load_a_m(A[J2][1], 1, min(s + 2, nk - 1));
          if constexpr (q < 3) read_b(bf[(q + 1) & 1], Bs[J], q + 1);
          else read_b(bf[0], Bs[J1], 0);
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NN; ++n)
              acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bf[q & 1][n]),
                                                                  __builtin_bit_cast(bf16x8_t, A[J][m][q]),
                                                                  acc[m][n], 0, 0, 0);
          dequant_pair(Bs[J2], C[J2], q_c);
          __builtin_amdgcn_sched_barrier(0);
        };
        sub_step(IC<0>{});
        sub_step(IC<1>{});
        sub_step(IC<2>{});
        sub_step(IC<3>{});
        __syncthreads();
      };

      // prologue: B tiles 0 and 1 in LDS, codes of 2 and 3 and A of 0 and 1
      // requested, B operands of stage 0's first sub-step read
      load_codes(C[0], 0);
      load_codes(C[1], min(1, nk - 1));
      load_codes(C[2], min(2, nk - 1));
      load_a(A[0], 0);
      load_a(A[1], min(1, nk - 1));
      dequant_store(Bs[0], C[0]);
      dequant_store(Bs[1], C[1]);
      load_codes(C[0], min(3, nk - 1));
      __syncthreads();
      read_b(bf[0], Bs[0], 0);
      int s = 0;
      for (; s + 3 <= nk; s += 3) {
        stage(IC<0>{}, s);
        stage(IC<1>{}, s + 1);
        stage(IC<2>{}, s + 2);
      }
      if (s < nk) stage(IC<0>{}, s);
      if (s + 1 < nk) stage(IC<1>{}, s + 1);
      // the next tile's rows into the other slot (read after the barrier that
      // starts the next tile)
      store_row((k + 1) & 1, min(k + 1, ntiles - 1), pnext);

      // acc[m][n][r]: row 32 (wv + 4 m) + lane % 32, column 32 n + 8 (r / 4) +
      // 4 (lane / 32) + r % 4 of the tile.
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int orow = outrow[32 * (wv + 4 * m) + (lane & 31)];
        if (orow < 0) continue;
        uint16_t *crow = g.c + (size_t)orow * g.ldc;
#pragma unroll
        for (int n = 0; n < (kGU ? NN / 2 : NN); ++n)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = n0 + 32 * n + 8 * gq + 4 * h;
            if (col >= g.ncols) continue;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (kGU)
                o[i] = swiglu(acc[m][n][4 * gq + i] * alpha, acc[m][n + NN / 2][4 * gq + i] * alpha);
              else o[i] = acc[m][n][4 * gq + i] * alpha;
            }
            *reinterpret_cast<uint2 *>(crow + col) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          }
      }
    };
    if (nm == 2) run(IC<2>{});
    else if (nm == 1) run(IC<1>{});
    else run(IC<0>{});
    __syncthreads();
  }
}

// Router logits of the grouped path: logits[t, c] = bf16(fp32 x[t] . R[c]).
// A block takes 16 tokens and up to 128 experts (blockIdx.y: which 128);
// wave w owns experts 32 w .. 32 w + 31 as two 16 x 16 tiles on
// v_mfma_f32_16x16x32_bf16 (tokens are the first operand), over all of K
// (in an order that starts at a chunk of the block's own).  K goes in chunks of 128: the block's x rows and router rows of a
// chunk are moved global -> LDS with direct loads (16 lanes read one row's
// 256 contiguous bytes), three chunks ahead in four buffers, then read in the MFMA's
// operand layout (lane l: row l % 16, k = 32 s + 8 (l / 16) + 0..7 of
// sub-step s).  The 16-byte chunk c of row r sits at position
// 16 r + (c ^ (r % 16)), so the 16 lanes of a read (16 rows, one chunk)
// hit 16 different bank groups.  (Reading the operands from memory in the
// MFMA layout, each load touching 32 rows, ran at a quarter of this rate.)
constexpr int kRouterTokens = 16;
constexpr int kRouterExperts = 128;
constexpr int kRouterK = 128;  // K per chunk

__device__ __forceinline__ int rt_pos(int r, int c) { return r * 16 + (c ^ (r & 15)); }

__global__ void __launch_bounds__(kGThreads, 1) router_kernel(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ R, int M, int K,
                                                              int E, uint16_t *__restrict__ logits) {
  // four chunk buffers, in separate arrays (a read of one does not wait for
  // the direct loads still in flight into another)
  __shared__ u32x4_t xa0[kRouterTokens * 16], xa1[kRouterTokens * 16], xa2[kRouterTokens * 16],
      xa3[kRouterTokens * 16];
  __shared__ u32x4_t rb0[kRouterExperts * 16], rb1[kRouterExperts * 16], rb2[kRouterExperts * 16],
      rb3[kRouterExperts * 16];
  const int lane = lane_id(), wv = wave_id();
  const int t0 = blockIdx.x * kRouterTokens, e0 = blockIdx.y * kRouterExperts;
  const int nc = K / kRouterK;
  // direct loads: wave w moves x rows (one instruction: 4 rows) when w == 0,
  // and router rows 32 w .. 32 w + 31 (eight instructions); lane j of an
  // instruction fills position 64 i + j = rt_pos(r, c')
  const int c_lane = (lane & 15);  // position within the row
  auto src_chunk = [&](int r) { return c_lane ^ (r & 15); };
  const uint16_t *xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    xrow[i] = x + (size_t)min(t0 + r, M - 1) * K + src_chunk(r) * 8;
  }
  const uint16_t *rrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 32 * wv + 4 * i + (lane >> 4);
    rrow[i] = R + (size_t)min(e0 + r, E - 1) * K + src_chunk(r) * 8;
  }
  // Each block starts at its own chunk of K and goes round: blocks that run
  // at the same time read different router rows' parts, not the same L2
  // lines at once.
  const int c_off = (int)blockIdx.x % nc;
  auto issue = [&](u32x4_t *xa, u32x4_t *rb, int c) {
    const int cc = c + c_off < nc ? c + c_off : c + c_off - nc;
    const int ko = cc * kRouterK;
    if (wv == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(xrow[i] + ko, (__attribute__((address_space(3))) void *)(xa + 64 * i), 16, 0,
                                         0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(rrow[i] + ko,
                                       (__attribute__((address_space(3))) void *)(rb + 64 * (8 * wv + i)), 16, 0, 0);
  };
  typedef __attribute__((ext_vector_type(4))) float f32x4_t;
  f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  auto mma_chunk = [&](const u32x4_t *xa, const u32x4_t *rb) {
#pragma unroll
    for (int s = 0; s < kRouterK / 32; ++s) {
      const int c = 4 * s + (lane >> 4);
      const u32x4_t av = xa[rt_pos(lane & 15, c)];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t bv = rb[rt_pos(32 * wv + 16 * j + (lane & 15), c)];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                         __builtin_bit_cast(bf16x8_t, bv), acc[j], 0, 0, 0);
      }
    }
  };
  auto bufs = [&](auto j_c, auto &&f) {
    constexpr int J = decltype(j_c)::value;
    if constexpr (J == 0) f(xa0, rb0);
    else if constexpr (J == 1) f(xa1, rb1);
    else if constexpr (J == 2) f(xa2, rb2);
    else f(xa3, rb3);
  };
  // Chunk c lives in buffer c % 4.  Every chunk step issues one chunk's
  // loads (past the end: the last chunk again, into a buffer no longer
  // read), so the count of loads issued after chunk c + 1's is always two
  // chunks' worth: wave 0 moves 12 per chunk, the others 8.  The barrier
  // after chunk c waits for chunk c + 1 and for every wave's reads of c.
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    if (wv == 0) __builtin_amdgcn_s_waitcnt(0x4078);  // vmcnt(24) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x4070);           // vmcnt(16) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  bufs(IC<0>{}, [&](u32x4_t *xa, u32x4_t *rb) { issue(xa, rb, 0); });
  bufs(IC<1>{}, [&](u32x4_t *xa, u32x4_t *rb) { issue(xa, rb, min(1, nc - 1)); });
  bufs(IC<2>{}, [&](u32x4_t *xa, u32x4_t *rb) { issue(xa, rb, min(2, nc - 1)); });
  barrier();  // chunk 0 (two chunks issued after it)
  auto step = [&](auto j_c, int c) {
    constexpr int J = decltype(j_c)::value;
    bufs(IC<(J + 3) % 4>{}, [&](u32x4_t *xa, u32x4_t *rb) { issue(xa, rb, min(c + 3, nc - 1)); });
    bufs(j_c, [&](u32x4_t *xa, u32x4_t *rb) { mma_chunk(xa, rb); });
    barrier();
  };
  for (int c = 0; c < nc; c += 4) {
    step(IC<0>{}, c);
    if (c + 1 >= nc) break;
    step(IC<1>{}, c + 1);
    if (c + 2 >= nc) break;
    step(IC<2>{}, c + 2);
    if (c + 3 >= nc) break;
    step(IC<3>{}, c + 3);
  }
  // acc[j][i]: token t0 + 4 (lane / 16) + i, expert e0 + 32 w + 16 j + lane % 16
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + 32 * wv + 16 * j + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * (lane >> 4) + i;
      if (t < M && e < E) logits[(size_t)t * E + e] = (uint16_t)f32_to_bf16(acc[j][i]);
    }
  }
}

// Router logits of decode-size batches: logits[t, c] = bf16(fp32 x[t] . R[c])
// for a tile of 16 tokens x 16 experts per block, K split in eighths over
// the block's eight waves (so a 64-token batch of 128 experts is 32 blocks
// of 256 lanes each, against 8 blocks of the 32 x 32 tiles above).  Each
// wave multiplies its K range on v_mfma_f32_16x16x32_bf16 with both
// operands straight from memory in the MFMA layout (operand lane l: row
// l % 16, k = 32 s + 8 (l / 16) + 0..7 of step s), eight steps of loads in
// flight; the eight partial tiles are added in wave order through LDS (a
// fixed order).  Rows past M or E are clamped to the last row and not
// stored.  K: a multiple of 256.
constexpr int kRsWaves = 8;
constexpr int kRsBatch = 8;  // K steps of 32 per batch of loads

__global__ void __launch_bounds__(kRsWaves * kWave) router_small_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ R, int M, int K, int E,
    uint16_t *__restrict__ logits) {
  typedef __attribute__((ext_vector_type(4))) float f32x4_t;
  __shared__ f32x4_t part[kRsWaves - 1][kWave];
  const int lane = lane_id(), wv = wave_id(), m = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.y * 16, e0 = blockIdx.x * 16;
  const int trow = min(t0 + m, M - 1), erow = min(e0 + m, E - 1);
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(x, (size_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rs_r = make_rsrc(R, (size_t)E * K * 2);
  const int kw = K / kRsWaves;  // this wave's K range [wv kw, wv kw + kw)
  const uint32_t xo = (uint32_t)trow * (uint32_t)(K * 2) + (uint32_t)(wv * kw + q * 8) * 2;
  const uint32_t ro = (uint32_t)erow * (uint32_t)(K * 2) + (uint32_t)(wv * kw + q * 8) * 2;
  const int steps = kw / 32;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < steps; s0 += kRsBatch) {
    u32x4_t a[kRsBatch], b[kRsBatch];
#pragma unroll
    for (int i = 0; i < kRsBatch; ++i) {
      const uint32_t so = s0 + i < steps ? (uint32_t)(s0 + i) * 64 : kOOB;
      a[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_r, ro, so, 0));
      b[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_x, xo, so, 0));
    }
#pragma unroll
    for (int i = 0; i < kRsBatch; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[i]),
                                                    __builtin_bit_cast(bf16x8_t, b[i]), acc, 0, 0, 0);
  }
  if (wv > 0) part[wv - 1][lane] = acc;
  __syncthreads();
  if (wv > 0) return;
#pragma unroll
  for (int w = 0; w < kRsWaves - 1; ++w) acc += part[w][lane];
  // acc[i]: expert e0 + 4 q + i, token t0 + m
  const int t = t0 + m;
  if (t < M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = e0 + 4 * q + i;
      if (c < E) logits[(size_t)t * E + c] = (uint16_t)f32_to_bf16(acc[i]);
    }
  }
}

bool router_small_supported(int M, int H, int E, int top_k) {
  return M >= 1 && M <= kSkinnyMaxM && H % (kRsWaves * 32) == 0 && (long)M * top_k <= kMaxDecodePairs &&
         E <= kMaxExperts;
}

// out[t, h] = bf16(bf16(sum_j tw[t, j] y[t*k + j, h]) + sh[t, h]) for 8
// consecutive h per thread: the k rows of y are loaded together (16 bytes
// each), the sum is exact in fp64 (every product has 16 significant bits)
// and rounded once to fp32.  sh == NULL: no shared expert.
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t *__restrict__ y,
                                                      const float *__restrict__ tw,
                                                      const int32_t *__restrict__ ids,
                                                      const uint16_t *__restrict__ sh, int M, int H,
                                                      int E, int k, uint16_t *__restrict__ out) {
  // block (t, c): token t, columns [2048 c, 2048 c + 2048); the token is the
  // block's, so its ids and weights are scalar loads
  const int t = blockIdx.x;
  const int h = ((int)blockIdx.y * 256 + (int)threadIdx.x) * 8;
  if (h >= H) return;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j0 = 0; j0 < k; j0 += 8) {
    u32x4_t v[8];
    float w[8];
    // every y row is loaded at once, independent of the ids (a dropped id
    // gets weight 0; rows past k repeat the last pair's row)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u < k ? j0 + u : k - 1;
      v[u] = load16(y + ((size_t)t * k + j) * H + h);
      const bool on = j0 + u < k && (unsigned)ids[(size_t)t * k + j] < (unsigned)E;
      w[u] = on ? tw[(size_t)t * k + j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += (double)w[u] * (double)bf16_lo(v[u][d]);
        acc[2 * d + 1] += (double)w[u] * (double)bf16_hi(v[u][d]);
      }
  }
  const u32x4_t s = sh ? load16(sh + (size_t)t * H + h) : u32x4_t{0, 0, 0, 0};
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = f32_to_bf16(round_bf16((float)acc[2 * d]) + bf16_lo(s[d]));
    const uint32_t hi = f32_to_bf16(round_bf16((float)acc[2 * d + 1]) + bf16_hi(s[d]));
    o[d] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x4_t *>(out + (size_t)t * H + h) = o;
}

// Pair lists per expert: block e compacts the pairs p (ascending) whose
// expert is e into lists[e][0 .. count), count into counts[e].  The ids are
// read in chunks of 8192 (coalesced, staged through LDS, the next chunk's
// loads in flight meanwhile); thread t takes 32 consecutive pairs of a
// chunk, so an exclusive scan of the per-thread match counts over the block
// gives every match its slot, in ascending order.
__global__ void __launch_bounds__(256) plan_lists_kernel(const int32_t *__restrict__ ids, int npairs,
                                                         int32_t *__restrict__ lists, int stride,
                                                         int32_t *__restrict__ counts) {
  constexpr int kPer = 32, kChunk = 256 * kPer;
  __shared__ int sid[kChunk];
  __shared__ int wsum[4];
  const int e = blockIdx.x;
  const int lane = lane_id(), wv = wave_id();
  int v[kPer];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = c0 + i * 256 + (int)threadIdx.x;
      v[i] = p < npairs ? ids[p] : -1;
    }
  };
  int base = 0;
  fetch(0);
  for (int c0 = 0; c0 < npairs; c0 += kChunk) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) sid[i * 256 + threadIdx.x] = v[i];
    __syncthreads();
    fetch(c0 + kChunk);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) m |= (uint32_t)(sid[threadIdx.x * kPer + j] == e) << j;
    const int n = __popc(m);
    int incl = n;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    int off = base + incl - n;
    for (int w = 0; w < wv; ++w) off += wsum[w];
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    while (m) {
      const int j = __ffs(m) - 1;
      m &= m - 1;
      if (off < stride) lists[(size_t)e * stride + off] = c0 + (int)threadIdx.x * kPer + j;
      ++off;
    }
    __syncthreads();  // sid and wsum are rewritten next chunk
  }
  if (threadIdx.x == 0) counts[e] = min(base, stride);  // an expert has <= 1 pair per token
}

template <int MODE>
hipError_t launch_gemm(const GemmArgs &g, int row_tiles, int col_tiles, hipStream_t st) {
  const int nblk = row_tiles * col_tiles;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<MODE>), dim3(nblk), dim3(kGThreads), 0, st, g);
  return hipGetLastError();
}

// The NVFP4 shared expert's row list: rows 0..M-1 of one "expert".
__global__ void __launch_bounds__(256) iota_list_kernel(int32_t *__restrict__ lists, int M,
                                                        int32_t *__restrict__ counts) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < M) lists[i] = i;
  if (i == 0) counts[0] = M;
}

// One block per CU (32 per XCD), more if an XCD's tiles would exceed
// kMaxTiles per block (row_tiles bounds the actual count, known on the
// device).
template <int MODE>
hipError_t launch_routed(const GemmArgs &g, int row_tiles, hipStream_t st) {
  const int colw = MODE == kRoutedGateUp ? kRBN / 2 : kRBN;
  const int col_tiles = (g.ncols + colw - 1) / colw;
  const long per_xcd = (long)(row_tiles + 7) / 8 * col_tiles;
  if (per_xcd <= 0) return hipSuccess;
  const int nblk = 8 * (int)std::max<long>(32, (per_xcd + kMaxTiles - 1) / kMaxTiles);
  hipLaunchKernelGGL((routed_gemm_kernel<MODE>), dim3(nblk), dim3(kGThreads), 0, st, g);
  return hipGetLastError();
}



// The shared expert's two GEMMs depend on x only; without stage events they
// run on a second stream of the device (created on first use, kept for the
// process, default priority) so their blocks fill the CUs the routed GEMMs
// leave idle at their ends.  The caller's stream forks to it after the
// router (an event) and joins it before the combine (another event).
// Enqueueing a call's fork and join is serialised per device by a mutex, so
// calls from several host threads cannot interleave their event records.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu[kMaxDevices];

hipError_t side_stream(int dev, SideStream **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream &sd = g_side[dev];
  if (!sd.s) {
    hipError_t e;
    if ((e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&sd.join, hipEventDisableTiming)) != hipSuccess) return e;
  }
  *out = &sd;
  return hipSuccess;
}

}  // namespace

bool grouped_shape_supported(int H, int I, int SI) {
  return H % 128 == 0 && I % 64 == 0 && H >= 128 && I >= 64 && H <= 8192 && I <= 8192 &&
         (SI == 0 || (SI % 64 == 0 && SI >= 64 && SI <= 8192));
}

hipError_t launch_grouped(const GroupedArgs &a, hipStream_t st) {
  const int M = a.M, H = a.H, E = a.E, I = a.I, k = a.top_k, SI = a.SI;
  const int P = M * k;
  hipError_t err;
  auto mark = [&](int i) -> hipError_t {
    return (a.events && a.events[i]) ? hipEventRecord((hipEvent_t)a.events[i], st) : hipSuccess;
  };
  // Few tokens (decode-size batches): every expert GEMM on the skinny
  // kernels, whose waves each stream their own weight rows and which find
  // their rows from the routing ids themselves (no pair lists).
  const bool sk = M <= kSkinnyMaxM && (long)P <= kMaxDecodePairs && skinny_shape_supported(H, I, true) &&
                  skinny_shape_supported(I, H, false) &&
                  (!a.sgu || (skinny_shape_supported(H, SI, true) && skinny_shape_supported(SI, H, false)));
  // 1. router logits and top-k (skipped with forced routing); decode-size
  // batches take the small-tile router
  if ((err = mark(0)) != hipSuccess) return err;
  if (!a.ids_in) {
    if (router_small_supported(M, H, E, k))
      hipLaunchKernelGGL(router_small_kernel, dim3((E + 15) / 16, (M + 15) / 16), dim3(kRsWaves * kWave),
                         0, st, a.x, a.router, M, H, E, a.logits);
    else
      hipLaunchKernelGGL(router_kernel,
                         dim3((M + kRouterTokens - 1) / kRouterTokens, (E + kRouterExperts - 1) / kRouterExperts),
                         dim3(kGThreads), 0, st, a.x, a.router, M, H, E, a.logits);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_topk(a.logits, M, E, k, a.ids, a.tw, nullptr, st)) != hipSuccess) return err;
  }
  // 2. pair lists per expert (not for the skinny GEMMs)
  if ((err = mark(1)) != hipSuccess) return err;
  if (!sk) {
    hipLaunchKernelGGL(plan_lists_kernel, dim3(E), dim3(256), 0, st, a.ids, P, a.lists, M, a.counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 3. shared gate/up (and 6. shared down): on the side stream unless
  // stage events are asked for
  if ((err = mark(2)) != hipSuccess) return err;
  // (the skinny GEMMs compute the shared expert in the routed launches)
  const bool side = a.sgu && !a.events && !a.inline_shared && !sk;
  auto sk_args = [&](const uint16_t *A, int a_rows, const void *w, const uint8_t *ws,
                     const float *alpha, uint16_t *c, int c_rows, const int32_t *ids, int E_, int K,
                     int wrows, int ncols) -> SkinnyArgs {
    SkinnyArgs g{};
    g.a = A;
    g.a_rows = a_rows;
    g.w = static_cast<const uint8_t *>(w);
    g.ws = ws;
    g.alpha = alpha;
    g.c = c;
    g.c_rows = c_rows;
    g.ids = ids;
    g.top_k = k;
    g.nrows = M;
    g.K = K;
    g.wrows = wrows;
    g.ncols = ncols;
    g.ldc = ncols;
    g.I = ncols;
    g.E = E_;
    return g;
  };
  hipStream_t sst = st;
  std::unique_lock<std::mutex> side_lock;
  SideStream *sd = nullptr;
  if (side) {
    int dev = 0;
    if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    side_lock = std::unique_lock<std::mutex>(g_side_mu[dev]);
    if ((err = side_stream(dev, &sd)) != hipSuccess) return err;
    if ((err = hipEventRecord(sd->fork, st)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(sd->s, sd->fork, 0)) != hipSuccess) return err;
    sst = sd->s;
  }
  // NVFP4 shared expert: the routed kernels with one expert whose list is
  // every row (its codes, scales and global scale in place of W13 / W2)
  auto nv_shared = [&](int mode) -> hipError_t {
    GemmArgs g{};
    g.top_k = 1;
    g.lists = a.sh_lists;
    g.counts = a.sh_counts;
    g.list_stride = M;
    g.E = 1;
    g.a_rows = M;
    if (mode == kRoutedGateUp) {
      g.a = a.x;
      g.b = reinterpret_cast<const uint8_t *>(a.sgu);
      g.bs = a.s_gu;
      g.alpha = a.a_gu;
      g.c = a.sact;
      g.K = H;
      g.ncols = SI;
      g.ldc = SI;
      g.I = SI;
      return launch_routed<kRoutedGateUp>(g, (M + kRBM - 1) / kRBM + 1, sst);
    }
    g.a = a.sact;
    g.b = reinterpret_cast<const uint8_t *>(a.sdown);
    g.bs = a.s_down;
    g.alpha = a.a_down;
    g.c = a.sh;
    g.K = SI;
    g.ncols = H;
    g.ldc = H;
    return launch_routed<kRoutedDown>(g, (M + kRBM - 1) / kRBM + 1, sst);
  };
  auto shared_down = [&]() -> hipError_t {
    if (a.s_gu) return nv_shared(kRoutedDown);
    GemmArgs sdn{};
    sdn.a = a.sact;
    sdn.b = reinterpret_cast<const uint8_t *>(a.sdown);
    sdn.c = a.sh;
    sdn.rows = M;
    sdn.a_rows = M;
    sdn.K = SI;
    sdn.ncols = H;
    sdn.ldc = H;
    return launch_gemm<kSharedDown>(sdn, (M + kBM - 1) / kBM, H / kBN, sst);
  };
  if (a.sgu && sk) {
    // with the routed gate/up below
  } else if (a.sgu && a.s_gu) {
    hipLaunchKernelGGL(iota_list_kernel, dim3((M + 255) / 256), dim3(256), 0, sst, a.sh_lists, M, a.sh_counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = nv_shared(kRoutedGateUp)) != hipSuccess) return err;
    if (side) {
      if ((err = shared_down()) != hipSuccess) return err;
      if ((err = hipEventRecord(sd->join, sst)) != hipSuccess) return err;
    }
  } else if (a.sgu) {
    GemmArgs s{};
    s.a = a.x;
    s.b = reinterpret_cast<const uint8_t *>(a.sgu);
    s.c = a.sact;
    s.rows = M;
    s.a_rows = M;
    s.K = H;
    s.ncols = SI;
    s.ldc = SI;
    s.I = SI;
    if ((err = launch_gemm<kSharedGateUp>(s, (M + kBM - 1) / kBM, SI / (kBN / 2), sst)) != hipSuccess)
      return err;
    if (side) {
      if ((err = shared_down()) != hipSuccess) return err;
      if ((err = hipEventRecord(sd->join, sst)) != hipSuccess) return err;
    }
  }
  // 4. routed gate/up: row tiles bounded by sum_e ceil(count_e / 256)
  if ((err = mark(3)) != hipSuccess) return err;
  const int max_row_tiles = (P + kRBM - 1) / kRBM + E;
  if (sk) {
    // gate/up of the routed experts and of the shared expert in one launch,
    // then their down projections in another (the shared units read sact,
    // which the first launch completed)
    const bool bf = a.bw13 != nullptr;
    const int rf = bf ? kBf16 : kNvfp4, sf = a.s_gu ? kNvfp4 : kBf16;
    const SkinnyArgs rgu = sk_args(a.x, M, bf ? (const void *)a.bw13 : (const void *)a.w13,
                                   bf ? nullptr : a.s13, bf ? nullptr : a.a13, a.act, P, a.ids, E, H,
                                   2 * I, I);
    const SkinnyArgs sgu = sk_args(a.x, M, a.sgu, a.s_gu, a.a_gu, a.sact, M, nullptr, 1, H, 2 * SI, SI);
    if ((err = launch_skinny(rgu, rf, a.sgu ? &sgu : nullptr, sf, true, st)) != hipSuccess) return err;
    // 5. routed down
    if ((err = mark(4)) != hipSuccess) return err;
    const SkinnyArgs rdn = sk_args(a.act, P, bf ? (const void *)a.bw2 : (const void *)a.w2,
                                   bf ? nullptr : a.s2, bf ? nullptr : a.a2, a.y, P, a.ids, E, I, H, H);
    const SkinnyArgs sdn = sk_args(a.sact, M, a.sdown, a.s_down, a.a_down, a.sh, M, nullptr, 1, SI, H, H);
    if ((err = launch_skinny(rdn, rf, a.sgu ? &sdn : nullptr, sf, false, st)) != hipSuccess) return err;
  } else if (a.bw13) {
    // BF16 experts: gemm_kernel on the pair lists (the row tiles of every
    // expert, in expert order; blocks past the last tile exit at once)
    GemmArgs gu{};
    gu.a = a.x;
    gu.a_rows = M;
    gu.b = reinterpret_cast<const uint8_t *>(a.bw13);
    gu.c = a.act;
    gu.K = H;
    gu.ncols = I;
    gu.ldc = I;
    gu.I = I;
    gu.top_k = k;
    gu.lists = a.lists;
    gu.counts = a.counts;
    gu.list_stride = M;
    gu.E = E;
    if ((err = launch_gemm<kBf16GateUp>(gu, max_row_tiles, I / (kBN / 2), st)) != hipSuccess) return err;
    // 5. routed down
    if ((err = mark(4)) != hipSuccess) return err;
    GemmArgs dn{};
    dn.a = a.act;
    dn.a_rows = P;
    dn.b = reinterpret_cast<const uint8_t *>(a.bw2);
    dn.c = a.y;
    dn.K = I;
    dn.ncols = H;
    dn.ldc = H;
    dn.top_k = k;
    dn.lists = a.lists;
    dn.counts = a.counts;
    dn.list_stride = M;
    dn.E = E;
    if ((err = launch_gemm<kBf16Down>(dn, max_row_tiles, H / kBN, st)) != hipSuccess) return err;
  } else {
    GemmArgs gu{};
    gu.a = a.x;
    gu.a_rows = M;
    gu.b = a.w13;
    gu.bs = a.s13;
    gu.alpha = a.a13;
    gu.c = a.act;
    gu.K = H;
    gu.ncols = I;
    gu.ldc = I;
    gu.I = I;
    gu.top_k = k;
    gu.lists = a.lists;
    gu.counts = a.counts;
    gu.list_stride = M;
    gu.E = E;
    if ((err = launch_routed<kRoutedGateUp>(gu, max_row_tiles, st)) != hipSuccess) return err;
    // 5. routed down
    if ((err = mark(4)) != hipSuccess) return err;
    GemmArgs dn{};
    dn.a = a.act;
    dn.a_rows = P;
    dn.b = a.w2;
    dn.bs = a.s2;
    dn.alpha = a.a2;
    dn.c = a.y;
    dn.K = I;
    dn.ncols = H;
    dn.ldc = H;
    dn.top_k = k;
    dn.lists = a.lists;
    dn.counts = a.counts;
    dn.list_stride = M;
    dn.E = E;
    if ((err = launch_routed<kRoutedDown>(dn, max_row_tiles, st)) != hipSuccess) return err;
  }
  // 6. shared down -> sh (already queued on the side stream: join it)
  if ((err = mark(5)) != hipSuccess) return err;
  if (side) {
    if ((err = hipStreamWaitEvent(st, sd->join, 0)) != hipSuccess) return err;
  } else if (a.sgu && !sk) {
    if ((err = shared_down()) != hipSuccess) return err;
  }
  // 7. combine + shared add (a precomputed shared output: once its event
  // has completed)
  if ((err = mark(6)) != hipSuccess) return err;
  if (a.sh_ext && a.sh_ready && (err = hipStreamWaitEvent(st, (hipEvent_t)a.sh_ready, 0)) != hipSuccess)
    return err;
  {
    const uint16_t *shp = a.sh_ext ? a.sh_ext : (a.sgu ? a.sh : nullptr);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)M, (unsigned)((H / 8 + 255) / 256)), dim3(256), 0, st,
                       a.y, a.tw,
                       a.ids, shp, M, H, E, k, a.out);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return mark(7);
}

}  // namespace flint
