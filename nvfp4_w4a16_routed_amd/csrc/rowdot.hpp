// Per-lane row dot products of the expert GEMVs (gfx950, wave64).
//
// A weight row of K elements is split in 16-byte chunks (32 NVFP4 codes or 8
// bf16 values).  LPR lanes share a row; lane q of a row owns chunks
// q + LPR * i (i < CPL), so every load instruction reads LPR * 16 contiguous
// bytes of the row and 64 / LPR rows are in flight per instruction.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace flint {

constexpr int pow2_divisor(int n, int cap) {
  int p = 1;
  while (p * 2 <= cap && n % (p * 2) == 0) p *= 2;
  return p;
}

// Lane mapping of a row: LPR, the largest power-of-two divisor of the chunk
// count (at most 64), lanes share a row and each holds CPL chunks, so every
// lane is busy (a 24-chunk NVFP4 row, I = 768, is 8 lanes x 3 chunks and a
// wave covers 8 rows per load).
template <int FMT, int K>
struct RowMap {
  static constexpr int CE = FMT == kNvfp4 ? 32 : 8;        // elements per chunk
  static constexpr int NC = K / CE;                          // chunks per row
  static constexpr int LPR = pow2_divisor(NC, kWave);        // lanes per row
  static constexpr int CPL = (NC + LPR - 1) / LPR;           // chunks per lane
  static constexpr bool PAD = LPR * CPL != NC;               // some lanes idle
  static constexpr int RS = kWave / LPR;                     // rows per slice
  static constexpr int ROW_BYTES = FMT == kNvfp4 ? K / 2 : K * 2;
  static_assert(K % CE == 0, "row length");
  static_assert(!PAD || CPL == 1, "padded rows hold one chunk per lane");
  __device__ static bool active(int q, int i) { return !PAD || q + LPR * i < NC; }
};

// Weight registers of one row for one lane: raw 16-byte chunks and, for
// NVFP4, the two E4M3 block-scale bytes of each chunk.
template <int FMT, int K>
struct RowRegs {
  using Map = RowMap<FMT, K>;
  u32x4_t raw[Map::CPL];
  uint32_t sc[Map::CPL];
};

// The lane's part of a bf16 vector matching one chunk of a row.
template <int FMT>
struct VecChunk {
  static constexpr int U4 = FMT == kNvfp4 ? 4 : 1;  // 16-byte loads per chunk
  u32x4_t v[U4];
};

// One row's chunks for lane q: codes (or bf16 values) at byte offset woff of
// descriptor w, NVFP4 scales at soff of descriptor s.  Every load is issued
// (idle lanes and rows past a share read out of range, which returns zero
// and costs no memory traffic), so the number of loads never varies.
template <int FMT, int K>
__device__ __forceinline__ void load_row(RowRegs<FMT, K> &r, __amdgpu_buffer_rsrc_t w,
                                         uint32_t woff, __amdgpu_buffer_rsrc_t s, uint32_t soff,
                                         int q) {
  using Map = RowMap<FMT, K>;
#pragma unroll
  for (int i = 0; i < Map::CPL; ++i) {
    const int c = q + Map::LPR * i;
    const bool on = Map::active(q, i);
    r.raw[i] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w, on ? woff + c * 16 : kOOB, 0, kPolicyStream));
    r.sc[i] = 0;
    if constexpr (FMT == kNvfp4)
      r.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(s, on ? soff + c * 2 : kOOB, 0, 0);
  }
}

// Where a vector is read from: an input in global memory (plain loads),
// data other waves of the grid wrote (device-scope loads; see the
// signalling notes in common.hpp), or a copy in LDS.
enum VecSrc { kSrcGlobal = 0, kSrcDevice = 1, kSrcLds = 2 };

// Chunk i of the lane's part of vector `vec` (K elements).
template <int FMT, int K, int SRC>
__device__ __forceinline__ void load_chunk(VecChunk<FMT> &x, const uint16_t *vec, int q, int i) {
  using Map = RowMap<FMT, K>;
  const uint16_t *p = vec + (size_t)(q + Map::LPR * i) * Map::CE;
  const bool on = Map::active(q, i);
#pragma unroll
  for (int u = 0; u < VecChunk<FMT>::U4; ++u) {
    if (!on)
      x.v[u] = u32x4_t{0, 0, 0, 0};
    else if constexpr (SRC == kSrcDevice)
      x.v[u] = ld_dev16(p + 8 * u);
    else
      x.v[u] = load16(p + 8 * u);  // global or LDS (address space inferred)
  }
}

// Partial dot product of one chunk of a row with the matching vector part.
// NVFP4: codes -> bf16 pairs (hardware converter), bf16 dot2 into fp32 per
// 16-element block, times the block's E4M3 scale (exact), summed in fp32.
template <int FMT>
__device__ __forceinline__ float chunk_dot(const u32x4_t &raw, uint32_t sc, const VecChunk<FMT> &x) {
  if constexpr (FMT == kNvfp4) {
    float part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t va = x.v[2 * h];
      const u32x4_t vb = x.v[2 * h + 1];
      uint32_t w0[4], w1[4];
      fp4x8_to_bf16(raw[2 * h], w0);
      fp4x8_to_bf16(raw[2 * h + 1], w1);
      float p = dot2_bf16(w0[0], va[0], 0.0f);
      p = dot2_bf16(w0[1], va[1], p);
      p = dot2_bf16(w0[2], va[2], p);
      p = dot2_bf16(w0[3], va[3], p);
      p = dot2_bf16(w1[0], vb[0], p);
      p = dot2_bf16(w1[1], vb[1], p);
      p = dot2_bf16(w1[2], vb[2], p);
      p = dot2_bf16(w1[3], vb[3], p);
      part[h] = p;
    }
    return part[0] * e4m3_to_f32(sc & 0xffu) + part[1] * e4m3_to_f32((sc >> 8) & 0xffu);
  } else {
    (void)sc;
    const u32x4_t va = x.v[0];
    float p = dot2_bf16(raw[0], va[0], 0.0f);
    p = dot2_bf16(raw[1], va[1], p);
    p = dot2_bf16(raw[2], va[2], p);
    return dot2_bf16(raw[3], va[3], p);
  }
}

// All chunks of the lane's part of one vector.
template <int FMT, int K>
struct VecRegs {
  VecChunk<FMT> c[RowMap<FMT, K>::CPL];
};

template <int FMT, int K, int SRC>
__device__ __forceinline__ void load_vec(VecRegs<FMT, K> &x, const uint16_t *vec, int q) {
#pragma unroll
  for (int i = 0; i < RowMap<FMT, K>::CPL; ++i) load_chunk<FMT, K, SRC>(x.c[i], vec, q, i);
}

// A copy of one chunk of weight registers that the compiler must treat as
// changed here: the caller converts codes to bf16 per use instead of
// hoisting the conversion of every row out of a loop over vectors (that
// would hold all rows' converted codes at once and exceed the register
// budget; converting per use costs half an instruction per element).
__device__ __forceinline__ u32x4_t opaque_chunk(u32x4_t raw) {
  asm volatile("" : "+v"(raw));
  return raw;
}

// Per-lane partial dot products of NR rows with a vector held in registers.
template <int FMT, int K, int NR>
__device__ __forceinline__ void rows_dot_regs(const RowRegs<FMT, K> (&rows)[NR],
                                              const VecRegs<FMT, K> &x, float (&acc)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < RowMap<FMT, K>::CPL; ++i)
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      acc[r] += chunk_dot<FMT>(opaque_chunk(rows[r].raw[i]), rows[r].sc[i], x.c[i]);
      // One row's converted codes live at a time (keeps the register budget).
      if constexpr (FMT == kNvfp4) __builtin_amdgcn_sched_barrier(0);
    }
}

// Per-lane partial dot products of NR rows (all with the same lane mapping)
// with one vector, chunk by chunk so each vector chunk is loaded once.
template <int FMT, int K, int SRC, int NR>
__device__ __forceinline__ void rows_dot(const RowRegs<FMT, K> (&rows)[NR], const uint16_t *vec,
                                         int q, float (&acc)[NR]) {
  using Map = RowMap<FMT, K>;
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < Map::CPL; ++i) {
    VecChunk<FMT> x;
    load_chunk<FMT, K, SRC>(x, vec, q, i);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      acc[r] += chunk_dot<FMT>(opaque_chunk(rows[r].raw[i]), rows[r].sc[i], x);
      if constexpr (FMT == kNvfp4) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Gate/up geometry: row pairs per wave item, whole row slices (2 NVFP4 row
// pairs = 4.6 KB at H = 2048, 1 bf16 row pair = 8 KB).
template <int FMT, int H>
struct GateUpGeo {
  using Map = RowMap<FMT, H>;
  static constexpr int RP_MIN = FMT == kNvfp4 ? 2 : 1;
  static constexpr int RP = Map::RS >= RP_MIN ? Map::RS : RP_MIN;
  static constexpr int NSL = RP / Map::RS;
};

// Down geometry: output rows per wave item, whole slices (8 NVFP4 rows =
// 3.4 KB at I = 768, 4 bf16 rows = 6 KB).
template <int FMT, int I>
struct DownGeo {
  using Map = RowMap<FMT, I>;
  static constexpr int RW_MIN = FMT == kNvfp4 ? 8 : 4;
  static constexpr int RW = Map::RS >= RW_MIN ? Map::RS : RW_MIN;
  static constexpr int NSL = RW / Map::RS;
};

// Weights of a gate/up wave item: rows[s] = gate row of slice s, rows[NSL + s]
// its up row (RP row pairs n_base .. n_base + RP - 1).
template <int FMT, int H, int I>
struct GateUpW {
  RowRegs<FMT, H> rows[2 * GateUpGeo<FMT, H>::NSL];
};

// wexp / sexp: byte offsets of the expert's [2I, ...] codes and scales in
// descriptors w / s (kOOB: no item, nothing is read).
template <int FMT, int H, int I>
__device__ __forceinline__ void gate_up_load(GateUpW<FMT, H, I> &W, __amdgpu_buffer_rsrc_t w,
                                             uint32_t wexp, __amdgpu_buffer_rsrc_t sc,
                                             uint32_t sexp, int n_base) {
  using Map = RowMap<FMT, H>;
  using Geo = GateUpGeo<FMT, H>;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane / Map::LPR, q = lane % Map::LPR;
#pragma unroll
  for (int s = 0; s < Geo::NSL; ++s) {
    const uint32_t n = n_base + s * Map::RS + r;
    load_row(W.rows[s], w, wexp + n * Map::ROW_BYTES, sc, sexp + n * (H / 16), q);
    load_row(W.rows[Geo::NSL + s], w, wexp + (I + n) * Map::ROW_BYTES, sc,
             sexp + (I + n) * (H / 16), q);
  }
}

// Weights of a down wave item: RW output rows h_base .. h_base + RW - 1.
template <int FMT, int I>
struct DownW {
  RowRegs<FMT, I> rows[DownGeo<FMT, I>::NSL];
};

template <int FMT, int I>
__device__ __forceinline__ void down_load(DownW<FMT, I> &W, __amdgpu_buffer_rsrc_t w,
                                          uint32_t wexp, __amdgpu_buffer_rsrc_t sc, uint32_t sexp,
                                          int h_base) {
  using Map = RowMap<FMT, I>;
  using Geo = DownGeo<FMT, I>;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane / Map::LPR, q = lane % Map::LPR;
#pragma unroll
  for (int s = 0; s < Geo::NSL; ++s) {
    const uint32_t h = h_base + s * Map::RS + r;
    load_row(W.rows[s], w, wexp + h * Map::ROW_BYTES, sc, sexp + h * (I / 16), q);
  }
}

}  // namespace flint
