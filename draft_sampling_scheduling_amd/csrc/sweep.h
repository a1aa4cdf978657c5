// sweep.h -- the vocabulary sweep shared by the draft step and verification.
//
// For a group of rows (requests at one draft position, or verified positions) and a
// contiguous range of 64-id vocabulary blocks, it forms
//     l(row, v) = sum_i B[row][i] * W2t[v][i]          (bias = W1[x_{k-1}] W2, eq. (5))
// on the matrix cores, 64 ids at a time, and hands every 64x(rows) tile of fp32 logits to
// an epilogue that folds it into per-row running state (normalisers, Gumbel maxima,
// distances), so no V-wide row is ever written to memory.
//
// Work split (one workgroup = 4 waves = 256 threads):
//   - grid = nranges x ngroups tasks; a task owns one vocabulary range and one row group.
//   - The W2t rows of the current 64-id block are staged in LDS (double-buffered, loaded
//     with coalesced 16-byte reads: a W2t row is r contiguous bf16), shared by all waves.
//   - Each wave owns NT*32 rows; their B rows (K = r) live in registers for the whole
//     sweep, so every LDS fragment of W2t feeds NT MFMAs.
//   - MFMA 32x32x16 bf16 with A = W2t tile (vocab on M) and B = B^T (rows on N): lane
//     (n, h) of the accumulator holds row n and 16 vocabulary ids; the tile's vocabulary
//     order is permuted so that these 16 ids are consecutive (v0 + 16h .. v0 + 16h + 15),
//     which makes the epilogue's per-row operand loads two 16-byte reads per tile.
#pragma once

#include "dev.h"

namespace dspark {

constexpr int kSweepThreads = 256;
constexpr int kMaxKS = 16;   // r <= 256
constexpr int kMaxStage = 8; // 16-byte W2t chunks staged per thread per block (r = 256)

struct SweepGeom {
  int nrows;      // rows (upper bound; an epilogue may know the exact count on device)
  int V, r;
  int CH;         // r / 8: 16-byte chunks per W2t row
  int nks;        // r / 16: MFMA k-steps
  int nblocks;    // ceil(V / 64)
  int nranges;    // vocabulary ranges (one per task column)
  int ngroups;    // row groups
  int blocks_lo;  // range i spans blocks_lo + (i < blocks_extra) blocks
  int blocks_extra;
  const uint16_t* W2t;  // [V][r] bf16
};

// position of the 16-byte chunk c of tile row m (0..31) of m-tile mt in an LDS buffer
__device__ __forceinline__ int lds_pos(const SweepGeom& g, int mt, int m, int c) {
  const int swz = m & ((g.CH < 16 ? g.CH : 16) - 1);
  return (mt * 32 + m) * g.CH + (c ^ swz);
}

// accumulator row m of a 32x32 tile holds vocabulary offset perm(m) inside the tile:
// perm(8q + 4h + t) = 16h + 4q + t.  Inverse: v -> 8((v & 15) >> 2) + 4(v >> 4) + (v & 3).
__device__ __forceinline__ int tile_row_of_vocab(int vv) {
  return 8 * ((vv & 15) >> 2) + 4 * (vv >> 4) + (vv & 3);
}

__device__ __forceinline__ void task_of(const SweepGeom& g, int& range, int& group) {
  const int ntask = g.nranges * g.ngroups;
  int t = blockIdx.x;
  // consecutive tasks share a vocabulary range; keep them on one XCD (round-robin
  // dispatch over 8 XCDs) so that the range's W2t rows are fetched into one L2
  if ((ntask & 7) == 0) t = (t & 7) * (ntask >> 3) + (t >> 3);
  range = t / g.ngroups;
  group = t - range * g.ngroups;
}

__device__ __forceinline__ void range_blocks(const SweepGeom& g, int range, int& b0, int& b1) {
  b0 = range * g.blocks_lo + (range < g.blocks_extra ? range : g.blocks_extra);
  b1 = b0 + g.blocks_lo + (range < g.blocks_extra ? 1 : 0);
}

// load the W2t rows of block b into staging registers (zero past V)
__device__ __forceinline__ void stage_load(const SweepGeom& g, int b, uint4 (&st)[kMaxStage]) {
  const int total = 64 * g.CH;
#pragma unroll
  for (int s = 0; s < kMaxStage; ++s) {
    const int c = threadIdx.x + s * kSweepThreads;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c < total) {
      const int vl = c / g.CH, ch = c - vl * g.CH;
      const int vocab = b * kVB + vl;
      if (vocab < g.V)
        v = *reinterpret_cast<const uint4*>(g.W2t + (size_t)vocab * g.r + ch * 8);
    }
    st[s] = v;
  }
}

__device__ __forceinline__ void stage_store(const SweepGeom& g, uint4* buf,
                                            const uint4 (&st)[kMaxStage]) {
  const int total = 64 * g.CH;
#pragma unroll
  for (int s = 0; s < kMaxStage; ++s) {
    const int c = threadIdx.x + s * kSweepThreads;
    if (c < total) {
      const int vl = c / g.CH, ch = c - vl * g.CH;
      buf[lds_pos(g, vl >> 5, tile_row_of_vocab(vl & 31), ch)] = st[s];
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// hi/lo bf16 split of 8 floats: x = hi + lo to ~16 significant bits
__device__ __forceinline__ void split8(const float (&x)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t a = f32_to_bf16(x[2 * i]), b = f32_to_bf16(x[2 * i + 1]);
    const uint16_t la = f32_to_bf16(x[2 * i] - bf16_to_f32(a));
    const uint16_t lb = f32_to_bf16(x[2 * i + 1] - bf16_to_f32(b));
    h[i] = (uint32_t)a | ((uint32_t)b << 16);
    l[i] = (uint32_t)la | ((uint32_t)lb << 16);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// The sweep kernel.  Epi provides:
//   struct Params; struct State; struct Pre;
//   static bool group_live(const Params&, int row0)          rows exist in this group
//   static int  nrows(const Params&)                         exact row count (device)
//   static const void* brow(const Params&, int row)          B row of a row (bf16 or f32)
//   static void init(const Params&, State&, int myrow)
//   template <int NT> static void prefetch(const Params&, Pre&, int b, int rowbase)
//   static void block(const Params&, State&, const Pre&, const f32x16 (&acc)[NT][2],
//                     int b, int rowbase, int myrow)
//   static void finish(const Params&, const State&, int myrow, int range)
// SPLIT: B rows are float and enter as hi + lo bf16 terms (two MFMAs each).
template <int NT, bool SPLIT, class Epi>
__global__ void __launch_bounds__(kSweepThreads, 1)
    sweep_kernel(SweepGeom g, typename Epi::Params ep) {
  extern __shared__ uint4 lds[];
  int range, group;
  task_of(g, range, group);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int group_row0 = group * (kSweepThreads / kWave) * NT * 32;
  if (!Epi::group_live(ep, group_row0)) return;
  const int nrows = Epi::nrows(ep);
  const int rowbase = group_row0 + wave * NT * 32;
  // the row this lane keeps running state for: n-tile h (NT == 2) or n-tile 0 (NT == 1)
  const int myrow = (NT == 2 || h == 0) ? rowbase + (NT == 2 ? 32 * h : 0) + n : -1;

  // B operand in registers: rows rowbase + 32*nt + n, k = 16*ks + 8*h .. + 8
  bf16x8 bh[NT][kMaxKS];
  bf16x8 bl[SPLIT ? NT : 1][SPLIT ? kMaxKS : 1];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = rowbase + 32 * nt + n;
    const bool live = row < nrows;
#pragma unroll
    for (int ks = 0; ks < kMaxKS; ++ks) {
      uint4 hi = make_uint4(0, 0, 0, 0), lo = make_uint4(0, 0, 0, 0);
      if (live && ks < g.nks) {
        const int k0 = 16 * ks + 8 * h;
        if (SPLIT) {
          const float* p = reinterpret_cast<const float*>(Epi::brow(ep, row)) + k0;
          const float4 a = *reinterpret_cast<const float4*>(p);
          const float4 c = *reinterpret_cast<const float4*>(p + 4);
          const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
          split8(x, hi, lo);
        } else {
          hi = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(Epi::brow(ep, row)) + k0);
        }
      }
      bh[nt][ks] = as_bf16x8(hi);
      if (SPLIT) bl[SPLIT ? nt : 0][SPLIT ? ks : 0] = as_bf16x8(lo);
    }
  }

  typename Epi::State st;
  Epi::init(ep, st, myrow);

  int b0, b1;
  range_blocks(g, range, b0, b1);
  const int buf_chunks = 64 * g.CH;
  uint4 stage[kMaxStage];
  if (b0 < b1) {
    stage_load(g, b0, stage);
    stage_store(g, lds, stage);
  }
  for (int b = b0; b < b1; ++b) {
    uint4* cur = lds + ((b - b0) & 1) * buf_chunks;
    uint4* nxt = lds + (((b - b0) & 1) ^ 1) * buf_chunks;
    const bool more = b + 1 < b1;
    if (more) stage_load(g, b + 1, stage);
    typename Epi::Pre pre;
    Epi::template prefetch<NT>(ep, pre, b, rowbase);
    __syncthreads();  // cur is complete; every wave is past its reads of nxt

    f32x16 acc[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[nt][mt][j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kMaxKS; ++ks) {
      if (ks < g.nks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = as_bf16x8(cur[lds_pos(g, mt, n, 2 * ks + h)]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[nt][ks], acc[nt][mt],
                                                                  0, 0, 0);
            if (SPLIT)
              acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  a, bl[SPLIT ? nt : 0][SPLIT ? ks : 0], acc[nt][mt], 0, 0, 0);
          }
        }
      }
    }
    Epi::template block<NT>(ep, st, pre, acc, b, rowbase, myrow);
    if (more) stage_store(g, nxt, stage);
  }
  Epi::finish(ep, st, myrow, range);
}

// host-side geometry
inline SweepGeom make_geom(int nrows, int V, int r, const uint16_t* W2t, int nt,
                           int target_tasks) {
  SweepGeom g{};
  g.nrows = nrows;
  g.V = V;
  g.r = r;
  g.CH = r / 8;
  g.nks = r / 16;
  g.nblocks = (V + kVB - 1) / kVB;
  const int rows_per_group = (kSweepThreads / kWave) * nt * 32;
  g.ngroups = (nrows + rows_per_group - 1) / rows_per_group;
  if (g.ngroups < 1) g.ngroups = 1;
  int nr = target_tasks / g.ngroups;
  if (nr < 1) nr = 1;
  if (nr > g.nblocks) nr = g.nblocks;
  g.nranges = nr;
  g.blocks_lo = g.nblocks / nr;
  g.blocks_extra = g.nblocks - g.blocks_lo * nr;
  g.W2t = W2t;
  return g;
}

inline size_t sweep_lds_bytes(int r) { return (size_t)2 * 64 * (r / 8) * 16; }

}  // namespace dspark
