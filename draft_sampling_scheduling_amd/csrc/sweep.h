// sweep.h -- the vocabulary sweep shared by the draft step and verification.
//
// For a group of up to 128 rows (requests at one draft position, or verified positions)
// and a contiguous range of 64-id vocabulary blocks, it forms
//     l(row, v) = sum_i B[row][i] * W2t[v][i] + stream_0[row][v]   (eq. (4) with eq. (5))
// on the matrix cores, 32 ids at a time, and hands each 32 x 128 tile of fp32 logits to an
// epilogue that folds it into per-row running state (normalisers, Gumbel maxima,
// distances), so no V-wide row is ever written to memory.
//
// Work split: workgroups of 4 waves, two per vocabulary range (grid = 2 x ranges, about two
// per CU, each with its own barrier domain so one's waits overlap the other's work); the
// workgroups of a range walk the row groups of 128 alternately, so a row count known only
// on the device costs no idle workgroups.
//   - Each wave owns 32 rows of the group; their B rows (K = r) live in registers for the
//     group's whole sweep.
//   - Per 32-id tile the workgroup stages in LDS the tile's W2t rows (32 x r bf16, shared by
//     all waves) and every wave's 32 x 32 slice of each streamed operand (U, and the target
//     logits in verification).  Staging is asynchronous: the loads go straight to LDS
//     (global_load_lds_dwordx4), two stages deep, so each tile's HBM traffic is issued one
//     tile ahead of its use (while the CU's other workgroup computes) and the matrix-core and
//     epilogue work of the current tile hides the memory latency.  The waits on those
//     loads are explicit vmcnt waits.
//   - Without the bias contraction (one streamed operand, no W2t tiles: the parallel block's
//     own sampling) U is staged a whole 64-id block at a time, one block ahead, in two block
//     buffers: 128 bytes of each row per copy.  Rows lie a position's stride apart in HBM, and
//     64-byte pieces of them (one tile's share) come at about 3.9 TB/s where 128-byte pieces
//     come at the 5.7 TB/s of a plain read.  With W2t tiles beside them the block buffers made
//     the draft sweep slower (32.7 against 31.2-31.9 us), so the sweeps with a bias keep the
//     tile's 64-byte slices.
//   - MFMA 32x32x16 bf16 with A = W2t tile (vocabulary on M) and B = B^T (rows on N):
//     accumulator lane (n, h) holds row n; its 16 registers are permuted (see
//     tile_row_of_vocab) to two runs of 8 consecutive ids, which the epilogue matches with
//     two 16-byte LDS reads per streamed operand.
#pragma once

#include <hip/hip_ext.h>

#include <type_traits>

#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kSweepThreads = 256;  // 4 waves; each wave owns 32 rows of the group
constexpr int kSweepWaves = kSweepThreads / kWave;
constexpr int kRowsPerGroup = kSweepWaves * 32;
constexpr int kTile = 32;           // vocabulary ids per pipeline step (one m-tile)

struct SweepGeom {
  int nrows;      // rows (upper bound; an epilogue may know the exact count on device)
  int V, r;
  int CH;         // r / 8: 16-byte chunks per W2t row
  int nks;        // r / 16: MFMA k-steps
  int nblocks;    // ceil(V / 64)
  int nranges;    // vocabulary ranges (one per task column)
  int ngroups;    // row groups
  int gsplit;     // workgroups per vocabulary range; each takes every gsplit-th row group
  int blocks_lo;  // range i spans blocks_lo + (i < blocks_extra) blocks
  int blocks_extra;
  const uint16_t* W2t;  // [V][r] bf16
};

// ---------------------------------------------------------------------------------------
// LDS layout of one pipeline stage (units of 16-byte chunks)
//   [W2t tile: 32 rows, row stride CH + 1 (the odd stride puts the 16 rows one
//    ds_read_b128 phase reads on distinct banks, so every fragment address is a per-lane
//    base plus an immediate); rounded up to whole 64-chunk copies]
//   [stream s: 4 waves x 32 rows x 4 chunks] for each streamed operand
// ---------------------------------------------------------------------------------------
__host__ __device__ constexpr int w2_copies(int CH) { return (32 * (CH + 1) + 63) / 64; }
__host__ __device__ constexpr int w2_tile_chunks(int CH) { return 64 * w2_copies(CH); }
__host__ __device__ constexpr int stream_tile_chunks() { return kSweepWaves * 32 * 4; }
__host__ __device__ constexpr int stage_chunks(int CH, int nstreams) {
  return w2_tile_chunks(CH) + nstreams * stream_tile_chunks();
}
// a sweep without the bias and with one stream stages U per block: its stages hold nothing
// (no W2t tiles), and two U block buffers of 128 rows x 8 chunks follow them
constexpr int kUBlkChunks = kSweepWaves * 32 * 8;
__host__ __device__ constexpr bool sweep_ublk(int nstreams, bool bias) {
  return nstreams == 1 && !bias;
}
__host__ __device__ constexpr int sweep_stage_chunks(int CH, int nstreams, bool bias) {
  return sweep_ublk(nstreams, bias) ? 0 : stage_chunks(CH, nstreams);
}
inline size_t sweep_lds_bytes(int r, int nstreams, int nstage, bool bias) {
  return (size_t)16 * (nstage * sweep_stage_chunks(r / 8, nstreams, bias) +
                       (sweep_ublk(nstreams, bias) ? 2 * kUBlkChunks : 0));
}

// 16-byte chunk c (0..3) of row n in a wave's 32 x 32 stream slice; the xor spreads the 16
// rows of one read phase over the banks
__device__ __forceinline__ int stream_pos(int n, int c) { return n * 4 + (c ^ ((n >> 2) & 3)); }
// chunk c (0..7) of row n in a wave's slice of a U block buffer; the xor puts the 16 rows of
// one read phase on distinct banks
__device__ __forceinline__ int ublk_pos(int n, int c) { return n * 8 + (c ^ ((n >> 1) & 7)); }

// Accumulator row m = 16c + 8a + 4h + t of a 32x32 tile holds vocabulary offset
// 16c + 8h + 4a + t (bits 2 and 3 swapped; the map is its own inverse), so register
// j = 8c + e of lane half h is vocabulary offset 16c + 8h + e: chunks h and 2 + h of the
// row's 32-id slice.
__device__ __forceinline__ int tile_row_of_vocab(int vv) {
  return 16 * (vv >> 4) + 8 * ((vv >> 2) & 1) + 4 * ((vv >> 3) & 1) + (vv & 3);
}
__device__ __forceinline__ int vocab_of_reg(int h, int j) { return 16 * (j >> 3) + 8 * h + (j & 7); }

__device__ __forceinline__ void range_blocks(const SweepGeom& g, int range, int& b0, int& b1) {
  b0 = range * g.blocks_lo + (range < g.blocks_extra ? range : g.blocks_extra);
  b1 = b0 + g.blocks_lo + (range < g.blocks_extra ? 1 : 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte chunk index of row q's chunk j (elements 8j .. 8j+7) in the packed B layout for
// r = 16 * nks: 32-row blocks of nks * 64 chunks, k-step major, lane (n, h) minor
__host__ __device__ __forceinline__ size_t bpack_index(int q, int j, int nks) {
  return (size_t)(q >> 5) * (size_t)(nks * 64) + (size_t)((j >> 1) * 64 + (j & 1) * 32 + (q & 31));
}
// rows the packed B buffer holds for R rows (whole row groups, so every wave's block exists)
__host__ __device__ __forceinline__ int bpack_rows(int R) {
  return (R + kRowsPerGroup - 1) / kRowsPerGroup * kRowsPerGroup;
}

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

// 8 bf16 of a 16-byte chunk, widened
__device__ __forceinline__ void widen8(uint4 u, float* o) {
  o[0] = bf16lo(u.x); o[1] = bf16hi(u.x); o[2] = bf16lo(u.y); o[3] = bf16hi(u.y);
  o[4] = bf16lo(u.z); o[5] = bf16hi(u.z); o[6] = bf16lo(u.w); o[7] = bf16hi(u.w);
}

// ---------------------------------------------------------------------------------------
// Asynchronous global -> LDS copies (global_load_lds_dwordx4): every lane moves 16 bytes to
// lds_byte_base + 16 * lane.  They are issued as inline assembly so that the compiler's own
// wait-count bookkeeping does not serialise later LDS reads behind them; the sweep waits
// for them explicitly (vm_wait) before the barrier that publishes a stage.
// ---------------------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// the same copy with a scalar base and a per-lane 32-bit byte offset: the per-tile cost is
// one scalar add per copy
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_byte_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_byte_base)
      : "memory", "m0");
}

// Workgroup barrier for the staging pipeline.  __syncthreads() carries a release fence,
// which the compiler implements by draining every outstanding vector-memory load first
// (vmcnt(0)) -- that would retire the prefetched tiles too and collapse the pipeline to
// depth one.  Here the copies are awaited explicitly (vm_wait), so the barrier only has to
// retire this wave's LDS reads before another wave may overwrite the stage; the memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// x of the lane 32 apart (lane l <-> l ^ 32) combined with op, on both halves: the swap
// returns (x[0..31], x[0..31]) and (x[32..63], x[32..63]), so op(first, second) is
// op(x[l], x[l ^ 32]) on every lane when op is commutative
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ void half_lse(float& m, float& s) {
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  m = __uint_as_float(rm[0]);
  s = __uint_as_float(rs[0]);
  lse_merge(m, s, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
}

// The sweep of one row group over one vocabulary range.  Lane (n, h) of wave w works on
// row = group*128 + 32w + n; the lanes with h == 0 own the row's running state.  Epi
// provides:
//   static constexpr int kStreams;       streamed operands: 1 (U) or 2 (U, target)
//   struct Params; struct State;
//   static bool group_live(const Params&, int row0)         rows exist in this group
//   static int  nrows(const Params&)                        exact row count (device)
//   static const void* brow(const Params&, int row)         B row of a live row
//   static const uint4* bpack(const Params&)                 the B rows in packed order,
//        or null (then brow is used): for row group g, wave w and k-step ks, lane l's
//        16-byte fragment sits at chunk (4g + w) * NKS * 64 + ks * 64 + l, so each k-step
//        is one coalesced 1 KB load per wave (see bpack_index)
//   static const uint16_t* sbase(const Params&, int s)      stream s array
//   static uint32_t srow(const Params&, int s, int row)     element offset of a live row
//   static void init(const Params&, State&, int row)        row < 0: not a live row
//   static void refresh(const Params&, State&, int b, int row)   random words of block b
//   template <int HALF, bool MASK>
//   static void tile(const Params&, State&, const f32x16& l, const uint4 (&x)[2], int b,
//                    int row, bool owner)
//        l: the 32-id tile (half HALF of block b) of logits U + bias in accumulator
//        layout; x: stream 1 of the tile (packed bf16, chunks h and 2 + h of the row's
//        slice) when kStreams == 2; MASK: ids past V may be present (last block only)
//   static void finish(const Params&, const State&, int row, bool owner, int range)
// NKS = r / 16 (compile time: the k loop is fully unrolled over register operands).
// SPLIT: B rows are float and enter as hi + lo bf16 terms (two MFMAs each).
// Host guarantees: every stream array is smaller than 4 GiB (32-bit byte offsets).
//
// An epilogue may declare `static constexpr bool kNoBias = true`: the logits are then the
// first streamed operand alone (no W2t tiles are copied and no matrix-core chain runs), the
// sampling of the parallel block without the sequential head.
template <class E, class = void>
struct epi_has_bias : std::true_type {};
template <class E>
struct epi_has_bias<E, std::void_t<decltype(E::kNoBias)>>
    : std::integral_constant<bool, !E::kNoBias> {};

// The work comes in two parts: prepare() fixes the per-lane copy offsets and issues the
// first tile into stage 0 (it reads nothing the B rows or the epilogue state need); run()
// loads the B rows, streams the range and hands the result to the epilogue.
template <int NKS, bool SPLIT, int NSTAGE, class Epi>
struct SweepTask {
  static constexpr int CH = 2 * NKS;
  static constexpr int RS = CH + 1;                 // W2t tile row stride (chunks)
  static constexpr int NI = w2_copies(CH);          // W2t copies per tile
  static constexpr int W2_MAX = (NI + kSweepWaves - 1) / kSweepWaves;
  static constexpr int NS = Epi::kStreams;
  static constexpr bool BIAS = epi_has_bias<Epi>::value;
  static constexpr bool UBLK = sweep_ublk(NS, BIAS);  // U staged per 64-id block
  static constexpr int SCH = sweep_stage_chunks(CH, NS, BIAS);
  static constexpr int UB0 = NSTAGE * SCH;          // first U block buffer (chunks)
  static constexpr int OPS_U = 4;                   // copies of one U block per wave
  static constexpr int D = NSTAGE - 1;              // prefetch distance in tiles
  // copies one tile puts in flight for a wave (W2t copies: W2_MAX or W2_MAX - 1)
  static constexpr int OPS_BIG = (BIAS ? W2_MAX : 0) + 2 * NS;
  static constexpr int OPS_SMALL = (BIAS ? W2_MAX - 1 : 0) + 2 * NS;

  const SweepGeom& g;
  const typename Epi::Params& ep;
  uint4* lds;
  int range, group_row0, lane, wave, n, h, nrows, row;
  bool live, owner, big;
  uint32_t w2off[W2_MAX];
  uint32_t soff[NS][2];
  int sx[2];
  uint32_t uoff[OPS_U];  // U block copies: row 8i + lane / 8 of the wave, a 16-byte piece
  int u_idx, u_sw;       // this lane's row in a U block buffer, and its xor
  const uint16_t* sb[NS];
  uint32_t lds0;
  int a_idx, s_idx0, s_idx1;
  int b0, b1, bp1, t0, t1;
  bool ragged;

  __device__ __forceinline__ SweepTask(const SweepGeom& g_, const typename Epi::Params& ep_,
                                       uint4* lds_)
      : g(g_), ep(ep_), lds(lds_) {}

  // copies of full tile t into stage stg (scalar bases; per-lane offsets fixed)
  __device__ __forceinline__ void issue(int t, int stg) {
    const uint32_t base = lds0 + 16u * stg * SCH;
    const uint16_t* w2b = g.W2t + (size_t)kTile * t * g.r;
#pragma unroll
    for (int i = 0; i < W2_MAX; ++i) {
      const int I = wave + kSweepWaves * i;
      if (BIAS && I < NI) dma16s(w2b, w2off[i], base + 16u * 64u * I);
    }
    if constexpr (!UBLK) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int k = 0; k < 2; ++k)
          dma16s(sb[s] + kTile * t, soff[s][k],
                 base + 16u * (w2_tile_chunks(CH) + s * stream_tile_chunks() + wave * 128 + 64 * k));
    }
  }
  // copies of U block b (128 bytes of each row) into block buffer ub
  __device__ __forceinline__ void issue_u(int b, int ub) {
    const uint32_t base = lds0 + 16u * (UB0 + ub * kUBlkChunks + wave * 256);
    const uint16_t* src = sb[0] + (size_t)kVB * b;
#pragma unroll
    for (int i = 0; i < OPS_U; ++i) dma16s(src, uoff[i], base + 16u * 64u * i);
  }
  // the same for the short last block: each piece's ids clamped into the row
  __device__ __forceinline__ void issue_u_ragged(int b, int ub) {
    const uint32_t base = lds0 + 16u * (UB0 + ub * kUBlkChunks + wave * 256);
#pragma unroll
    for (int i = 0; i < OPS_U; ++i) {
      const int rl = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ ((rl >> 1) & 7);
      int v = kVB * b + 8 * c;
      if (v > g.V - 8) v = g.V - 8;
      dma16s(sb[0], uoff[i] + (uint32_t)(v - 8 * c) * 2u, base + 16u * 64u * i);
    }
  }
  // the same for the short last tile: clamp each lane's source into the arrays
  __device__ __forceinline__ void issue_ragged(int t, int stg) {
    const uint32_t base = lds0 + 16u * stg * SCH;
#pragma unroll
    for (int i = 0; i < W2_MAX; ++i) {
      const int I = wave + kSweepWaves * i;
      const int P = 64 * I + lane;
      const int m = P / RS, c = P - m * RS;
      int v = kTile * t + (m < 32 ? tile_row_of_vocab(m) : 0);
      if (v >= g.V) v = g.V - 1;
      const uint32_t off = (m < 32 && c < CH) ? (uint32_t)(v * g.r + 8 * c) * 2u : 0u;
      if (BIAS && I < NI) dma16s(g.W2t, off, base + 16u * 64u * I);
    }
    if constexpr (!UBLK) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          int v = kTile * t + sx[k];
          if (v > g.V - 8) v = g.V - 8;
          dma16s(sb[s], soff[s][k] + (uint32_t)(v - sx[k]) * 2u,
                 base + 16u * (w2_tile_chunks(CH) + s * stream_tile_chunks() + wave * 128 + 64 * k));
        }
    }
  }
  // wait until at most `left` (0 .. D-1) tiles' copies are still in flight (loads complete
  // in order)
  __device__ __forceinline__ void wait_tiles(int left) {
    if (left <= 0) {
      vm_wait<0>();
    } else if (left == 1 || D < 3) {
      if (big) vm_wait<OPS_BIG>(); else vm_wait<OPS_SMALL>();
    } else {
      if (big) vm_wait<2 * OPS_BIG>(); else vm_wait<2 * OPS_SMALL>();
    }
  }

  // the per-lane copy offsets of row group `group` and the first tile's copies
  __device__ __forceinline__ void prepare(int range_, int group) {
    range = range_;
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    n = lane & 31;
    h = lane >> 5;
    nrows = Epi::nrows(ep);
    // values derived from the group are recomputed per group rather than hoisted out of
    // the group loop and held (the scalar register file is the tight resource here)
    group_row0 = group * kRowsPerGroup;
    asm volatile("" : "+s"(group_row0));
    row = group_row0 + wave * 32 + n;
    live = row < nrows;
    owner = live && h == 0;

    // per-lane byte offsets of the copies (constant over tiles)
    //   W2t copy i (index I = wave + 8i): lane -> padded position P = 64I + lane -> tile row
    //   m = P / RS, chunk c = P % RS; the pad chunk and positions past the tile read row 0
    //   stream copy k: lane -> chunk lane & 3 (xor-permuted) of the wave's row 16k + lane/4;
    //   rows past the end read the last live row
#pragma unroll
    for (int i = 0; i < W2_MAX; ++i) {
      const int P = 64 * (wave + kSweepWaves * i) + lane;
      const int m = P / RS, c = P - m * RS;
      w2off[i] = (m < 32 && c < CH) ? (uint32_t)(tile_row_of_vocab(m) * g.r + 8 * c) * 2u : 0u;
    }
    if constexpr (UBLK) {
      //   U block copy i: lane -> row 8i + lane / 8 of the wave, piece (lane & 7) xor the row's
      //   swizzle, so that the 64 lanes land on ublk_pos order in LDS
#pragma unroll
      for (int i = 0; i < OPS_U; ++i) {
        const int rl = 8 * i + (lane >> 3);
        int rr = group_row0 + wave * 32 + rl;
        if (rr >= nrows) rr = nrows - 1;
        const int c = (lane & 7) ^ ((rl >> 1) & 7);
        uoff[i] = (Epi::srow(ep, 0, rr) + (uint32_t)(8 * c)) * 2u;
      }
      u_idx = UB0 + wave * 256 + n * 8;
      u_sw = (n >> 1) & 7;
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int rl = 16 * k + (lane >> 2);
        int rr = group_row0 + wave * 32 + rl;
        if (rr >= nrows) rr = nrows - 1;
        sx[k] = 8 * ((lane & 3) ^ ((rl >> 2) & 3));  // element offset inside the 32-id slice
#pragma unroll
        for (int s = 0; s < NS; ++s) soff[s][k] = (Epi::srow(ep, s, rr) + (uint32_t)sx[k]) * 2u;
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) sb[s] = Epi::sbase(ep, s);
    lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    // LDS chunk indices this lane reads (stage 0): A fragments at a_idx + 2*ks, stream chunks
    a_idx = n * RS + h;
    s_idx0 = w2_tile_chunks(CH) + wave * 128 + stream_pos(n, h);
    s_idx1 = w2_tile_chunks(CH) + wave * 128 + stream_pos(n, 2 + h);
    big = wave < NI - kSweepWaves * (W2_MAX - 1);

    int rg = range + (group_row0 & 0);
    asm volatile("" : "+s"(rg));
    range_blocks(g, rg, b0, b1);
    // the last block of the vocabulary is short when V % 64 != 0: it leaves the pipeline
    ragged = (b1 * kVB > g.V);
    bp1 = ragged ? b1 - 1 : b1;  // pipelined blocks [b0, bp1)
    t0 = 2 * b0;
    t1 = 2 * bp1;
    // the first tile goes out before anything else (it depends on nothing the B rows or
    // the epilogue state need); the rest of the pipeline fills once they are in, so the
    // first step waits for one tile rather than D
    if (t0 < t1) {
      issue(t0, 0);
      if constexpr (UBLK) issue_u(b0, 0);
    }
  }

  // matrix-core chain of the tile in stage stg, seeded with its U slice
  __device__ __forceinline__ void mma(int stg, f32x16& acc, uint4 (&x)[2], const bf16x8 (&bh)[NKS],
                                      const bf16x8 (&bl)[SPLIT ? NKS : 1]) {
    const uint4* sl = lds + stg * SCH;
    float u[16];
    widen8(sl[s_idx0], u);
    widen8(sl[s_idx1], u + 8);
    if (NS == 2) {
      x[0] = sl[s_idx0 + stream_tile_chunks()];
      x[1] = sl[s_idx1 + stream_tile_chunks()];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = u[j];
    if (!BIAS) return;
    const uint4* ab = sl + a_idx;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = as_bf16x8(ab[2 * ks]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], acc, 0, 0, 0);
      if (SPLIT) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[SPLIT ? ks : 0], acc, 0, 0, 0);
    }
  }

  // the one-stream form: U from block buffer ub, half HALF of the block
  template <int HALF>
  __device__ __forceinline__ void mma_ublk(int stg, int ub, f32x16& acc, const bf16x8 (&bh)[NKS],
                                           const bf16x8 (&bl)[SPLIT ? NKS : 1]) {
    const uint4* up = lds + u_idx + ub * kUBlkChunks;
    float u[16];
    widen8(up[(4 * HALF + h) ^ u_sw], u);
    widen8(up[(4 * HALF + 2 + h) ^ u_sw], u + 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = u[j];
    if (!BIAS) return;
    const uint4* ab = lds + stg * SCH + a_idx;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = as_bf16x8(ab[2 * ks]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], acc, 0, 0, 0);
      if (SPLIT) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[SPLIT ? ks : 0], acc, 0, 0, 0);
    }
  }

  // the B rows, the streamed tiles and the epilogue of the prepared group
  __device__ __forceinline__ void run() {
    if constexpr (UBLK)
      run_ublk();
    else
      run_tiles();
  }

  // B operand in registers: k = 16*ks + 8*h .. + 8 of this lane's row; from the packed
  // copy when the epilogue has one (coalesced; rows past the end read padding)
  __device__ __forceinline__ void load_b(bf16x8 (&bh)[NKS], bf16x8 (&bl)[SPLIT ? NKS : 1]) {
    const uint4* bpk = SPLIT ? nullptr : Epi::bpack(ep);
    if (!BIAS) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) bh[ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
    } else if (bpk) {
      const uint4* src = bpk + (size_t)(group_row0 / 32 + wave) * (NKS * kWave) + lane;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) bh[ks] = as_bf16x8(src[ks * kWave]);
    } else {
      const void* brow = live ? Epi::brow(ep, row) : nullptr;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 hi = make_uint4(0, 0, 0, 0), lo = make_uint4(0, 0, 0, 0);
        if (live) {
          const int k0 = 16 * ks + 8 * h;
          if (SPLIT) {
            const float* p = reinterpret_cast<const float*>(brow) + k0;
            const float4 a = *reinterpret_cast<const float4*>(p);
            const float4 c = *reinterpret_cast<const float4*>(p + 4);
            const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            split8(x, hi, lo);
          } else {
            hi = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(brow) + k0);
          }
        }
        bh[ks] = as_bf16x8(hi);
        if (SPLIT) bl[SPLIT ? ks : 0] = as_bf16x8(lo);
      }
    }
  }

  // The sweep without the bias: block b + 1's U rows go out when block b starts (one block
  // ahead).  A block's first half waits for its own rows; its second half lets the next
  // block's copies stay in flight.  (The W2t calls are kept in the form the bias needs:
  // without it they issue nothing and the matrix chain is skipped.)
  __device__ __forceinline__ void run_ublk() {
    bf16x8 bh[NKS];
    bf16x8 bl[SPLIT ? NKS : 1];
    typename Epi::State st;
    load_b(bh, bl);
    Epi::init(ep, st, live ? row : -1);
    // a wait the compiler sees: the first block's copies, the B rows and the epilogue
    // state have landed
    __builtin_amdgcn_s_waitcnt(0);
    f32x16 accA, accB;
    uint4 xz[2];
    xz[0] = xz[1] = make_uint4(0, 0, 0, 0);
    for (int b = b0; b < bp1; ++b) {
      const int ub = (b - b0) & 1;
      const bool more = b + 1 < bp1;
      // -- first half of block b (stage 0); epilogue of the second half of block b - 1
      if (b > b0) {
        Epi::refresh(ep, st, b - 1, row);
        vm_wait<0>();
      }
      stage_barrier();
      issue(2 * b + 1, 1);
      if (more) issue_u(b + 1, ub ^ 1);
      mma_ublk<0>(0, ub, accA, bh, bl);
      if (b > b0) Epi::template tile<1, false>(ep, st, accB, xz, b - 1, row, owner);
      // -- second half of block b (stage 1); epilogue of its first half
      if (more)
        vm_wait<OPS_U>();
      else
        vm_wait<0>();
      stage_barrier();
      if (more) issue(2 * b + 2, 0);
      mma_ublk<1>(1, ub, accB, bh, bl);
      Epi::template tile<0, false>(ep, st, accA, xz, b, row, owner);
    }
    if (bp1 > b0) {
      Epi::refresh(ep, st, bp1 - 1, row);
      Epi::template tile<1, false>(ep, st, accB, xz, bp1 - 1, row, owner);
    }
    if (ragged) {  // the short last block, unpipelined
      const int b = b1 - 1;
      vm_wait<0>();
      __syncthreads();
      issue_ragged(2 * b, 0);
      issue_ragged(2 * b + 1, 1);
      issue_u_ragged(b, 0);
      vm_wait<0>();
      __syncthreads();
      mma_ublk<0>(0, 0, accA, bh, bl);
      Epi::template tile<0, true>(ep, st, accA, xz, b, row, owner);
      mma_ublk<1>(1, 0, accB, bh, bl);
      Epi::refresh(ep, st, b, row);
      Epi::template tile<1, true>(ep, st, accB, xz, b, row, owner);
    }
    vm_wait<0>();
    Epi::finish(ep, st, row, owner, range);
  }

  // The sweep with per-tile streamed slices (the bias contraction, or two streams).
  __device__ __forceinline__ void run_tiles() {
    bf16x8 bh[NKS];  // B operand (filled once the first tiles are in flight)
    bf16x8 bl[SPLIT ? NKS : 1];
    typename Epi::State st;
    load_b(bh, bl);
    Epi::init(ep, st, live ? row : -1);

    // a wait the compiler sees: every load issued so far (first tile, B rows, epilogue
    // state) has landed, so none of them is pending at the loop header
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int d = 1; d < D; ++d)
      if (t0 + d < t1) issue(t0 + d, d);
    f32x16 accA, accB;
    uint4 xA[2], xB[2];
    xA[0] = xA[1] = xB[0] = xB[1] = make_uint4(0, 0, 0, 0);
    int stg = 0;
    // one pipeline step: tile t's copies are awaited, tile t+D's issued, tile t's matrix
    // chain runs, and the epilogue of tile t-1 (HALF = 1 - half of t) is interleaved with it
    // (the first pair has no previous tile and is peeled off)
    auto next_stage = [&](int sg) { return sg + 1 == NSTAGE ? 0 : sg + 1; };
    auto ahead = [&](int sg) { return sg + D >= NSTAGE ? sg + D - NSTAGE : sg + D; };
    if (t1 > t0) {
      wait_tiles(min(D - 1, t1 - 1 - t0));
      stage_barrier();
      if (t0 + D < t1) issue(t0 + D, ahead(stg));
      mma(stg, accA, xA, bh, bl);
      stg = next_stage(stg);
      wait_tiles(min(D - 1, t1 - 2 - t0));
      stage_barrier();
      if (t0 + 1 + D < t1) issue(t0 + 1 + D, ahead(stg));
      mma(stg, accB, xB, bh, bl);
      Epi::template tile<0, false>(ep, st, accA, xA, t0 >> 1, row, owner);
      stg = next_stage(stg);
    }
    for (int t = t0 + 2; t < t1; t += 2) {
      const int b = t >> 1;
      Epi::refresh(ep, st, b - 1, row);
      // -- tile t = 2b (half 0); epilogue of tile 2b-1 (half 1 of block b-1)
      wait_tiles(min(D - 1, t1 - 1 - t));
      stage_barrier();
      if (t + D < t1) issue(t + D, ahead(stg));
      mma(stg, accA, xA, bh, bl);
      Epi::template tile<1, false>(ep, st, accB, xB, b - 1, row, owner);
      stg = next_stage(stg);
      // -- tile t + 1 (half 1); epilogue of tile t (half 0 of block b)
      wait_tiles(min(D - 1, t1 - 2 - t));
      stage_barrier();
      if (t + 1 + D < t1) issue(t + 1 + D, ahead(stg));
      mma(stg, accB, xB, bh, bl);
      Epi::template tile<0, false>(ep, st, accA, xA, b, row, owner);
      stg = next_stage(stg);
    }
    if (t1 > t0) {
      Epi::refresh(ep, st, bp1 - 1, row);
      Epi::template tile<1, false>(ep, st, accB, xB, bp1 - 1, row, owner);
    }
    if (ragged) {  // the short last block, unpipelined
      const int b = b1 - 1;
      vm_wait<0>();
      __syncthreads();
      issue_ragged(2 * b, 0);
      issue_ragged(2 * b + 1, 1);
      vm_wait<0>();
      __syncthreads();
      mma(0, accA, xA, bh, bl);
      Epi::template tile<0, true>(ep, st, accA, xA, b, row, owner);
      mma(1, accB, xB, bh, bl);
      Epi::refresh(ep, st, b, row);
      Epi::template tile<1, true>(ep, st, accB, xB, b, row, owner);
    }
    vm_wait<0>();
    Epi::finish(ep, st, row, owner, range);
  }
};

// task -> (vocabulary range, first row group); the gsplit workgroups of one range are
// dispatched to the same XCD (round-robin dispatch over 8 XCDs) so its W2t tiles come from
// HBM once and from that XCD's L2 after
__device__ __forceinline__ void sweep_task_of(const SweepGeom& g, int bid, int& range, int& g0) {
  const int G = g.gsplit;
  if ((g.nranges & 7) == 0) {
    const int slot = bid >> 3;
    range = (slot / G) * 8 + (bid & 7);
    g0 = slot - (slot / G) * G;
  } else {
    range = bid / G;
    g0 = bid - range * G;
  }
}

// The sweep kernel: workgroup (range, g0) sweeps row groups g0, g0 + gsplit, ... over its
// range.
template <int NKS, bool SPLIT, int NSTAGE, class Epi>
__global__ void __launch_bounds__(kSweepThreads, 2)
    sweep_kernel(SweepGeom g, typename Epi::Params ep) {
  extern __shared__ uint4 lds[];
  int range, g0;
  sweep_task_of(g, blockIdx.x, range, g0);
  for (int group = g0; Epi::group_live(ep, group * kRowsPerGroup); group += g.gsplit) {
    SweepTask<NKS, SPLIT, NSTAGE, Epi> task(g, ep, lds);
    task.prepare(range, group);
    task.run();
    __syncthreads();  // the next group reuses the stages
  }
}

// host-side geometry: target_ranges vocabulary ranges, row groups of 128
inline SweepGeom make_geom(int nrows, int V, int r, const uint16_t* W2t, int target_ranges) {
  SweepGeom g{};
  g.nrows = nrows;
  g.V = V;
  g.r = r;
  g.CH = r / 8;
  g.nks = r / 16;
  g.nblocks = (V + kVB - 1) / kVB;
  g.ngroups = (nrows + kRowsPerGroup - 1) / kRowsPerGroup;
  if (g.ngroups < 1) g.ngroups = 1;
  int nr = target_ranges;
  if (nr < 1) nr = 1;
  if (nr > g.nblocks) nr = g.nblocks;
  g.nranges = nr;
  g.gsplit = g.ngroups >= 2 ? 2 : 1;
  g.blocks_lo = g.nblocks / nr;
  g.blocks_extra = g.nblocks - g.blocks_lo * nr;
  g.W2t = W2t;
  return g;
}

// ev0/ev1 (both or neither): events the dispatch itself timestamps at the kernel's start
// and end, so their elapsed time is the kernel's own duration
template <int NKS, bool SPLIT, int NSTAGE, class Epi>
inline void launch_sweep_nks(const SweepGeom& g, const typename Epi::Params& p, hipStream_t s,
                             hipEvent_t ev0, hipEvent_t ev1) {
  auto kern = sweep_kernel<NKS, SPLIT, NSTAGE, Epi>;
  const size_t sh = sweep_lds_bytes(g.r, Epi::kStreams, NSTAGE, epi_has_bias<Epi>::value);
  static std::atomic<uint64_t> lds_raised{0};
  ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)sh, lds_raised);
  if (ev0 && ev1)
    hipExtLaunchKernelGGL(kern, dim3(g.nranges * g.gsplit), dim3(kSweepThreads), (uint32_t)sh, s,
                          ev0, ev1, 0, g, p);
  else
    kern<<<g.nranges * g.gsplit, kSweepThreads, sh, s>>>(g, p);
}

// launch with NKS = r / 16 fixed at compile time (r in {16, 32, 64, 128, 256}) and two
// pipeline stages.  A third stage still fits two one-stream workgroups in a CU's LDS, but the
// draft sweep at R = 256, V = 151936, r = 256 ran 32.4-35.4 us with three against
// 29.8-31.8 us with two (interleaved runs on one device).
template <int NKS, bool SPLIT, class Epi>
inline void launch_sweep_stages(const SweepGeom& g, const typename Epi::Params& p, hipStream_t s,
                                hipEvent_t ev0, hipEvent_t ev1) {
  launch_sweep_nks<NKS, SPLIT, 2, Epi>(g, p, s, ev0, ev1);
}

template <bool SPLIT, class Epi>
inline void launch_sweep(const SweepGeom& g, const typename Epi::Params& p, hipStream_t s,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
  switch (g.nks) {
    case 1: launch_sweep_stages<1, SPLIT, Epi>(g, p, s, ev0, ev1); break;
    case 2: launch_sweep_stages<2, SPLIT, Epi>(g, p, s, ev0, ev1); break;
    case 4: launch_sweep_stages<4, SPLIT, Epi>(g, p, s, ev0, ev1); break;
    case 8: launch_sweep_stages<8, SPLIT, Epi>(g, p, s, ev0, ev1); break;
    default: launch_sweep_stages<16, SPLIT, Epi>(g, p, s, ev0, ev1);
  }
}

}  // namespace dspark
