// draft_epi.h -- the draft sweep's epilogue (sweep.h's Epi interface): per row and
// vocabulary range, the running normaliser of l = U_k + bias_k and the first level of the
// two-level Gumbel-max sampler (digest, Module B and the sampling notes: block scores
// LSE_b + g_b over 64-id blocks).  Together with sweep.h and dev.h this is the whole source
// of the draft sweep kernel.
#pragma once

#include "dev.h"
#include "sweep.h"

namespace dspark {

struct DraftSweepParams {
  const uint16_t* U;     // U + (k-1)*V; row q at U + q*ustride  (bf16)
  size_t ustride;        // gamma * V
  int V, R;
  const int32_t* prev;   // x_{k-1} of row q at prev[q * prev_stride]
  int prev_stride;
  const uint16_t* W1;    // Markov B rows: W1[x_{k-1}]
  const float* orow;     // RNN B rows: tanh(W_o z_k), [R][r] float
  const uint4* bpack;    // Markov B rows W1[x_{k-1}] in the sweep's packed order
  int r;
  uint32_t k;            // position, 1-based
  uint64_t seed, cycle;
  float4* partials;      // [R][nranges]: (max, sum exp, best G, best block)
  int nranges;
  int32_t* status;
};

// BIAS = false: the sampling of the parallel block alone (logits U_k, no head bias), the
// drafter the sequential head is measured against
template <bool RNN, bool BIAS = true>
struct DraftEpi {
  static constexpr int kStreams = 1;  // U_k
  static constexpr bool kNoBias = !BIAS;
  using Params = DraftSweepParams;
  // Row state, kept alike in the row's two lanes except for the partial sums: one running
  // reference ref (log2 units: the largest l * log2(e) seen so far), so each tile's
  // exponentials are taken against it directly and only the sums rescale when it grows.
  struct State {
    float ref;    // running reference of the row (log2 units)
    float S;      // this lane's sum of exp2(l log2e - ref) over finished blocks
    float hs;     // this lane's sum over the first half of the current block
    float G;      // best first-level score LSE_b + g_b of the range so far
    int B;        // its block
    int grp;      // block group (4 blocks) whose random words are cached
    uint4 words;
  };
  __device__ static bool group_live(const Params& p, int row0) { return row0 < p.R; }
  __device__ static int nrows(const Params& p) { return p.R; }
  __device__ static const void* brow(const Params& p, int row) {
    if (RNN) return p.orow + (size_t)row * p.r;
    const int32_t t = checked_token(p.prev[(size_t)row * p.prev_stride], p.V, p.status);
    return p.W1 + (size_t)t * p.r;
  }
  __device__ static const uint4* bpack(const Params& p) { return RNN ? nullptr : p.bpack; }
  __device__ static const uint16_t* sbase(const Params& p, int) { return p.U; }
  __device__ static uint32_t srow(const Params& p, int, int row) {
    return (uint32_t)((size_t)row * p.ustride);
  }
  __device__ static void init(const Params&, State& s, int) {
    s.ref = -FLT_MAX;  // finite: ref - new_ref never forms inf - inf
    s.S = 0.0f;
    s.hs = 0.0f;
    s.G = -INFINITY;
    s.B = 0x7fffffff;
    s.grp = -1;
    s.words = make_uint4(0, 0, 0, 0);
  }
  // random words of block b's group of four (uniform value across the wave)
  __device__ static void refresh(const Params& p, State& s, int b, int row) {
    if ((b >> 2) != s.grp) {
      s.grp = b >> 2;
      s.words = Rng(p.seed, p.cycle).block(kStreamDraftBlk, (uint32_t)row, p.k, (uint32_t)s.grp);
    }
  }
  // one 32-id tile (half HALF of block b): its exponentials join the lane's sums; after the
  // second half, the block's LSE_b + g_b enters the running first-level Gumbel-max.
  // Branch-free unless MASK.  Rows past R compute on clamped data and are never written.
  template <int HALF, bool MASK>
  __device__ static void tile(const Params& p, State& s, const f32x16& acc, const uint4 (&)[2],
                              int b, int, bool) {
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kLn2 = 0.69314718055994531f;
    const int h = (threadIdx.x & 63) >> 5;
    float l[16];  // U_k + bias (the accumulator was seeded with U_k)
#pragma unroll
    for (int j = 0; j < 16; ++j) l[j] = acc[j];
    if (MASK) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (b * kVB + kTile * HALF + vocab_of_reg(h, j) >= p.V) l[j] = -INFINITY;
    }
    float m = fmaxf(fmaxf(l[0], l[1]), l[2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) m = fmaxf(fmaxf(m, l[j]), l[j + 1]);
    m = fmaxf(m, l[15]);
    const float ref = fmaxf(s.ref, half_max(m * kLog2e));
    const float sc = __builtin_amdgcn_exp2f(s.ref - ref);
    s.S *= sc;
    if (HALF == 1) s.hs *= sc;
    s.ref = ref;
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += __builtin_amdgcn_exp2f(fmaf(l[j], kLog2e, -ref));
    if (HALF == 0) {
      s.hs = sum;
      return;
    }
    const float own = s.hs + sum;  // this lane's share of block b
    s.S += own;
    const float lse_b = (ref + __builtin_amdgcn_logf(half_sum(own))) * kLn2;
    const float G = lse_b + gumbel_of(pick_word(s.words, (uint32_t)b & 3u));
    const bool better = G > s.G;
    s.G = better ? G : s.G;
    s.B = better ? b : s.B;
  }
  __device__ static void finish(const Params& p, const State& s, int row, bool owner, int range) {
    const float S = half_sum(s.S);
    if (!owner) return;
    p.partials[(size_t)row * p.nranges + range] =
        make_float4(s.ref * 0.69314718055994531f, S, s.G, __int_as_float(s.B));
  }
};

}  // namespace dspark
