// verify.hip -- lossless verification of the scheduled prefixes (digest page, overall cycle
// step 3; explainer page, section 06 single-token rule; eq. (8) for the analytic
// acceptance c*).
//
// Rows are flattened the way the digest's production section describes variable-length
// verification: the scheduled positions of all requests form one ragged list, so no row
// is padded.  Launches:
//   prep    one workgroup: exclusive scans of ell; list A = (q, j) for j = 1..ell_q + 1
//           (every row whose target normaliser is needed, the bonus row included), list B
//           = (q, j) for j = 1..ell_q (every verified position);
//   lse     each list-A row in wave items of 64 blocks of 64 ids (a grid of at most four
//           workgroups per CU walks the items, whose count is known on the device only;
//           loads coalesced, 8 lanes per block): (max, sum exp) of the target logits; on
//           the bonus row also the first level of the bonus sample (stream 5);
//   decide  one wave per request, one lane per position: merges the lse items into the
//           target normalisers (and the bonus block), then the acceptance tests
//           u < p_j(x_j)/q_j(x_j) (stream 2), the first rejection j*, the accepted tokens;
//   sweep   matrix cores over list B (sweep.h): q_j recomputed from U_j + bias_j W2 and
//           normalised by the drafted lse; sum |p - q| per row, and on the row j* the
//           residual max(0, p - q) per 64-id block with its first-level Gumbel score
//           (stream 3);
//   final   one workgroup of four waves per request: c* for every verified row, then the
//           second level of the correction (stream 4) or of the bonus (stream 6), written
//           as the last emitted token (and, when asked, as the next cycle's anchor).
#include <type_traits>

#include "dev.h"
#include "host.h"
#include "sweep.h"

namespace dspark {

constexpr int kLseThreads = 256;  // lse pass: four independent waves per workgroup

// the lse pass works in wave items: 64 consecutive 64-id blocks (4096 ids) of one row
__host__ __device__ inline int lse_witems(int V) { return ((V + kVB - 1) / kVB + kWave - 1) / kWave; }

struct VerifyWs {
  int* hdr;        // [0] = |A|, [1] = |B|
  int* offA;       // [R]
  int* offB;       // [R]
  int4* rowA;      // [R*(gamma+1)] (q, j, 1 if j is the bonus row, 0)
  int2* rowB;      // [R*gamma]
  float* lset;     // [R*(gamma+1)] target log-sum-exp of list-A rows
  float4* lpart;   // [R*(gamma+1)][lse_witems(V)] (max, sum exp, best G, block) per item
  float2* bonus;   // [R] (best G, block) of the bonus row
  int* jstar;      // [R] first rejected position, 0 = none
  float4* partials;  // [R*gamma][nranges]: (sum |p-q|, best G, block, residual mass)
  uint4* bpack;      // list-B bias rows (bf16) in the sweep's packed order, or null
  size_t bytes;
};

static VerifyWs carve_verify(void* ws, int R, int gamma, int V, int r) {
  Carve cv(ws);
  VerifyWs w{};
  w.hdr = cv.take<int>(4);
  w.offA = cv.take<int>((size_t)R);
  w.offB = cv.take<int>((size_t)R);
  w.rowA = cv.take<int4>((size_t)R * (gamma + 1));
  w.rowB = cv.take<int2>((size_t)R * gamma);
  w.lset = cv.take<float>((size_t)R * (gamma + 1));
  w.lpart = cv.take<float4>((size_t)R * (gamma + 1) * lse_witems(V));
  w.bonus = cv.take<float2>((size_t)R);
  w.jstar = cv.take<int>((size_t)R);
  const int nblocks = (V + kVB - 1) / kVB;
  w.partials = cv.take<float4>((size_t)R * gamma * (nblocks < kMaxRanges ? nblocks : kMaxRanges));
  w.bpack = cv.take<uint4>((size_t)bpack_rows(R * gamma) * r / 8);
  w.bytes = cv.bytes();
  return w;
}

// ---------------------------------------------------------------------------------------
// prep: ragged row lists from ell
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) verify_prep_kernel(int R, int gamma, const int32_t* ell_in,
                                                           VerifyWs ws, int32_t* status) {
  __shared__ int totA[1024 / kWave], totB[1024 / kWave];
  const int per = (R + 1023) / 1024;
  const int lo = threadIdx.x * per, hi = min(R, lo + per);
  int sa = 0, sb = 0;
  for (int q = lo; q < hi; ++q) {
    int L = ell_in[q];
    if (L < 0 || L > gamma) {
      raise_fault(status, DSPARK_FAULT_LEN);
      L = L < 0 ? 0 : gamma;
    }
    sa += L + 1;
    sb += L;
  }
  // exclusive prefix sums of the per-thread totals: inclusive scans inside each wave, then a
  // scan of the 16 wave totals (two barriers)
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int ia = sa, ib = sb;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int ua = __shfl_up(ia, o, kWave), ub = __shfl_up(ib, o, kWave);
    if (lane >= o) {
      ia += ua;
      ib += ub;
    }
  }
  if (lane == kWave - 1) {
    totA[wave] = ia;
    totB[wave] = ib;
  }
  __syncthreads();
  if (wave == 0) {
    int xa = lane < 1024 / kWave ? totA[lane] : 0, xb = lane < 1024 / kWave ? totB[lane] : 0;
#pragma unroll
    for (int o = 1; o < 1024 / kWave; o <<= 1) {
      const int ua = __shfl_up(xa, o, kWave), ub = __shfl_up(xb, o, kWave);
      if (lane >= o) {
        xa += ua;
        xb += ub;
      }
    }
    if (lane < 1024 / kWave) {
      totA[lane] = xa;  // inclusive totals through wave `lane`
      totB[lane] = xb;
    }
  }
  __syncthreads();
  int oa = ia - sa + (wave > 0 ? totA[wave - 1] : 0);
  int ob = ib - sb + (wave > 0 ? totB[wave - 1] : 0);
  for (int q = lo; q < hi; ++q) {
    int L = ell_in[q];
    L = L < 0 ? 0 : (L > gamma ? gamma : L);
    ws.offA[q] = oa;
    ws.offB[q] = ob;
    for (int j = 1; j <= L + 1; ++j) ws.rowA[oa + j - 1] = make_int4(q, j, j == L + 1, 0);
    for (int j = 1; j <= L; ++j) ws.rowB[ob + j - 1] = make_int2(q, j);
    oa += L + 1;
    ob += L;
  }
  if (threadIdx.x == 1023) {
    ws.hdr[0] = totA[1024 / kWave - 1];
    ws.hdr[1] = totB[1024 / kWave - 1];
  }
}

__device__ __forceinline__ int clamp_len(int L, int gamma) { return L < 0 ? 0 : (L > gamma ? gamma : L); }

// ---------------------------------------------------------------------------------------
// lse: (max, sum exp) of every 4096-id wave item of the list-A rows (+ first level of the
// bonus sample)
// ---------------------------------------------------------------------------------------
// reductions over the 8 lanes 8k .. 8k+7 on the DPP network (xor 1, xor 2, then the
// half-row mirror, which pairs the two quads)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  return fmaxf(x, dpp_f<0x141>(x));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  return x + dpp_f<0x141>(x);
}

// one wave's eight chunks of a 64-block window, held raw until they are used
template <class T>
struct LseRaw;
template <>
struct LseRaw<uint16_t> {
  uint4 c[8];
  __device__ __forceinline__ void load(const uint16_t* row, const int (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = *reinterpret_cast<const uint4*>(row + v[k]);
  }
  __device__ __forceinline__ void widen_one(int k, float (&x)[8]) const { widen8(c[k], x); }
};
template <>
struct LseRaw<float> {
  float4 c[16];
  __device__ __forceinline__ void load(const float* row, const int (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      c[2 * k] = *reinterpret_cast<const float4*>(row + v[k]);
      c[2 * k + 1] = *reinterpret_cast<const float4*>(row + v[k] + 4);
    }
  }
  __device__ __forceinline__ void widen_one(int k, float (&x)[8]) const {
    const float4 a = c[2 * k], b = c[2 * k + 1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

template <class T>
__global__ void __launch_bounds__(kLseThreads) verify_lse_kernel(int R, int gamma, int V,
                                                                 const T* __restrict__ target,
                                                                 const int32_t* ell, VerifyWs ws,
                                                                 uint64_t seed, uint64_t cycle) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.69314718055994531f;
  const int per_row = lse_witems(V);
  const int nitems = ws.hdr[0] * per_row;
  const int nblocks = (V + kVB - 1) / kVB;
  const int lane = threadIdx.x & 63;
  // every wave is an independent worker over the wave items (no barriers, no LDS): the
  // next item's descriptor loads while the current one streams
  const int gw = blockIdx.x * (kLseThreads / kWave) + (threadIdx.x >> 6);
  const int W = gridDim.x * (kLseThreads / kWave);
  const Rng rng(seed, cycle);
  // Wave item wi of a row covers blocks 64 wi .. 64 wi + 64 in 8 coalesced rounds: in round
  // c lane l holds chunk l & 7 of block 8c + l/8.  One reference serves the whole window
  // (its largest logit), so the row needs no per-block max; on the bonus row the block sums
  // are 8-lane reductions on the DPP network.
  auto offsets = [&](int item, int4 inf, const T*& row, int (&v)[8]) {
    row = target + ((size_t)inf.x * (gamma + 1) + (inf.y - 1)) * V;
    const int bw = (item % per_row) * kWave;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[c] = (bw + 8 * c + (lane >> 3)) * kVB + 8 * (lane & 7);
      v[c] = v[c] < V ? v[c] : V - 8;  // clamped, unconditional loads (V % 8 == 0)
    }
  };
  // the row descriptor of the next item is fetched while the current one streams (clamped
  // index: an unconditional global load)
  if (gw >= nitems) return;
  int4 info = ws.rowA[gw / per_row];
  for (int item = gw; item < nitems; item += W) {
    const int nxt = item + W < nitems ? item + W : item;
    const int4 info1 = ws.rowA[nxt / per_row];
    LseRaw<T> cur;
    {
      const T* row;
      int v[8];
      offsets(item, info, row, v);
      cur.load(row, v);
    }
    __builtin_amdgcn_sched_barrier(0);  // all eight loads go out before their first use
    const int q = info.x, j = info.y;
    const bool bonus = info.z != 0;
    const int bw = (item % per_row) * kWave;  // first block of this wave item
    // The item's arithmetic, with ids past V masked only in a window that reaches the end
    // of the row (MASK); every other window skips the per-element selects.
    float mx, ref, S, G;
    int Bk;
    auto item_math = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // chunk c widened on demand (twice: for the max, then for the sums), which keeps the
      // register footprint at two raw items
      auto chunk = [&](int c, float (&x)[8]) {
        cur.widen_one(c, x);
        if (MASK) {
          const int v = (bw + 8 * c + (lane >> 3)) * kVB + 8 * (lane & 7);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = v < V ? x[e] : -INFINITY;
        }
      };
      mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float x[8];
        chunk(c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[e]);
      }
      mx = wave_max(mx);
      ref = mx == -INFINITY ? 0.0f : mx * kLog2e;
      // bonus row: lane l owns block bw + l (its Gumbel noise, and its sum gathered from
      // the chunk that holds it)
      float gb = 0.0f;
      if (bonus) {
        const uint32_t b = (uint32_t)(bw + lane);
        gb = gumbel_of(pick_word(rng.block(kStreamBonusBlk, (uint32_t)q, (uint32_t)j, b >> 2), b & 3u));
      }
      float bmine = 0.0f;
      S = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float x[8];
        chunk(c, x);
        float sb = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb += __builtin_amdgcn_exp2f(fmaf(x[e], kLog2e, -ref));
        S += sb;
        if (bonus) {
          // block 8c + m sums over lanes 8m .. 8m+7; lane 8c + m takes it from lane 8m
          const float bs = __shfl(sum8(sb), 8 * (lane & 7), kWave);
          bmine = (lane >> 3) == c ? bs : bmine;
        }
      }
      G = -INFINITY;
      Bk = 0x7fffffff;
      if (bonus) {
        const int b = bw + lane;
        if (b < nblocks && bmine > 0.0f) {
          G = (ref + __builtin_amdgcn_logf(bmine)) * kLn2 + gb;
          Bk = b;
        }
      }
    };
    if ((bw + kWave) * kVB <= V)
      item_math(std::false_type{});
    else
      item_math(std::true_type{});
    S = wave_sum(S);
    const float M = mx == -INFINITY ? -INFINITY : ref * kLn2;
    wave_argmax(G, Bk);
    if (lane == 0) ws.lpart[item] = make_float4(M, S, G, __int_as_float(Bk));
    info = info1;
  }
}

// ---------------------------------------------------------------------------------------
// decide: acceptance tests in order
// ---------------------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(64) verify_decide_kernel(
    int R, int gamma, int V, const T* __restrict__ target, const int32_t* __restrict__ x,
    const float* __restrict__ lse, const float* __restrict__ logit_x, const int32_t* ell,
    VerifyWs ws, uint64_t seed, uint64_t cycle, int32_t* n_acc, int32_t* y, int32_t* status,
    const uint16_t* __restrict__ brows, int r) {
  // one wave per request; lane j - 1 tests position j (gamma <= 64)
  const int q = blockIdx.x, lane = threadIdx.x, j = lane + 1;
  const int L = clamp_len(ell[q], gamma);
  // the acceptance test's operands first (they do not depend on the normalisers, so this
  // chain of loads overlaps the packing and the merges below): x_j, its target logit,
  // log q_j(x_j) and the uniform
  bool bad = false;
  int xj = 0;
  float tv = 0.0f, lq = 0.0f, u_acc = 0.0f;
  if (j <= L) {
    const size_t rj = (size_t)q * gamma + (j - 1);
    const int32_t t = x[rj];
    bad = t < 0 || t >= V;
    xj = bad ? 0 : t;
    tv = ld<T>(target, ((size_t)q * (gamma + 1) + (j - 1)) * V + xj);
    lq = logit_x[rj] - lse[rj];  // log q_j(x_j)
    u_acc = uniform_of(Rng(seed, cycle).word(kStreamAccept, (uint32_t)q, (uint32_t)j, 0u));
  }
  if (brows) {
    // the sweep's B rows for this request's list-B rows, in its packed order: half-waves
    // take one row each, lane & 31 its 16-byte chunk; four row pairs in flight per pass
    const int ob = ws.offB[q], cpr = r / 8, ch = lane & 31;
    for (int j0 = 0; j0 < L; j0 += 8) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jr = j0 + 2 * u + (lane >> 5);
        const int jc = jr < L ? jr : 0;
        v[u] = reinterpret_cast<const uint4*>(brows + ((size_t)q * gamma + jc) * r)[ch < cpr ? ch : 0];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jr = j0 + 2 * u + (lane >> 5);
        if (jr < L && ch < cpr) ws.bpack[bpack_index(ob + jr, ch, r / 16)] = v[u];
      }
    }
  }
  // target normaliser of rows 1..L+1 from their lse items, lane jj - 1 taking row jj: all of
  // a row's items in flight together (up to 40 per pass: one round trip for rows of up to
  // 40 x 4096 ids), then the largest maximum and one rescaled sum, so the exponentials are
  // independent; the best (G, block) with ties to the lowest block; the bonus row's winner
  const int tiles = lse_witems(V);
  float lset_j = 0.0f;
  for (int jj = j; jj <= L + 1; jj += kWave) {
    const int i = ws.offA[q] + jj - 1;
    float M = -INFINITY, S = 0.0f, G = -INFINITY;
    int Bk = 0x7fffffff;
    constexpr int kPass = 40;
    for (int pc0 = 0; pc0 < tiles; pc0 += kPass) {
      float4 o[kPass];  // clamped, unconditional loads
#pragma unroll
      for (int u = 0; u < kPass; ++u)
        o[u] = ws.lpart[(size_t)i * tiles + (pc0 + u < tiles ? pc0 + u : tiles - 1)];
      // predicates, not breaks: the loops stay fully unrolled over registers
      float mp = -INFINITY;
#pragma unroll
      for (int u = 0; u < kPass; ++u)
        if (pc0 + u < tiles) mp = fmaxf(mp, o[u].x);
      const float ref = mp == -INFINITY ? 0.0f : mp;
      float sp = 0.0f;
#pragma unroll
      for (int u = 0; u < kPass; ++u)
        if (pc0 + u < tiles && o[u].x != -INFINITY) sp += o[u].y * __expf(o[u].x - ref);
      lse_merge(M, S, mp, sp);
#pragma unroll
      for (int u = 0; u < kPass; ++u) {
        const int ob = __float_as_int(o[u].w);
        if (pc0 + u < tiles && (o[u].z > G || (o[u].z == G && ob < Bk))) {
          G = o[u].z;
          Bk = ob;
        }
      }
    }
    const float ls = M + __logf(S);
    ws.lset[i] = ls;
    if (jj == j) lset_j = ls;
    if (jj == L + 1) ws.bonus[q] = make_float2(G, __int_as_float(Bk));
  }
  bool reject = false;
  if (j <= L) {
    const float lp = tv - lset_j;  // log p_j(x_j)
    reject = !(u_acc < __expf(lp - lq));
  }
  // the tests run in order: the first rejection ends them
  const unsigned long long rm = __ballot(reject);
  const int js = rm ? __ffsll(rm) : 0;
  const int na = js ? js - 1 : L;
  if (bad && j <= (js ? js : L)) raise_fault(status, DSPARK_FAULT_TOKEN);
  if (lane == 0) {
    ws.jstar[q] = js;
    n_acc[q] = na;
  }
  int32_t* yq = y + (size_t)q * (gamma + 1);
  if (lane <= gamma) yq[lane] = lane < na ? xj : -1;  // lane j - 1 holds x_j
  if (gamma == kWave && lane == 0) yq[kWave] = -1;
}

// ---------------------------------------------------------------------------------------
// sweep epilogue over list B
// ---------------------------------------------------------------------------------------
struct VerifySweepParams {
  const uint16_t* U;        // [R][gamma][V]
  const uint16_t* target;   // [R][gamma+1][V]
  const void* brows;        // [R][gamma][r] bf16 or float
  const float* lse;         // [R][gamma]
  int R, gamma, V, r;
  VerifyWs ws;
  uint64_t seed, cycle;
  int nranges;
};

template <bool SPLIT>
struct VerifyEpi {
  static constexpr int kStreams = 2;  // U_j, target row j
  using Params = VerifySweepParams;
  struct State {
    float tv;          // sum |p - q| over this range
    float G, mass;     // residual: best block score, total mass
    int B;
    int q, j, resid;   // this lane's row
    float lq, lp;      // normalisers (draft lse, target lse)
    float hr;          // residual mass of the first half of the current block
    int grp;
    uint4 words;
  };
  __device__ static bool group_live(const Params& p, int row0) { return row0 < p.ws.hdr[1]; }
  __device__ static int nrows(const Params& p) { return p.ws.hdr[1]; }
  __device__ static const void* brow(const Params& p, int row) {
    const int2 qj = p.ws.rowB[row];
    const size_t off = ((size_t)qj.x * p.gamma + (qj.y - 1)) * p.r;
    if (SPLIT) return static_cast<const float*>(p.brows) + off;
    return static_cast<const uint16_t*>(p.brows) + off;
  }
  __device__ static const uint4* bpack(const Params& p) { return SPLIT ? nullptr : p.ws.bpack; }
  __device__ static const uint16_t* sbase(const Params& p, int s) { return s == 0 ? p.U : p.target; }
  __device__ static uint32_t srow(const Params& p, int s, int row) {
    const int2 qj = p.ws.rowB[row];
    if (s == 0) return (uint32_t)(((size_t)qj.x * p.gamma + (qj.y - 1)) * p.V);
    return (uint32_t)(((size_t)qj.x * (p.gamma + 1) + (qj.y - 1)) * p.V);
  }
  __device__ static void init(const Params& p, State& s, int row) {
    s.tv = 0.0f;
    s.G = -INFINITY;
    s.mass = 0.0f;
    s.B = 0x7fffffff;
    s.grp = -1;
    s.words = make_uint4(0, 0, 0, 0);
    s.q = 0;
    s.j = 1;
    s.resid = 0;
    s.lq = s.lp = 0.0f;
    s.hr = 0.0f;
    if (row >= 0) {
      const int2 qj = p.ws.rowB[row];
      s.q = qj.x;
      s.j = qj.y;
      s.resid = (p.ws.jstar[qj.x] == qj.y);
      s.lq = p.lse[(size_t)qj.x * p.gamma + (qj.y - 1)];
      s.lp = p.ws.lset[p.ws.offA[qj.x] + qj.y - 1];
    }
  }
  __device__ static void refresh(const Params& p, State& s, int b, int) {
    if (s.resid && (b >> 2) != s.grp) {
      s.grp = b >> 2;
      s.words = Rng(p.seed, p.cycle).block(kStreamResidBlk, (uint32_t)s.q, (uint32_t)s.j,
                                           (uint32_t)s.grp);
    }
  }
  // one 32-id tile: q from the logits and the draft normaliser, p from the target and its
  // normaliser; sum |p - q| always, and on the first rejected row the residual mass of the
  // 64-id block with its first-level Gumbel score
  template <int HALF, bool MASK>
  __device__ static void tile(const Params& p, State& s, const f32x16& acc, const uint4 (&x)[2],
                              int b, int, bool owner) {
    const int h = (threadIdx.x & 63) >> 5;
    float t[16];  // target logits of the tile; acc holds U_j + bias
    widen8(x[0], t);
    widen8(x[1], t + 8);
    float tv = 0.0f, rho = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool ok = !MASK || b * kVB + kTile * HALF + vocab_of_reg(h, j) < p.V;
      const float qv = ok ? __expf(acc[j] - s.lq) : 0.0f;
      const float pv = ok ? __expf(t[j] - s.lp) : 0.0f;
      tv += fabsf(pv - qv);
      rho += fmaxf(pv - qv, 0.0f);
    }
    tv = half_sum(tv);
    rho = half_sum(rho);
    s.tv += owner ? tv : 0.0f;
    if (HALF == 0) {
      s.hr = rho;
      return;
    }
    rho += s.hr;  // the whole 64-id block
    const bool mine = owner && s.resid;
    const float G = (rho > 0.0f) ? __logf(rho) + gumbel_of(pick_word(s.words, (uint32_t)b & 3u))
                                 : -INFINITY;
    const bool better = mine && G > s.G;
    s.mass += mine ? rho : 0.0f;
    s.G = better ? G : s.G;
    s.B = better ? b : s.B;
  }
  __device__ static void finish(const Params& p, const State& s, int row, bool owner, int range) {
    if (!owner) return;
    p.ws.partials[(size_t)row * p.nranges + range] = make_float4(s.tv, s.G, __int_as_float(s.B), s.mass);
  }
};

// float operands: one wave per (list-B row, range), VALU only
__global__ void __launch_bounds__(64) verify_sweep_f32_kernel(
    int gamma, int V, int r, const float* __restrict__ U, const float* __restrict__ target,
    const float* __restrict__ W2t, const float* __restrict__ brows,
    const float* __restrict__ lse, VerifyWs ws, uint64_t seed, uint64_t cycle, int nranges,
    int nblocks) {
  const int row = blockIdx.y, range = blockIdx.x, lane = threadIdx.x;
  if (row >= ws.hdr[1]) return;
  const int2 qj = ws.rowB[row];
  const int q = qj.x, j = qj.y;
  const size_t rj = (size_t)q * gamma + (j - 1);
  const float* e = brows + rj * r;
  const float* trow = target + ((size_t)q * (gamma + 1) + (j - 1)) * V;
  const float lq = lse[rj], lp = ws.lset[ws.offA[q] + j - 1];
  const bool resid = ws.jstar[q] == j;
  const int per = (nblocks + nranges - 1) / nranges;
  const int b0 = range * per, b1 = min(nblocks, b0 + per);
  const Rng rng(seed, cycle);
  float tv = 0.0f, G = -INFINITY, mass = 0.0f;
  int Bk = 0x7fffffff;
  for (int b = b0; b < b1; ++b) {
    const int v = b * kVB + lane;
    float d = 0.0f, rho = 0.0f;
    if (v < V) {
      float acc = 0.0f;
      for (int i = 0; i < r; ++i) acc = fmaf(e[i], W2t[(size_t)v * r + i], acc);
      const float qv = __expf(U[rj * V + v] + acc - lq);
      const float pv = __expf(trow[v] - lp);
      d = fabsf(pv - qv);
      rho = fmaxf(pv - qv, 0.0f);
    }
    tv += wave_sum(d);
    const float m = wave_sum(rho);
    if (resid) {
      mass += m;
      if (m > 0.0f) {
        const float Gb = __logf(m) + gumbel_of(rng.word(kStreamResidBlk, (uint32_t)q, (uint32_t)j, (uint32_t)b));
        if (Gb > G) {
          G = Gb;
          Bk = b;
        }
      }
    }
  }
  if (lane == 0) ws.partials[(size_t)row * nranges + range] = make_float4(tv, G, __int_as_float(Bk), mass);
}

// two-level Gumbel-max over a whole row of logits, one wave (fallback of the correction
// when the residual mass is zero in floating point)
template <class T>
__device__ int sample_row_wave(const T* row, int V, const Rng& rng, uint32_t sblk, uint32_t sin,
                               uint32_t q, uint32_t k) {
  const int lane = threadIdx.x & 63;
  const int nblocks = (V + kVB - 1) / kVB;
  float G = -INFINITY;
  int Bk = 0;
  for (int b = 0; b < nblocks; ++b) {
    const int v = b * kVB + lane;
    const float l = v < V ? ld<T>(row, v) : -INFINITY;
    const float m = wave_max(l);
    const float s = wave_sum(l == -INFINITY ? 0.0f : __expf(l - m));
    const float Gb = m + __logf(s) + gumbel_of(rng.word(sblk, q, k, (uint32_t)b));
    if (Gb > G) {
      G = Gb;
      Bk = b;
    }
  }
  const int v = Bk * kVB + lane;
  float score = v < V ? ld<T>(row, v) + gumbel_of(rng.word(sin, q, k, (uint32_t)v)) : -INFINITY;
  int idx = v;
  wave_argmax(score, idx);
  return idx;
}

// ---------------------------------------------------------------------------------------
// final: c* of every verified row, then the correction or the bonus token
// ---------------------------------------------------------------------------------------
constexpr int kFinalThreads = 256;  // per request in the final step

template <class T, class BT>
__global__ void __launch_bounds__(kFinalThreads) verify_final_kernel(
    int R, int gamma, int V, int r, const T* __restrict__ target, const T* __restrict__ U,
    const T* __restrict__ W2t, const BT* __restrict__ brows, const float* __restrict__ lse,
    const int32_t* ell, VerifyWs ws, int nranges, uint64_t seed, uint64_t cycle,
    const int32_t* n_acc, int32_t* y, float* c_star, int32_t* x_next) {
  constexpr int kWaves = kFinalThreads / kWave;
  constexpr int kJ = 8;  // verified rows whose range sums are in flight together
  __shared__ float tvs[kWaves][kJ];
  __shared__ float4 red[kWaves];
  __shared__ float dotp[kWaves][kWave];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = clamp_len(ell[q], gamma);
  const int nblocks = (V + kVB - 1) / kVB;
  const int js = ws.jstar[q];
  const size_t offB = (size_t)ws.offB[q];

  // c* = 1 - 1/2 sum |p - q| for every verified row (eq. (8)); NaN past the scheduled length
  for (int j0 = 1; j0 <= gamma; j0 += kJ) {
    float sum[kJ];
    // every range of the kJ rows at once (unconditional loads of clamped addresses, so
    // they are all in flight together)
#pragma unroll
    for (int u = 0; u < kJ; ++u) sum[u] = 0.0f;
    for (int i0 = 0; i0 < nranges; i0 += kFinalThreads) {
      const int i = i0 + tid;
      float v[kJ];
#pragma unroll
      for (int u = 0; u < kJ; ++u) {
        const int jj = j0 + u <= L ? j0 + u : 1;
        v[u] = ws.partials[(offB + jj - 1) * nranges + (i < nranges ? i : 0)].x;
      }
#pragma unroll
      for (int u = 0; u < kJ; ++u) sum[u] += (j0 + u <= L && i < nranges) ? v[u] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      const float t = wave_sum(sum[u]);
      if (lane == 0) tvs[wave][u] = t;
    }
    __syncthreads();
    if (tid < kJ && j0 + tid <= gamma) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += tvs[w][tid];
      c_star[(size_t)q * gamma + (j0 + tid - 1)] =
          (j0 + tid <= L) ? 1.0f - 0.5f * t : __int_as_float(0x7fc00000);
    }
    __syncthreads();
  }

  const Rng rng(seed, cycle);
  // the block the token is drawn from: the residual's winning block at the first rejected
  // row, or the bonus row's
  int Bk;
  float mass = 1.0f;
  if (js > 0) {
    const size_t row = offB + js - 1;
    float G = -INFINITY, m = 0.0f;
    int B = 0x7fffffff;
    for (int i = tid; i < nranges; i += kFinalThreads) {
      const float4 pr = ws.partials[row * nranges + i];
      const int pb = __float_as_int(pr.z);
      m += pr.w;
      if (pr.y > G || (pr.y == G && pb < B)) {
        G = pr.y;
        B = pb;
      }
    }
    m = wave_sum(m);
    wave_argmax(G, B);
    if (lane == 0) red[wave] = make_float4(G, m, __int_as_float(B), 0.0f);
    __syncthreads();
    G = red[0].x;
    m = red[0].y;
    B = __float_as_int(red[0].z);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float4 o = red[w];
      m += o.y;
      const int ob = __float_as_int(o.z);
      if (o.x > G || (o.x == G && ob < B)) {
        G = o.x;
        B = ob;
      }
    }
    mass = m;
    Bk = B;
  } else {
    Bk = __float_as_int(ws.bonus[q].y);
  }
  const bool resid_ok = js > 0 && mass > 0.0f && Bk >= 0 && Bk < nblocks;
  if (Bk < 0 || Bk >= nblocks) Bk = 0;
  const int jrow = js > 0 ? js : L + 1;  // target row of the draw
  const T* trow = target + ((size_t)q * (gamma + 1) + (jrow - 1)) * V;
  const int v = Bk * kVB + lane;

  // residual: q over the winning block, the k sum split over the waves in 8-element chunks
  if (resid_ok) {
    const size_t rj = (size_t)q * gamma + (js - 1);
    float part = 0.0f;
    if (v < V) {
      const BT* e = brows + rj * r;
      const T* wr = W2t + (size_t)v * r;
      // r <= 256: at most 8 chunks per wave, all loads in flight together
      float a[8][8], bv[8][8];
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int ch = wave + kWaves * it < r / 8 ? wave + kWaves * it : 0;
        ld8<T>(wr + ch * 8, a[it]);
        ld8<BT>(e + ch * 8, bv[it]);
      }
#pragma unroll
      for (int it = 0; it < 8; ++it)
        if (wave + kWaves * it < r / 8)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) part = fmaf(bv[it][jj], a[it][jj], part);
    }
    dotp[wave][lane] = part;
    __syncthreads();
  }
  if (wave != 0) return;
  int token;
  if (js > 0) {
    if (resid_ok) {
      const size_t rj = (size_t)q * gamma + (js - 1);
      const float lq = lse[rj], lp = ws.lset[ws.offA[q] + js - 1];
      float score = -INFINITY;
      if (v < V) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += dotp[w][lane];
        const float qv = __expf(ld<T>(U, rj * V + v) + acc - lq);
        const float pv = __expf(ld<T>(trow, v) - lp);
        const float rho = pv - qv;
        if (rho > 0.0f)
          score = __logf(rho) + gumbel_of(rng.word(kStreamResidIn, (uint32_t)q, (uint32_t)js, (uint32_t)v));
      }
      int idx = v;
      wave_argmax(score, idx);
      // The block was chosen from the sweep's residual masses; recomputed here in another
      // order, every rho of a block with rounding-level mass can come out <= 0.  No id of
      // it may be emitted then (its residual probability is zero): the draw falls back to
      // the target row, as for a zero residual mass.  The whole wave holds the same score.
      token = score > -INFINITY
                  ? idx
                  : sample_row_wave<T>(trow, V, rng, kStreamResidBlk, kStreamResidIn,
                                       (uint32_t)q, (uint32_t)js);
    } else {
      // the residual mass is zero in floating point: draw from the target row instead
      token = sample_row_wave<T>(trow, V, rng, kStreamResidBlk, kStreamResidIn, (uint32_t)q,
                                 (uint32_t)js);
    }
  } else {
    float score = v < V ? ld<T>(trow, v) + gumbel_of(rng.word(kStreamBonusIn, (uint32_t)q,
                                                               (uint32_t)jrow, (uint32_t)v))
                        : -INFINITY;
    int idx = v;
    wave_argmax(score, idx);
    token = idx;
  }
  if (lane == 0) {
    y[(size_t)q * (gamma + 1) + n_acc[q]] = token;
    if (x_next) x_next[q] = token;  // the next cycle's anchor
  }
}

// ---------------------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------------------
template <class T, class BT>
static int verify_run(int R, int gamma, int V, int r, const void* target_, const void* U_,
                      const void* W2t_, const void* brows_, const int32_t* x, const float* lse,
                      const float* logit_x, const int32_t* ell, uint64_t seed, uint64_t cycle,
                      int32_t* n_acc, int32_t* y, float* c_star, int32_t* x_next,
                      int32_t* status, const VerifyWs& ws, hipStream_t stream) {
  const T* target = static_cast<const T*>(target_);
  const T* U = static_cast<const T*>(U_);
  const T* W2t = static_cast<const T*>(W2t_);
  const BT* brows = static_cast<const BT*>(brows_);
  constexpr bool BF = sizeof(T) == 2;
  constexpr bool SPLIT = BF && sizeof(BT) == 4;

  verify_prep_kernel<<<1, 1024, 0, stream>>>(R, gamma, ell, ws, status);
  {
    // a grid-stride walk over the items of list A (its length is known on the device only)
    const int wgs = (R * (gamma + 1) * lse_witems(V) + 3) / 4, cap = 4 * device_cus();
    verify_lse_kernel<T><<<wgs < cap ? wgs : cap, kLseThreads, 0, stream>>>(
        R, gamma, V, target, ell, ws, seed, cycle);
  }
  // bf16 bias rows go to the sweep in its packed order (float ones, split hi + lo, do not)
  const uint16_t* brows16 =
      (BF && !SPLIT) ? reinterpret_cast<const uint16_t*>(brows_) : nullptr;
  verify_decide_kernel<T><<<R, 64, 0, stream>>>(R, gamma, V, target, x, lse, logit_x, ell, ws,
                                                seed, cycle, n_acc, y, status, brows16, r);

  const int rows_max = R * gamma;
  int nranges;
  if (BF) {
    // one workgroup per vocabulary range; each walks the row groups of list B, whose
    // length is known on the device only
    SweepGeom g = make_geom(rows_max, V, r, reinterpret_cast<const uint16_t*>(W2t),
                            device_cus() < kMaxRanges ? device_cus() : kMaxRanges);
    nranges = g.nranges;
    VerifySweepParams p{};
    p.U = reinterpret_cast<const uint16_t*>(U);
    p.target = reinterpret_cast<const uint16_t*>(target);
    p.brows = brows;
    p.lse = lse;
    p.R = R;
    p.gamma = gamma;
    p.V = V;
    p.r = r;
    p.ws = ws;
    p.seed = seed;
    p.cycle = cycle;
    p.nranges = nranges;
    launch_sweep<SPLIT, VerifyEpi<SPLIT>>(g, p, stream);
  } else {
    const int nblocks = (V + kVB - 1) / kVB;
    nranges = nblocks < 64 ? nblocks : 64;
    dim3 grid(nranges, rows_max);
    verify_sweep_f32_kernel<<<grid, 64, 0, stream>>>(
        gamma, V, r, reinterpret_cast<const float*>(U), reinterpret_cast<const float*>(target),
        reinterpret_cast<const float*>(W2t), reinterpret_cast<const float*>(brows), lse, ws,
        seed, cycle, nranges, nblocks);
  }
  verify_final_kernel<T, BT><<<R, kFinalThreads, 0, stream>>>(R, gamma, V, r, target, U, W2t, brows, lse,
                                                    ell, ws, nranges, seed, cycle, n_acc, y, c_star,
                                                    x_next);
  return launch_status();
}

}  // namespace dspark

extern "C" {

size_t dspark_verify_workspace_bytes(int R, int gamma, int V, int r) {
  if (!dspark::dims_ok(R, gamma, V, r, 0)) return 0;
  return dspark::carve_verify(nullptr, R, gamma, V, r).bytes;
}

int dspark_verify(int R, int gamma, int V, int r, dspark_dtype dt, const void* target,
                  const void* U, const void* W2t, const void* bias_rows, dspark_dtype bias_dt,
                  const int32_t* x, const float* lse, const float* logit_x, const int32_t* ell,
                  uint64_t seed, uint64_t cycle, int32_t* n_acc, int32_t* y, float* c_star,
                  int32_t* x_next, int32_t* dev_status, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  using namespace dspark;
  if (!dims_ok(R, gamma, V, r, 0) || (dt != DSPARK_F32 && dt != DSPARK_BF16)) return DSPARK_EINVAL;
  if (bias_dt != DSPARK_F32 && bias_dt != dt) return DSPARK_EINVAL;
  if (cycle >= ((uint64_t)1 << 28)) return DSPARK_EINVAL;
  if (R == 0) return DSPARK_OK;
  if ((long)R * (gamma + 1) > (long)0x7fffffff / 2) return DSPARK_EINVAL;
  if (!target || !U || !W2t || !bias_rows || !x || !lse || !logit_x || !ell || !n_acc || !y ||
      !c_star || !ws)
    return DSPARK_EINVAL;
  if (!aligned16(target) || !aligned16(U) || !aligned16(W2t) || !aligned16(bias_rows))
    return DSPARK_EINVAL;
  // the bf16 sweep addresses U and target rows with 32-bit byte offsets
  if (dt == DSPARK_BF16 && (uint64_t)R * (gamma + 1) * V * 2 >= ((uint64_t)1 << 32))
    return DSPARK_EINVAL;
  if (ws_bytes < carve_verify(nullptr, R, gamma, V, r).bytes) return DSPARK_EWORKSPACE;
  if (!aligned16(ws)) return DSPARK_EINVAL;
  const VerifyWs lay = carve_verify(ws, R, gamma, V, r);
  if (dt == DSPARK_BF16) {
    if (bias_dt == DSPARK_BF16)
      return verify_run<uint16_t, uint16_t>(R, gamma, V, r, target, U, W2t, bias_rows, x, lse,
                                            logit_x, ell, seed, cycle, n_acc, y, c_star,
                                            x_next, dev_status, lay, stream);
    return verify_run<uint16_t, float>(R, gamma, V, r, target, U, W2t, bias_rows, x, lse,
                                       logit_x, ell, seed, cycle, n_acc, y, c_star, x_next,
                                       dev_status, lay, stream);
  }
  return verify_run<float, float>(R, gamma, V, r, target, U, W2t, bias_rows, x, lse, logit_x,
                                  ell, seed, cycle, n_acc, y, c_star, x_next, dev_status, lay,
                                  stream);
}

const char* dspark_version(void) { return "dspark-mi355x 0.1 (gfx950)"; }

}  // extern "C"
