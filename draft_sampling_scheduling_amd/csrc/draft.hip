// draft.hip -- the sequential block's draft loop (Markov head eq. (5), RNN head eq. (6)),
// the confidence head (eq. (7)) and the two-level Gumbel-max sampler.
//
// One draft position k costs two launches:
//   sweep   (matrix cores, see sweep.h): per request and per vocabulary range, the running
//           normaliser (max, sum exp) of l = U_k + bias_k and the best block score
//           LSE_b + g_b of the sampler's first level;
//   combine (one workgroup of four waves per request): merge the ranges, take the winning
//           block, recompute its 64 logits (the r-long dot products split over the waves),
//           draw x_k inside it (second level), and write lse, l(x_k), c_k and the bias row.
// The position-independent half of the confidence, w_h . h_k, is computed for all k by one
// launch up front; the RNN head adds one state-update launch per position and one
// h-projection launch up front.
#include "dev.h"
#include "draft_epi.h"
#include "host.h"
#include "sweep.h"

namespace dspark {

// ---------------------------------------------------------------------------------------
// w_h . h_k for every (request, position): one wave per row of h
// ---------------------------------------------------------------------------------------
// the sweep's packed B rows for step 1: row q's chunk j = W1[x0[q]][8j .. 8j+8)
__device__ __forceinline__ void bpack_gather_one(int gid, int R, int r, int V,
                                                 const int32_t* __restrict__ x0,
                                                 const uint16_t* __restrict__ W1, uint4* bpack,
                                                 int32_t* status) {
  const int cpr = r / 8;  // chunks per row
  if (gid >= R * cpr) return;
  const int q = gid / cpr, j = gid - q * cpr;
  const int32_t t = checked_token(x0[q], V, status);
  bpack[bpack_index(q, j, r / 16)] = reinterpret_cast<const uint4*>(W1 + (size_t)t * r)[j];
}

__global__ void __launch_bounds__(256) bpack_gather_kernel(int R, int r, int V,
                                                           const int32_t* __restrict__ x0,
                                                           const uint16_t* __restrict__ W1,
                                                           uint4* bpack, int32_t* status) {
  bpack_gather_one(blockIdx.x * 256 + threadIdx.x, R, r, V, x0, W1, bpack, status);
}

template <class T>
__global__ void __launch_bounds__(256) conf_h_kernel(int rows, int d, const T* __restrict__ h,
                                                     const float* __restrict__ w,
                                                     float* __restrict__ zh, int R, int r,
                                                     int V, const int32_t* __restrict__ x0,
                                                     const uint16_t* __restrict__ W1,
                                                     uint4* bpack, int32_t* status) {
  // the step-1 packed B rows ride along (bf16 Markov head only)
  if (bpack) bpack_gather_one(blockIdx.x * 256 + threadIdx.x, R, r, V, x0, W1, bpack, status);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* hr = h + (size_t)row * d;
  float acc = 0.0f;
  // eight 8-element chunks per lane in flight together (a whole row of d = 4096 in one
  // round trip; clamped addresses, masked sums)
  constexpr int kDepth = 8;
  for (int i0 = lane * 8; i0 < d; i0 += kDepth * 64 * 8) {
    float x[kDepth][8], wv[kDepth][8];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int i = i0 + u * 64 * 8 < d ? i0 + u * 64 * 8 : i0;
      ld8<T>(hr + i, x[u]);
      ld8<float>(w + i, wv[u]);
    }
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
      if (i0 + u * 64 * 8 < d)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(wv[u][j], x[u][j], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) zh[row] = acc;
}

// ---------------------------------------------------------------------------------------
// the same step for float operands: plain VALU, one wave per (request, range); lane = id
// inside a 64-id block.  Used by the float workload only.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) draft_sweep_f32_kernel(
    int R, int V, int r, const float* __restrict__ U, size_t ustride, const int32_t* prev,
    int prev_stride, const float* __restrict__ W1, const float* __restrict__ orow,
    const float* __restrict__ W2t, uint32_t k, uint64_t seed, uint64_t cycle, float4* partials,
    int nranges, int nblocks, int32_t* status) {
  const int q = blockIdx.y, range = blockIdx.x, lane = threadIdx.x;
  const int per = (nblocks + nranges - 1) / nranges;
  const int b0 = range * per, b1 = min(nblocks, b0 + per);
  const float* e;
  if (orow) {
    e = orow + (size_t)q * r;
  } else {
    const int32_t t = checked_token(prev[(size_t)q * prev_stride], V, status);
    e = W1 + (size_t)t * r;
  }
  const Rng rng(seed, cycle);
  float M = -INFINITY, S = 0.0f, G = -INFINITY;
  int Bk = 0x7fffffff;
  for (int b = b0; b < b1; ++b) {
    const int v = b * kVB + lane;
    float l = -INFINITY;
    if (v < V) {
      float acc = 0.0f;
      for (int i = 0; i < r; ++i) acc = fmaf(e[i], W2t[(size_t)v * r + i], acc);
      l = U[(size_t)q * ustride + v] + acc;
    }
    const float m = wave_max(l);
    const float sum = wave_sum(l == -INFINITY ? 0.0f : __expf(l - m));
    lse_merge(M, S, m, sum);
    const float g = gumbel_of(rng.word(kStreamDraftBlk, (uint32_t)q, k, (uint32_t)b));
    const float Gb = m + __logf(sum) + g;
    if (Gb > G) {
      G = Gb;
      Bk = b;
    }
  }
  if (lane == 0) partials[(size_t)q * nranges + range] = make_float4(M, S, G, __int_as_float(Bk));
}

// ---------------------------------------------------------------------------------------
// combine: one workgroup per request
// ---------------------------------------------------------------------------------------
constexpr int kCombineThreads = 256;
constexpr int kCombineWaves = kCombineThreads / kWave;

struct CombineLds {
  float4 red[kCombineWaves];
  float dotp[kCombineWaves][kWave];
  float zred[kCombineWaves];
};

// The combine of request q at position k, for a workgroup of kCombineThreads threads.  It
// first does the work that depends on x_{k-1} only (the embedding part of the confidence,
// and the bias row verification reuses), while the first range partial is in flight; then
// it merges the vocabulary ranges' partials (normaliser and winning block), recomputes the
// winning block's 64 logits, draws x_k inside it (second level of the sampler), and writes
// x, c, z, lse, logit_x (and W1[x_k] in the next sweep's packed order when bpack is set).
// BIAS = false: the logits are U_k (the parallel block's own sampling).
template <class T, bool RNN, bool BIAS>
__device__ void combine_request(CombineLds& sm, int q, int R, int gamma, int V, int r, int d,
                               const T* __restrict__ U, const T* __restrict__ W1,
                               const T* __restrict__ W2t, const float* __restrict__ w,
                               const float* __restrict__ temps, const float* zh,
                               int32_t tprev, const float* __restrict__ orow,
                               const float4* partials, int nranges, uint32_t k, uint64_t seed,
                               uint64_t cycle, int32_t* x, float* c, float* zout, float* lse,
                               float* logit_x, void* bias_rows, uint4* bpack, int32_t* status) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t rk = (size_t)q * gamma + (k - 1);
  const T* e = W1 + (size_t)tprev * r;
  // this thread's first range partial is loaded before anything else, so it is in flight
  // with the x_{k-1} work
  const float4* prow = partials + (size_t)q * nranges;
  const float4 pr0 = tid < nranges ? prow[tid]
                                   : make_float4(0.0f, 0.0f, 0.0f, __int_as_float(0x7fffffff));
  // confidence head, embedding part: w_e . W1[x_{k-1}], and the bias row this step used (for
  // verification): both depend on x_{k-1} only
  {
    float ze = 0.0f;
    for (int i = tid; i < r; i += kCombineThreads) ze = fmaf(w[d + i], ld<T>(e, i), ze);
    ze = wave_sum(ze);
    if (lane == 0) sm.zred[wave] = ze;
    if (RNN) {
      float* br = static_cast<float*>(bias_rows) + rk * r;
      for (int i = tid; i < r; i += kCombineThreads) br[i] = orow[(size_t)q * r + i];
    } else {
      T* br = static_cast<T*>(bias_rows) + rk * r;
      for (int i = tid; i < r; i += kCombineThreads) br[i] = e[i];
    }
  }

  // the range partials: per wave the largest reference, one rescale per lane and a plain
  // sum
  float M = -INFINITY, S = 0.0f, G = -INFINITY;
  int Bk = 0x7fffffff;
  for (int i = tid; i < nranges; i += kCombineThreads) {
    const float4 pr = i == tid ? pr0 : prow[i];
    const int pb = __float_as_int(pr.w);
    if (pb == 0x7fffffff) continue;
    lse_merge(M, S, pr.x, pr.y);
    if (pr.z > G || (pr.z == G && pb < Bk)) {
      G = pr.z;
      Bk = pb;
    }
  }
  {
    const float Mw = wave_max(M);
    S = (M == -INFINITY) ? 0.0f : S * __expf(M - Mw);
    S = wave_sum(S);
    M = Mw;
  }
  wave_argmax(G, Bk);
  if (lane == 0) sm.red[wave] = make_float4(M, S, G, __int_as_float(Bk));
  __syncthreads();
  {
    const float4 r0 = sm.red[0];
    M = r0.x; S = r0.y; G = r0.z; Bk = __float_as_int(r0.w);
#pragma unroll
    for (int i = 1; i < kCombineWaves; ++i) {
      const float4 ri = sm.red[i];
      lse_merge(M, S, ri.x, ri.y);
      const int bi = __float_as_int(ri.w);
      if (ri.z > G || (ri.z == G && bi < Bk)) {
        G = ri.z;
        Bk = bi;
      }
    }
  }
  const int nblocks = (V + kVB - 1) / kVB;
  if (Bk < 0 || Bk >= nblocks) Bk = 0;  // only if every partial was empty (cannot happen)

  // second level: the winning block's 64 logits, the k sum split over the waves in
  // 8-element chunks
  const int v = Bk * kVB + lane;
  const int vc = v < V ? v : V - 1;  // lanes past V load row V-1 and are masked below
  // zh[rk] is independent of the block: in flight with the rest
  const float zh_k = wave == 0 ? zh[rk] : 0.0f;
  float part = 0.0f;
  float gn = 0.0f;  // in-block Gumbel noise (wave 0), formed while the block's rows load
  T ur = T();       // wave 0: U_k at this lane's id, kept raw until after the barrier so
                    // that the wait for it does not hold back the row loads issued before it
  if (BIAS) {
    const T* wr = W2t + (size_t)vc * r;
    // r <= 256: at most 8 chunks per wave, all loads in flight together
    float a[8][8], bv[8][8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int ch = wave + kCombineWaves * it < r / 8 ? wave + kCombineWaves * it : 0;
      ld8<T>(wr + ch * 8, a[it]);
      if (RNN) {
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[it][j] = orow[(size_t)q * r + ch * 8 + j];
      } else {
        ld8<T>(e + ch * 8, bv[it]);
      }
    }
    if (wave == 0) {
      ur = U[rk * V + vc];
      gn = gumbel_of(Rng(seed, cycle).word(kStreamDraftIn, (uint32_t)q, k, (uint32_t)v));
    }
#pragma unroll
    for (int it = 0; it < 8; ++it)
      if (wave + kCombineWaves * it < r / 8)
#pragma unroll
        for (int j = 0; j < 8; ++j) part = fmaf(bv[it][j], a[it][j], part);
  } else if (wave == 0) {
    ur = U[rk * V + vc];
    gn = gumbel_of(Rng(seed, cycle).word(kStreamDraftIn, (uint32_t)q, k, (uint32_t)v));
  }
  sm.dotp[wave][lane] = part;
  __syncthreads();
  if (wave == 0) {
    const float u = ld<T>(&ur, 0);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) acc += sm.dotp[i][lane];
    const float l = (v < V) ? u + acc : -INFINITY;
    float score = (v < V) ? l + gn : -INFINITY;
    int idx = v;
    wave_argmax(score, idx);  // every lane of the wave holds the pick
    // W1[x_k] in the next sweep's packed order, one 16-byte chunk per lane: loaded here,
    // stored after the outputs
    // (the row index is clamped: only NaN logits can make a lane past V win, and the token
    // itself then raises the fault bit when the next position reads it)
    const bool pack = sizeof(T) == 2 && !RNN && bpack && lane < r / 8;
    const int gidx = idx < V ? idx : V - 1;
    const uint4 prow_next = pack ? reinterpret_cast<const uint4*>(W1 + (size_t)gidx * r)[lane]
                                 : make_uint4(0, 0, 0, 0);
    const float lx = __shfl(l, idx - Bk * kVB, kWave);
    float z = zh_k;
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) z += sm.zred[i];
    if (lane == 0) {
      // the position's STS temperature (Module D); a non-positive one is a data fault
      float Tk = temps ? temps[k - 1] : 1.0f;
      if (!(Tk > 0.0f)) {
        raise_fault(status, DSPARK_FAULT_CONF);
        Tk = 1.0f;
      }
      x[rk] = idx;
      c[rk] = 1.0f / (1.0f + __expf(-z / Tk));
      if (zout) zout[rk] = z;
      lse[rk] = M + __logf(S);
      logit_x[rk] = lx;
    }
    if (pack) bpack[bpack_index(q, lane, r / 16)] = prow_next;
  }
}

template <class T, bool RNN, bool BIAS = true>
__global__ void __launch_bounds__(kCombineThreads) draft_combine_kernel(
    int R, int gamma, int V, int r, int d, const T* __restrict__ U, const T* __restrict__ W1,
    const T* __restrict__ W2t, const float* __restrict__ w, const float* __restrict__ temps,
    const float* __restrict__ zh, const int32_t* prev, int prev_stride,
    const float* __restrict__ orow, const float4* __restrict__ partials, int nranges,
    uint32_t k, uint64_t seed, uint64_t cycle, int32_t* x, float* c, float* zout, float* lse,
    float* logit_x, void* bias_rows, uint4* bpack, int32_t* status) {
  __shared__ CombineLds sm;
  const int q = blockIdx.x;
  const int32_t tprev = checked_token(prev[(size_t)q * prev_stride], V, status);
  combine_request<T, RNN, BIAS>(sm, q, R, gamma, V, r, d, U, W1, W2t, w, temps, zh, tprev,
                                orow, partials, nranges, k, seed, cycle, x, c, zout, lse,
                                logit_x, bias_rows, bpack, status);
}

// ---------------------------------------------------------------------------------------
// RNN head (eq. (6)).  Gh[q][k][o] = sum_i W_gco[o][2r + i] h_k[i] for all k up front;
// per step: G = W_gco[:, :2r] [s; e] + Gh, gate/candidate/output nonlinearities, s update.
// ---------------------------------------------------------------------------------------
// Gh = h W_h^T: [rows][d] x [3r][d]^T -> [rows][3r] fp32, on the matrix cores.
// A workgroup computes a 128-row x 96-output tile over one half of the inputs (split-K: the
// halves go to two partial buffers, added by the step kernel, so the sum has a fixed order
// and needs no atomics).  Its four waves own 32 rows each and all three 32-output blocks.
// The inputs advance in chunks of 64 through a two-stage LDS ring, copied straight from
// global memory with global_load_lds_dwordx4: one copy moves 8 whole 128-byte row segments
// (8 lanes per row), and row rho of the stage keeps its 16-byte piece c in slot
// c ^ ((rho / 2) % 8).  A ds_read_b128 is served 16 lanes at a time over 64 four-byte
// banks, and a 128-byte row spans half of them (even rows one half, odd rows the other),
// so the fragment reads of 16 consecutive lanes (lane l: row l % 32, piece 2 ks + l / 32)
// land on 8 different slots in each half: conflict-free.  Wave w copies
// rows 8w .. 8w + 8 of every 32-row block of h and W_h.  Rows and outputs past the end are
// clamped to the last one (their results are not stored); inputs past d occur only in the
// last chunk, are read clamped and zeroed in registers.  Tiles that share rows are placed
// on one XCD (workgroup b runs on XCD b % 8), so h comes from HBM about once.
constexpr int kHpRows = 128, kHpOut = 96, kHpKC = 64, kHpKS = kHpKC / 16;
constexpr int kHpStageBytes = (kHpRows + kHpOut) * kHpKC * 2;  // 28 KB
constexpr int kHpSplit = 2;

template <bool MASK>
__device__ __forceinline__ void hproj_chunk(const uint8_t* buf, int wave, int lane, int kc,
                                            int d, f32x16 (&acc)[3]) {
  const int rl = lane & 31, sw = (rl >> 1) & 7;
#pragma unroll
  for (int ks = 0; ks < kHpKS; ++ks) {
    const int slot = 16 * ((2 * ks + (lane >> 5)) ^ sw);
    uint4 bf = *reinterpret_cast<const uint4*>(buf + (32 * wave + rl) * 128 + slot);
    uint4 af[3];
#pragma unroll
    for (int ob = 0; ob < 3; ++ob)
      af[ob] = *reinterpret_cast<const uint4*>(buf + (kHpRows + 32 * ob + rl) * 128 + slot);
    if (MASK && kc + 16 * ks + 8 * (lane >> 5) >= d) {
      bf = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int ob = 0; ob < 3; ++ob) af[ob] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int ob = 0; ob < 3; ++ob)
      acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[ob]), as_bf16x8(bf),
                                                          acc[ob], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(256, 2) rnn_hproj_bf16_kernel(
    int rows, int d, int r3, int ldw, int nN, int per_xcd, const uint16_t* __restrict__ h,
    const uint16_t* __restrict__ Wh, float* __restrict__ Gh) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kHpStageBytes];
  const int nM = (rows + kHpRows - 1) / kHpRows;
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= nM * nN * kHpSplit) return;
  const int split = t % kHpSplit, tn = (t / kHpSplit) % nN, tm = t / (kHpSplit * nN);
  const int row0 = tm * kHpRows, o0 = tn * kHpOut;
  const int nchunks = (d + kHpKC - 1) / kHpKC, cper = (nchunks + kHpSplit - 1) / kHpSplit;
  const int c0 = split * cper;
  const int c1 = c0 + cper < nchunks ? c0 + cper : nchunks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, ln = lane & 31, hh = lane >> 5;

  // copy lane: row 8 wave + lane / 8 of each 32-row block, piece (lane % 8) ^ (lane / 8)
  const int crow = 8 * wave + (lane >> 3), cpiece = (lane & 7) ^ ((crow >> 1) & 7);
  uint32_t hoff[4], woff[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 32 * i + crow < rows ? row0 + 32 * i + crow : rows - 1;
    hoff[i] = (uint32_t)row * (uint32_t)d * 2u;
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int o = o0 + 32 * i + crow < r3 ? o0 + 32 * i + crow : r3 - 1;
    woff[i] = (uint32_t)o * (uint32_t)ldw * 2u;
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int c, int sb) {
    int k = c * kHpKC + 8 * cpiece;
    if (k > d - 8) k = d - 8;
    const uint32_t kb = (uint32_t)k * 2u;
    const uint32_t base = lds0 + sb * kHpStageBytes + (8 * wave) * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16s(h, hoff[i] + kb, base + (32 * i) * 128);
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16s(Wh, woff[i] + kb, base + (kHpRows + 32 * i) * 128);
  };

  f32x16 acc[3];
#pragma unroll
  for (int ob = 0; ob < 3; ++ob)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[ob][j] = 0.0f;

  if (c0 < c1) issue(c0, 0);
  for (int c = c0; c < c1; ++c) {
    const int sb = (c - c0) & 1;
    vm_wait<0>();     // this wave's copies of chunk c have landed
    stage_barrier();  // everyone's have; everyone is done reading chunk c - 1
    if (c + 1 < c1) issue(c + 1, sb ^ 1);
    const uint8_t* buf = lds + sb * kHpStageBytes;
    if ((c + 1) * kHpKC > d)
      hproj_chunk<true>(buf, wave, lane, c * kHpKC, d, acc);
    else
      hproj_chunk<false>(buf, wave, lane, c * kHpKC, d, acc);
  }

  // accumulator: output o0 + 32 ob + 8 (j / 4) + 4 hh + j % 4, row row0 + 32 wave + ln
  const int row = row0 + 32 * wave + ln;
  if (row < rows) {
    float* dst = Gh + (size_t)split * rows * r3 + (size_t)row * r3;
#pragma unroll
    for (int ob = 0; ob < 3; ++ob)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int o = o0 + 32 * ob + 8 * jj + 4 * hh;  // r3 % 4 == 0: a group is in or out
        if (o < r3)
          *reinterpret_cast<float4*>(dst + o) =
              make_float4(acc[ob][4 * jj], acc[ob][4 * jj + 1], acc[ob][4 * jj + 2],
                          acc[ob][4 * jj + 3]);
      }
  }
}

template <class T>
__global__ void __launch_bounds__(64) rnn_hproj_f32_kernel(int rows, int d, int r3, int ldw,
                                                           const T* __restrict__ h,
                                                           const T* __restrict__ Wh,
                                                           float* __restrict__ Gh) {
  const int row = blockIdx.y, o = blockIdx.x * 64 + threadIdx.x;
  if (row >= rows || o >= r3) return;
  float acc = 0.0f;
  for (int i = 0; i < d; ++i) acc = fmaf(ld<T>(Wh, (size_t)o * ldw + i), ld<T>(h, (size_t)row * d + i), acc);
  Gh[(size_t)row * r3 + o] = acc;
}

// one workgroup per request: z_se = [s_{k-1}; W1[x_{k-1}]] in LDS, 3r dot products of
// length 2r, then the nonlinearities.  Writes o_k (float) and s_k in place.
template <class T>
__global__ void __launch_bounds__(256) rnn_step_kernel(int R, int gamma, int V, int r, int d,
                                                       const T* __restrict__ W1,
                                                       const T* __restrict__ Wg,
                                                       const float* __restrict__ Gh,
                                                       const int32_t* prev, int prev_stride,
                                                       uint32_t k, float* s, float* orow,
                                                       int32_t* status) {
  extern __shared__ float zs[];  // [2r] then G [3r]
  const int q = blockIdx.x;
  float* G = zs + 2 * r;
  const int32_t t = checked_token(prev[(size_t)q * prev_stride], V, status);
  for (int i = threadIdx.x; i < r; i += blockDim.x) {
    zs[i] = s[(size_t)q * r + i];
    zs[r + i] = ld<T>(W1, (size_t)t * r + i);
  }
  __syncthreads();
  const int K = 2 * r + d;
  const float* gh = Gh + ((size_t)q * gamma + (k - 1)) * 3 * r;
  for (int o = threadIdx.x; o < 3 * r; o += blockDim.x) {
    float acc = gh[o];
    const T* wr = Wg + (size_t)o * K;
    for (int i = 0; i < 2 * r; i += 8) {
      float a[8];
      ld8<T>(wr + i, a);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf(a[j], zs[i + j], acc);
    }
    G[o] = acc;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < r; i += blockDim.x) {
    const float g = 1.0f / (1.0f + expf(-G[i]));
    const float cand = tanhf(G[r + i]);
    const float out = tanhf(G[2 * r + i]);
    orow[(size_t)q * r + i] = out;
    s[(size_t)q * r + i] = g * zs[i] + (1.0f - g) * cand;
  }
}

// The [s; e] columns of W_gco regrouped for the batched step: chunk (k8, o) holds
// W_gco[o][8 k8 .. 8 k8 + 8), so a workgroup's threads (consecutive outputs) read one
// contiguous 16-byte chunk each per 8 inputs.
__global__ void __launch_bounds__(256) rnn_wpack_kernel(int r, int ldw,
                                                        const uint16_t* __restrict__ Wg,
                                                        uint4* __restrict__ Wp) {
  const int r3 = 3 * r, nk8 = 2 * r / 8;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= r3 * nk8) return;
  const int k8 = gid / r3, o = gid - k8 * r3;
  Wp[gid] = *reinterpret_cast<const uint4*>(Wg + (size_t)o * ldw + 8 * k8);
}

constexpr int kRnnReq = 4;     // requests per workgroup of the batched step
constexpr int kRnnUnits = 64;  // units per workgroup (r >= 64), else r
constexpr int kRnnKSplit = 4;  // input quarters, one thread group each

// The RNN step for kRnnReq requests and a slice of U units.  Threads form kRnnKSplit
// groups of 3U; thread t of group p computes output o = (t / U) * r + u0 + t % U (gate,
// candidate or output row of unit u0 + t % U) over the p-th quarter of the 2r inputs, for
// all the workgroup's requests, so each weight chunk is read once for all of them.  The
// quarters are added in order, then one thread per (request, unit) applies the
// nonlinearities.  s is double-buffered across steps (s_in -> s_out), since other
// workgroups still read s_{k-1} of these requests.
__global__ void __launch_bounds__(kRnnKSplit * 3 * kRnnUnits) rnn_step_batched_kernel(
    int R, int gamma, int V, int r, const uint16_t* __restrict__ W1,
    const uint4* __restrict__ Wp, const float* __restrict__ Gh, const int32_t* prev,
    int prev_stride, uint32_t k, const float* __restrict__ s_in, float* __restrict__ s_out,
    float* __restrict__ orow, int32_t* status) {
  // z [kRnnReq][2r], then partial G [kRnnKSplit][kRnnReq][3U]
  extern __shared__ float sh[];
  const int U = r < kRnnUnits ? r : kRnnUnits;
  const int q0 = blockIdx.x * kRnnReq, u0 = blockIdx.y * U;
  const int nq = R - q0 < kRnnReq ? R - q0 : kRnnReq;
  float* z = sh;
  float* G = sh + kRnnReq * 2 * r;
  const int t = threadIdx.x;
  __shared__ int toks[kRnnReq];
  if (t < kRnnReq)
    toks[t] = t < nq ? checked_token(prev[(size_t)(q0 + t) * prev_stride], V, status) : 0;
  __syncthreads();
  // z_se = [s_{k-1}; W1[x_{k-1}]] of the workgroup's requests, four values per item
  for (int i = t; i < kRnnReq * r / 4; i += blockDim.x) {
    const int qq = (4 * i) / r, c = 4 * i - qq * r;
    const bool live = qq < nq;
    const int q = live ? q0 + qq : q0;
    const float4 sv = *reinterpret_cast<const float4*>(s_in + (size_t)q * r + c);
    const uint2 ev = *reinterpret_cast<const uint2*>(W1 + (size_t)toks[qq] * r + c);
    float* zs = z + qq * 2 * r + c;
    zs[0] = live ? sv.x : 0.0f;
    zs[1] = live ? sv.y : 0.0f;
    zs[2] = live ? sv.z : 0.0f;
    zs[3] = live ? sv.w : 0.0f;
    zs[r + 0] = live ? bf16lo(ev.x) : 0.0f;
    zs[r + 1] = live ? bf16hi(ev.x) : 0.0f;
    zs[r + 2] = live ? bf16lo(ev.y) : 0.0f;
    zs[r + 3] = live ? bf16hi(ev.y) : 0.0f;
  }
  __syncthreads();
  const int part = t / (3 * U), tt = t - part * 3 * U;
  const int g = tt / U, u = u0 + tt - g * U, o = g * r + u;
  const int r3 = 3 * r, nk8 = 2 * r / 8, per = nk8 / kRnnKSplit;  // per >= 1 (r >= 16)
  float acc[kRnnReq];
#pragma unroll
  for (int qq = 0; qq < kRnnReq; ++qq) acc[qq] = 0.0f;
  for (int kb = part * per; kb < (part + 1) * per; kb += 2) {
    // two weight chunks in flight per pass (per is even for r >= 32; r = 16 takes one)
    uint4 wv[2];
#pragma unroll
    for (int v2 = 0; v2 < 2; ++v2) {
      const int kk = kb + v2 < (part + 1) * per ? kb + v2 : kb;
      wv[v2] = Wp[(size_t)kk * r3 + o];
    }
#pragma unroll
    for (int v2 = 0; v2 < 2; ++v2) {
      if (kb + v2 >= (part + 1) * per) break;
      float a[8];
      a[0] = bf16lo(wv[v2].x); a[1] = bf16hi(wv[v2].x); a[2] = bf16lo(wv[v2].y); a[3] = bf16hi(wv[v2].y);
      a[4] = bf16lo(wv[v2].z); a[5] = bf16hi(wv[v2].z); a[6] = bf16lo(wv[v2].w); a[7] = bf16hi(wv[v2].w);
#pragma unroll
      for (int qq = 0; qq < kRnnReq; ++qq) {
        const float* zq = z + qq * 2 * r + 8 * (kb + v2);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[qq] = fmaf(a[j], zq[j], acc[qq]);
      }
    }
  }
#pragma unroll
  for (int qq = 0; qq < kRnnReq; ++qq) G[(part * kRnnReq + qq) * 3 * U + tt] = acc[qq];
  __syncthreads();
  for (int i = t; i < nq * U; i += blockDim.x) {
    const int qq = i / U, uu = i - qq * U, q = q0 + qq, unit = u0 + uu;
    const float* gh = Gh + ((size_t)q * gamma + (k - 1)) * 3 * r;
    const float* gh1 = gh + (size_t)R * gamma * 3 * r;  // the second K half
    float gv[3];
#pragma unroll
    for (int gi = 0; gi < 3; ++gi) {
      float a = gh[gi * r + unit] + gh1[gi * r + unit];
#pragma unroll
      for (int pp = 0; pp < kRnnKSplit; ++pp) a += G[(pp * kRnnReq + qq) * 3 * U + gi * U + uu];
      gv[gi] = a;
    }
    const float gt = 1.0f / (1.0f + expf(-gv[0]));
    const float cand = tanhf(gv[1]);
    const float out = tanhf(gv[2]);
    orow[(size_t)q * r + unit] = out;
    s_out[(size_t)q * r + unit] = gt * z[qq * 2 * r + unit] + (1.0f - gt) * cand;
  }
}

// The RNN step on the matrix cores (r >= 32).  Workgroup (request block, unit block) forms
// G = W_gco[:, :2r] [s_{k-1}; e] for 32 requests x 32 units of each of the gate, candidate
// and output rows: three 32x32 accumulators (units on M, requests on N) that share the B
// operand.  The four waves take quarters of the 2r inputs (two of s, two of e), each
// issuing all of its loads before its matrix chain: A is the packed [s; e] weight chunk of
// 32 consecutive rows (one coalesced load per half-wave), B is s_{k-1} entered as hi + lo
// bf16 terms (two MFMAs) or the bf16 row W1[x_{k-1}] (one).  The accumulators meet
// in LDS; wave w then finishes accumulator registers 4w .. 4w + 4 (four consecutive units
// of every request): the four quarters in order, the two h-projection halves, the
// nonlinearities and the state update.  s is double-buffered across steps (s_in -> s_out).
constexpr int kStepWaves = 4;
__global__ void __launch_bounds__(kStepWaves * kWave) rnn_step_mfma_kernel(
    int R, int gamma, int V, int r, const uint16_t* __restrict__ W1,
    const uint4* __restrict__ Wp, const float* __restrict__ Gh, const int32_t* prev,
    int prev_stride, uint32_t k, const float* __restrict__ s_in, float* __restrict__ s_out,
    float* __restrict__ orow, int32_t* status) {
  __shared__ float part[kStepWaves][3][16][kWave];
  const int q0 = blockIdx.x * 32, u0 = blockIdx.y * 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5;
  const int qn = q0 + n < R ? q0 + n : R - 1;  // this lane's request (clamped for loads)
  const int r3 = 3 * r, cps = r / 8, per = r / 32;
  // the finishing step's operands first (they depend on nothing computed here): the two
  // h-projection halves and s_{k-1} of this lane's four units (accumulator registers
  // 4 wave .. 4 wave + 4: units u0 + 8 wave + 4 h .. + 4 of request q0 + n)
  const int ub = u0 + 8 * wave + 4 * h;
  const float* gh0 = Gh + ((size_t)qn * gamma + (k - 1)) * r3;
  const float* gh1 = gh0 + (size_t)R * gamma * r3;  // the second K half
  float4 gp[3][2];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    gp[g][0] = *reinterpret_cast<const float4*>(gh0 + g * r + ub);
    gp[g][1] = *reinterpret_cast<const float4*>(gh1 + g * r + ub);
  }
  const float4 sp = *reinterpret_cast<const float4*>(s_in + (size_t)qn * r + ub);

  // k-steps (16 inputs) over [s; e]: r / 16 in each part; r >= 32 makes their count a
  // multiple of 4, so waves 0 and 1 take s and waves 2 and 3 take e, per = r / 32 each;
  // every load of the wave goes out first (clamped k-steps past `per`), then its chain
  constexpr int kMaxPer = 8;  // r <= 256
  const int ks0 = (wave & 1) * per;  // k-step inside the wave's part
  f32x16 acc[3];
#pragma unroll
  for (int g = 0; g < 3; ++g)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[g][j] = 0.0f;
  uint4 a[kMaxPer][3];
  const int kbase = wave < 2 ? 0 : cps;  // chunk offset of the wave's part in [s; e]
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c8 = 2 * (ks0 + (i < per ? i : 0)) + h;  // chunk inside the part
#pragma unroll
    for (int g = 0; g < 3; ++g) a[i][g] = Wp[(size_t)(kbase + c8) * r3 + g * r + u0 + n];
  }
  if (wave < 2) {  // s_{k-1} as hi + lo bf16 terms
    float4 xs[kMaxPer][2];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int c8 = 2 * (ks0 + (i < per ? i : 0)) + h;
      xs[i][0] = *reinterpret_cast<const float4*>(s_in + (size_t)qn * r + 8 * c8);
      xs[i][1] = *reinterpret_cast<const float4*>(s_in + (size_t)qn * r + 8 * c8 + 4);
    }
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (i < per) {
        const float x[8] = {xs[i][0].x, xs[i][0].y, xs[i][0].z, xs[i][0].w,
                            xs[i][1].x, xs[i][1].y, xs[i][1].z, xs[i][1].w};
        uint4 hi, lo;
        split8(x, hi, lo);
#pragma unroll
        for (int g = 0; g < 3; ++g) {
          acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i][g]), as_bf16x8(hi), acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i][g]), as_bf16x8(lo), acc[g], 0, 0, 0);
        }
      }
    }
  } else {  // the bf16 row W1[x_{k-1}]
    const int32_t tk = checked_token(prev[(size_t)qn * prev_stride], V, status);
    const uint16_t* erow = W1 + (size_t)tk * r;
    uint4 ev[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int c8 = 2 * (ks0 + (i < per ? i : 0)) + h;
      ev[i] = *reinterpret_cast<const uint4*>(erow + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (i < per) {
#pragma unroll
        for (int g = 0; g < 3; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i][g]), as_bf16x8(ev[i]), acc[g], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 3; ++g)
#pragma unroll
    for (int j = 0; j < 16; ++j) part[wave][g][j][lane] = acc[g][j];
  __syncthreads();
  const int q = q0 + n;
  if (q >= R) return;
  float G[3][4];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    const float b[4] = {gp[g][0].x + gp[g][1].x, gp[g][0].y + gp[g][1].y,
                        gp[g][0].z + gp[g][1].z, gp[g][0].w + gp[g][1].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float v = b[t];
#pragma unroll
      for (int w = 0; w < kStepWaves; ++w) v += part[w][g][4 * wave + t][lane];
      G[g][t] = v;
    }
  }
  const float sv[4] = {sp.x, sp.y, sp.z, sp.w};
  float so[4], oo[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float gt = 1.0f / (1.0f + expf(-G[0][t]));
    so[t] = gt * sv[t] + (1.0f - gt) * tanhf(G[1][t]);
    oo[t] = tanhf(G[2][t]);
  }
  *reinterpret_cast<float4*>(s_out + (size_t)q * r + ub) = make_float4(so[0], so[1], so[2], so[3]);
  *reinterpret_cast<float4*>(orow + (size_t)q * r + ub) = make_float4(oo[0], oo[1], oo[2], oo[3]);
}

// ---------------------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------------------
static int nranges_for(int V, int ngroups) {
  const int nblocks = (V + kVB - 1) / kVB;
  int nr = device_cus() / (ngroups > 0 ? ngroups : 1);
  if (nr < 1) nr = 1;
  if (nr > nblocks) nr = nblocks;
  if (nr > kMaxRanges) nr = kMaxRanges;
  return nr;
}

struct DraftWs {
  float* zh;
  float4* partials;
  uint4* bpack;  // Markov: the next sweep's B rows in packed order
  float* Gh;
  float* s;
  float* s2;     // RNN state, the other buffer of the step's ping-pong
  float* orow;
  uint4* wpack;  // RNN [s; e] weights regrouped for the batched step
  size_t bytes;
};

static DraftWs carve_draft(void* ws, int R, int gamma, int V, int r, int d, bool rnn) {
  Carve cv(ws);
  DraftWs w{};
  w.zh = cv.take<float>((size_t)R * gamma);
  const int nblocks = (V + kVB - 1) / kVB;
  w.partials = cv.take<float4>((size_t)R * (nblocks < kMaxRanges ? nblocks : kMaxRanges));
  if (rnn) {
    w.Gh = cv.take<float>((size_t)kHpSplit * R * gamma * 3 * r);  // bf16: two K halves
    w.s = cv.take<float>((size_t)R * r);
    w.s2 = cv.take<float>((size_t)R * r);
    w.orow = cv.take<float>((size_t)R * r);
    w.wpack = cv.take<uint4>((size_t)(2 * r / 8) * 3 * r);
  } else {
    w.bpack = cv.take<uint4>((size_t)bpack_rows(R) * r / 8);
  }
  (void)d;
  w.bytes = cv.bytes();
  return w;
}

// Enqueues the whole draft call on `stream`: the confidence pre-projection (and the RNN
// head's set-up), then per position [state update], sweep, combine.  evb/eve (nullable
// arrays of gamma events) time each position's sweep; returns the launch status.
template <class T>
static int draft_run(bool rnn, bool bias, int R, int gamma, int V, int r, int d, const void* U_,
                     const void* h_, const void* W1_, const void* W2t_, const void* Wg_,
                     const float* w, const float* temps, const int32_t* x0, uint64_t seed,
                     uint64_t cycle, int32_t* x, float* c, float* z, float* lse, float* logit_x,
                     void* bias_rows, int32_t* status, const DraftWs& ws, hipStream_t stream,
                     hipEvent_t* evb, hipEvent_t* eve) {
  const T* U = static_cast<const T*>(U_);
  const T* h = static_cast<const T*>(h_);
  const T* W1 = static_cast<const T*>(W1_);
  const T* W2t = static_cast<const T*>(W2t_);
  const T* Wg = static_cast<const T*>(Wg_);
  constexpr bool BF = sizeof(T) == 2;
  const int rows = R * gamma;

  uint4* bpack = (BF && !rnn) ? ws.bpack : nullptr;
  const uint16_t* W1b = reinterpret_cast<const uint16_t*>(W1_);
  if (d > 0) {
    conf_h_kernel<T><<<(rows + 3) / 4, 256, 0, stream>>>(rows, d, h, w, ws.zh, R, r, V, x0, W1b,
                                                         bpack, status);
  } else {
    fill_kernel<<<(rows + 255) / 256, 256, 0, stream>>>(ws.zh, (size_t)rows, 0.0f);
    if (bpack)
      bpack_gather_kernel<<<(R * (r / 8) + 255) / 256, 256, 0, stream>>>(R, r, V, x0, W1b,
                                                                          bpack, status);
  }
  if (rnn) {
    const int r3 = 3 * r, K = 2 * r + d;
    if (d > 0) {
      if (BF) {
        const int nN = (r3 + kHpOut - 1) / kHpOut;
        const int tiles = (rows + kHpRows - 1) / kHpRows * nN * kHpSplit;
        const int per = (tiles + 7) / 8;
        rnn_hproj_bf16_kernel<<<8 * per, 256, 0, stream>>>(
            rows, d, r3, K, nN, per, reinterpret_cast<const uint16_t*>(h),
            reinterpret_cast<const uint16_t*>(Wg) + 2 * r, ws.Gh);
      } else {
        dim3 grid((r3 + 63) / 64, rows);
        rnn_hproj_f32_kernel<T><<<grid, 64, 0, stream>>>(rows, d, r3, K, h, Wg + 2 * r, ws.Gh);
      }
    } else {
      const size_t n3 = (size_t)kHpSplit * rows * r3;  // both partial buffers
      fill_kernel<<<(unsigned)((n3 + 255) / 256), 256, 0, stream>>>(ws.Gh, n3, 0.0f);
    }
    fill_kernel<<<(R * r + 255) / 256, 256, 0, stream>>>(ws.s, (size_t)R * r, 0.0f);  // s_0 = 0
    if (BF) {
      const int n = (2 * r / 8) * 3 * r;
      rnn_wpack_kernel<<<(n + 255) / 256, 256, 0, stream>>>(
          r, K, reinterpret_cast<const uint16_t*>(Wg), ws.wpack);
    }
  }

  SweepGeom g{};
  int nranges;
  if (BF) {
    g = make_geom(R, V, r, reinterpret_cast<const uint16_t*>(W2t), nranges_for(V, 1));
    nranges = g.nranges;
  } else {
    nranges = nranges_for(V, R);
    if (nranges > 64) nranges = 64;
  }

  for (int k = 1; k <= gamma; ++k) {
    const int32_t* prev = (k == 1) ? x0 : x + (k - 2);
    const int ps = (k == 1) ? 1 : gamma;
    if (rnn && BF && r >= 32) {
      float* s_in = (k & 1) ? ws.s : ws.s2;  // s_0 sits in ws.s
      float* s_out = (k & 1) ? ws.s2 : ws.s;
      const dim3 grid((R + 31) / 32, r / 32);
      rnn_step_mfma_kernel<<<grid, kStepWaves * kWave, 0, stream>>>(
          R, gamma, V, r, reinterpret_cast<const uint16_t*>(W1), ws.wpack, ws.Gh, prev, ps,
          (uint32_t)k, s_in, s_out, ws.orow, status);
    } else if (rnn && BF) {
      const int U = r < kRnnUnits ? r : kRnnUnits;
      const size_t sh = sizeof(float) * kRnnReq * (2 * r + kRnnKSplit * 3 * U);
      const dim3 grid((R + kRnnReq - 1) / kRnnReq, r / U);
      float* s_in = (k & 1) ? ws.s : ws.s2;  // s_0 sits in ws.s
      float* s_out = (k & 1) ? ws.s2 : ws.s;
      rnn_step_batched_kernel<<<grid, kRnnKSplit * 3 * U, sh, stream>>>(
          R, gamma, V, r, reinterpret_cast<const uint16_t*>(W1), ws.wpack, ws.Gh, prev, ps,
          (uint32_t)k, s_in, s_out, ws.orow, status);
    } else if (rnn) {
      const size_t sh = sizeof(float) * 5 * r;
      rnn_step_kernel<T><<<R, 256, sh, stream>>>(R, gamma, V, r, d, W1, Wg, ws.Gh, prev, ps,
                                                 (uint32_t)k, ws.s, ws.orow, status);
    }
    // the timed variant: the bf16 sweep's dispatch timestamps its own start and end
    hipEvent_t e0 = (evb && eve) ? evb[k - 1] : nullptr, e1 = (evb && eve) ? eve[k - 1] : nullptr;
    if (!BF && e0 && e1) (void)hipEventRecord(e0, stream);
    if (BF) {
      DraftSweepParams p{};
      p.U = reinterpret_cast<const uint16_t*>(U) + (size_t)(k - 1) * V;
      p.ustride = (size_t)gamma * V;
      p.V = V;
      p.R = R;
      p.prev = prev;
      p.prev_stride = ps;
      p.W1 = reinterpret_cast<const uint16_t*>(W1);
      p.orow = ws.orow;
      p.bpack = bpack;
      p.r = r;
      p.k = (uint32_t)k;
      p.seed = seed;
      p.cycle = cycle;
      p.partials = ws.partials;
      p.nranges = nranges;
      p.status = status;
      if (rnn)
        launch_sweep<true, DraftEpi<true>>(g, p, stream, e0, e1);
      else if (bias)
        launch_sweep<false, DraftEpi<false>>(g, p, stream, e0, e1);
      else
        launch_sweep<false, DraftEpi<false, false>>(g, p, stream, e0, e1);
    } else {
      const int nblocks = (V + kVB - 1) / kVB;
      dim3 grid(nranges, R);
      draft_sweep_f32_kernel<<<grid, 64, 0, stream>>>(
          R, V, r, reinterpret_cast<const float*>(U) + (size_t)(k - 1) * V, (size_t)gamma * V,
          prev, ps, reinterpret_cast<const float*>(W1), rnn ? ws.orow : nullptr,
          reinterpret_cast<const float*>(W2t), (uint32_t)k, seed, cycle, ws.partials, nranges,
          nblocks, status);
    }
    if (!BF && e0 && e1) (void)hipEventRecord(e1, stream);
    if (rnn)
      draft_combine_kernel<T, true><<<R, kCombineThreads, 0, stream>>>(
          R, gamma, V, r, d, U, W1, W2t, w, temps, ws.zh, prev, ps, ws.orow, ws.partials,
          nranges, (uint32_t)k, seed, cycle, x, c, z, lse, logit_x, bias_rows, nullptr,
          status);
    else if (bias)
      draft_combine_kernel<T, false><<<R, kCombineThreads, 0, stream>>>(
          R, gamma, V, r, d, U, W1, W2t, w, temps, ws.zh, prev, ps, nullptr, ws.partials,
          nranges, (uint32_t)k, seed, cycle, x, c, z, lse, logit_x, bias_rows,
          k < gamma ? bpack : nullptr, status);
    else
      draft_combine_kernel<T, false, false><<<R, kCombineThreads, 0, stream>>>(
          R, gamma, V, r, d, U, W1, W2t, w, temps, ws.zh, prev, ps, nullptr, ws.partials,
          nranges, (uint32_t)k, seed, cycle, x, c, z, lse, logit_x, bias_rows,
          k < gamma ? bpack : nullptr, status);
  }
  return launch_status();
}

static int draft_entry(bool rnn, bool bias, int R, int gamma, int V, int r, int d, dspark_dtype dt,
                       const void* U, const void* h, const void* W1, const void* W2t,
                       const void* Wg, const float* w, const float* temps, const int32_t* x0,
                       uint64_t seed, uint64_t cycle, int32_t* x, float* c, float* z,
                       float* lse, float* logit_x, void* bias_rows, int32_t* status, void* ws,
                       size_t ws_bytes, hipStream_t stream, hipEvent_t* evb = nullptr,
                       hipEvent_t* eve = nullptr) {
  if (!dims_ok(R, gamma, V, r, d) || (dt != DSPARK_F32 && dt != DSPARK_BF16)) return DSPARK_EINVAL;
  if (cycle >= ((uint64_t)1 << 28)) return DSPARK_EINVAL;
  if (R == 0) return DSPARK_OK;
  if (!U || !W1 || (bias && !W2t) || !w || !x0 || !x || !c || !lse || !logit_x || !bias_rows ||
      !ws)
    return DSPARK_EINVAL;
  if (d > 0 && !h) return DSPARK_EINVAL;
  if (rnn && !Wg) return DSPARK_EINVAL;
  if (!bias && (rnn || dt != DSPARK_BF16)) return DSPARK_EINVAL;  // the parallel drafter: bf16
  // the bf16 h projection addresses h with 32-bit byte offsets
  if (rnn && dt == DSPARK_BF16 && (uint64_t)R * gamma * d * 2 >= ((uint64_t)1 << 32))
    return DSPARK_EINVAL;
  // the bf16 sweep addresses U rows with 32-bit byte offsets
  if (dt == DSPARK_BF16 && (uint64_t)R * gamma * V * 2 >= ((uint64_t)1 << 32)) return DSPARK_EINVAL;
  if (!aligned16(U) || !aligned16(h) || !aligned16(W1) || !aligned16(W2t) || !aligned16(Wg) ||
      !aligned16(bias_rows) || !aligned16(w))
    return DSPARK_EINVAL;
  const DraftWs probe = carve_draft(nullptr, R, gamma, V, r, d, rnn);
  if (ws_bytes < probe.bytes) return DSPARK_EWORKSPACE;
  if (!aligned16(ws)) return DSPARK_EINVAL;
  const DraftWs lay = carve_draft(ws, R, gamma, V, r, d, rnn);
  if (dt == DSPARK_BF16)
    return draft_run<uint16_t>(rnn, bias, R, gamma, V, r, d, U, h, W1, W2t, Wg, w, temps, x0, seed,
                               cycle, x, c, z, lse, logit_x, bias_rows, status, lay, stream,
                               evb, eve);
  return draft_run<float>(rnn, bias, R, gamma, V, r, d, U, h, W1, W2t, Wg, w, temps, x0, seed, cycle,
                          x, c, z, lse, logit_x, bias_rows, status, lay, stream, evb, eve);
}

// ---------------------------------------------------------------------------------------
// allocation-free variant: the workspace is a library-owned device array, one per GPU
// (each device's code object holds its own copy until the process ends).  In host code the
// array's name is only a stand-in for the symbol, so its device address is looked up once
// per device with hipGetSymbolAddress and that address is what the kernels receive.
// ---------------------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// the scratch array's device address on the current device (null on failure); the first
// call on a device looks it up, later calls read the per-device cache (concurrent first
// calls both look it up and store the same address)
static void* scratch_on_device() {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  addr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace dspark

extern "C" {

size_t dspark_draft_markov_noalloc_max_bytes(void) { return dspark::kNoAllocScratchBytes; }

int dspark_draft_markov_noalloc(int R, int gamma, int V, int r, int d, dspark_dtype dt,
                                const void* U, const void* h, const void* W1, const void* W2t,
                                const float* w, const float* temps, const int32_t* x0,
                                uint64_t seed, uint64_t cycle, int32_t* x, float* c, float* z,
                                float* lse, float* logit_x, void* bias_rows,
                                int32_t* dev_status, hipStream_t stream) {
  using namespace dspark;
  if (!dims_ok(R, gamma, V, r, d)) return DSPARK_EINVAL;
  if (carve_draft(nullptr, R, gamma, V, r, d, false).bytes > kNoAllocScratchBytes)
    return DSPARK_ERANGE;
  if (R == 0) return DSPARK_OK;
  void* ws = scratch_on_device();
  if (!ws) return DSPARK_EDEVICE;
  return draft_entry(false, true, R, gamma, V, r, d, dt, U, h, W1, W2t, nullptr, w, temps, x0, seed,
                     cycle, x, c, z, lse, logit_x, bias_rows, dev_status, ws,
                     kNoAllocScratchBytes, stream);
}

size_t dspark_draft_workspace_bytes(int R, int gamma, int V, int r, int d) {
  if (!dspark::dims_ok(R, gamma, V, r, d)) return 0;
  return dspark::carve_draft(nullptr, R, gamma, V, r, d, false).bytes;
}

size_t dspark_draft_rnn_workspace_bytes(int R, int gamma, int V, int r, int d) {
  if (!dspark::dims_ok(R, gamma, V, r, d)) return 0;
  return dspark::carve_draft(nullptr, R, gamma, V, r, d, true).bytes;
}

int dspark_draft_markov(int R, int gamma, int V, int r, int d, dspark_dtype dt, const void* U,
                        const void* h, const void* W1, const void* W2t, const float* w,
                        const float* temps, const int32_t* x0, uint64_t seed, uint64_t cycle,
                        int32_t* x, float* c, float* z, float* lse, float* logit_x,
                        void* bias_rows, int32_t* dev_status, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  return dspark::draft_entry(false, true, R, gamma, V, r, d, dt, U, h, W1, W2t, nullptr, w, temps, x0,
                             seed, cycle, x, c, z, lse, logit_x, bias_rows, dev_status, ws,
                             ws_bytes, stream);
}

int dspark_draft_markov_timed(int R, int gamma, int V, int r, int d, dspark_dtype dt,
                              const void* U, const void* h, const void* W1, const void* W2t,
                              const float* w, const float* temps, const int32_t* x0,
                              uint64_t seed, uint64_t cycle, int32_t* x, float* c, float* z,
                              float* lse, float* logit_x, void* bias_rows, int32_t* dev_status,
                              void* ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t* ev_begin, hipEvent_t* ev_end) {
  if (!ev_begin || !ev_end) return DSPARK_EINVAL;
  return dspark::draft_entry(false, true, R, gamma, V, r, d, dt, U, h, W1, W2t, nullptr, w, temps, x0,
                             seed, cycle, x, c, z, lse, logit_x, bias_rows, dev_status, ws,
                             ws_bytes, stream, ev_begin, ev_end);
}

int dspark_draft_parallel(int R, int gamma, int V, int r, int d, dspark_dtype dt, const void* U,
                          const void* h, const void* W1, const float* w, const float* temps,
                          const int32_t* x0, uint64_t seed, uint64_t cycle, int32_t* x, float* c,
                          float* z, float* lse, float* logit_x, void* bias_rows,
                          int32_t* dev_status, void* ws, size_t ws_bytes, hipStream_t stream) {
  return dspark::draft_entry(false, false, R, gamma, V, r, d, dt, U, h, W1, nullptr, nullptr, w,
                             temps, x0, seed, cycle, x, c, z, lse, logit_x, bias_rows, dev_status,
                             ws, ws_bytes, stream);
}

int dspark_draft_rnn(int R, int gamma, int V, int r, int d, dspark_dtype dt, const void* U,
                     const void* h, const void* W1, const void* W2t, const void* W_gco,
                     const float* w, const float* temps, const int32_t* x0, uint64_t seed,
                     uint64_t cycle, int32_t* x, float* c, float* z, float* lse, float* logit_x,
                     float* bias_rows, int32_t* dev_status, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return dspark::draft_entry(true, true, R, gamma, V, r, d, dt, U, h, W1, W2t, W_gco, w, temps, x0,
                             seed, cycle, x, c, z, lse, logit_x, bias_rows, dev_status, ws,
                             ws_bytes, stream);
}

}  // extern "C"
