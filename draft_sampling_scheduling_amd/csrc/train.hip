// train.hip -- forward pass of the drafter's training objective (DSpark digest page,
// Module F, eqs. (8)-(12)) with the Markov head, on teacher-forced blocks: position k of a
// block conditions on the reference token x*_{k-1} (x*_0 = the anchor), so all R * gamma
// rows are independent and one vocabulary sweep covers them all (W2t is read once per
// sweep, not once per position as in drafting).
//
//   sweep 1 (TrainLseEpi)  l = U_k + W1[x*_{k-1}] W2 on the matrix cores, with the target
//                          row streamed beside U: online log-sum-exp of both, per range
//   merge                  per row: both normalisers, log q_k(x*_k) from one 256-term dot,
//                          the confidence logit z_k = w . [h_k ; W1[x*_{k-1}]]
//   sweep 2 (TrainTvEpi)   sum_v |p_k(v) - q_k(v)| per range, both normalisers known
//   final                  per block: tv, c* = 1 - tv/2 (eq. (8)), c = sigmoid(z), and the
//                          weighted losses L_ce, L_tv, L_conf and their mix (eqs. (9)-(12))
#include "dev.h"
#include "host.h"
#include "sweep.h"

namespace dspark {

struct TrainSweepParams {
  const uint16_t* U;       // [R][gamma][V]
  const uint16_t* target;  // [R][gamma][V]
  const uint16_t* W1;      // [V][r]
  const int32_t* x0;       // [R]
  const int32_t* xstar;    // [R][gamma]
  int R, gamma, V, r, nrows, nranges;
  float4* part1;           // [rows][nranges]: (ref_q ln2, S_q, ref_p ln2, S_p)
  float* part2;            // [rows][nranges]: partial sum |p - q|
  const float2* lse;       // [rows]: (lse_q, lse_p) for sweep 2
  const uint4* bpack;      // W1[x*_{k-1}] of every row in the sweep's packed order
  int32_t* status;
};

// previous token of row = q * gamma + (k - 1)
__device__ __forceinline__ int32_t train_prev(const TrainSweepParams& p, int row) {
  const int k1 = row % p.gamma;
  const int32_t t = k1 == 0 ? p.x0[row / p.gamma] : p.xstar[row - 1];
  return checked_token(t, p.V, p.status);
}

struct TrainRowsBase {
  static constexpr int kStreams = 2;  // U_k, target row k
  using Params = TrainSweepParams;
  __device__ static bool group_live(const Params& p, int row0) { return row0 < p.nrows; }
  __device__ static int nrows(const Params& p) { return p.nrows; }
  __device__ static const void* brow(const Params& p, int row) {
    return p.W1 + (size_t)train_prev(p, row) * p.r;
  }
  __device__ static const uint4* bpack(const Params& p) { return p.bpack; }
  __device__ static const uint16_t* sbase(const Params& p, int s) {
    return s == 0 ? p.U : p.target;
  }
  __device__ static uint32_t srow(const Params& p, int, int row) {
    return (uint32_t)((size_t)row * p.V);
  }
};

// both normalisers in one pass: running references (log2 units) and this lane's sums
struct TrainLseEpi : TrainRowsBase {
  struct State {
    float rq, Sq, rp, Sp;
  };
  __device__ static void init(const Params&, State& s, int) {
    s.rq = s.rp = -FLT_MAX;
    s.Sq = s.Sp = 0.0f;
  }
  __device__ static void refresh(const Params&, State&, int, int) {}
  template <int HALF, bool MASK>
  __device__ static void tile(const Params& p, State& s, const f32x16& acc, const uint4 (&x)[2],
                              int b, int, bool) {
    constexpr float kLog2e = 1.4426950408889634f;
    const int h = (threadIdx.x & 63) >> 5;
    float l[16], t[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) l[j] = acc[j];
    widen8(x[0], t);
    widen8(x[1], t + 8);
    if (MASK) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (b * kVB + kTile * HALF + vocab_of_reg(h, j) >= p.V) l[j] = t[j] = -INFINITY;
    }
    float mq = l[0], mp = t[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) {
      mq = fmaxf(mq, l[j]);
      mp = fmaxf(mp, t[j]);
    }
    const float rq = fmaxf(s.rq, half_max(mq * kLog2e));
    const float rp = fmaxf(s.rp, half_max(mp * kLog2e));
    s.Sq *= __builtin_amdgcn_exp2f(s.rq - rq);
    s.Sp *= __builtin_amdgcn_exp2f(s.rp - rp);
    s.rq = rq;
    s.rp = rp;
    float sq = 0.0f, sp = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sq += __builtin_amdgcn_exp2f(fmaf(l[j], kLog2e, -rq));
      sp += __builtin_amdgcn_exp2f(fmaf(t[j], kLog2e, -rp));
    }
    s.Sq += sq;
    s.Sp += sp;
  }
  __device__ static void finish(const Params& p, const State& s, int row, bool owner, int range) {
    constexpr float kLn2 = 0.69314718055994531f;
    const float Sq = half_sum(s.Sq), Sp = half_sum(s.Sp);
    if (!owner) return;
    p.part1[(size_t)row * p.nranges + range] = make_float4(s.rq * kLn2, Sq, s.rp * kLn2, Sp);
  }
};

// sum_v |p(v) - q(v)| with both normalisers known
struct TrainTvEpi : TrainRowsBase {
  struct State {
    float tv, lq, lp;
  };
  __device__ static void init(const Params& p, State& s, int row) {
    s.tv = 0.0f;
    s.lq = s.lp = 0.0f;
    if (row >= 0) {
      const float2 n = p.lse[row];
      s.lq = n.x;
      s.lp = n.y;
    }
  }
  __device__ static void refresh(const Params&, State&, int, int) {}
  template <int HALF, bool MASK>
  __device__ static void tile(const Params& p, State& s, const f32x16& acc, const uint4 (&x)[2],
                              int b, int, bool) {
    const int h = (threadIdx.x & 63) >> 5;
    float t[16];
    widen8(x[0], t);
    widen8(x[1], t + 8);
    float tv = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool ok = !MASK || b * kVB + kTile * HALF + vocab_of_reg(h, j) < p.V;
      const float d = __expf(t[j] - s.lp) - __expf(acc[j] - s.lq);
      tv += ok ? fabsf(d) : 0.0f;
    }
    s.tv += tv;
  }
  __device__ static void finish(const Params& p, const State& s, int row, bool owner, int range) {
    const float tv = half_sum(s.tv);
    if (!owner) return;
    p.part2[(size_t)row * p.nranges + range] = tv;
  }
};

// the B rows of both sweeps, W1[x*_{k-1}] per row, in the sweep's packed order
__global__ void __launch_bounds__(256) train_pack_kernel(TrainSweepParams p, uint4* bpack) {
  const int cpr = p.r / 8;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= p.nrows * cpr) return;
  const int row = gid / cpr, ch = gid - row * cpr;
  const int32_t t = train_prev(p, row);
  bpack[bpack_index(row, ch, p.r / 16)] =
      reinterpret_cast<const uint4*>(p.W1 + (size_t)t * p.r)[ch];
}

constexpr int kTrainMergeRows = 4;  // one wave per row

// per row: normalisers from the range partials, log q(x*), confidence logit
__global__ void __launch_bounds__(64 * kTrainMergeRows) train_merge_kernel(
    TrainSweepParams p, int d, const uint16_t* __restrict__ h, const uint16_t* __restrict__ W2t,
    const float* __restrict__ w, float2* __restrict__ lse, float* __restrict__ logq,
    float* __restrict__ zlogit, float* __restrict__ logq_out) {
  const int row = blockIdx.x * kTrainMergeRows + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.nrows) return;
  float mq = -INFINITY, sq = 0.0f, mp = -INFINITY, sp = 0.0f;
  const float4* part = p.part1 + (size_t)row * p.nranges;
  for (int i = lane; i < p.nranges; i += kWave) {
    const float4 v = part[i];
    lse_merge(mq, sq, v.x, v.y);
    lse_merge(mp, sp, v.z, v.w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mq2 = __shfl_xor(mq, o, kWave), sq2 = __shfl_xor(sq, o, kWave);
    const float mp2 = __shfl_xor(mp, o, kWave), sp2 = __shfl_xor(sp, o, kWave);
    lse_merge(mq, sq, mq2, sq2);
    lse_merge(mp, sp, mp2, sp2);
  }
  const float lq = mq + __logf(sq), lp = mp + __logf(sp);
  // l(x*) = U[row][x*] + W1[prev] . W2t[x*]; z = w[:d] . h_row + w[d:] . W1[prev]
  const int32_t prev = train_prev(p, row);
  const int32_t xs = checked_token(p.xstar[row], p.V, p.status);
  const uint16_t* e = p.W1 + (size_t)prev * p.r;
  const uint16_t* wx = W2t + (size_t)xs * p.r;
  float dl = 0.0f, dz = 0.0f;
  for (int i = lane; i < p.r; i += kWave) {
    const float ei = bf16_to_f32(e[i]);
    dl = fmaf(ei, bf16_to_f32(wx[i]), dl);
    dz = fmaf(ei, w[d + i], dz);
  }
  const uint16_t* hr = h + (size_t)row * d;
  for (int i = lane * 8; i < d; i += kWave * 8) {
    float x[8];
    ld8<uint16_t>(hr + i, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) dz = fmaf(w[i + j], x[j], dz);
  }
  dl = wave_sum(dl);
  dz = wave_sum(dz);
  if (lane == 0) {
    lse[row] = make_float2(lq, lp);
    const float lx = bf16_to_f32(p.U[(size_t)row * p.V + xs]) + dl - lq;
    logq[row] = lx;
    if (logq_out) logq_out[row] = lx;
    zlogit[row] = dz;
  }
}

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x)));
}

constexpr int kTrainFinalThreads = 256;

// one workgroup per block: wave w takes positions w, w + 4, ...; the block's sums run in
// position order
__global__ void __launch_bounds__(kTrainFinalThreads) train_final_kernel(
    int gamma, int nranges, const float* __restrict__ part2, const float* __restrict__ logq,
    const float* __restrict__ zlogit, float a_ce, float a_tv, float a_conf,
    float* __restrict__ c_star, float* __restrict__ c, float* __restrict__ tv_out,
    float* __restrict__ loss) {
  __shared__ float terms[3][kMaxGamma];
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int k = wave; k < gamma; k += kTrainFinalThreads / kWave) {
    const size_t row = (size_t)q * gamma + k;
    const float* part = part2 + row * nranges;
    float tv = 0.0f;
    for (int i = lane; i < nranges; i += kWave) tv += part[i];
    tv = wave_sum(tv);
    if (lane == 0) {
      const float cs = 1.0f - 0.5f * tv;
      const float z = zlogit[row];
      const float wk = __expf(-(float)k / (float)gamma);
      if (c_star) c_star[row] = cs;
      if (c) c[row] = 1.0f / (1.0f + __expf(-z));
      if (tv_out) tv_out[row] = tv;
      terms[0][k] = -wk * logq[row];
      terms[1][k] = wk * tv;
      terms[2][k] = wk * (cs * softplus_f(-z) + (1.0f - cs) * softplus_f(z));
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && loss) {
    float Lce = 0.0f, Ltv = 0.0f, Lconf = 0.0f;
    for (int k = 0; k < gamma; ++k) {
      Lce += terms[0][k];
      Ltv += terms[1][k];
      Lconf += terms[2][k];
    }
    float* o = loss + (size_t)q * 4;
    o[0] = Lce;
    o[1] = Ltv;
    o[2] = Lconf;
    o[3] = a_ce * Lce + a_tv * Ltv + a_conf * Lconf;
  }
}

struct TrainWs {
  uint4* bpack;
  float4* part1;
  float* part2;
  float2* lse;
  float* logq;
  float* z;
  size_t bytes;
};

// Vocabulary ranges of the two sweeps.  Every (range, row group) pair is one workgroup, and
// each workgroup pays a prologue (its B rows, the first tile) before its tiles stream; with
// many row groups, fewer and longer ranges spread that over more tiles.  The count aims at
// about four workgroups per CU over the whole grid (two resident at a time) and never exceeds
// one range per CU.  At 2048 rows (16 groups) over V = 151936 that is 64 ranges: a call took
// 0.72-0.74 ms against 0.76-0.78 ms with 256 ranges, and 32 ranges timed like 64.
inline int train_nranges(int V, int rows) {
  const int nblocks = (V + kVB - 1) / kVB;
  const int ngroups = rows > 0 ? (rows + kRowsPerGroup - 1) / kRowsPerGroup : 1;
  int nr = (4 * device_cus() + ngroups - 1) / ngroups;
  if (nr > device_cus()) nr = device_cus();
  if (nr >= 8) nr &= ~7;  // a multiple of 8 keeps each range's workgroups on one XCD
  if (nr > kMaxRanges) nr = kMaxRanges;
  if (nr > nblocks) nr = nblocks;
  return nr < 1 ? 1 : nr;
}

inline TrainWs train_carve(void* base, int rows, int nranges) {
  Carve cv(base);
  TrainWs w;
  w.bpack = cv.take<uint4>((size_t)bpack_rows(rows) * 32);  // r <= 256: 32 chunks per row
  w.part1 = cv.take<float4>((size_t)rows * nranges);
  w.part2 = cv.take<float>((size_t)rows * nranges);
  w.lse = cv.take<float2>((size_t)rows);
  w.logq = cv.take<float>((size_t)rows);
  w.z = cv.take<float>((size_t)rows);
  w.bytes = cv.bytes();
  return w;
}

// the U and target arrays are addressed with 32-bit byte offsets inside the sweep
inline bool train_dims_ok(int R, int gamma, int V, int r, int d) {
  return dims_ok(R, gamma, V, r, d) && (size_t)R * gamma * V * 2 < ((size_t)1 << 32);
}

}  // namespace dspark

extern "C" {

size_t dspark_train_forward_workspace_bytes(int R, int gamma, int V, int r, int d) {
  using namespace dspark;
  if (!train_dims_ok(R, gamma, V, r, d)) return 0;
  // sized for the largest range count any device may pick
  return train_carve(nullptr, R * gamma, kMaxRanges).bytes;
}

int dspark_train_forward(int R, int gamma, int V, int r, int d, dspark_dtype dt, const void* U,
                         const void* h, const void* W1, const void* W2t, const float* w,
                         const void* target, const int32_t* x0, const int32_t* xstar,
                         float a_ce, float a_tv, float a_conf, float* c_star, float* c,
                         float* logq, float* tv, float* loss, int32_t* dev_status, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  using namespace dspark;
  if (dt != DSPARK_BF16) return DSPARK_EINVAL;
  if (!train_dims_ok(R, gamma, V, r, d)) return DSPARK_EINVAL;
  if (R == 0) return DSPARK_OK;
  if (!U || !W1 || !W2t || !w || !target || !x0 || !xstar || !ws) return DSPARK_EINVAL;
  if (d > 0 && !h) return DSPARK_EINVAL;
  if (!aligned16(U) || !aligned16(h) || !aligned16(W1) || !aligned16(W2t) ||
      !aligned16(target))
    return DSPARK_EINVAL;
  const int rows = R * gamma;
  const int nranges = train_nranges(V, rows);
  const TrainWs wsl = train_carve(ws, rows, nranges);
  if (ws_bytes < train_carve(nullptr, rows, kMaxRanges).bytes) return DSPARK_EWORKSPACE;

  TrainSweepParams p{};
  p.U = static_cast<const uint16_t*>(U);
  p.target = static_cast<const uint16_t*>(target);
  p.W1 = static_cast<const uint16_t*>(W1);
  p.x0 = x0;
  p.xstar = xstar;
  p.R = R;
  p.gamma = gamma;
  p.V = V;
  p.r = r;
  p.nrows = rows;
  p.nranges = nranges;
  p.part1 = wsl.part1;
  p.part2 = wsl.part2;
  p.lse = wsl.lse;
  p.status = dev_status;
  p.bpack = wsl.bpack;
  SweepGeom g = make_geom(rows, V, r, static_cast<const uint16_t*>(W2t), nranges);
  // one workgroup per (range, row group): the dispatch order runs a range's groups together on
  // one XCD, so each W2t tile comes from HBM about once and from that XCD's L2 for the rest,
  // and one workgroup's start overlaps another's sweep instead of following it
  g.gsplit = g.ngroups;
  train_pack_kernel<<<(rows * (r / 8) + 255) / 256, 256, 0, stream>>>(p, wsl.bpack);
  launch_sweep<false, TrainLseEpi>(g, p, stream);
  train_merge_kernel<<<(rows + kTrainMergeRows - 1) / kTrainMergeRows, 64 * kTrainMergeRows, 0,
                       stream>>>(p, d, static_cast<const uint16_t*>(h),
                                 static_cast<const uint16_t*>(W2t), w, wsl.lse, wsl.logq,
                                 wsl.z, logq);
  launch_sweep<false, TrainTvEpi>(g, p, stream);
  train_final_kernel<<<R, kTrainFinalThreads, 0, stream>>>(gamma, nranges, wsl.part2, wsl.logq,
                                                           wsl.z, a_ce, a_tv, a_conf, c_star,
                                                           c, tv, loss);
  return launch_status();
}

}  // extern "C"
