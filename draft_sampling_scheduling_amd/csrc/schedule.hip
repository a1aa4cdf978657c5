// schedule.hip -- the hardware-aware prefix scheduler (digest page, Module E, Algorithm 1,
// and the production variants without the break and with the two-step lag).
//
// Entry e = (q, j) of a batch has the prefix survival a_e = c_{q,1} * ... * c_{q,j} (float,
// left to right) and the 64-bit key
//     key_e = (~bits(a_e)) << 32 | (q * gamma + j - 1),
// so ascending keys are descending a with ties broken by q, then j (a is non-negative, so
// its bit pattern orders like its value, and the j order keeps every request's admitted set
// a prefix).  Entries with a = 0 are not candidates.  Algorithm 1 admits the candidates in
// that order; entry e is admitted n_e = rho_e + 1 -th, where
//     rho_e = #{candidates f : key_f < key_e},   S_e = sum of floor(a_f * 2^32) over them,
// and tau after it is exactly R + (S_e + floor(a_e * 2^32)) * 2^-32.  Both are dominance
// counts over all pairs, so no sorted array is needed, and Theta_{n_e} and Theta_{n_e - 1}
// (the break's comparison) follow from e alone.  The increments are integers, so tau never
// depends on a summation order, and every decision is the one the sequential loop of
// Algorithm 1 takes.
//
// One launch.  Every workgroup rebuilds its batch's keys in LDS; each wave takes XW entries
// and sweeps all keys in its lanes (one 64-bit compare and one 64-bit conditional add per
// pair: the increment carries 2^48, so the count rides in the high bits of the same sum).
// A workgroup then publishes its decisive entry: the first key that drops Theta (break),
// the key with the largest Theta (no break), the count n at the largest Theta (lagged batch
// of the two-step lag), or its number of candidates (current batch of the two-step lag).
// The last workgroup to publish (every workgroup checks whether all others have) reduces the
// publications.  With the break or without it, that gives the first key not admitted, and
// its LDS still holds every key: n, tau and ell_q are counts and sums over the keys below
// it.  In the two-step-lag mode the lagged batch's workgroups run beside the current batch's
// and the admitted set is read back from each entry's rank.
//
// Publication without a zeroed counter and without cache maintenance: the workspace holds an
// epoch word; a call's workgroups read it at their start and publish with tag = epoch + 1,
// and the finishing workgroup stores epoch + 1 back, so a replayed graph reads the epoch
// afresh and words left by earlier calls never carry the current tag.  A publication is two
// payload words and a check word, the tag's hash mixed with the payload words' hashes, all
// stored at device scope (written through to the point of coherence that every XCD shares).
// A reader that loads the three words and finds the check consistent with the current tag
// has the current payload: a stale word changes the check by a hash difference.  A
// workgroup waits until its own three stores are acknowledged before it loads the others'
// words, so the owner of the last acknowledged publication sees every publication.  Two
// workgroups that both see all of them compute and store the same results.
#include <climits>

#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / kWave;  // 16
constexpr int kRankUnroll = 4;                    // key rows in flight per lane
constexpr int kRankMaxBlocks = 256;               // workgroups per batch (XW is picked to fit)
constexpr unsigned long long kCountUnit = 1ull << 48;  // S < N * 2^32 <= 2^45 < 2^48
constexpr unsigned long long kNoKey = ~0ull;           // non-candidates and "none"
constexpr unsigned long long kNegInfBits = 0xFFF0000000000000ull;  // -inf as a double
constexpr int kPubWords = 4;  // words per publication slot (payload, payload, check, unused)

enum SchedEval { kEvalNone = 0, kEvalBreak = 1, kEvalArgmax = 2 };

struct SchedBatch {
  const float* c;           // [R][gamma]
  int R;
  int nblocks;              // workgroups of this batch
  int eval;                 // SchedEval
  bool lagged;              // the lagged batch (argmax publishes n instead of the key)
  int32_t* rank;            // [R * gamma] rho_e (INT_MAX for non-candidates), or null
  unsigned long long* tau;  // [R * gamma] tau through e in 2^-32 units, or null
  float* a_out;             // [R][gamma] prefix survival, or null
};

struct SchedOut {
  int mode;
  int32_t* ell;
  double* stats;
  unsigned long long* epoch;  // one word
  unsigned long long* pub;    // [b0.nblocks + b1.nblocks][kPubWords]: payload, payload, check
};

__device__ __forceinline__ double theta_of(unsigned long long tau_fx, float sps) {
  return ((double)tau_fx * 0x1p-32) * (double)sps;
}

// floor(a * 2^32) for a in [0, 1] from the float's fields (exact)
__device__ __forceinline__ unsigned long long incr_of_bits(uint32_t b) {
  const int e = (int)(b >> 23);
  if (e == 0) return 0ull;  // zero and subnormals: a * 2^32 < 1
  const unsigned long long m = (b & 0x7FFFFFu) | 0x800000u;
  const int sh = e - 118;  // a * 2^32 = m * 2^(e - 150 + 32), e <= 127
  return sh >= 0 ? m << sh : (sh > -32 ? m >> (-sh) : 0ull);
}

// 64-bit finalizer of MurmurHash3 (fmix64): a bijection that spreads every input bit
__device__ __forceinline__ unsigned long long mix64(unsigned long long x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdull;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ull;
  x ^= x >> 33;
  return x;
}

__device__ __forceinline__ unsigned long long pub_check(unsigned long long tag,
                                                        unsigned long long w0,
                                                        unsigned long long w1) {
  return mix64(tag) ^ mix64(w0 ^ 0x9e3779b97f4a7c15ull) ^ mix64(w1 ^ 0x632be59bd9b4e019ull);
}

// s_waitcnt vmcnt(0) (gfx9 encoding; expcnt and lgkmcnt left free): every memory access
// this wave issued has completed, stores included
constexpr int kWaitStores = 0x0F70;

__device__ __forceinline__ void st_dev(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// this wave's device-scope stores are acknowledged before anything after this point issues
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // keeps the compiler's order
  __builtin_amdgcn_s_waitcnt(kWaitStores);
}

// a 64-bit value of the partner lane of butterfly step STEP (the DPP network of dev.h)
template <int STEP>
__device__ __forceinline__ unsigned long long partner64(unsigned long long v) {
  const uint32_t lo = xlane_partner<STEP>((uint32_t)v);
  const uint32_t hi = xlane_partner<STEP>((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
// the values of lanes l and l ^ 32, in the order (lower half, upper half)
__device__ __forceinline__ void halves64(unsigned long long v, unsigned long long& a,
                                         unsigned long long& b) {
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32),
                                                   false, false);
  a = ((unsigned long long)hi[0] << 32) | lo[0];
  b = ((unsigned long long)hi[1] << 32) | lo[1];
}

// sum across the wave (exact integers: every lane ends with the same total)
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  v += partner64<0>(v);
  v += partner64<1>(v);
  v += partner64<2>(v);
  v += partner64<3>(v);
  v += partner64<4>(v);
  unsigned long long a, b;
  halves64(v, a, b);
  return a + b;
}

// the published quantity of one batch: (theta, order) for the argmax (largest theta, then
// smallest order), the smallest order for the break, the sum of counts otherwise
struct Pub {
  unsigned long long o;  // key or n ("none": kNoKey); candidate count for kEvalNone
  double th;             // -inf if none
};

__device__ __forceinline__ Pub pub_none(int eval) {
  Pub p;
  p.o = eval == kEvalNone ? 0ull : kNoKey;
  p.th = -INFINITY;
  return p;
}

__device__ __forceinline__ void pub_merge(Pub& a, const Pub& b, int eval) {
  if (eval == kEvalNone) {
    a.o += b.o;
  } else if (eval == kEvalBreak) {
    a.o = b.o < a.o ? b.o : a.o;
  } else if (b.th > a.th || (b.th == a.th && b.o < a.o)) {
    a = b;
  }
}

template <int STEP>
__device__ __forceinline__ Pub partner_pub(const Pub& p) {
  Pub q;
  q.o = partner64<STEP>(p.o);
  q.th = __longlong_as_double((long long)partner64<STEP>((unsigned long long)__double_as_longlong(p.th)));
  return q;
}

__device__ __forceinline__ Pub wave_pub(Pub p, int eval) {
  pub_merge(p, partner_pub<0>(p), eval);
  pub_merge(p, partner_pub<1>(p), eval);
  pub_merge(p, partner_pub<2>(p), eval);
  pub_merge(p, partner_pub<3>(p), eval);
  pub_merge(p, partner_pub<4>(p), eval);
  Pub lo, hi;
  halves64(p.o, lo.o, hi.o);
  unsigned long long tl, th;
  halves64((unsigned long long)__double_as_longlong(p.th), tl, th);
  lo.th = __longlong_as_double((long long)tl);
  hi.th = __longlong_as_double((long long)th);
  pub_merge(lo, hi, eval);
  return lo;
}

__host__ __device__ __forceinline__ int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Workgroups [0, b0.nblocks) take batch b0 (the current batch), the rest batch b1 (the lagged
// batch of the two-step-lag mode).  Workgroup blk of a batch owns entries [blk * XB, blk * XB
// + XB) in request-major order; wave w of it entries blk * XB + w * XW + i, i < XW.
// LDS: the batch's keys with their increments (+ 2^48), entry (q, j) at slot j * R + q so
// that the threads building them write consecutive slots, padded with non-candidates; then,
// with SPS_LDS, the table slice SPS(R .. R + N).
template <int XW, bool SPS_LDS>
__global__ void __launch_bounds__(kRankThreads) schedule_kernel(
    int gamma, SchedBatch b0, SchedBatch b1, const float* __restrict__ sps, int sps_B0,
    int npad_max, SchedOut out, int32_t* status) {
  constexpr int XB = XW * kRankWaves;
  extern __shared__ ulonglong2 ent[];
  __shared__ Pub e_pub[XB];
  __shared__ Pub s_cur, s_lag;
  __shared__ unsigned long long s_red[kRankWaves];
  __shared__ int s_last;
  const bool second = (int)blockIdx.x >= b0.nblocks;
  const SchedBatch B = second ? b1 : b0;
  const int blk = second ? (int)blockIdx.x - b0.nblocks : (int)blockIdx.x;
  const int R = B.R, N = R * gamma;
  const int npad = round_up(N, kWave * kRankUnroll);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nwg = b0.nblocks + b1.nblocks;

  // The confidences of this thread's first request go out first and the keys are built from
  // them; the SPS slice and the epoch are issued after the keys (loads retire in order, so
  // the keys never wait for them) and stay in flight through the pair sweep, which reads LDS
  // only; the slice is stored to LDS just before the evaluation.
  const int q0 = threadIdx.x;
  float cv0[8];
  {
    const float* cq = B.c + (size_t)(q0 < R ? q0 : 0) * gamma;
#pragma unroll
    for (int u = 0; u < 8; ++u) cv0[u] = cq[u < gamma ? u : gamma - 1];
  }
  float* lsps = reinterpret_cast<float*>(ent + npad_max);
  const float* tsps = SPS_LDS ? lsps : sps + (R - sps_B0);  // SPS(R + n) for n = 0..N
  constexpr int kSpsPer = SPS_LDS ? (4096 + kRankThreads) / kRankThreads : 1;  // N <= 4096

  // keys of every entry of the batch: chunk j0 .. j0 + 7 of request q, the running product
  // carried in run
  auto chunk = [&](int q, int j0, const float (&cv)[8], float& run) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      if (j >= gamma) break;
      float cj = cv[u];
      if (!(cj >= 0.0f && cj <= 1.0f)) {
        if (blk == 0) raise_fault(status, DSPARK_FAULT_CONF);
        cj = (cj > 1.0f) ? 1.0f : 0.0f;  // NaN and negatives -> 0
      }
      run = (j == 0) ? cj : __fmul_rn(run, cj);
      const uint32_t bits = __float_as_uint(run);
      ent[j * R + q] = run > 0.0f
                           ? make_ulonglong2(((unsigned long long)(~bits) << 32) |
                                                 (unsigned)(q * gamma + j),
                                             incr_of_bits(bits) + kCountUnit)
                           : make_ulonglong2(kNoKey, 0ull);
    }
  };
  // the first chunk of the first request straight from the registers loaded first (no loop
  // around it, so its wait leaves the later loads in flight)
  float run0 = 1.0f;
  if (q0 < R) chunk(q0, 0, cv0, run0);
  for (int q = q0; q < R; q += kRankThreads) {
    const float* cq = B.c + (size_t)q * gamma;
    float run = run0;
    for (int j0 = q == q0 ? 8 : 0; j0 < gamma; j0 += 8) {
      float cv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) cv[u] = cq[j0 + u < gamma ? j0 + u : gamma - 1];
      chunk(q, j0, cv, run);
    }
  }
  for (int s = N + threadIdx.x; s < npad; s += kRankThreads) ent[s] = make_ulonglong2(kNoKey, 0ull);
  __builtin_amdgcn_sched_barrier(0);  // the loads below stay after the keys
  float sv[kSpsPer];
  if (SPS_LDS) {
#pragma unroll
    for (int u = 0; u < kSpsPer; ++u) {
      const int n = (int)threadIdx.x + u * kRankThreads;
      sv[u] = n <= N ? sps[R - sps_B0 + n] : 0.0f;
    }
  }
  const float sps_R = sps[b0.R - sps_B0];  // SPS(R) of the current batch
  const float sps_Rl = b1.nblocks > 0 ? sps[b1.R - sps_B0] : 0.0f;
  const unsigned long long tag = ld_dev(out.epoch) + 1ull;  // needed only to publish
  __syncthreads();

  // this wave's entries (uniform across the wave: broadcast reads)
  const int e0 = blk * XB + wave * XW;
  unsigned long long xk[XW];
#pragma unroll
  for (int i = 0; i < XW; ++i) {
    const int e = e0 + i;
    xk[i] = e < N ? ent[(e % gamma) * R + e / gamma].x : kNoKey;
  }
  unsigned long long acc[XW];
#pragma unroll
  for (int i = 0; i < XW; ++i) acc[i] = 0ull;
  for (int s0 = lane; s0 < npad; s0 += kWave * kRankUnroll) {
    ulonglong2 y[kRankUnroll];
#pragma unroll
    for (int u = 0; u < kRankUnroll; ++u) y[u] = ent[s0 + u * kWave];
#pragma unroll
    for (int u = 0; u < kRankUnroll; ++u)
#pragma unroll
      for (int i = 0; i < XW; ++i) acc[i] += (y[u].x < xk[i]) ? y[u].y : 0ull;
  }
#pragma unroll
  for (int i = 0; i < XW; ++i) acc[i] = wave_sum_u64(acc[i]);
  if (SPS_LDS) {
#pragma unroll
    for (int u = 0; u < kSpsPer; ++u) {
      const int n = (int)threadIdx.x + u * kRankThreads;
      if (n <= N) lsps[n] = sv[u];
    }
    __syncthreads();
  }

  // lane i < XW evaluates entry e0 + i
  if (lane < XW) {
    const int i = lane;
    const int e = e0 + i;
    unsigned long long A = acc[0], key = xk[0];
#pragma unroll
    for (int k = 1; k < XW; ++k)
      if (i == k) {
        A = acc[k];
        key = xk[k];
      }
    Pub p = pub_none(B.eval);
    if (e < N) {
      const bool valid = key != kNoKey;
      if (B.a_out) B.a_out[e] = valid ? __uint_as_float(~(uint32_t)(key >> 32)) : 0.0f;
      if (B.rank) st_dev(B.rank + e, valid ? (int)(A >> 48) : INT_MAX);
      if (valid) {
        const int rho = (int)(A >> 48);
        const unsigned long long before = ((unsigned long long)R << 32) + (A & (kCountUnit - 1));
        const unsigned long long through = before + incr_of_bits(~(uint32_t)(key >> 32));
        if (B.tau) st_dev(B.tau + e, through);
        if (B.eval == kEvalNone) {
          p.o = 1ull;
        } else {
          const double t1 = theta_of(through, tsps[rho + 1]);
          if (B.eval == kEvalArgmax) {
            p.o = B.lagged ? (unsigned long long)(rho + 1) : key;
            p.th = t1;
          } else if (!(t1 > theta_of(before, tsps[rho]))) {
            p.o = key;
          }
        }
      }
    }
    e_pub[wave * XW + i] = p;
  }
  // the ranks and taus that the finishing workgroup reads back (two-step lag) are
  // acknowledged before this workgroup publishes
  if (B.rank) stores_done();
  __syncthreads();

  // publish; then load every publication and check whether all are current
  if (wave == 0) {
    if (lane == 0) {
      Pub p = e_pub[0];
      for (int k = 1; k < XB; ++k) pub_merge(p, e_pub[k], B.eval);
      const unsigned long long w1 = (unsigned long long)__double_as_longlong(p.th);
      unsigned long long* w = out.pub + kPubWords * (size_t)blockIdx.x;
      st_dev(w + 0, p.o);
      st_dev(w + 1, w1);
      st_dev(w + 2, pub_check(tag, p.o, w1));
      stores_done();
    }
    Pub cur = pub_none(b0.eval), lag = pub_none(kEvalArgmax);
    bool ok = true;
    for (int k = lane; k < nwg; k += kWave) {
      const unsigned long long* w = out.pub + kPubWords * (size_t)k;
      Pub p;
      p.o = ld_dev(w + 0);
      // the second word is -inf unless the batch publishes a maximum
      const bool arg = k < b0.nblocks ? b0.eval == kEvalArgmax : true;
      const unsigned long long w1 = arg ? ld_dev(w + 1) : kNegInfBits;
      ok &= ld_dev(w + 2) == pub_check(tag, p.o, w1);
      p.th = __longlong_as_double((long long)w1);
      if (k < b0.nblocks)
        pub_merge(cur, p, b0.eval);
      else
        pub_merge(lag, p, kEvalArgmax);
    }
    const bool all = __ballot(!ok) == 0ull;
    cur = wave_pub(cur, b0.eval);
    lag = wave_pub(lag, kEvalArgmax);
    if (lane == 0) {
      s_last = all ? 1 : 0;
      s_cur = cur;
      s_lag = lag;
    }
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the finishing workgroup: the admitted count, ell and the stats ----
  const int Rc = b0.R;
  const Pub cur = s_cur;
  int n;
  unsigned long long tau_n;
  if (out.mode != DSPARK_SCHED_ASYNC_LAG2) {
    // a current-batch workgroup: its LDS holds every key; the admitted entries are the keys
    // below thr
    unsigned long long thr;
    if (out.mode == DSPARK_SCHED_SYNC_BREAK)
      thr = cur.o;  // the first key that drops Theta, or kNoKey: all candidates
    else
      thr = (cur.o != kNoKey && cur.th > theta_of((unsigned long long)Rc << 32, sps_R))
                ? cur.o + 1ull  // keys are distinct: the keys up to the best one
                : 0ull;
    unsigned long long a = 0ull;
    for (int s = threadIdx.x; s < npad; s += kRankThreads) {
      const ulonglong2 y = ent[s];
      a += y.x < thr ? y.y : 0ull;
    }
    a = wave_sum_u64(a);
    if (lane == 0) s_red[wave] = a;
    for (int q = threadIdx.x; q < Rc; q += kRankThreads) {
      int cnt = 0;
      for (int j = 0; j < gamma; ++j) cnt += ent[j * Rc + q].x < thr ? 1 : 0;
      out.ell[q] = cnt;
    }
    __syncthreads();
    a = 0ull;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) a += s_red[w];
    n = (int)(a >> 48);
    tau_n = ((unsigned long long)Rc << 32) + (a & (kCountUnit - 1));
  } else {
    // the lagged batch's no-break count gives the capacity; the admitted set by rank (this
    // workgroup's LDS may hold the other batch); the entry of rank n - 1 gives tau
    const Pub lag = s_lag;
    const int Rl = b1.R;
    const int nl =
        (lag.o != kNoKey && lag.th > theta_of((unsigned long long)Rl << 32, sps_Rl)) ? (int)lag.o : 0;
    const int K = Rl + nl - Rc;
    const int nE = (int)cur.o;
    n = K > 0 ? (K < nE ? K : nE) : 0;
    tau_n = (unsigned long long)Rc << 32;
    for (int q = threadIdx.x; q < Rc; q += kRankThreads) {
      int cnt = 0;
      for (int j = 0; j < gamma; ++j) {
        const int rk = ld_dev(b0.rank + q * gamma + j);
        cnt += rk < n ? 1 : 0;
        if (out.stats && n > 0 && rk == n - 1) {
          const unsigned long long t = ld_dev(b0.tau + q * gamma + j);
          const int Bn = Rc + n;
          out.stats[0] = (double)Bn;
          out.stats[1] = (double)t * 0x1p-32;
          out.stats[2] = theta_of(t, sps[Bn - sps_B0]);
          out.stats[3] = (double)n;
        }
      }
      out.ell[q] = cnt;
    }
  }
  if (threadIdx.x == 0) {
    if (out.stats && (out.mode != DSPARK_SCHED_ASYNC_LAG2 || n == 0)) {
      const int Bn = Rc + n;
      out.stats[0] = (double)Bn;
      out.stats[1] = (double)tau_n * 0x1p-32;
      out.stats[2] = theta_of(tau_n, (SPS_LDS && !second) ? lsps[n] : sps[Bn - sps_B0]);
      out.stats[3] = (double)n;
    }
    st_dev(out.epoch, tag);
  }
}

// entries per wave so that a batch of N entries takes at most kRankMaxBlocks workgroups
static int rank_xw(int N) { return N <= kRankWaves * kRankMaxBlocks ? 1 : 2; }

struct SchedWs {
  unsigned long long* epoch;
  unsigned long long* pub;
  unsigned long long* tau;
  int32_t* rank;
  size_t bytes;
};

// the epoch and the publications first, at offsets that do not depend on the shape
static SchedWs carve_sched(void* ws, int R, int gamma) {
  const size_t N = (size_t)R * gamma;
  Carve cv(ws);
  SchedWs w{};
  w.epoch = cv.take<unsigned long long>(1);
  w.pub = cv.take<unsigned long long>(kPubWords * 2 * kRankMaxBlocks);
  w.tau = cv.take<unsigned long long>(N);
  w.rank = cv.take<int32_t>(N);
  w.bytes = cv.bytes();
  return w;
}

// the table slice goes to LDS beside the keys up to 4096 entries (8192 keys fill 128 KB)
template <int XW>
static void launch_schedule(int gamma, const SchedBatch& b0, const SchedBatch& b1,
                            const float* sps, int sps_B0, int nmax, const SchedOut& out,
                            int32_t* status, hipStream_t stream) {
  constexpr bool kSpsLds = XW == 1;
  const int npad_max = round_up(nmax, kWave * kRankUnroll);
  const size_t lds =
      (size_t)npad_max * sizeof(ulonglong2) + (kSpsLds ? (size_t)(nmax + 1) * sizeof(float) : 0);
  static std::atomic<uint64_t> raised{0};
  ensure_dynamic_lds(reinterpret_cast<const void*>(schedule_kernel<XW, kSpsLds>),
                     (int)(round_up(kMaxSchedN, kWave * kRankUnroll) * sizeof(ulonglong2)),
                     raised);
  schedule_kernel<XW, kSpsLds><<<b0.nblocks + b1.nblocks, kRankThreads, lds, stream>>>(
      gamma, b0, b1, sps, sps_B0, npad_max, out, status);
}

}  // namespace dspark

extern "C" {

size_t dspark_schedule_workspace_bytes(int R, int gamma) {
  using namespace dspark;
  if (R < 1 || gamma < 1 || gamma > kMaxGamma || (long)R * gamma > kMaxSchedN) return 0;
  return carve_sched(nullptr, R, gamma).bytes;
}

int dspark_schedule(int R, int gamma, const float* c, const float* c_lag, int R_lag,
                    const float* sps, int sps_B0, int sps_len, dspark_sched_mode mode,
                    int32_t* ell, float* a, double* stats, int32_t* dev_status, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  using namespace dspark;
  if (R < 0 || gamma < 1 || gamma > kMaxGamma || sps_len < 1) return DSPARK_EINVAL;
  if (mode != DSPARK_SCHED_SYNC_BREAK && mode != DSPARK_SCHED_GLOBAL &&
      mode != DSPARK_SCHED_ASYNC_LAG2)
    return DSPARK_EINVAL;
  if (R == 0) return DSPARK_OK;
  if ((long)R * gamma > kMaxSchedN) return DSPARK_EINVAL;
  if (!c || !sps || !ell) return DSPARK_EINVAL;
  const bool lag = mode == DSPARK_SCHED_ASYNC_LAG2;
  if (lag && (!c_lag || R_lag < 1 || (long)R_lag * gamma > kMaxSchedN)) return DSPARK_EINVAL;
  if (sps_B0 > R || (long)sps_B0 + sps_len - 1 < (long)R * (1 + gamma)) return DSPARK_ERANGE;
  if (lag && (sps_B0 > R_lag || (long)sps_B0 + sps_len - 1 < (long)R_lag * (1 + gamma)))
    return DSPARK_ERANGE;
  const SchedWs w = carve_sched(ws, R, gamma);
  if (!ws || ws_bytes < w.bytes) return DSPARK_EWORKSPACE;

  const int N = R * gamma, Nl = lag ? R_lag * gamma : 0;
  const int nmax = N > Nl ? N : Nl;
  const int xw = rank_xw(nmax);
  const int xb = xw * kRankWaves;
  const SchedBatch b0{c,
                      R,
                      (N + xb - 1) / xb,
                      mode == DSPARK_SCHED_SYNC_BREAK
                          ? kEvalBreak
                          : (mode == DSPARK_SCHED_GLOBAL ? kEvalArgmax : kEvalNone),
                      false,
                      lag ? w.rank : nullptr,
                      lag ? w.tau : nullptr,
                      a};
  const SchedBatch b1{lag ? c_lag : c, lag ? R_lag : R, lag ? (Nl + xb - 1) / xb : 0,
                      kEvalArgmax, true, nullptr, nullptr, nullptr};
  const SchedOut out{(int)mode, ell, stats, w.epoch, w.pub};
  if (xw == 1)
    launch_schedule<1>(gamma, b0, b1, sps, sps_B0, nmax, out, dev_status, stream);
  else
    launch_schedule<2>(gamma, b0, b1, sps, sps_B0, nmax, out, dev_status, stream);
  return launch_status();
}

}  // extern "C"
