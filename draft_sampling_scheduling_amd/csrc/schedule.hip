// schedule.hip -- the hardware-aware prefix scheduler (digest page, Module E, Algorithm 1,
// and the production variants without the break and with the two-step lag).
//
// The whole scheduler is one workgroup (1024 threads) working in LDS:
//   1. prefix survival a_{q,j} = a_{q,j-1} * c_{q,j} in float, one request per thread;
//   2. 64-bit keys (~bits(a) << 32 | q*gamma + j-1) sorted ascending (bitonic), which is
//      descending a with ties broken by q, then j -- a is non-negative, so its bit pattern
//      orders like its value, and the j order keeps every request's admitted set a prefix;
//   3. an exact integer prefix sum of floor(a * 2^32): tau of every prefix of the order is
//      then independent of summation order, so the parallel search below decides exactly
//      as the sequential loop of Algorithm 1 would;
//   4. Theta_n = tau_n * SPS(R + n) in double for every n, and the admitted count n:
//      first non-improving n minus one (break), first maximiser (no break), or the
//      capacity of the lagged batch (two-step lag);
//   5. ell_q = number of q's entries among the first n.
#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kSchedThreads = 1024;

struct SchedShared {
  unsigned long long* key;  // [npad]
  unsigned long long* pre;  // [npad] inclusive prefix sums of the increments
};

__device__ __forceinline__ double theta_of(unsigned long long tau_fx, float sps) {
  return ((double)tau_fx * 0x1p-32) * (double)sps;
}

__device__ __forceinline__ unsigned long long incr_of_key(unsigned long long key) {
  const float a = __uint_as_float(~(uint32_t)(key >> 32));
  return (unsigned long long)((double)a * 4294967296.0);
}

// smallest power of two >= x (x >= 1)
__device__ __forceinline__ int pow2_ceil(int x) { return x <= 1 ? 1 : 1 << (32 - __clz(x - 1)); }

// steps 1-3 for one batch of confidences; returns the candidate count |E|.  *npad_io is the
// sorted length on entry (bitonic layout) and on return (the layout actually used).
//
// Each request's keys already ascend (a falls along j, ties keep j order), so when the
// padded layout fits, the order is R runs merged pairwise: round r merges runs of length
// P * 2^r, every key finding its place by one binary search in the partner run (keys are
// unique; the even run counts partner keys below it, the odd run those not above it, which
// also keeps the padding keys of the two runs apart).  Otherwise a bitonic sort.
__device__ int sched_sort_scan(int R, int gamma, const float* __restrict__ c, float* a_out,
                               int* npad_io, SchedShared sh, unsigned long long* red_u64,
                               int* red_i, int32_t* status) {
  (void)(R * gamma);
  const int P = pow2_ceil(gamma), Rp = pow2_ceil(R);
  const bool merge = (long)Rp * P <= *npad_io;  // both buffers hold *npad_io keys
  const int npad = merge ? Rp * P : *npad_io;
  *npad_io = npad;
  // merge layout: request q's run at [q * P, q * P + P) of the source buffer (sh.pre)
  unsigned long long* src = merge ? sh.pre : sh.key;
  for (int i = threadIdx.x; i < npad; i += kSchedThreads) src[i] = ~0ull;
  __syncthreads();
  for (int q = threadIdx.x; q < R; q += kSchedThreads) {
    float run = 1.0f;
    for (int j = 0; j < gamma; ++j) {
      float cj = c[(size_t)q * gamma + j];
      if (!(cj >= 0.0f && cj <= 1.0f)) {
        raise_fault(status, DSPARK_FAULT_CONF);
        cj = (cj > 1.0f) ? 1.0f : 0.0f;  // NaN and negatives -> 0
      }
      run = (j == 0) ? cj : __fmul_rn(run, cj);
      const int idx = q * gamma + j;
      if (a_out) a_out[idx] = run;
      src[merge ? q * P + j : idx] =
          (run > 0.0f) ? (((unsigned long long)(~__float_as_uint(run)) << 32) | (unsigned)idx)
                       : ~0ull;
    }
  }
  __syncthreads();

  if (merge) {
    unsigned long long* in = sh.pre;
    unsigned long long* out = sh.key;
    for (int L = P; L < npad; L <<= 1) {
      for (int i = threadIdx.x; i < npad; i += kSchedThreads) {
        const unsigned long long k = in[i];
        const int run0 = i & ~(2 * L - 1);  // first run of the pair
        const bool odd = (i & L) != 0;
        const int pos = i & (L - 1);
        const unsigned long long* other = in + run0 + (odd ? 0 : L);
        // number of partner keys below k (even run) or not above k (odd run)
        int lo = 0, len = L;
        while (len > 0) {
          const int half = len >> 1;
          const unsigned long long o = other[lo + half];
          if (odd ? (o <= k) : (o < k)) {
            lo += half + 1;
            len -= half + 1;
          } else {
            len = half;
          }
        }
        out[run0 + pos + lo] = k;
      }
      __syncthreads();
      unsigned long long* t = in;
      in = out;
      out = t;
    }
    if (in != sh.key) {  // the sorted keys belong in sh.key
      for (int i = threadIdx.x; i < npad; i += kSchedThreads) sh.key[i] = in[i];
      __syncthreads();
    }
  }

  // bitonic sort, ascending (when the merge layout does not fit)
  for (int k = 2; !merge && k <= npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < npad; i += kSchedThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = sh.key[i], y = sh.key[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            sh.key[i] = y;
            sh.key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // |E| = index of the first padding key
  if (threadIdx.x == 0) *red_i = npad;
  __syncthreads();
  for (int i = threadIdx.x; i < npad; i += kSchedThreads)
    if (sh.key[i] == ~0ull && (i == 0 || sh.key[i - 1] != ~0ull)) atomicMin(red_i, i);
  __syncthreads();
  const int nE = *red_i;

  // inclusive prefix sums of the increments: contiguous chunks per thread, then a scan of
  // the per-thread totals
  const int per = npad / kSchedThreads > 0 ? npad / kSchedThreads : 1;
  const int lo = threadIdx.x * per;
  unsigned long long run = 0;
  if (lo < npad) {
    for (int i = lo; i < lo + per; ++i) {
      run += (i < nE) ? incr_of_key(sh.key[i]) : 0ull;
      sh.pre[i] = run;
    }
  }
  red_u64[threadIdx.x] = (lo < npad) ? run : 0ull;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const unsigned long long v = (threadIdx.x >= off) ? red_u64[threadIdx.x - off] : 0ull;
    __syncthreads();
    red_u64[threadIdx.x] += v;
    __syncthreads();
  }
  const unsigned long long base = threadIdx.x > 0 ? red_u64[threadIdx.x - 1] : 0ull;
  if (lo < npad)
    for (int i = lo; i < lo + per; ++i) sh.pre[i] += base;
  __syncthreads();
  return nE;
}

__device__ __forceinline__ unsigned long long tau_at(int R, const SchedShared& sh, int n) {
  return ((unsigned long long)R << 32) + (n > 0 ? sh.pre[n - 1] : 0ull);
}

// step 4 without the break: smallest n in [0, nE] reaching the largest Theta_n
__device__ int sched_argmax(int R, int nE, const float* __restrict__ sps, int sps_B0,
                            const SchedShared& sh, double* red_d, int* red_i) {
  double best = -INFINITY;
  int bi = 0x7fffffff;
  for (int n = threadIdx.x; n <= nE; n += kSchedThreads) {
    const double t = theta_of(tau_at(R, sh, n), sps[R + n - sps_B0]);
    if (t > best) {  // n increases within a thread: strict keeps the smallest
      best = t;
      bi = n;
    }
  }
  red_d[threadIdx.x] = best;
  red_i[threadIdx.x] = bi;
  __syncthreads();
  for (int off = kSchedThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      const double t2 = red_d[threadIdx.x + off];
      const int i2 = red_i[threadIdx.x + off];
      const double t1 = red_d[threadIdx.x];
      const int i1 = red_i[threadIdx.x];
      if (t2 > t1 || (t2 == t1 && i2 < i1)) {
        red_d[threadIdx.x] = t2;
        red_i[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  const int n = red_i[0];
  __syncthreads();
  return n;
}

// step 4 with the break: (first n >= 1 with Theta_n <= Theta_{n-1}) - 1, or nE
__device__ int sched_first_drop(int R, int nE, const float* __restrict__ sps, int sps_B0,
                                const SchedShared& sh, int* red_i) {
  if (threadIdx.x == 0) *red_i = 0x7fffffff;
  __syncthreads();
  for (int n = 1 + threadIdx.x; n <= nE; n += kSchedThreads) {
    const double t1 = theta_of(tau_at(R, sh, n), sps[R + n - sps_B0]);
    const double t0 = theta_of(tau_at(R, sh, n - 1), sps[R + n - 1 - sps_B0]);
    if (!(t1 > t0)) atomicMin(red_i, n);
  }
  __syncthreads();
  const int first = *red_i;
  __syncthreads();
  return first == 0x7fffffff ? nE : first - 1;
}

__global__ void __launch_bounds__(kSchedThreads) schedule_kernel(
    int R, int gamma, const float* __restrict__ c, const float* __restrict__ c_lag, int R_lag,
    const float* __restrict__ sps, int sps_B0, int mode, int npad, int npad_lag, int32_t* ell,
    float* a_out, double* stats, int32_t* status) {
  extern __shared__ unsigned long long smem[];
  __shared__ unsigned long long red_u64[kSchedThreads];
  __shared__ double red_d[kSchedThreads];
  __shared__ int red_i[kSchedThreads];
  __shared__ int red_one;
  const int np = npad > npad_lag ? npad : npad_lag;
  SchedShared sh{smem, smem + np};

  int K = -1;  // admitted-count cap from the lagged batch
  if (mode == DSPARK_SCHED_ASYNC_LAG2) {
    int np_lag = npad_lag;
    const int nEl = sched_sort_scan(R_lag, gamma, c_lag, nullptr, &np_lag, sh, red_u64,
                                    &red_one, status);
    const int nl = sched_argmax(R_lag, nEl, sps, sps_B0, sh, red_d, red_i);
    const int cap = R_lag + nl;
    K = cap - R > 0 ? cap - R : 0;
    __syncthreads();
  }
  int np_cur = npad;
  const int nE = sched_sort_scan(R, gamma, c, a_out, &np_cur, sh, red_u64, &red_one, status);
  int n;
  if (mode == DSPARK_SCHED_SYNC_BREAK)
    n = sched_first_drop(R, nE, sps, sps_B0, sh, &red_one);
  else if (mode == DSPARK_SCHED_GLOBAL)
    n = sched_argmax(R, nE, sps, sps_B0, sh, red_d, red_i);
  else
    n = K < nE ? K : nE;

  const unsigned long long tau = tau_at(R, sh, n);
  __syncthreads();
  // count admitted entries per request (reuse the prefix array as int counters)
  int* cnt = reinterpret_cast<int*>(sh.pre);
  for (int q = threadIdx.x; q < R; q += kSchedThreads) cnt[q] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kSchedThreads)
    atomicAdd(&cnt[(int)(sh.key[i] & 0xffffffffull) / gamma], 1);
  __syncthreads();
  for (int q = threadIdx.x; q < R; q += kSchedThreads) ell[q] = cnt[q];
  if (threadIdx.x == 0 && stats) {
    const int B = R + n;
    stats[0] = (double)B;
    stats[1] = (double)tau * 0x1p-32;
    stats[2] = theta_of(tau, sps[B - sps_B0]);
    stats[3] = (double)n;
  }
}

static int pow2_at_least(int n) {
  int p = 2;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace dspark

extern "C" {

size_t dspark_schedule_workspace_bytes(int R, int gamma) {
  (void)R;
  (void)gamma;
  return 0;
}

int dspark_schedule(int R, int gamma, const float* c, const float* c_lag, int R_lag,
                    const float* sps, int sps_B0, int sps_len, dspark_sched_mode mode,
                    int32_t* ell, float* a, double* stats, int32_t* dev_status, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  using namespace dspark;
  (void)ws;
  (void)ws_bytes;
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
  const int npad = pow2_at_least(R * gamma);
  const int npad_lag = lag ? pow2_at_least(R_lag * gamma) : 2;
  const int np = npad > npad_lag ? npad : npad_lag;
  const size_t sh = (size_t)2 * np * sizeof(unsigned long long);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(schedule_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)(2 * kMaxSchedN * sizeof(unsigned long long)));
    attr_set = true;
  }
  schedule_kernel<<<1, kSchedThreads, sh, stream>>>(R, gamma, c, lag ? c_lag : nullptr,
                                                    lag ? R_lag : 0, sps, sps_B0, (int)mode,
                                                    npad, npad_lag, ell, a, stats, dev_status);
  return launch_status();
}

}  // extern "C"
