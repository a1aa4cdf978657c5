// schedule.hip -- the hardware-aware prefix scheduler (digest page, Module E, Algorithm 1,
// and the production variants without the break and with the two-step lag).
//
// The whole scheduler is one workgroup (1024 threads) working in LDS:
//   1. prefix survival a_{q,j} = a_{q,j-1} * c_{q,j} in float, one request per thread;
//   2. 64-bit keys (~bits(a) << 32 | q*gamma + j-1) sorted ascending (bitonic, in registers
//      and shuffles up to a wave's span, through LDS beyond), which is
//      descending a with ties broken by q, then j -- a is non-negative, so its bit pattern
//      orders like its value, and the j order keeps every request's admitted set a prefix;
//   3. an exact integer prefix sum of floor(a * 2^32): tau of every prefix of the order is
//      then independent of summation order, so the parallel search below decides exactly
//      as the sequential loop of Algorithm 1 would;
//   4. Theta_n = tau_n * SPS(R + n) in double for every n, and the admitted count n:
//      first non-improving n minus one (break), first maximiser (no break), or the
//      capacity of the lagged batch (two-step lag);
//   5. ell_q = number of q's entries among the first n.
#include <type_traits>

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

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int d) {
  const int lo = __shfl_xor((int)(uint32_t)v, d, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), d, kWave);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// the key of lane ^ d for d < 32: a swizzle in xor mode (and-mask 31, xor-mask d) moves
// both halves without an address operand
template <int D>
__device__ __forceinline__ unsigned long long swz_xor_u64(unsigned long long v) {
  constexpr int kPat = (D << 10) | 0x1F;
  const int lo = __builtin_amdgcn_ds_swizzle((int)(uint32_t)v, kPat);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(uint32_t)(v >> 32), kPat);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// the key of lane ^ D for D = 1, 2: a quad permutation on the DPP network (no LDS pipe)
template <int D>
__device__ __forceinline__ unsigned long long dpp_xor_u64(unsigned long long v) {
  constexpr int kCtrl = D == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, 0xF, 0xF, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// compare-exchange seen from one side: the kept key is the smaller of (x, y) when keep_min,
// else the larger (one compare, one 64-bit select)
__device__ __forceinline__ unsigned long long cx_keep(unsigned long long x, unsigned long long y,
                                                      bool keep_min) {
  return ((y < x) == keep_min) ? y : x;
}

// Bitonic sort of npad keys (a power of two, npad <= 1024 * KP), ascending, starting at
// stage kstart (blocks of kstart / 2 already sorted, alternately ascending and descending).
// Thread t holds keys t*KP .. t*KP + KP-1 in registers: partners less than KP apart are in
// the same thread, less than 64*KP apart in the same wave (one shuffle per key), farther
// through LDS (two buffers used in turn, so each such step needs a single barrier).
// Threads past npad / KP hold nothing but join the barriers.
template <int KP>
__device__ void sched_bitonic(unsigned long long (&key)[KP], int npad, int kstart,
                              unsigned long long* buf0, unsigned long long* buf1) {
  const int t = threadIdx.x;
  const int i0 = t * KP;
  const bool active = i0 < npad;
  int which = 0;
  // one in-wave step at lane distance D (compile time), when the stage has it
  auto wave_step = [&](auto dc, int k) {
    constexpr int D = decltype(dc)::value;
    const int j = D * KP;
    if (j >= k) return;
    const bool keep_min = ((i0 & j) == 0) == ((i0 & k) == 0);
#pragma unroll
    for (int s = 0; s < KP; ++s) {
      const unsigned long long y = D == 32 ? shfl_xor_u64(key[s], 32)
                                   : (D <= 2 ? dpp_xor_u64<D>(key[s]) : swz_xor_u64<D>(key[s]));
      key[s] = cx_keep(key[s], y, keep_min);
    }
  };
  for (int k = kstart; k <= npad; k <<= 1) {
    // partners a wave or more apart: through LDS
    for (int j = k >> 1; j >= kWave * KP; j >>= 1) {
      unsigned long long* b = which ? buf1 : buf0;
      if (active)
#pragma unroll
        for (int s = 0; s < KP; ++s) b[i0 + s] = key[s];
      __syncthreads();
      const bool keep_min = ((i0 & j) == 0) == ((i0 & k) == 0);
      if (active)
#pragma unroll
        for (int s = 0; s < KP; ++s) key[s] = cx_keep(key[s], b[(i0 + s) ^ j], keep_min);
      which ^= 1;
    }
    // partners in the same wave (j >= KP and k > j lie above the slot bits, so one
    // direction serves all KP keys)
    wave_step(std::integral_constant<int, 32>{}, k);
    wave_step(std::integral_constant<int, 16>{}, k);
    wave_step(std::integral_constant<int, 8>{}, k);
    wave_step(std::integral_constant<int, 4>{}, k);
    wave_step(std::integral_constant<int, 2>{}, k);
    wave_step(std::integral_constant<int, 1>{}, k);
    // partners in the same thread
#pragma unroll
    for (int j = KP / 2; j > 0; j >>= 1) {
      if (j >= k) continue;
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        const int p = s ^ j;
        if (p > s) {
          const bool up = ((i0 + s) & k) == 0;
          const unsigned long long x = key[s], y = key[p];
          const bool sw = (x > y) == up;
          key[s] = sw ? y : x;
          key[p] = sw ? x : y;
        }
      }
    }
  }
}

template <int KP>
__device__ void sched_sort_lds(int npad, int kstart, SchedShared sh) {
  unsigned long long key[KP];
  const int t = threadIdx.x;
  const bool active = t * KP < npad;
#pragma unroll
  for (int s = 0; s < KP; ++s) key[s] = active ? sh.key[t * KP + s] : ~0ull;
  __syncthreads();  // every key is in registers before the buffers are reused
  sched_bitonic<KP>(key, npad, kstart, sh.pre, sh.key);
  __syncthreads();
  if (active)
#pragma unroll
    for (int s = 0; s < KP; ++s) sh.key[t * KP + s] = key[s];
  __syncthreads();
}

// inclusive scan of v over the workgroup (wave scans, then the wave totals)
__device__ __forceinline__ unsigned long long block_scan_u64(unsigned long long v,
                                                             unsigned long long* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int lo = __shfl_up((int)(uint32_t)v, o, kWave);
    const int hi = __shfl_up((int)(uint32_t)(v >> 32), o, kWave);
    const unsigned long long up = ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
    if (lane >= o) v += up;
  }
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    unsigned long long x = lane < kSchedThreads / kWave ? wsum[lane] : 0ull;
#pragma unroll
    for (int o = 1; o < kSchedThreads / kWave; o <<= 1) {
      const int lo = __shfl_up((int)(uint32_t)x, o, kWave);
      const int hi = __shfl_up((int)(uint32_t)(x >> 32), o, kWave);
      const unsigned long long up = ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
      if (lane >= o) x += up;
    }
    if (lane < kSchedThreads / kWave) wsum[lane] = x;
  }
  __syncthreads();
  const unsigned long long base = wave > 0 ? wsum[wave - 1] : 0ull;
  __syncthreads();  // wsum is reused by the next scan
  return v + base;
}

// steps 1-3 for one batch of confidences; returns the candidate count |E|.  *npad_io is the
// sorted length on entry (the padded layout) and on return (the layout actually used).
//
// Each request's keys already ascend (a falls along j, ties keep j order).  When the padded
// run layout fits, request q's keys sit at [q * P, q * P + P) with the odd runs reversed,
// which is the state a bitonic sort reaches after its stage P, so the sort starts at 2P;
// otherwise the keys sit at q*gamma + j - 1 and the sort starts from pairs.
__device__ int sched_sort_scan(int R, int gamma, const float* __restrict__ c, float* a_out,
                               int* npad_io, SchedShared sh, unsigned long long* red_u64,
                               int* red_i, int32_t* status) {
  const int P = pow2_ceil(gamma), Rp = pow2_ceil(R);
  const bool runs = (long)Rp * P <= *npad_io;
  const int npad = runs ? Rp * P : *npad_io;
  *npad_io = npad;
  for (int i = threadIdx.x; i < npad; i += kSchedThreads) sh.key[i] = ~0ull;
  __syncthreads();
  for (int q = threadIdx.x; q < R; q += kSchedThreads) {
    const float* cq = c + (size_t)q * gamma;
    float run = 1.0f;
    for (int j0 = 0; j0 < gamma; j0 += 8) {
      float cv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) cv[u] = cq[j0 + u < gamma ? j0 + u : gamma - 1];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j >= gamma) break;
        float cj = cv[u];
        if (!(cj >= 0.0f && cj <= 1.0f)) {
          raise_fault(status, DSPARK_FAULT_CONF);
          cj = (cj > 1.0f) ? 1.0f : 0.0f;  // NaN and negatives -> 0
        }
        run = (j == 0) ? cj : __fmul_rn(run, cj);
        const int idx = q * gamma + j;
        if (a_out) a_out[idx] = run;
        const int pos = runs ? q * P + ((q & 1) ? P - 1 - j : j) : idx;
        sh.key[pos] = (run > 0.0f)
                          ? (((unsigned long long)(~__float_as_uint(run)) << 32) | (unsigned)idx)
                          : ~0ull;
      }
    }
  }
  __syncthreads();
  const int kstart = runs ? 2 * P : 2;
  if (npad <= 2048)
    sched_sort_lds<2>(npad, kstart, sh);
  else if (npad <= 4096)
    sched_sort_lds<4>(npad, kstart, sh);
  else
    sched_sort_lds<8>(npad, kstart, sh);

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
  const unsigned long long incl = block_scan_u64(lo < npad ? run : 0ull, red_u64);
  const unsigned long long base = incl - (lo < npad ? run : 0ull);
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
  // wave, then workgroup: the largest Theta, ties to the smaller n
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double t2 = __shfl_xor(best, o, kWave);
    const int i2 = __shfl_xor(bi, o, kWave);
    if (t2 > best || (t2 == best && i2 < bi)) {
      best = t2;
      bi = i2;
    }
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) {
    red_d[wave] = best;
    red_i[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kSchedThreads / kWave; ++w)
      if (red_d[w] > best || (red_d[w] == best && red_i[w] < bi)) {
        best = red_d[w];
        bi = red_i[w];
      }
    red_i[0] = bi;
  }
  __syncthreads();
  const int n = red_i[0];
  __syncthreads();
  return n;
}

// step 4 with the break: (first n >= 1 with Theta_n <= Theta_{n-1}) - 1, or nE
__device__ int sched_first_drop(int R, int nE, const float* __restrict__ sps, int sps_B0,
                                const SchedShared& sh, int* red_i) {
  if (threadIdx.x == 0) *red_i = 0x7fffffff;
  __syncthreads();
  int first = 0x7fffffff;  // this thread's first drop (n increases within a thread)
  for (int n = 1 + threadIdx.x; n <= nE; n += kSchedThreads) {
    const double t1 = theta_of(tau_at(R, sh, n), sps[R + n - sps_B0]);
    const double t0 = theta_of(tau_at(R, sh, n - 1), sps[R + n - 1 - sps_B0]);
    if (!(t1 > t0)) {
      first = n;
      break;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0 && first != 0x7fffffff) atomicMin(red_i, first);
  __syncthreads();
  const int f = *red_i;
  __syncthreads();
  return f == 0x7fffffff ? nE : f - 1;
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
  static std::atomic<uint64_t> lds_raised{0};
  ensure_dynamic_lds(reinterpret_cast<const void*>(schedule_kernel),
                     (int)(2 * kMaxSchedN * sizeof(unsigned long long)), lds_raised);
  schedule_kernel<<<1, kSchedThreads, sh, stream>>>(R, gamma, c, lag ? c_lag : nullptr,
                                                    lag ? R_lag : 0, sps, sps_B0, (int)mode,
                                                    npad, npad_lag, ell, a, stats, dev_status);
  return launch_status();
}

}  // extern "C"
