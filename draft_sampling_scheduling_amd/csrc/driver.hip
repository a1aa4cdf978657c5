// driver.hip -- multi-cycle decode on a toy chain (DSpark digest page, overall cycle;
// explainer, section 06), with the diagnostics the pages report: per-position conditional
// acceptance, the mean verified length, and the fixed-length and static-threshold
// baselines beside the scheduler's modes.
//
// The target is a bigram model (its logits after token t are row t of Tb) and the parallel
// backbone a table (U_k, h_k for anchor a are rows (a, k-1) of Ub, Hb).  One cycle:
//   gather     U, h from the anchors' table rows
//   draft      dspark_draft_markov (gamma sweeps + combines)
//   lengths    dspark_schedule (Algorithm 1 and its production variants), or the policy
//              kernel (every position, or the positions whose prefix survival is at least a
//              threshold)
//   gather     the target rows Tb[anchor], Tb[x_1], ..., Tb[x_gamma]
//   verify     dspark_verify
//   account    append the emitted tokens, move the anchor to the last one, count
// All on the caller's stream; the host only enqueues.
#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kGatherThreads = 256;
constexpr int kAccountThreads = 1024;

// rows of a table into per-request rows: dst[q][k] (row_len elements of esz bytes) =
// table[key(q)][k] for k < nk; 16-byte chunks
__global__ void __launch_bounds__(kGatherThreads) gather_anchor_rows_kernel(
    int R, int nk, size_t row_chunks, const uint4* __restrict__ table,
    const int32_t* __restrict__ anchor, int V, uint4* __restrict__ dst, int32_t* status) {
  const size_t per_req = (size_t)nk * row_chunks;
  const size_t total = (size_t)R * per_req;
  for (size_t i = (size_t)blockIdx.x * kGatherThreads + threadIdx.x; i < total;
       i += (size_t)gridDim.x * kGatherThreads) {
    const int q = (int)(i / per_req);
    const size_t rest = i - (size_t)q * per_req;
    int32_t a = anchor[q];
    if (a < 0 || a >= V) {
      raise_fault(status, DSPARK_FAULT_TOKEN);
      a = 0;
    }
    dst[i] = table[(size_t)a * per_req + rest];
  }
}

// target rows: dst[q][j] = Tb[prev_j], prev_0 = anchor, prev_j = x_j (j = 1..gamma)
__global__ void __launch_bounds__(kGatherThreads) gather_target_rows_kernel(
    int R, int gamma, size_t row_chunks, const uint4* __restrict__ Tb,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ x, int V,
    uint4* __restrict__ dst, int32_t* status) {
  const size_t per_req = (size_t)(gamma + 1) * row_chunks;
  const size_t total = (size_t)R * per_req;
  for (size_t i = (size_t)blockIdx.x * kGatherThreads + threadIdx.x; i < total;
       i += (size_t)gridDim.x * kGatherThreads) {
    const int q = (int)(i / per_req);
    const size_t rest = i - (size_t)q * per_req;
    const int j = (int)(rest / row_chunks);
    int32_t t = j == 0 ? anchor[q] : x[(size_t)q * gamma + j - 1];
    if (t < 0 || t >= V) {
      raise_fault(status, DSPARK_FAULT_TOKEN);
      t = 0;
    }
    dst[i] = Tb[(size_t)t * row_chunks + (rest - (size_t)j * row_chunks)];
  }
}

// lengths without the scheduler: every position (threshold <= 0 reaches them all), or the
// leading positions whose prefix survival a_j = c_1 ... c_j (fp32, left to right) is at
// least the threshold
__global__ void __launch_bounds__(256) policy_lengths_kernel(int R, int gamma,
                                                             const float* __restrict__ c,
                                                             int fixed, float threshold,
                                                             int32_t* __restrict__ ell) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= R) return;
  if (fixed) {
    ell[q] = gamma;
    return;
  }
  float run = 1.0f;
  int l = 0;
  for (int j = 1; j <= gamma; ++j) {
    const float cj = c[(size_t)q * gamma + j - 1];
    run = j == 1 ? cj : __fmul_rn(run, cj);
    if (run >= threshold && l == j - 1) l = j;
  }
  ell[q] = l;
}

// start state: anchors, empty sequences, zero counters (kernels, not memsets, so that a
// captured graph holds kernels only)
__global__ void __launch_bounds__(256) decode_init_kernel(int R, int gamma, size_t ntok,
                                                          const int32_t* __restrict__ x0,
                                                          int32_t* anchor, int32_t* tokens,
                                                          int32_t* n_emitted, long long* stats) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t t = i; t < ntok; t += stride) tokens[t] = -1;
  if (i < (size_t)R) {
    anchor[i] = x0[i];
    n_emitted[i] = 0;
  }
  if (i < (size_t)(2 * gamma + 3)) stats[i] = 0;
}

// one workgroup: per request append y[0..n_acc], move the anchor, count into LDS; then
// the counters join the running totals (only this kernel writes them, in stream order)
__global__ void __launch_bounds__(kAccountThreads) decode_account_kernel(
    int R, int gamma, int maxlen, const int32_t* __restrict__ ell,
    const int32_t* __restrict__ n_acc, const int32_t* __restrict__ y, int32_t* anchor,
    int32_t* tokens, int32_t* n_emitted, long long* stats) {
  __shared__ int cnt[2 * kMaxGamma + 3];
  for (int i = threadIdx.x; i < 2 * gamma + 3; i += kAccountThreads) cnt[i] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < R; q += kAccountThreads) {
    int l = ell[q];
    l = l < 0 ? 0 : (l > gamma ? gamma : l);
    int na = n_acc[q];
    na = na < 0 ? 0 : (na > l ? l : na);
    for (int k = 1; k <= l; ++k) {
      if (na >= k - 1) atomicAdd(&cnt[k - 1], 1);
      if (na >= k) atomicAdd(&cnt[gamma + k - 1], 1);
    }
    atomicAdd(&cnt[2 * gamma], l);
    atomicAdd(&cnt[2 * gamma + 1], na + 1);
    atomicAdd(&cnt[2 * gamma + 2], 1);
    const int32_t* yq = y + (size_t)q * (gamma + 1);
    const int base = n_emitted[q];
    for (int i = 0; i <= na; ++i)
      if (base + i < maxlen) tokens[(size_t)q * maxlen + base + i] = yq[i];
    n_emitted[q] = base + na + 1;
    anchor[q] = yq[na];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * gamma + 3; i += kAccountThreads) stats[i] += cnt[i];
}

struct DecodeWs {
  void* U;
  void* h;
  void* tg;
  void* brows;
  int32_t *anchor, *x, *ell, *n_acc, *y;
  float* c[3];
  float *lse, *logit_x, *c_star;
  void* dws;
  size_t dws_bytes;
  void* vws;
  size_t vws_bytes;
  void* sws;
  size_t sws_bytes;
  size_t bytes;
};

inline DecodeWs decode_carve(void* base, int R, int gamma, int V, int r, int d, size_t esz) {
  Carve cv(base);
  DecodeWs w{};
  const size_t RG = (size_t)R * gamma;
  w.U = cv.take<char>(esz * RG * V);
  w.h = cv.take<char>(esz * RG * (size_t)(d > 0 ? d : 1));
  w.tg = cv.take<char>(esz * (size_t)R * (gamma + 1) * V);
  w.brows = cv.take<char>(esz * RG * r);
  w.anchor = cv.take<int32_t>(R);
  w.x = cv.take<int32_t>(RG);
  w.ell = cv.take<int32_t>(R);
  w.n_acc = cv.take<int32_t>(R);
  w.y = cv.take<int32_t>((size_t)R * (gamma + 1));
  for (int i = 0; i < 3; ++i) w.c[i] = cv.take<float>(RG);
  w.lse = cv.take<float>(RG);
  w.logit_x = cv.take<float>(RG);
  w.c_star = cv.take<float>(RG);
  w.dws_bytes = dspark_draft_workspace_bytes(R, gamma, V, r, d);
  w.dws = cv.take<char>(w.dws_bytes);
  w.vws_bytes = dspark_verify_workspace_bytes(R, gamma, V, r);
  w.vws = cv.take<char>(w.vws_bytes);
  w.sws_bytes = dspark_schedule_workspace_bytes(R, gamma);
  w.sws = cv.take<char>(w.sws_bytes);
  w.bytes = cv.bytes();
  return w;
}

inline int grid_for(size_t n, int threads) {
  const size_t g = (n + threads - 1) / threads;
  return (int)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

}  // namespace dspark

extern "C" {

size_t dspark_decode_workspace_bytes(int R, int gamma, int V, int r, int d, dspark_dtype dt) {
  using namespace dspark;
  if (R < 1 || !dims_ok(R, gamma, V, r, d) || (dt != DSPARK_BF16 && dt != DSPARK_F32)) return 0;
  if (dspark_draft_workspace_bytes(R, gamma, V, r, d) == 0) return 0;
  return decode_carve(nullptr, R, gamma, V, r, d, dt == DSPARK_BF16 ? 2 : 4).bytes;
}

int dspark_decode_run(int R, int gamma, int V, int r, int d, dspark_dtype dt, int ncycles,
                      const void* Ub, const void* Hb, const void* W1, const void* W2t,
                      const float* w, const float* temps, const void* Tb, const int32_t* x0,
                      dspark_decode_policy policy, float threshold, const float* sps,
                      int sps_B0, int sps_len, uint64_t seed, int32_t* tokens,
                      int32_t* n_emitted, int64_t* stats, int32_t* dev_status, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  using namespace dspark;
  if (R < 1 || !dims_ok(R, gamma, V, r, d) || ncycles < 0) return DSPARK_EINVAL;
  if (dt != DSPARK_BF16 && dt != DSPARK_F32) return DSPARK_EINVAL;
  if ((long)ncycles * (gamma + 1) > 0x7fffffffL / (R > 0 ? R : 1)) return DSPARK_EINVAL;
  if ((uint64_t)ncycles > (1ull << 28)) return DSPARK_EINVAL;
  if (dt == DSPARK_BF16 && (uint64_t)R * (gamma + 1) * V * 2 >= ((uint64_t)1 << 32))
    return DSPARK_EINVAL;
  if (policy < DSPARK_DECODE_SYNC_BREAK || policy > DSPARK_DECODE_THRESHOLD) return DSPARK_EINVAL;
  if (!Ub || !W1 || !W2t || !w || !Tb || !x0 || !n_emitted || !stats || !ws) return DSPARK_EINVAL;
  if (ncycles > 0 && !tokens) return DSPARK_EINVAL;  // empty when there are no cycles
  if (d > 0 && !Hb) return DSPARK_EINVAL;
  if (!aligned16(Ub) || !aligned16(Hb) || !aligned16(Tb)) return DSPARK_EINVAL;
  const bool scheduled = policy <= DSPARK_DECODE_ASYNC_LAG2;
  if (scheduled) {
    if (!sps || sps_len < 1) return DSPARK_EINVAL;
    if (sps_B0 > R || (long)sps_B0 + sps_len - 1 < (long)R * (1 + gamma)) return DSPARK_ERANGE;
    if ((long)R * gamma > kMaxSchedN) return DSPARK_EINVAL;
  }
  const size_t esz = dt == DSPARK_BF16 ? 2 : 4;
  const DecodeWs wl = decode_carve(ws, R, gamma, V, r, d, esz);
  if (wl.dws_bytes == 0 || ws_bytes < wl.bytes) return DSPARK_EWORKSPACE;
  const int maxlen = ncycles * (gamma + 1);
  const size_t ntok = (size_t)R * maxlen;

  size_t ninit = ntok > (size_t)R ? ntok : (size_t)R;
  if (ninit < (size_t)(2 * gamma + 3)) ninit = (size_t)(2 * gamma + 3);
  decode_init_kernel<<<grid_for(ninit, 256), 256, 0, stream>>>(
      R, gamma, ntok, x0, wl.anchor, tokens, n_emitted, reinterpret_cast<long long*>(stats));
  int rc = launch_status();
  const size_t u_chunks = (size_t)V * esz / 16, h_chunks = (size_t)d * esz / 16;
  for (int cyc = 0; cyc < ncycles && rc == DSPARK_OK; ++cyc) {
    gather_anchor_rows_kernel<<<grid_for((size_t)R * gamma * u_chunks, kGatherThreads),
                                kGatherThreads, 0, stream>>>(
        R, gamma, u_chunks, static_cast<const uint4*>(Ub), wl.anchor, V,
        static_cast<uint4*>(wl.U), dev_status);
    if (d > 0)
      gather_anchor_rows_kernel<<<grid_for((size_t)R * gamma * h_chunks, kGatherThreads),
                                  kGatherThreads, 0, stream>>>(
          R, gamma, h_chunks, static_cast<const uint4*>(Hb), wl.anchor, V,
          static_cast<uint4*>(wl.h), dev_status);
    float* ccur = wl.c[cyc % 3];
    rc = dspark_draft_markov(R, gamma, V, r, d, dt, wl.U, d > 0 ? wl.h : nullptr, W1, W2t, w,
                             temps, wl.anchor, seed, (uint64_t)cyc, wl.x, ccur, nullptr, wl.lse,
                             wl.logit_x, wl.brows, dev_status, wl.dws, wl.dws_bytes, stream);
    if (rc != DSPARK_OK) break;
    if (scheduled) {
      const bool lag = policy == DSPARK_DECODE_ASYNC_LAG2 && cyc >= 2;
      const dspark_sched_mode mode =
          lag ? DSPARK_SCHED_ASYNC_LAG2
              : (policy == DSPARK_DECODE_SYNC_BREAK ? DSPARK_SCHED_SYNC_BREAK : DSPARK_SCHED_GLOBAL);
      rc = dspark_schedule(R, gamma, ccur, lag ? wl.c[(cyc - 2) % 3] : nullptr, lag ? R : 0, sps,
                           sps_B0, sps_len, mode, wl.ell, nullptr, nullptr, dev_status, wl.sws,
                           wl.sws_bytes, stream);
      if (rc != DSPARK_OK) break;
    } else {
      policy_lengths_kernel<<<(R + 255) / 256, 256, 0, stream>>>(
          R, gamma, ccur, policy == DSPARK_DECODE_FIXED ? 1 : 0, threshold, wl.ell);
    }
    gather_target_rows_kernel<<<grid_for((size_t)R * (gamma + 1) * u_chunks, kGatherThreads),
                                kGatherThreads, 0, stream>>>(
        R, gamma, u_chunks, static_cast<const uint4*>(Tb), wl.anchor, wl.x, V,
        static_cast<uint4*>(wl.tg), dev_status);
    rc = dspark_verify(R, gamma, V, r, dt, wl.tg, wl.U, W2t, wl.brows, dt, wl.x, wl.lse,
                       wl.logit_x, wl.ell, seed, (uint64_t)cyc, wl.n_acc, wl.y, wl.c_star,
                       nullptr, dev_status, wl.vws, wl.vws_bytes, stream);
    if (rc != DSPARK_OK) break;
    decode_account_kernel<<<1, kAccountThreads, 0, stream>>>(
        R, gamma, maxlen, wl.ell, wl.n_acc, wl.y, wl.anchor, tokens, n_emitted,
        reinterpret_cast<long long*>(stats));
    rc = launch_status();
  }
  return rc;
}

}  // extern "C"
