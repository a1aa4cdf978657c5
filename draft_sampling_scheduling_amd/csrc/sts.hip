// sts.hip -- Sequential Temperature Scaling of the confidence head (DSpark digest page,
// Module D): per draft position k, left to right, the temperature T_k from a candidate grid
// whose scaled confidences sigma(z_k / T_k) make the running product
// P_k = prod_{j<=k} sigma(z_j / T_j) best calibrated against held-out acceptance outcomes
// (o = 1 when the accepted prefix reaches position k), measured by the expected calibration
// error over equal-width bins of [0, 1]:  ECE = sum_bins |sum_{n in bin} (o_n - P_n)| / N.
// The positions before k keep the temperatures already chosen; scaling by a positive T
// keeps each position's ranking of the samples.
//
// Per position three launches:
//   sts_bins   one pass over the samples: the running product of the earlier positions
//              (kept in the workspace, one double per sample), then for every grid entry
//              the sample's bin and its (o - P) in 2^-38 fixed point, added into per-
//              workgroup LDS bins with 64-bit LDS atomics; each workgroup writes its bins.
//   sts_reduce column sums of the per-workgroup bins (integers: exact, order-free).
//   sts_pick   per grid entry sum_b |bin sum|, the smallest wins (ties: earlier entry);
//              writes T_k and its ECE.
// Fixed point makes the bin sums exact and independent of launch shape and atomic order;
// each term is rounded once to 2^-38, far below the ECE differences the grid separates.
#include <hip/hip_runtime.h>
#include <cmath>
#include <stdint.h>

#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kStsThreads = 256;
constexpr int kStsMaxG = 128;
constexpr int kStsMaxBins = 256;
constexpr int kStsMaxCells = 4096;  // G * nbins: 32 KiB of int64 LDS bins
constexpr int kStsMaxN = 1 << 24;   // |bin sum| <= N * 2^38 < 2^63
constexpr int kStsMaxWG = 512;
constexpr double kStsScale = 0x1p38;

struct StsGrid {
  float v[kStsMaxG];
};

__device__ __forceinline__ double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

__global__ __launch_bounds__(kStsThreads) void sts_bins_kernel(
    int N, int gamma, int k, const float* __restrict__ z, const int32_t* __restrict__ n_acc,
    StsGrid grid, int G, int nbins, const float* __restrict__ T, double* __restrict__ pref,
    long long* __restrict__ partials) {
  __shared__ unsigned long long bins[kStsMaxCells];
  const int cells = G * nbins;
  for (int i = threadIdx.x; i < cells; i += kStsThreads) bins[i] = 0ull;
  __syncthreads();
  const double Tprev = k > 0 ? (double)T[k - 1] : 1.0;
  const double nb = (double)nbins;
  for (int n = blockIdx.x * kStsThreads + threadIdx.x; n < N; n += gridDim.x * kStsThreads) {
    const float* zn = z + (size_t)n * gamma;
    double p = 1.0;
    if (k > 0) {
      if (k > 1) p = pref[n];
      p = p * sigmoid_d((double)zn[k - 1] / Tprev);
      if (k + 1 < gamma) pref[n] = p;
    }
    const double zk = (double)zn[k];
    const double o = n_acc[n] > k ? 1.0 : 0.0;
    for (int g = 0; g < G; ++g) {
      const double P = p * sigmoid_d(zk / (double)grid.v[g]);
      const double f = P * nb;
      // floor into [0, nbins-1]; P = 1 (and a non-finite P) lands in the top bin
      const int b = f < nb - 1.0 ? (f > 0.0 ? (int)f : 0) : nbins - 1;
      const long long inc = (long long)rint((o - P) * kStsScale);
      atomicAdd(&bins[g * nbins + b], (unsigned long long)inc);
    }
  }
  __syncthreads();
  long long* out = partials + (size_t)blockIdx.x * cells;
  for (int i = threadIdx.x; i < cells; i += kStsThreads) out[i] = (long long)bins[i];
}

// one workgroup per 64 cells: lane = cell, the 16 waves split the rows (independent
// loads, several in flight per lane)
constexpr int kStsReduceThreads = 1024;

__global__ __launch_bounds__(kStsReduceThreads) void sts_reduce_kernel(
    int nwg, int cells, const long long* __restrict__ partials, long long* __restrict__ sums) {
  constexpr int kWaves = kStsReduceThreads / kWave;
  __shared__ unsigned long long part[kWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int cell = blockIdx.x * kWave + lane;
  unsigned long long acc = 0ull;
  if (cell < cells) {
#pragma unroll 8
    for (int w = wave; w < nwg; w += kWaves)
      acc += (unsigned long long)partials[(size_t)w * cells + cell];
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && cell < cells) {
    unsigned long long s = 0ull;
    for (int i = 0; i < kWaves; ++i) s += part[i][lane];
    sums[cell] = (long long)s;
  }
}

__global__ __launch_bounds__(kStsMaxG) void sts_pick_kernel(
    int N, int k, int G, int nbins, const long long* __restrict__ sums, StsGrid grid,
    float* __restrict__ T, double* __restrict__ ece) {
  __shared__ unsigned long long err[kStsMaxG];
  const int g = threadIdx.x;
  if (g < G) {
    unsigned long long e = 0ull;
    for (int b = 0; b < nbins; ++b) {
      const long long s = sums[g * nbins + b];
      e += (unsigned long long)(s < 0 ? -s : s);
    }
    err[g] = e;
  }
  __syncthreads();
  if (g == 0) {
    int best = 0;
    for (int i = 1; i < G; ++i)
      if (err[i] < err[best]) best = i;
    T[k] = grid.v[best];
    if (ece) ece[k] = (double)err[best] * (1.0 / kStsScale) / (double)N;
  }
}

struct StsWs {
  double* pref;
  long long* partials;
  long long* sums;
  size_t bytes;
};

inline int sts_groups(int N) {
  const int need = (N + kStsThreads - 1) / kStsThreads;
  return need < kStsMaxWG ? need : kStsMaxWG;
}

inline StsWs sts_carve(void* base, int N, int G, int nbins) {
  Carve cv(base);
  StsWs w;
  const size_t cells = (size_t)G * nbins;
  w.pref = cv.take<double>((size_t)N);
  w.partials = cv.take<long long>((size_t)sts_groups(N) * cells);
  w.sums = cv.take<long long>(cells);
  w.bytes = cv.bytes();
  return w;
}

inline bool sts_dims_ok(int N, int G, int nbins) {
  return N >= 1 && N <= kStsMaxN && G >= 1 && G <= kStsMaxG && nbins >= 1 &&
         nbins <= kStsMaxBins && G * nbins <= kStsMaxCells;
}

}  // namespace dspark

extern "C" {

size_t dspark_sts_workspace_bytes(int N, int G, int nbins) {
  using namespace dspark;
  if (!sts_dims_ok(N, G, nbins)) return 0;
  return sts_carve(nullptr, N, G, nbins).bytes;
}

int dspark_sts_fit(int N, int gamma, const float* z, const int32_t* n_acc, const float* grid,
                   int G, int nbins, float* T, double* ece, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  using namespace dspark;
  if (!sts_dims_ok(N, G, nbins) || gamma < 1 || gamma > kMaxGamma) return DSPARK_EINVAL;
  if (!z || !n_acc || !grid || !T || !ws) return DSPARK_EINVAL;
  StsGrid gv = {};
  for (int g = 0; g < G; ++g) {
    if (!(grid[g] > 0.0f) || !std::isfinite(grid[g])) return DSPARK_EINVAL;
    gv.v[g] = grid[g];
  }
  const StsWs w = sts_carve(ws, N, G, nbins);
  if (ws_bytes < w.bytes) return DSPARK_EWORKSPACE;
  const int nwg = sts_groups(N);
  const int cells = G * nbins;
  for (int k = 0; k < gamma; ++k) {
    sts_bins_kernel<<<nwg, kStsThreads, 0, stream>>>(N, gamma, k, z, n_acc, gv, G, nbins, T,
                                                    w.pref, w.partials);
    sts_reduce_kernel<<<(cells + kWave - 1) / kWave, kStsReduceThreads, 0, stream>>>(
        nwg, cells, w.partials, w.sums);
    sts_pick_kernel<<<1, kStsMaxG, 0, stream>>>(N, k, G, nbins, w.sums, gv, T, ece);
  }
  return launch_status();
}

}  // extern "C"
