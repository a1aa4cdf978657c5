// layout.hip -- the one re-layout a caller makes before the hot path: the low-rank output
// factor W2 in R^{r x V} of the Markov head (digest, Module B eq. (5)), stored as the pages
// write it ([r][V], row i = coordinate i over the vocabulary), becomes W2t [V][r], the
// layout the vocabulary sweeps read (a 32-id tile of W2t is one contiguous run of
// 32 * r elements).  Done once per weight load.
#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kTrTile = 64;  // 64 x 64 element tiles through LDS

// one workgroup per (64-id, 64-coordinate) tile: coalesced reads along V, coalesced writes
// along r; the LDS row pitch of 65 elements keeps the transposed reads on distinct banks
template <class T>
__global__ void __launch_bounds__(256) w2_transpose_kernel(int V, int r, const T* __restrict__ W2,
                                                           T* __restrict__ W2t) {
  __shared__ T tile[kTrTile][kTrTile + 1];
  const int v0 = blockIdx.x * kTrTile, i0 = blockIdx.y * kTrTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4 threads
  for (int ii = ty; ii < kTrTile; ii += 4) {
    const int i = i0 + ii, v = v0 + tx;
    if (i < r && v < V) tile[ii][tx] = W2[(size_t)i * V + v];
  }
  __syncthreads();
  for (int vv = ty; vv < kTrTile; vv += 4) {
    const int v = v0 + vv, i = i0 + tx;
    if (i < r && v < V) W2t[(size_t)v * r + i] = tile[tx][vv];
  }
}

}  // namespace dspark

extern "C" int dspark_w2_relayout(int V, int r, dspark_dtype dt, const void* W2, void* W2t,
                                  hipStream_t stream) {
  using namespace dspark;
  if (V < 8 || V % 8 != 0 || !rank_ok(r) || (dt != DSPARK_F32 && dt != DSPARK_BF16))
    return DSPARK_EINVAL;
  if (!W2 || !W2t || W2 == W2t) return DSPARK_EINVAL;
  const dim3 grid((V + kTrTile - 1) / kTrTile, (r + kTrTile - 1) / kTrTile);
  if (dt == DSPARK_BF16)
    w2_transpose_kernel<uint16_t><<<grid, 256, 0, stream>>>(
        V, r, static_cast<const uint16_t*>(W2), static_cast<uint16_t*>(W2t));
  else
    w2_transpose_kernel<float><<<grid, 256, 0, stream>>>(V, r, static_cast<const float*>(W2),
                                                         static_cast<float*>(W2t));
  return launch_status();
}
