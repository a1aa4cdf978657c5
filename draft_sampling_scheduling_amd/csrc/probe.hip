// probe.hip -- a plain streaming read of device memory, measured beside the roofline: the
// rate at which a kernel that only reads (one 4-byte write per workgroup) draws bytes from
// HBM on this device, the practical ceiling against which the published peak is read.
// Not part of the method; bench.py reports it next to the sweep's achieved rate.
#include <hip/hip_ext.h>

#include "dev.h"
#include "host.h"

namespace dspark {

constexpr int kProbeThreads = 256;
constexpr int kProbeDepth = 16;  // 16-byte loads in flight per thread (64 KB per workgroup)

// Workgroup b reads its own contiguous slice (HBM serves one stream per workgroup faster
// than the whole grid striding through a shared window) and writes the XOR of every 32-bit
// word it read to sink[b], so that no load can be dropped.
__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const uint4* __restrict__ a,
                                                                   size_t n, uint32_t* sink) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n ? b0 + per : n;
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (size_t)(kProbeDepth - 1) * kProbeThreads < b1; i += kProbeDepth * kProbeThreads) {
    uint4 x[kProbeDepth];
#pragma unroll
    for (int u = 0; u < kProbeDepth; ++u) x[u] = a[i + (size_t)u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeDepth; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < b1; i += kProbeThreads) {
    const uint4 x = a[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
  __shared__ uint32_t red[kProbeThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / kWave; ++w) s ^= red[w];
    sink[blockIdx.x] = s;
  }
}

}  // namespace dspark

extern "C" int dspark_read_probe(const void* buf, size_t bytes, int grid, uint32_t* sink,
                                 hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  using namespace dspark;
  if (!buf || !sink || bytes % 16 != 0 || !aligned16(buf) || grid < 1 || grid > 65536)
    return DSPARK_EINVAL;
  if (!ev_begin != !ev_end) return DSPARK_EINVAL;
  const uint4* a = static_cast<const uint4*>(buf);
  const size_t n = bytes / 16;
  if (ev_begin)  // the dispatch itself timestamps its start and end
    hipExtLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, ev_begin,
                          ev_end, 0, a, n, sink);
  else
    read_probe_kernel<<<grid, kProbeThreads, 0, stream>>>(a, n, sink);
  return launch_status();
}
