// host.h -- host-side helpers of the C ABI: argument checks, device properties, workspace
// carving.  No allocation, no synchronisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

constexpr int kMaxGamma = 64;
constexpr int kMaxRanges = 1024;
constexpr int kMaxSchedN = 8192;  // R * gamma handled by the one-workgroup scheduler

inline bool rank_ok(int r) { return r == 16 || r == 32 || r == 64 || r == 128 || r == 256; }

inline bool dims_ok(int R, int gamma, int V, int r, int d) {
  return R >= 0 && gamma >= 1 && gamma <= kMaxGamma && V >= 8 && V % 8 == 0 && rank_ok(r) &&
         d >= 0 && d % 8 == 0;
}

// 16-byte alignment of the operands read with vector loads (null passes)
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// compute units of the current device (cached per device id)
inline int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev] = cus;
  return cus;
}

// bump allocator over the caller's workspace (256-byte aligned slices)
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return (off + 255) & ~(size_t)255; }
};

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

}  // namespace dspark
