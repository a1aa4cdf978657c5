// host.h -- host-side helpers of the C ABI: argument checks, device properties, workspace
// carving.  No allocation, no synchronisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

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

// Device attributes are cached per device id in relaxed atomics: concurrent first calls
// may both query the runtime, and store the same value.
inline int cached_device_attribute(std::atomic<int> (&cache)[64], hipDeviceAttribute_t attr,
                                   int fallback) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fallback;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) v = fallback;
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// compute units of the current device
inline int device_cus() {
  static std::atomic<int> cache[64];
  return cached_device_attribute(cache, hipDeviceAttributeMultiprocessorCount, 256);
}

// Raises a kernel's dynamic-LDS ceiling to `bytes` on the current device, once per device
// (`done` is the kernel's own set of devices already raised).
inline void ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) ==
          hipSuccess &&
      bit)
    done.fetch_or(bit, std::memory_order_relaxed);
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
