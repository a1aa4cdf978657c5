// dev.h -- device helpers shared by the DSpark kernels (gfx950, wave64).
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), the uniform/Gumbel mapping of the
// library's random convention, bf16 encoding, and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;
constexpr int kVB = 64;  // block of the two-level Gumbel-max sampler (consecutive ids)

// random streams (low nibble of counter word 3)
enum : uint32_t {
  kStreamDraftBlk = 0,
  kStreamDraftIn = 1,
  kStreamAccept = 2,
  kStreamResidBlk = 3,
  kStreamResidIn = 4,
  kStreamBonusBlk = 5,
  kStreamBonusIn = 6
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ----------------------------------------------------------------------------------------
// Philox4x32 with 10 rounds.  Round: with products P0 = 0xD2511F53 * w0 and
// P1 = 0xCD9E8D57 * w2 (64-bit), the block becomes
// (hi(P1) ^ w1 ^ k0, lo(P1), hi(P0) ^ w3 ^ k1, lo(P0)); the key is bumped by
// (0x9E3779B9, 0xBB67AE85) before every round after the first.
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox10(uint4 w, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * w.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * w.z;
    const uint4 n = make_uint4((uint32_t)(p1 >> 32) ^ w.y ^ k0, (uint32_t)p1,
                               (uint32_t)(p0 >> 32) ^ w.w ^ k1, (uint32_t)p0);
    w = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return w;
}

struct Rng {
  uint32_t k0, k1;  // key = seed
  uint32_t w3hi;    // cycle << 4
  __device__ __forceinline__ Rng(uint64_t seed, uint64_t cycle)
      : k0((uint32_t)seed), k1((uint32_t)(seed >> 32)), w3hi((uint32_t)(cycle << 4)) {}
  // the four words of counter (i4, r, k, cycle<<4 | stream)
  __device__ __forceinline__ uint4 block(uint32_t stream, uint32_t r, uint32_t k,
                                         uint32_t i4) const {
    return philox10(make_uint4(i4, r, k, w3hi | stream), k0, k1);
  }
  __device__ __forceinline__ uint32_t word(uint32_t stream, uint32_t r, uint32_t k,
                                           uint32_t i) const {
    const uint4 b = block(stream, r, k, i >> 2);
    const uint32_t s = i & 3u;
    return s == 0 ? b.x : (s == 1 ? b.y : (s == 2 ? b.z : b.w));
  }
};

__device__ __forceinline__ uint32_t pick_word(uint4 b, uint32_t s) {
  return s == 0 ? b.x : (s == 1 ? b.y : (s == 2 ? b.z : b.w));
}

// u = (2*(w >> 9) + 1) * 2^-24: odd multiples of 2^-24, exact in float, never 0 or 1
__device__ __forceinline__ float uniform_of(uint32_t w) {
  return (float)(2u * (w >> 9) + 1u) * 0x1p-24f;
}

// g = -ln(-ln u), branch-free.  -ln u is taken from the hardware log2 except when
// e = 1 - u (exact: u is an odd multiple of 2^-24) is below 2^-7, where the series
// e + e^2/2 + e^3/3 + e^4/4 keeps full relative accuracy for the largest noise values,
// which decide the argmax.
__device__ __forceinline__ float gumbel_of(uint32_t w) {
  constexpr float kLn2 = 0.69314718055994531f;
  const uint32_t k = w >> 9;
  const float u = (float)(2u * k + 1u) * 0x1p-24f;
  const float e = (float)(0xFFFFFFu - 2u * k) * 0x1p-24f;
  const float t_log = -__builtin_amdgcn_logf(u) * kLn2;
  const float t_ser = e * (1.0f + e * (0.5f + e * (0.333333343f + e * 0.25f)));
  const float t = (e < 0x1p-7f) ? t_ser : t_log;
  return -__builtin_amdgcn_logf(t) * kLn2;
}

// ----------------------------------------------------------------------------------------
// bf16
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) {
  return __uint_as_float(pair & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ----------------------------------------------------------------------------------------
// wave reductions (wave64), every lane ending with the result.  The partner values come
// from the cross-lane network rather than LDS permutes: DPP quad permutes (lanes 1 and 2
// apart), the DPP 8- and 16-lane mirrors (after the quad steps each lane holds its quad's
// result, so pairing lane i with 7 - i, then with 15 - i, joins disjoint groups), a swizzle
// for lanes 16 apart inside each half, and the 32-lane swap.  Each step combines a lane's
// value with its partner's under a commutative operation, so all lanes compute the same
// tree and hold bit-identical results.  Call with the whole wave active.
// ----------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t xlane_dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t xlane_swz16(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (0x10 << 10) | 0x1F);
}
// value of the partner lane at butterfly step STEP (0..4: 1, 2, mirror 8, mirror 16, 16)
template <int STEP>
__device__ __forceinline__ uint32_t xlane_partner(uint32_t x) {
  if (STEP == 0) return xlane_dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if (STEP == 1) return xlane_dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if (STEP == 2) return xlane_dpp<0x141>(x);  // row_half_mirror
  if (STEP == 3) return xlane_dpp<0x140>(x);  // row_mirror
  return xlane_swz16(x);                      // lane ^ 16 inside each half
}
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, __uint_as_float(xlane_partner<0>(__float_as_uint(v))));
  v = op(v, __uint_as_float(xlane_partner<1>(__float_as_uint(v))));
  v = op(v, __uint_as_float(xlane_partner<2>(__float_as_uint(v))));
  v = op(v, __uint_as_float(xlane_partner<3>(__float_as_uint(v))));
  v = op(v, __uint_as_float(xlane_partner<4>(__float_as_uint(v))));
  // the swap gives every lane the lower half's value and the upper half's, in that order
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// merge of two (max, sum of exp(l - max)) pairs; -inf maxima carry zero mass (branch-free)
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  const float ref = (mm == -INFINITY) ? 0.0f : mm;
  s = s * __expf(m - ref) + s2 * __expf(m2 - ref);
  m = mm;
}

// argmax with ties to the lower index, across the wave (the same network as wave_reduce;
// value and index travel together, and the order is total, so every lane ends alike)
__device__ __forceinline__ void wave_argmax(float& val, int& idx) {
  auto take = [&](float v2, int i2) {
    if (v2 > val || (v2 == val && i2 < idx)) {
      val = v2;
      idx = i2;
    }
  };
  take(__uint_as_float(xlane_partner<0>(__float_as_uint(val))), (int)xlane_partner<0>((uint32_t)idx));
  take(__uint_as_float(xlane_partner<1>(__float_as_uint(val))), (int)xlane_partner<1>((uint32_t)idx));
  take(__uint_as_float(xlane_partner<2>(__float_as_uint(val))), (int)xlane_partner<2>((uint32_t)idx));
  take(__uint_as_float(xlane_partner<3>(__float_as_uint(val))), (int)xlane_partner<3>((uint32_t)idx));
  take(__uint_as_float(xlane_partner<4>(__float_as_uint(val))), (int)xlane_partner<4>((uint32_t)idx));
  const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(val), __float_as_uint(val), false, false);
  const auto ri = __builtin_amdgcn_permlane32_swap((uint32_t)idx, (uint32_t)idx, false, false);
  val = __uint_as_float(rv[0]);
  idx = (int)ri[0];
  take(__uint_as_float(rv[1]), (int)ri[1]);
}

// plain fill (used instead of memset so that captured graphs hold only kernels)
static __global__ void __launch_bounds__(256) fill_kernel(float* p, size_t n, float v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__device__ __forceinline__ void raise_fault(int32_t* status, int32_t bit) {
  if (status) atomicOr(status, bit);
}

// ---------------------------------------------------------------------------------------
// element loads for the two operand types
// ---------------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) {
  return p[i];
}

// 8 consecutive elements (16 or 32 bytes, aligned)
template <class T>
__device__ __forceinline__ void ld8(const T* p, float (&o)[8]);
template <>
__device__ __forceinline__ void ld8<uint16_t>(const uint16_t* p, float (&o)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
  o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
}
template <>
__device__ __forceinline__ void ld8<float>(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}


// a token read from device data: out-of-range values raise the fault bit and read as 0
__device__ __forceinline__ int32_t checked_token(int32_t t, int V, int32_t* status) {
  if (t < 0 || t >= V) {
    raise_fault(status, 1 /* DSPARK_FAULT_TOKEN */);
    return 0;
  }
  return t;
}

}  // namespace dspark
