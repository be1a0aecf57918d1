// Device-side helpers shared by the ZHA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zha.h"

namespace zha {

constexpr int kWave = 64;
constexpr int kMaxLevels = 16;

// ---------------------------------------------------------------------------
// Geometry as the kernels see it.  Byte offsets of every level inside one
// tree; trees of (b, kvh) pairs follow each other at `stride` bytes.
// ---------------------------------------------------------------------------
struct TreeLayout {
  int32_t L;
  int32_t R;
  int32_t C;
  int64_t stride;
  int64_t n[kMaxLevels + 1];     // n[l], l = 1..L (n[0] unused): nodes of the T cached tokens
  int64_t ncap[kMaxLevels + 1];  // rows of capacity per level (offsets and strides)
  int64_t khat[kMaxLevels + 1];  // byte offset of k_hat_l
  int64_t bhat[kMaxLevels + 1];  // byte offset of b_hat_l
};

// ---------------------------------------------------------------------------
// Storage types.  bf16 is kept as raw 16-bit patterns.
// ---------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// double -> bf16 in a single rounding step (nearest even).  A double rounded
// to float first and then to bf16 can land on the wrong neighbour; this
// rounds the 53-bit significand straight to bf16's 8 bits.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int e = (int)((u >> 52) & 0x7ff);
  const uint64_t frac = u & ((1ull << 52) - 1);
  if (e == 0x7ff) return (uint16_t)(sign | 0x7f80u | (frac ? 0x40u : 0u));
  if (e == 0) return (uint16_t)sign;  // |x| < 2^-1022: rounds to zero in bf16
  const int E = e - 1023;
  const uint64_t sig = frac | (1ull << 52);
  if (E >= -126) {  // bf16 normal range: keep 1 + 7 bits
    uint64_t q = sig >> 45;
    const uint64_t rem = sig & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rem > half || (rem == half && (q & 1))) ++q;
    int Eb = E + 127;
    if (q == (1ull << 8)) {
      q >>= 1;
      ++Eb;
    }
    if (Eb >= 255) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | ((uint32_t)Eb << 7) | (uint32_t)(q & 0x7f));
  }
  // bf16 subnormal range: multiples of 2^-133.
  const int shift = -81 - E;  // sig * 2^(E-52) / 2^-133 = sig >> shift
  if (shift >= 64) return (uint16_t)sign;
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  return (uint16_t)(sign | (uint32_t)q);  // q == 0x80 becomes the smallest normal
}

// 16-byte vector of storage elements widened to fp32.
template <typename T>
struct Vec;

template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
};

template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const uint4& v, float* out) {
    out[0] = bf16_lo(v.x);
    out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y);
    out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z);
    out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w);
    out[7] = bf16_hi(v.w);
  }
};

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const bf16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i].bits << 16);
}
__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(bf16_t* p, int64_t i, float v) {
  p[i].bits = f32_to_bf16(v);
}
__device__ __forceinline__ void store_elem64(float* p, int64_t i, double v) { p[i] = (float)v; }
__device__ __forceinline__ void store_elem64(bf16_t* p, int64_t i, double v) {
  p[i].bits = f64_to_bf16(v);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef ZHA_NT_LOADS
#define ZHA_NT_LOADS 1
#endif

// Streaming 16-byte load (data read once).
__device__ __forceinline__ uint4 ld16(const void* p) {
#if ZHA_NT_LOADS
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}
// 16-byte load through the caches (data likely reused).
__device__ __forceinline__ uint4 ld16c(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Raw buffer loads.  A buffer resource covers [base, base + bytes) with
// bytes < 2^31; a load whose offset lies past the end returns zeros and reads
// no memory, so a load whose lane has no row is issued unconditionally with
// offset kBufNone (every wait can then count exactly the loads after it).
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr uint32_t kBufNone = 0x80000000u;
__device__ __forceinline__ buf_t make_buf(const void* base, int64_t bytes) {
  // Fourth descriptor word for gfx9 raw buffers: 32-bit data format.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Streaming (non-temporal) 16-byte buffer load.
__device__ __forceinline__ uint4 bld16(buf_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, ZHA_NT_LOADS ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Cached 16-byte and 4-byte buffer loads.
__device__ __forceinline__ uint4 bld16c(buf_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float bld4c(buf_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// ---------------------------------------------------------------------------
// Reductions inside aligned lane groups of size W (power of two, <= 64).
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
template <int W>
__device__ __forceinline__ double group_sum64(double v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int W>
__device__ __forceinline__ double group_max64(double v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}


// Order-preserving map float -> uint32 (ascending floats give ascending keys).
__device__ __forceinline__ uint32_t ord_f32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace zha
