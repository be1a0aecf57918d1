// Wavefront primitives for gfx950 (wave64) built on DPP lane moves.
//
// A DPP move is a VALU operand modifier: a few cycles, against the LDS
// round trip of ds_bpermute (what __shfl_* compiles to).  Reductions first
// combine the 16 lanes of each DPP row, then the four row results are read
// into scalar registers and combined there, so the result is wave-uniform.
#pragma once

#include "zha_common.hpp"

namespace zha {

// DPP controls (gfx9 encoding).
constexpr int kDppQpXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQpXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i inside each half row
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v), __float_as_uint(v)));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t old, uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)old, (uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
  __device__ __forceinline__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
  __device__ __forceinline__ uint64_t operator()(uint64_t a, uint64_t b) const {
    return a > b ? a : b;
  }
};
struct OpMin {
  __device__ __forceinline__ float operator()(float a, float b) const { return fminf(a, b); }
  __device__ __forceinline__ uint64_t operator()(uint64_t a, uint64_t b) const {
    return a < b ? a : b;
  }
};

// All-reduce inside aligned groups of W lanes (W = 2, 4, 8, 16, 32 or 64);
// every lane of a group gets the group's result.
template <int W, typename Op>
__device__ __forceinline__ float group_allreduce(float v, Op op) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  if constexpr (W == 8) {
    v = op(v, dpp_f32<kDppRowHalfMirror>(v));
  } else if constexpr (W >= 16) {
    v = op(v, dpp_f32<kDppRowRor8>(v));
    v = op(v, dpp_f32<kDppRowRor4>(v));
  }
  if constexpr (W >= 4) v = op(v, dpp_f32<kDppQpXor2>(v));
  v = op(v, dpp_f32<kDppQpXor1>(v));
  if constexpr (W >= 32) v = op(v, __shfl_xor(v, 16, kWave));
  if constexpr (W == 64) v = op(v, __shfl_xor(v, 32, kWave));
  return v;
}

// Row (16-lane) all-reduce of a 64-bit value.
template <typename Op>
__device__ __forceinline__ uint64_t row_allreduce_u64(uint64_t v, Op op) {
  v = op(v, dpp_u64<kDppRowRor8>(v, v));
  v = op(v, dpp_u64<kDppRowRor4>(v, v));
  v = op(v, dpp_u64<kDppQpXor2>(v, v));
  v = op(v, dpp_u64<kDppQpXor1>(v, v));
  return v;
}

// Whole-wave reductions; the result is uniform (scalar).
template <typename Op>
__device__ __forceinline__ float wave_allreduce_f32(float v, Op op) {
  v = group_allreduce<16>(v, op);
  return op(op(readlane_f32(v, 0), readlane_f32(v, 16)),
            op(readlane_f32(v, 32), readlane_f32(v, 48)));
}
template <typename Op>
__device__ __forceinline__ uint64_t wave_allreduce_u64(uint64_t v, Op op) {
  v = row_allreduce_u64(v, op);
  return op(op(readlane_u64(v, 0), readlane_u64(v, 16)),
            op(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// Whole-wave max of a float (uniform result), on order-preserving integer
// images so each step is one integer op: all-reduce inside each 16-lane row,
// then row_bcast15 / row_bcast31 carry the row results into lane 63.
__device__ __forceinline__ float wave_max_f32_bcast(float v) {
  uint32_t u = ord_f32(v);
  u = max(u, dpp_u32<kDppRowRor8>(u, u));
  u = max(u, dpp_u32<kDppRowRor4>(u, u));
  u = max(u, dpp_u32<kDppQpXor2>(u, u));
  u = max(u, dpp_u32<kDppQpXor1>(u, u));
  u = max(u, dpp_u32<kDppRowBcast15, 0xA>(u, u));
  u = max(u, dpp_u32<kDppRowBcast31, 0xC>(u, u));
  return unord_f32((uint32_t)__builtin_amdgcn_readlane((int)u, kWave - 1));
}

// Maximum of integer images over aligned groups of W lanes (W = 2 .. 64), DPP
// only.  For W <= 16 every lane of a group holds the group's maximum; for W = 32
// and 64, the row_bcast steps carry it into the group's last 16-lane row only.
template <int W>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t u) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  if constexpr (W == 8) {
    u = max(u, dpp_u32<kDppRowHalfMirror>(u, u));
  } else if constexpr (W >= 16) {
    u = max(u, dpp_u32<kDppRowRor8>(u, u));
    u = max(u, dpp_u32<kDppRowRor4>(u, u));
  }
  if constexpr (W >= 4) u = max(u, dpp_u32<kDppQpXor2>(u, u));
  u = max(u, dpp_u32<kDppQpXor1>(u, u));
  if constexpr (W >= 32) u = max(u, dpp_u32<kDppRowBcast15, 0xA>(u, u));
  if constexpr (W == 64) u = max(u, dpp_u32<kDppRowBcast31, 0xC>(u, u));
  return u;
}

// Whole-wave sum of a 64-bit value (uniform result), same pattern.
__device__ __forceinline__ uint64_t wave_sum_u64_bcast(uint64_t v) {
  v = row_allreduce_u64(v, OpAdd());
  v += dpp_u64<kDppRowBcast15, 0xA>(0ull, v);
  v += dpp_u64<kDppRowBcast31, 0xC>(0ull, v);
  return readlane_u64(v, kWave - 1);
}

// Inclusive prefix sum over the 64 lanes of a 64-bit value.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp_u64<kDppRowShr1>(0ull, v);
  v += dpp_u64<kDppRowShr2>(0ull, v);
  v += dpp_u64<kDppRowShr4>(0ull, v);
  v += dpp_u64<kDppRowShr8>(0ull, v);
  v += dpp_u64<kDppRowBcast15, 0xA>(0ull, v);
  v += dpp_u64<kDppRowBcast31, 0xC>(0ull, v);
  return v;
}

}  // namespace zha
