// device.h -- small device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest, ties to even.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Order-preserving map of a float onto uint32 (larger float -> larger uint).
// -0 is folded onto +0 first so that the two compare equal, as IEEE says.
__device__ __forceinline__ uint32_t float_order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_key_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// ---- cross-lane moves without LDS round trips (DPP). Within each row of 16
// lanes: quad_perm [1,0,3,2] and [2,3,0,1] read lanes i^1 and i^2; once quads
// are uniform, row_half_mirror (lane i <- 7-i of its half-row) reads the other
// quad, and once half-rows are uniform, row_mirror (lane i <- 15-i) the other
// half-row. Rows are combined through scalar lane reads.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_move(uint64_t v) {
  return ((uint64_t)dpp_move<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_move<CTRL>((uint32_t)v);
}
template <int CTRL>
__device__ __forceinline__ int32_t dpp_move(int32_t v) {
  return (int32_t)dpp_move<CTRL>((uint32_t)v);
}
template <int CTRL>
__device__ __forceinline__ int64_t dpp_move(int64_t v) {
  return (int64_t)dpp_move<CTRL>((uint64_t)v);
}
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
  return __longlong_as_double((long long)dpp_move<CTRL>((uint64_t)__double_as_longlong(v)));
}
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int l) {
  return ((uint64_t)lane_value((uint32_t)(v >> 32), l) << 32) | lane_value((uint32_t)v, l);
}
__device__ __forceinline__ int32_t lane_value(int32_t v, int l) {
  return (int32_t)lane_value((uint32_t)v, l);
}
__device__ __forceinline__ int64_t lane_value(int64_t v, int l) {
  return (int64_t)lane_value((uint64_t)v, l);
}
__device__ __forceinline__ double lane_value(double v, int l) {
  return __longlong_as_double((long long)lane_value((uint64_t)__double_as_longlong(v), l));
}

// op-reduction over aligned groups of G lanes (G a power of two <= 64); every
// lane of a group ends with the same result. The whole wave must be active.
template <typename V, typename Op>
__device__ __forceinline__ V group_reduce(V v, int G, Op op) {
  if (G >= 2) v = op(v, dpp_move<kDppXor1>(v));
  if (G >= 4) v = op(v, dpp_move<kDppXor2>(v));
  if (G >= 8) v = op(v, dpp_move<kDppHalfMirror>(v));
  if (G >= 16) v = op(v, dpp_move<kDppMirror>(v));
  if (G >= 32) {
    const V lo = op(lane_value(v, 0), lane_value(v, 16));
    const V hi = op(lane_value(v, 32), lane_value(v, 48));
    v = (G == 64) ? op(lo, hi) : ((__lane_id() < 32) ? lo : hi);
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = __lane_id();
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// 16-byte vector as a native clang vector (the non-temporal builtins need one).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load/store: data touched once. On this
// path they keep large single-use streams from displacing each other in the
// caches; measured on gfx950 they speed up the cold gathers of the combine and
// the expert stream by 15-45%.
__device__ __forceinline__ v4u load_stream(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(v4u* p, v4u v) { __builtin_nontemporal_store(v, p); }

}  // namespace moe
