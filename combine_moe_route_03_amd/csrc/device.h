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
