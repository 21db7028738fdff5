// route_token.h -- top-k gating of one token by a group of lanes (MoE systems
// survey, crad.ict.ac.cn, section 1.1, eq. (2): the k largest router logits,
// equal logits ordered by ascending expert id, and the softmax over those k).
// Shared by the routing kernels and the one-launch decode dispatch.
#pragma once

#include "device.h"

namespace moe {

// Top-k of token t by the G-lane group this lane belongs to (lane g of the
// group). Each logit becomes a 64-bit key: the order-preserving uint32 of the
// value above ~e, so the larger key is the larger logit and, on equal logits,
// the lower expert id; key 0 marks "empty or taken" (every finite float maps
// above it). Each of the k rounds takes the lane-local maximum and a DPP max
// over the group; the lane holding that key clears it. Lane g < k keeps pick g.
// The softmax over the k kept logits is evaluated in double (group sum by DPP,
// identical on every lane) and rounded once to fp32. Returns id -1 on lanes
// g >= k and for inactive tokens.
template <int V, bool kVec4>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int64_t t,
                                            bool active, int E, int k, int G, int g,
                                            int& pick_id, float& pick_w) {
  uint64_t key[V];
  const float* row = logits + t * (int64_t)E;
  auto make = [](float f, int e) -> uint64_t {
    return ((uint64_t)float_order_key(f) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
  };
  if constexpr (kVec4) {
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const int e0 = g * V + 4 * j;
      const bool ok = active && e0 < E;  // E % 4 == 0: the four are all in range or all out
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) f = *reinterpret_cast<const float4*>(row + e0);
      key[4 * j + 0] = ok ? make(f.x, e0 + 0) : 0ull;
      key[4 * j + 1] = ok ? make(f.y, e0 + 1) : 0ull;
      key[4 * j + 2] = ok ? make(f.z, e0 + 2) : 0ull;
      key[4 * j + 3] = ok ? make(f.w, e0 + 3) : 0ull;
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = g * V + v;
      key[v] = (active && e < E) ? make(row[e], e) : 0ull;
    }
  }

  const auto kmax = [](uint64_t x, uint64_t y) { return x > y ? x : y; };
  uint64_t top = 0, mine = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int v = 1; v < V; ++v) best = kmax(best, key[v]);
    const uint64_t gm = group_reduce(best, G, kmax);
    if (r == 0) top = gm;
    if (g == r) mine = gm;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (key[v] == gm) key[v] = 0ull;  // keys are unique: one slot of the group
  }

  const float vtop = order_key_float((uint32_t)(top >> 32));
  const float vmine = order_key_float((uint32_t)(mine >> 32));
  const double ex = (g < k) ? exp((double)vmine - (double)vtop) : 0.0;
  const double s = group_reduce(ex, G, [](double x, double y) { return x + y; });
  pick_id = (active && g < k) ? (int)(0xFFFFFFFFu - (uint32_t)mine) : -1;
  pick_w = (float)(ex / s);
}

}  // namespace moe
