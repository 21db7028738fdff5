// route.hip -- top-k gating on gfx950: per token, the k largest router logits
// (equal logits ordered by ascending expert id) and the softmax over those k
// (MoE systems survey, crad.ict.ac.cn, section 1.1, eq. (2): the non-kept
// logits act as -inf, so only the k kept ones enter the softmax).
//
// One aligned group of G = 2^glog lanes of a wave64 handles one token. Lane g
// holds V consecutive logits (experts g*V .. g*V+V-1) as order-preserving
// uint32 keys. Each of the k rounds takes the lane-local maximum (first index
// on ties), a butterfly max over the group, and a ballot: the lowest lane
// holding the maximum also holds the lowest expert id with that value. G >= k,
// so lane i keeps pick i and writes it. The softmax is evaluated in double and
// rounded once to fp32.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

template <int V, bool kVec4>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int glog,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
  const int G = 1 << glog;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = gtid >> glog;
  const int g = (int)(gtid & (G - 1));
  const bool active = t < T;
  const int gbase = (int)(threadIdx.x & (kWave - 1)) & ~(G - 1);
  const uint64_t gbits = (G == 64) ? ~0ull : ((1ull << G) - 1ull);

  uint32_t key[V];
  const float* row = logits + t * (int64_t)E;
  if constexpr (kVec4) {
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const int e0 = g * V + 4 * j;
      const bool ok = active && e0 < E;  // E % 4 == 0: the four are all in range or all out
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) f = *reinterpret_cast<const float4*>(row + e0);
      key[4 * j + 0] = ok ? float_order_key(f.x) : 0u;
      key[4 * j + 1] = ok ? float_order_key(f.y) : 0u;
      key[4 * j + 2] = ok ? float_order_key(f.z) : 0u;
      key[4 * j + 3] = ok ? float_order_key(f.w) : 0u;
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = g * V + v;
      key[v] = (active && e < E) ? float_order_key(row[e]) : 0u;
    }
  }

  // Key 0 marks "empty or taken": every finite float maps above it.
  float top = 0.f, mine = 0.f;
  int mine_id = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
    int bi = 0;
#pragma unroll
    for (int v = 1; v < V; ++v) {
      if (key[v] > best) {
        best = key[v];
        bi = v;
      }
    }
    uint32_t gm = best;
    for (int off = 1; off < G; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)gm, off);
      gm = o > gm ? o : gm;
    }
    const uint64_t holders = (__ballot(best == gm) >> gbase) & gbits;
    const int wl = __ffsll((unsigned long long)holders) - 1;
    const int wbi = __shfl(bi, gbase + wl);
    const int e = wl * V + wbi;
    const float val = order_key_float(gm);
    if (r == 0) top = val;
    if (g == r) {
      mine = val;
      mine_id = e;
    }
    if (g == wl) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == wbi) key[v] = 0u;
    }
  }

  const double ex = (g < k) ? exp((double)mine - (double)top) : 0.0;
  double s = ex;
  for (int off = 1; off < G; off <<= 1) s += __shfl_xor(s, off);
  if (active && g < k) {
    idx[t * k + g] = mine_id;
    w[t * k + g] = (float)(ex / s);
  }
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <int V, bool kVec4>
hipError_t go(const float* logits, int T, int E, int k, int G, int32_t* idx, float* w,
              hipStream_t s) {
  const int64_t threads = (int64_t)T * G;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  return launch(route_kernel<V, kVec4>, dim3(blocks), dim3(256), 0, s, logits, T, E, k, ilog2(G),
                idx, w);
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  int ge = next_pow2((E + 3) / 4);
  if (ge > kWave) ge = kWave;
  const int G = ge > next_pow2(k) ? ge : next_pow2(k);  // k <= 32, so G <= 64
  const int V = next_pow2((E + G - 1) / G);              // E <= 1024, so V <= 16
  const bool vec4 = (V % 4 == 0) && (E % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  switch (V) {
    case 1: return go<1, false>(logits, T, E, k, G, idx, w, s);
    case 2: return go<2, false>(logits, T, E, k, G, idx, w, s);
    case 4: return vec4 ? go<4, true>(logits, T, E, k, G, idx, w, s)
                        : go<4, false>(logits, T, E, k, G, idx, w, s);
    case 8: return vec4 ? go<8, true>(logits, T, E, k, G, idx, w, s)
                        : go<8, false>(logits, T, E, k, G, idx, w, s);
    case 16: return vec4 ? go<16, true>(logits, T, E, k, G, idx, w, s)
                         : go<16, false>(logits, T, E, k, G, idx, w, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
