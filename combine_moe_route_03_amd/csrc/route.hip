// route.hip -- top-k gating on gfx950: per token, the k largest router logits
// (equal logits ordered by ascending expert id) and the softmax over those k
// (MoE systems survey, crad.ict.ac.cn, section 1.1, eq. (2): the non-kept
// logits act as -inf, so only the k kept ones enter the softmax).
//
// One aligned group of G = 2^glog lanes of a wave64 handles one token; lane g
// holds V consecutive logits (experts g*V .. g*V+V-1). G >= k, so lane i keeps
// pick i and writes it. The fused variant also histograms the picks of its
// block for the placing pass.
#include "device.h"
#include "launch.h"
#include "route_token.h"

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
  int id;
  float wt;
  route_token<V, kVec4>(logits, t, t < T, E, k, G, g, id, wt);
  if (id >= 0) {
    idx[t * k + g] = id;
    w[t * k + g] = wt;
  }
}

// Routing fused with the counting pass of dispatch: block b routes tokens
// [b*tpb, (b+1)*tpb) (1024/G tokens per pass) and writes the histogram of its
// picks to hist[b][0..E) (LDS integer atomics: order-free, exact). Its picks
// are exactly chunk b of the placing pass when chunks are tpb*k picks long.
template <int V, bool kVec4>
__global__ __launch_bounds__(kIndexBlock) void route_count_kernel(
    const float* __restrict__ logits, int T, int E, int k, int glog, int tpb,
    int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ hist) {
  __shared__ int32_t h[1024];
  const int G = 1 << glog;
  const int tid = threadIdx.x;
  if (tid < E) h[tid] = 0;
  __syncthreads();
  const int g = tid & (G - 1);
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t t1 = (t0 + tpb < T) ? t0 + tpb : T;
  for (int64_t tb = t0; tb < t1; tb += kIndexBlock >> glog) {
    const int64_t t = tb + (tid >> glog);
    int id;
    float wt;
    route_token<V, kVec4>(logits, t, t < t1, E, k, G, g, id, wt);
    if (id >= 0) {
      idx[t * k + g] = id;
      w[t * k + g] = wt;
      atomicAdd(&h[id], 1);
    }
  }
  __syncthreads();
  if (tid < E) hist[(int64_t)blockIdx.x * E + tid] = h[tid];
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

template <int V, bool kVec4>
hipError_t go_count(const float* logits, int T, int E, int k, int G, int tpb, int32_t* idx,
                    float* w, int32_t* hist, hipStream_t s) {
  const unsigned blocks = (unsigned)((T + tpb - 1) / tpb);
  return launch(route_count_kernel<V, kVec4>, dim3(blocks), dim3(kIndexBlock), 0, s, logits, T, E,
                k, ilog2(G), tpb, idx, w, hist);
}

// Lanes per token: enough for E/4 logits a lane, at least k (k <= 32), <= 64.
int route_group(int E, int k) {
  int ge = next_pow2((E + 3) / 4);
  if (ge > kWave) ge = kWave;
  return ge > next_pow2(k) ? ge : next_pow2(k);
}

// Fused routing + counting: at most max_index_chunks(E) blocks of 1024 threads
// (the placing pass reads one histogram row per block). Lanes per token shrink
// (down to k and E/16, i.e. V <= 16 logits a lane) until one pass of a block
// covers its tokens, then extra passes are added.
void route_count_geometry(int T, int E, int k, int& G, int& tpb) {
  const int64_t max_blocks = max_index_chunks(E);
  const int gmin_k = next_pow2(k), gmin_e = next_pow2((E + 15) / 16);
  const int gmin = gmin_k > gmin_e ? gmin_k : gmin_e;
  G = route_group(E, k);
  while (G > gmin && (int64_t)T > max_blocks * (kIndexBlock / G)) G >>= 1;
  const int per_pass = kIndexBlock / G;
  int64_t passes = 1;
  while ((int64_t)T > max_blocks * per_pass * passes) ++passes;
  tpb = (int)(per_pass * passes);
}

}  // namespace

int route_count_tokens_per_block(int T, int E, int k) {
  int G, tpb;
  route_count_geometry(T, E, k, G, tpb);
  return tpb;
}

hipError_t launch_route_count(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                              int32_t* hist, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int G, tpb;
  route_count_geometry(T, E, k, G, tpb);
  const int V = next_pow2((E + G - 1) / G);  // G >= E/16, so V <= 16
  const bool vec4 = (V % 4 == 0) && (E % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  switch (V) {
    case 1: return go_count<1, false>(logits, T, E, k, G, tpb, idx, w, hist, s);
    case 2: return go_count<2, false>(logits, T, E, k, G, tpb, idx, w, hist, s);
    case 4: return vec4 ? go_count<4, true>(logits, T, E, k, G, tpb, idx, w, hist, s)
                        : go_count<4, false>(logits, T, E, k, G, tpb, idx, w, hist, s);
    case 8: return vec4 ? go_count<8, true>(logits, T, E, k, G, tpb, idx, w, hist, s)
                        : go_count<8, false>(logits, T, E, k, G, tpb, idx, w, hist, s);
    case 16: return vec4 ? go_count<16, true>(logits, T, E, k, G, tpb, idx, w, hist, s)
                         : go_count<16, false>(logits, T, E, k, G, tpb, idx, w, hist, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int G = route_group(E, k);
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
