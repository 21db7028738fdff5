// expert.hip -- identity-scaled experts of the synthetic workloads: expert e
// multiplies its rows by (e + 1). Rows of one expert are contiguous in the send
// buffer (survey section 1.1, EP flow step 3 runs on contiguous same-expert
// rows), so a row's expert is found by binary search over the bucket starts
// staged in LDS. Each thread moves kU 16-byte vectors (all loads first). The
// send rows are read once (streaming loads); the output rows are stored through
// the caches when the whole output fits the cache-reuse budget (the combine
// then finds them in the Infinity Cache), streamed otherwise.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxE = 1024;
constexpr int kU = 2;

template <bool kBF16>
__device__ __forceinline__ v4u scale_vec(v4u v, float sc) {
  v4u o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kBF16)
      o[j] = pack_bf16x2(sc * bf16_lo(v[j]), sc * bf16_hi(v[j]));
    else
      o[j] = __float_as_uint(sc * __uint_as_float(v[j]));
  }
  return o;
}

template <bool kBF16, bool kCacheOut>
__global__ __launch_bounds__(kBlock) void expert_scale_kernel(
    const v4u* __restrict__ in, uint32_t nvec, uint32_t total, int E, int R, int W,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ cnts, v4u* __restrict__ out) {
  __shared__ int32_t start[kMaxE];  // bucket starts in (wave, rank, slot) order
  __shared__ int32_t stop[kMaxE];   // bucket ends
  __shared__ int32_t bexp[kMaxE];   // expert of each bucket
  const uint32_t q0 = blockIdx.x * (uint32_t)(kBlock * kU) + threadIdx.x;
  v4u v[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const uint32_t q = q0 + u * kBlock;
    v[u] = (q < total) ? load_stream(in + q) : v4u{0u, 0u, 0u, 0u};
  }
  const int L = E / R, LW = L / W;
  for (int j = threadIdx.x; j < E; j += kBlock) {
    const int e = bucket_expert(j, R, L, LW);
    start[j] = offs[e];
    stop[j] = offs[e] + cnts[e];
    bexp[j] = e;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const uint32_t q = q0 + u * kBlock;
    if (q >= total) continue;
    const int n = (int)(q / nvec);
    int lo = 0, hi = E - 1;  // last bucket whose start is <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= n) lo = mid;
      else hi = mid - 1;
    }
    if (n < start[lo] || n >= stop[lo]) continue;  // row outside every bucket
    const v4u o = scale_vec<kBF16>(v[u], (float)(bexp[lo] + 1));
    if constexpr (kCacheOut) out[q] = o;
    else store_stream(out + q, o);
  }
}

// The rows [wave_offsets[w], wave_offsets[w+1]) of one expert wave (bounds read
// on the device, clamped to [0, rows_max)), grid-stride; the same per-row
// arithmetic as expert_scale_kernel.
template <bool kBF16, bool kCacheOut>
__global__ __launch_bounds__(kBlock) void expert_scale_wave_kernel(
    const v4u* __restrict__ in, uint32_t nvec, int64_t rows_max, int E, int R, int W,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ cnts,
    const int32_t* __restrict__ wave_offsets, int w, v4u* __restrict__ out) {
  __shared__ int32_t start[kMaxE];
  __shared__ int32_t stop[kMaxE];
  __shared__ int32_t bexp[kMaxE];
  int64_t a = wave_offsets[w], b = wave_offsets[w + 1];
  a = a < 0 ? 0 : (a > rows_max ? rows_max : a);
  b = b < a ? a : (b > rows_max ? rows_max : b);
  const int L = E / R, LW = L / W;
  for (int j = threadIdx.x; j < E; j += kBlock) {
    const int e = bucket_expert(j, R, L, LW);
    start[j] = offs[e];
    stop[j] = offs[e] + cnts[e];
    bexp[j] = e;
  }
  __syncthreads();
  const int64_t n_vec = (b - a) * nvec;
  const int64_t step = (int64_t)gridDim.x * kBlock * kU;
  for (int64_t q0 = (int64_t)blockIdx.x * kBlock * kU + threadIdx.x; q0 < n_vec; q0 += step) {
    v4u v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t q = q0 + u * kBlock;
      v[u] = (q < n_vec) ? load_stream(in + a * nvec + q) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t q = q0 + u * kBlock;
      if (q >= n_vec) continue;
      const int n = (int)(a + q / nvec);
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= n) lo = mid;
        else hi = mid - 1;
      }
      if (n < start[lo] || n >= stop[lo]) continue;
      const v4u o = scale_vec<kBF16>(v[u], (float)(bexp[lo] + 1));
      if constexpr (kCacheOut) out[a * nvec + q] = o;
      else store_stream(out + a * nvec + q, o);
    }
  }
}

}  // namespace

hipError_t launch_expert_scale_wave(const void* in, int dtype, int64_t rows_max, int64_t H, int E,
                                    int R, int W, const int32_t* expert_offsets,
                                    const int32_t* expert_counts, const int32_t* wave_offsets,
                                    int w, void* out, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  const bool bf16 = dtype == 1;
  const uint32_t nvec = (uint32_t)(H * (bf16 ? 2 : 4) / 16);
  // a wave holds at most all rows: enough blocks for that, at most 2048
  // (grid-stride beyond), the per-wave share of the whole-buffer policy below
  const int64_t want = (rows_max * nvec + kBlock * kU - 1) / (kBlock * kU);
  const unsigned grid = (unsigned)(want < 2048 ? (want < 1 ? 1 : want) : 2048);
  const bool cache = rows_max * nvec * 16 <= kCacheReuseBytes;
  auto go = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kBlock), 0, s, static_cast<const v4u*>(in), nvec,
                  rows_max, E, R, W, expert_offsets, expert_counts, wave_offsets, w,
                  static_cast<v4u*>(out));
  };
  if (bf16)
    return cache ? go(expert_scale_wave_kernel<true, true>) : go(expert_scale_wave_kernel<true, false>);
  return cache ? go(expert_scale_wave_kernel<false, true>) : go(expert_scale_wave_kernel<false, false>);
}

hipError_t launch_expert_scale(const void* in, int dtype, int64_t rows, int64_t H, int E, int R,
                               int W, const int32_t* expert_offsets,
                               const int32_t* expert_counts, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const bool bf16 = dtype == 1;
  const uint32_t nvec = (uint32_t)(H * (bf16 ? 2 : 4) / 16);
  const uint32_t total = (uint32_t)rows * nvec;
  const unsigned grid = (total + kBlock * kU - 1) / (kBlock * kU);
  const v4u* src = static_cast<const v4u*>(in);
  v4u* dst = static_cast<v4u*>(out);
  const bool cache = (int64_t)total * 16 <= kCacheReuseBytes;
  auto go = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kBlock), 0, s, src, nvec, total, E, R, W,
                  expert_offsets, expert_counts, dst);
  };
  if (bf16) return cache ? go(expert_scale_kernel<true, true>) : go(expert_scale_kernel<true, false>);
  return cache ? go(expert_scale_kernel<false, true>) : go(expert_scale_kernel<false, false>);
}

}  // namespace moe
