// combine_waves.hip -- the combine of the wave schedule (irregular AllToAll
// page, "Wave-Scheduled pipelining": W waves of E / W experts, each wave
// running dispatch -> compute -> combine).
//
// A token's weighted sum needs the outputs of all its kept picks, whose
// experts may sit in several waves; it is complete after the last of them. The
// order kernels list the tokens by that completion wave (ascending token id
// within a wave); the wave combine then sums the tokens of a range of
// completion waves with the one-pass combine's per-column arithmetic (the fp32
// fma chain in pick order, combine_column.h), so every token's bits equal the
// one-pass combine's, whatever the wave split.
//
// The wave of a row: rows are in (wave, rank, slot) bucket order, so row r is
// in the largest wave w with wave_offsets[w] <= r (empty waves share an
// offset with the next one and are skipped by that rule). The completion
// wave of a token is the wave of its largest row; a token with no row is
// complete before any wave (wave 0).
#include <type_traits>

#include "combine_column.h"
#include "device.h"
#include "index_tables.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kOrderBlock = 1024;
// 256-thread blocks: the grid covers all T tokens whatever the range, and
// with 128 the launches of empty early waves cost more (dirichlet_waves,
// W = 8, the eight waves one call each: 525 against 445 us).
constexpr int kBlock = 256;

__device__ __forceinline__ int wave_of_row(const int32_t* s_wo, int W, int32_t r) {
  int lo = 0, hi = W - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_wo[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int completion_wave(const int32_t* __restrict__ pos, int k, int t,
                                               uint32_t nrows, const int32_t* s_wo, int W) {
  int32_t last = -1;
  for (int i = 0; i < k; ++i) {
    const int32_t p = pos[(int64_t)t * k + i];
    if ((uint32_t)p < nrows && p > last) last = p;
  }
  return last < 0 ? 0 : wave_of_row(s_wo, W, last);
}

// The order in two launches, as the dispatch's index stage: block b of
// the count kernel histograms the completion waves of its tokens [b*tpb,
// (b+1)*tpb) into row b of hist [nb][W]; block b of the place kernel sums the
// rows before b and all rows, scans the wave totals (the first entry of each
// wave) and ranks its tokens 1024 at a time (stable: ballot match on the wave
// id, as the placing kernel ranks picks).
__global__ __launch_bounds__(kOrderBlock) void order_count_kernel(
    const int32_t* __restrict__ pos, int T, int k, const int32_t* __restrict__ wave_offsets,
    int W, int tpb, int32_t* __restrict__ hist) {
  __shared__ int32_t s_wo[kIndexMaxE + 1];
  __shared__ int32_t h[kIndexMaxE];
  const int tid = threadIdx.x, b = blockIdx.x;
  const uint32_t nrows = (uint32_t)T * (uint32_t)k;
  for (int w = tid; w <= W; w += kOrderBlock) s_wo[w] = wave_offsets[w];
  for (int w = tid; w < W; w += kOrderBlock) h[w] = 0;
  __syncthreads();
  const int t0 = b * tpb, t1 = min(T, t0 + tpb);
  for (int t = t0 + tid; t < t1; t += kOrderBlock)
    atomicAdd(&h[completion_wave(pos, k, t, nrows, s_wo, W)], 1);
  __syncthreads();
  for (int w = tid; w < W; w += kOrderBlock) hist[(int64_t)b * W + w] = h[w];
}

__global__ __launch_bounds__(kOrderBlock) void order_place_kernel(
    const int32_t* __restrict__ pos, int T, int k, const int32_t* __restrict__ wave_offsets,
    int W, int nbits, int tpb, int nb, const int32_t* __restrict__ hist,
    int32_t* __restrict__ token_wave_offsets, int32_t* __restrict__ order) {
  __shared__ int32_t s_wo[kIndexMaxE + 1];
  __shared__ int32_t run[kIndexMaxE];
  __shared__ int32_t wcnt[kOrderBlock / kWave][kIndexMaxE];
  __shared__ int32_t part[kOrderBlock / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave, b = blockIdx.x;
  const uint32_t nrows = (uint32_t)T * (uint32_t)k;
  for (int w = tid; w <= W; w += kOrderBlock) s_wo[w] = wave_offsets[w];
  if (tid < W) {
#pragma unroll
    for (int q = 0; q < kOrderBlock / kWave; ++q) wcnt[q][tid] = 0;
  }
  // thread w < W: tokens of wave w in the blocks before this one, and in all
  int pre = 0, all = 0;
  if (tid < W) {
    for (int q = 0; q < nb; ++q) {
      const int v = hist[(int64_t)q * W + tid];
      all += v;
      pre += q < b ? v : 0;
    }
  }
  const int cj = tid < W ? all : 0;
  const int incl = wave_incl_scan(cj);
  if (lane == kWave - 1) part[wid] = incl;
  __syncthreads();
  int excl = incl - cj;
  for (int q = 0; q < wid; ++q) excl += part[q];
  if (tid < W) {
    run[tid] = excl + pre;
    if (b == 0) token_wave_offsets[tid] = excl;
  }
  if (b == 0 && tid == 0) token_wave_offsets[W] = T;
  __syncthreads();

  const int t0 = b * tpb, t1 = min(T, t0 + tpb);
  for (int base = t0; base < t1; base += kOrderBlock) {
    const int t = base + tid;
    const bool valid = t < t1;
    const int c = valid ? completion_wave(pos, k, t, nrows, s_wo, W) : 0;
    const int at = batch_rank(c, valid, nbits, wcnt, run, base + kOrderBlock >= t1);
    if (valid) order[at] = t;
  }
}

// The tokens of completion waves [w0, w1): entries [twoff[w0], twoff[w1]) of
// the order as (token, 16-byte column) pairs, one per thread of a grid sized
// for all T tokens (the range's count is known only on the device; threads
// past it exit). On dirichlet_waves, all waves in one call: 365 us against
// 354 for the one-pass combine; a grid-stride loop over 2048 blocks took 400
// and over 16384 blocks 389 (one gather in flight per thread, chained behind
// the order and position loads).
template <int KMAX, bool kBF16, bool kCacheIn, bool kUniform>
__global__ __launch_bounds__(kBlock) void combine_wave_kernel(
    const v4u* __restrict__ eo, const float* __restrict__ w, const int32_t* __restrict__ pos,
    int k, uint32_t nvec, uint32_t nrows, const int32_t* __restrict__ order,
    const int32_t* __restrict__ twoff, int w0, int w1, int T, v4u* __restrict__ y) {
  // entries [a, b) of the order, clamped to [0, T] (T * nvec < 2^31)
  const int a = min(max(twoff[w0], 0), T), b = min(max(twoff[w1], a), T);
  const uint32_t n = (uint32_t)(b - a) * nvec;
  const uint32_t q = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
  if (q >= n) return;
  uint32_t j = q / nvec;
  if constexpr (kUniform) j = __builtin_amdgcn_readfirstlane(j);  // nvec % 64 == 0
  const uint32_t col = q - j * nvec;
  const int32_t t = order[a + j];
  if ((uint32_t)t >= (uint32_t)T) return;  // not a token: nothing to write
  store_stream(y + (size_t)t * nvec + col,
               combine_column<KMAX, kBF16, kCacheIn>(eo, w + (size_t)t * k, pos + (size_t)t * k, k,
                                                     nvec, col, nrows));
}

template <int KMAX>
hipError_t go(const void* eo, bool bf16, const float* w, const int32_t* pos, int k, uint32_t nvec,
              int T, uint32_t nrows, const int32_t* order, const int32_t* twoff, int w0, int w1,
              void* y, hipStream_t s) {
  const uint32_t total = (uint32_t)T * nvec;
  const unsigned grid = (total + kBlock - 1) / kBlock;  // total = T * nvec > 0
  const v4u* in = static_cast<const v4u*>(eo);
  v4u* out = static_cast<v4u*>(y);
  // the same cache and uniformity policy as the one-pass combine
  const bool cache = (int64_t)nrows * nvec * 16 <= kCacheReuseBytes;
  const bool uniform = kCombineUniform && nvec % kWave == 0 && (cache || kStreamUniform);
  auto run = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kBlock), 0, s, in, w, pos, k, nvec, nrows, order,
                  twoff, w0, w1, T, out);
  };
  auto pick = [&](auto bf, auto ca) {
    constexpr bool B = decltype(bf)::value, C = decltype(ca)::value;
    return uniform ? run(combine_wave_kernel<KMAX, B, C, true>)
                   : run(combine_wave_kernel<KMAX, B, C, false>);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (bf16) return cache ? pick(T_{}, T_{}) : pick(T_{}, F_{});
  return cache ? pick(F_{}, T_{}) : pick(F_{}, F_{});
}

}  // namespace

void combine_order_blocks(int64_t T, int W, int64_t& tpb, int64_t& nb) {
  // at most min(512, 65536 / W) blocks: the place kernel's threads each read
  // one column of the [nb][W] count matrix
  int64_t cap = 65536 / (W < 1 ? 1 : W);
  cap = cap > 512 ? 512 : (cap < 1 ? 1 : cap);
  tpb = (T + cap - 1) / cap;
  tpb = (tpb + kOrderBlock - 1) / kOrderBlock * kOrderBlock;
  if (tpb < kOrderBlock) tpb = kOrderBlock;
  nb = T > 0 ? (T + tpb - 1) / tpb : 1;
}

hipError_t launch_combine_order(const int32_t* pos, int T, int k, const int32_t* wave_offsets,
                                int W, int32_t* token_wave_offsets, int32_t* token_order,
                                int32_t* hist, hipStream_t s) {
  int64_t tpb, nb;
  combine_order_blocks(T, W, tpb, nb);
  int nbits = 0;
  while ((1 << nbits) < W) ++nbits;
  hipError_t e = launch(order_count_kernel, dim3((unsigned)nb), dim3(kOrderBlock), 0, s, pos, T,
                        k, wave_offsets, W, (int)tpb, hist);
  if (e != hipSuccess) return e;
  return launch(order_place_kernel, dim3((unsigned)nb), dim3(kOrderBlock), 0, s, pos, T, k,
                wave_offsets, W, nbits, (int)tpb, (int)nb, hist, token_wave_offsets, token_order);
}

hipError_t launch_combine_waves(const void* expert_out, int dtype, const float* w,
                                const int32_t* pos, int T, int k, int64_t H,
                                const int32_t* token_order, const int32_t* token_wave_offsets,
                                int w0, int w1, void* y, hipStream_t s) {
  if (T == 0 || w0 >= w1) return hipSuccess;
  const bool bf16 = dtype == 1;
  const uint32_t nvec = (uint32_t)(H * (bf16 ? 2 : 4) / 16);
  const uint32_t nrows = (uint32_t)T * (uint32_t)k;
  const int32_t* o = token_order;
  const int32_t* tw = token_wave_offsets;
  if (k <= 2) return go<2>(expert_out, bf16, w, pos, k, nvec, T, nrows, o, tw, w0, w1, y, s);
  if (k <= 4) return go<4>(expert_out, bf16, w, pos, k, nvec, T, nrows, o, tw, w0, w1, y, s);
  if (k <= 8) return go<8>(expert_out, bf16, w, pos, k, nvec, T, nrows, o, tw, w0, w1, y, s);
  if (k <= 16) return go<16>(expert_out, bf16, w, pos, k, nvec, T, nrows, o, tw, w0, w1, y, s);
  return go<32>(expert_out, bf16, w, pos, k, nvec, T, nrows, o, tw, w0, w1, y, s);
}

}  // namespace moe
