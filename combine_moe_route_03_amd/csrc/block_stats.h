// block_stats.h -- skew statistics of the send-count matrix S computed by one
// block from counts held in LDS (DODOCO summary, "metrics"): per-expert
// max/mean and the Gini coefficient of per-rank loads (per-expert Gini
// alongside). Numerators are exact 64-bit integer sums of |v_a - v_b| over all
// ordered pairs; each ratio is a single double division. Used by the
// standalone statistics kernel and by the dispatch place kernel.
#pragma once

#include "../../include/moe_route.h"
#include "device.h"

namespace moe {

// LDS scratch of block_stats: per-rank loads, per-wave partial reductions and
// the sort buffer of the large-n pair sums.
struct StatsScratch {
  int64_t vr[1024];
  int64_t red[7][16];
  int32_t key[1024];
};

// Up to this many values the pair sum runs over all pairs (n^2 / threads
// differences each); beyond it the values are sorted first (statistics kernel:
// E = 256 9.7 -> 6.9 us, E = 1024 68.6 -> 12.2 us, E = R = 1024 115 -> 18 us).
constexpr int kPairSumMax = 128;

namespace stats_detail {

// Wave-wide reductions (DPP within rows, scalar lane reads across rows).
template <typename V>
__device__ __forceinline__ V wave_sum(V v) {
  return group_reduce(v, kWave, [](V x, V y) { return x + y; });
}
template <typename V>
__device__ __forceinline__ V wave_max(V v) {
  return group_reduce(v, kWave, [](V x, V y) { return x > y ? x : y; });
}
template <typename V>
__device__ __forceinline__ V wave_min(V v) {
  return group_reduce(v, kWave, [](V x, V y) { return x < y ? x : y; });
}

// Sum over ordered pairs (a, b) of |v[a] - v[b]| for n values in LDS, spread
// over all nt threads: with n <= nt, thread t takes a = t mod n and one of the
// nt / n slices of b; otherwise a strides over the threads. |difference| fits
// in 32 bits (values are counts below 2^31), the running sum is 64-bit.
template <typename V>
__device__ __forceinline__ int64_t pair_abs_sum(const V* v, int n, int tid, int nt) {
  int64_t acc = 0;
  if (n <= nt) {
    const int S = nt / n;
    if (tid < S * n) {
      const int a = tid % n, sl = tid / n;
      const int len = (n + S - 1) / S, b0 = sl * len, b1 = (b0 + len < n) ? b0 + len : n;
      const int64_t va = v[a];
#pragma unroll 8
      for (int b = b0; b < b1; ++b) {
        const int64_t d = va - (int64_t)v[b];
        acc += d < 0 ? -d : d;
      }
    }
  } else {
    for (int a = tid; a < n; a += nt) {
      const int64_t va = v[a];
#pragma unroll 8
      for (int b = 0; b < n; ++b) {
        const int64_t d = va - (int64_t)v[b];
        acc += d < 0 ? -d : d;
      }
    }
  }
  return acc;
}

// The same sum through the sorted values x_0 <= ... <= x_{n-1}:
// sum over ordered pairs |v_a - v_b| = 2 * sum_k x_k (2k - n + 1), exact in
// 64-bit integers. Thread i holds element i (padded with INT32_MAX to a power
// of two np <= nt, so the pads sort last); a bitonic network orders them,
// partners less than 64 apart exchanging by lane shuffles and farther ones
// through `key` in LDS (two barriers a stage); then each thread adds its
// term. Every thread of the block calls it (barriers); returns this thread's
// part of the sum.
template <typename V>
__device__ int64_t sorted_pair_abs_sum(const V* v, int n, int32_t* key, int tid, int nt) {
  int np = 1;
  while (np < n) np <<= 1;
  int32_t x = tid < n ? (int32_t)v[tid] : INT32_MAX;
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      int32_t y;
      if (stride < kWave) {
        y = __shfl_xor(x, stride);
      } else {  // uniform branch
        key[tid] = x;
        __syncthreads();
        y = key[tid ^ stride];
        __syncthreads();
      }
      const bool up = (tid & size) == 0, lower = (tid & stride) == 0;
      x = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
    }
  }
  return tid < n ? 2 * (int64_t)x * (2 * tid - n + 1) : 0;
}

}  // namespace stats_detail

// Statistics of the E counts in LDS `cnt`, written to `out` by thread 0. Every
// thread of the block must call it (it has barriers); E <= 1024, blockDim a
// multiple of 64, <= 1024 and at least E rounded up to a power of two.
// Counts are below 2^31 in total, so totals, maxima and minima are 32-bit; only
// the two pair sums need 64 bits.
__device__ inline void block_stats(const int32_t* cnt, int E, int R, StatsScratch& sc,
                                   moe_stats_t* out) {
  using namespace stats_detail;
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nw = (nt + kWave - 1) / kWave;
  const int L = E / R;
  // per-rank loads: one rank per thread, its L slots summed with independent loads
  for (int r = tid; r < R; r += nt) {
    int64_t s = 0;
#pragma unroll 8
    for (int j = 0; j < L; ++j) s += cnt[r * L + j];
    sc.vr[r] = s;
  }
  __syncthreads();

  // uniform over the block: the sorted variant has barriers
  int64_t ge = E <= kPairSumMax ? pair_abs_sum(cnt, E, tid, nt)
                                : sorted_pair_abs_sum(cnt, E, sc.key, tid, nt);
  int64_t gr = R <= kPairSumMax ? pair_abs_sum(sc.vr, R, tid, nt)
                                : sorted_pair_abs_sum(sc.vr, R, sc.key, tid, nt);
  int32_t tot = 0, emax = INT32_MIN, emin = INT32_MAX, rmax = INT32_MIN, rmin = INT32_MAX;
  for (int a = tid; a < E; a += nt) {
    const int32_t va = cnt[a];
    tot += va;
    emax = va > emax ? va : emax;
    emin = va < emin ? va : emin;
  }
  for (int a = tid; a < R; a += nt) {
    const int32_t va = (int32_t)sc.vr[a];
    rmax = va > rmax ? va : rmax;
    rmin = va < rmin ? va : rmin;
  }
  // two-level reduction: within each wave, then wave 0 over the per-wave partials
  ge = wave_sum(ge);
  gr = wave_sum(gr);
  tot = wave_sum(tot);
  emax = wave_max(emax);
  emin = wave_min(emin);
  rmax = wave_max(rmax);
  rmin = wave_min(rmin);
  if (lane == 0) {
    sc.red[0][wid] = ge;
    sc.red[1][wid] = gr;
    sc.red[2][wid] = tot;
    sc.red[3][wid] = emax;
    sc.red[4][wid] = emin;
    sc.red[5][wid] = rmax;
    sc.red[6][wid] = rmin;
  }
  __syncthreads();
  if (wid == 0) {
    const bool in = lane < nw;
    ge = wave_sum(in ? sc.red[0][lane] : (int64_t)0);
    gr = wave_sum(in ? sc.red[1][lane] : (int64_t)0);
    tot = wave_sum(in ? (int32_t)sc.red[2][lane] : 0);
    emax = wave_max(in ? (int32_t)sc.red[3][lane] : INT32_MIN);
    emin = wave_min(in ? (int32_t)sc.red[4][lane] : INT32_MAX);
    rmax = wave_max(in ? (int32_t)sc.red[5][lane] : INT32_MIN);
    rmin = wave_min(in ? (int32_t)sc.red[6][lane] : INT32_MAX);
    if (lane == 0) {
      const int64_t T = tot;
      moe_stats_t st;
      st.total = T;
      st.expert_max = emax;
      st.expert_min = emin;
      st.rank_max = rmax;
      st.rank_min = rmin;
      st.expert_max_over_mean = T ? (double)((int64_t)E * emax) / (double)T : 0.0;
      st.rank_max_over_mean = T ? (double)((int64_t)R * rmax) / (double)T : 0.0;
      st.expert_gini = T ? (double)ge / (double)(2 * (int64_t)E * T) : 0.0;
      st.rank_gini = T ? (double)gr / (double)(2 * (int64_t)R * T) : 0.0;
      *out = st;
    }
  }
}

}  // namespace moe
