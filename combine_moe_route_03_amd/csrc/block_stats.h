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

// LDS scratch of block_stats: per-rank loads and per-wave partial reductions.
struct StatsScratch {
  int64_t vr[1024];
  int64_t red[7][16];
};

namespace stats_detail {

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_down(v, o);
  return v;
}
__device__ __forceinline__ int64_t wave_max(int64_t v) {
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const int64_t u = __shfl_down(v, o);
    v = u > v ? u : v;
  }
  return v;
}
__device__ __forceinline__ int64_t wave_min(int64_t v) {
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const int64_t u = __shfl_down(v, o);
    v = u < v ? u : v;
  }
  return v;
}

}  // namespace stats_detail

// Statistics of the E counts in LDS `cnt`, written to `out` by thread 0. Every
// thread of the block must call it (it has barriers); E <= 1024, blockDim <= 1024.
__device__ inline void block_stats(const int32_t* cnt, int E, int R, StatsScratch& sc,
                                   moe_stats_t* out) {
  using namespace stats_detail;
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int L = E / R;
  for (int r = tid; r < R; r += nt) {
    int64_t s = 0;
    for (int j = 0; j < L; ++j) s += cnt[r * L + j];
    sc.vr[r] = s;
  }
  __syncthreads();

  int64_t ge = 0, gr = 0, tot = 0;
  int64_t emax = INT64_MIN, emin = INT64_MAX, rmax = INT64_MIN, rmin = INT64_MAX;
  for (int a = tid; a < E; a += nt) {
    const int64_t va = cnt[a];
    for (int b = 0; b < E; ++b) {
      const int64_t d = va - cnt[b];
      ge += d < 0 ? -d : d;
    }
    tot += va;
    emax = va > emax ? va : emax;
    emin = va < emin ? va : emin;
  }
  for (int a = tid; a < R; a += nt) {
    const int64_t va = sc.vr[a];
    for (int b = 0; b < R; ++b) {
      const int64_t d = va - sc.vr[b];
      gr += d < 0 ? -d : d;
    }
    rmax = va > rmax ? va : rmax;
    rmin = va < rmin ? va : rmin;
  }
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
  if (tid == 0) {
    const int nw = (nt + kWave - 1) / kWave;
    for (int q = 1; q < nw; ++q) {
      sc.red[0][0] += sc.red[0][q];
      sc.red[1][0] += sc.red[1][q];
      sc.red[2][0] += sc.red[2][q];
      sc.red[3][0] = sc.red[3][q] > sc.red[3][0] ? sc.red[3][q] : sc.red[3][0];
      sc.red[4][0] = sc.red[4][q] < sc.red[4][0] ? sc.red[4][q] : sc.red[4][0];
      sc.red[5][0] = sc.red[5][q] > sc.red[5][0] ? sc.red[5][q] : sc.red[5][0];
      sc.red[6][0] = sc.red[6][q] < sc.red[6][0] ? sc.red[6][q] : sc.red[6][0];
    }
    const int64_t T = sc.red[2][0];
    moe_stats_t st;
    st.total = T;
    st.expert_max = (int32_t)sc.red[3][0];
    st.expert_min = (int32_t)sc.red[4][0];
    st.rank_max = (int32_t)sc.red[5][0];
    st.rank_min = (int32_t)sc.red[6][0];
    st.expert_max_over_mean = T ? (double)((int64_t)E * sc.red[3][0]) / (double)T : 0.0;
    st.rank_max_over_mean = T ? (double)((int64_t)R * sc.red[5][0]) / (double)T : 0.0;
    st.expert_gini = T ? (double)sc.red[0][0] / (double)(2 * (int64_t)E * T) : 0.0;
    st.rank_gini = T ? (double)sc.red[1][0] / (double)(2 * (int64_t)R * T) : 0.0;
    *out = st;
  }
}

}  // namespace moe
