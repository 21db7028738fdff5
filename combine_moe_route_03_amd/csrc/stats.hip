// stats.hip -- skew statistics of the send-count matrix S (DODOCO summary,
// "metrics"): per-expert max/mean and the Gini coefficient of per-rank loads
// (per-expert Gini alongside). Numerators are exact 64-bit integer sums of
// |v_a - v_b| over all ordered pairs; each ratio is a single double division.
#include "../../include/moe_route.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 1024;
constexpr int kMaxE = 1024;

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

__global__ __launch_bounds__(kBlock) void stats_kernel(const int32_t* __restrict__ counts, int E,
                                                       int R, moe_stats_t* __restrict__ out) {
  __shared__ int64_t ve[kMaxE];
  __shared__ int64_t vr[kMaxE];
  __shared__ int64_t red[7][kBlock / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int L = E / R;
  for (int e = tid; e < E; e += kBlock) ve[e] = counts[e];
  __syncthreads();
  for (int r = tid; r < R; r += kBlock) {
    int64_t s = 0;
    for (int j = 0; j < L; ++j) s += ve[r * L + j];
    vr[r] = s;
  }
  __syncthreads();

  int64_t ge = 0, gr = 0, tot = 0;
  int64_t emax = INT64_MIN, emin = INT64_MAX, rmax = INT64_MIN, rmin = INT64_MAX;
  for (int a = tid; a < E; a += kBlock) {
    const int64_t va = ve[a];
    for (int b = 0; b < E; ++b) {
      const int64_t d = va - ve[b];
      ge += d < 0 ? -d : d;
    }
    tot += va;
    emax = va > emax ? va : emax;
    emin = va < emin ? va : emin;
  }
  for (int a = tid; a < R; a += kBlock) {
    const int64_t va = vr[a];
    for (int b = 0; b < R; ++b) {
      const int64_t d = va - vr[b];
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
    red[0][wid] = ge;
    red[1][wid] = gr;
    red[2][wid] = tot;
    red[3][wid] = emax;
    red[4][wid] = emin;
    red[5][wid] = rmax;
    red[6][wid] = rmin;
  }
  __syncthreads();
  if (tid == 0) {
    for (int q = 1; q < kBlock / kWave; ++q) {
      red[0][0] += red[0][q];
      red[1][0] += red[1][q];
      red[2][0] += red[2][q];
      red[3][0] = red[3][q] > red[3][0] ? red[3][q] : red[3][0];
      red[4][0] = red[4][q] < red[4][0] ? red[4][q] : red[4][0];
      red[5][0] = red[5][q] > red[5][0] ? red[5][q] : red[5][0];
      red[6][0] = red[6][q] < red[6][0] ? red[6][q] : red[6][0];
    }
    const int64_t T = red[2][0];
    moe_stats_t st;
    st.total = T;
    st.expert_max = (int32_t)red[3][0];
    st.expert_min = (int32_t)red[4][0];
    st.rank_max = (int32_t)red[5][0];
    st.rank_min = (int32_t)red[6][0];
    st.expert_max_over_mean = T ? (double)((int64_t)E * red[3][0]) / (double)T : 0.0;
    st.rank_max_over_mean = T ? (double)((int64_t)R * red[5][0]) / (double)T : 0.0;
    st.expert_gini = T ? (double)red[0][0] / (double)(2 * (int64_t)E * T) : 0.0;
    st.rank_gini = T ? (double)red[1][0] / (double)(2 * (int64_t)R * T) : 0.0;
    *out = st;
  }
}

}  // namespace

hipError_t launch_stats(const int32_t* counts, int E, int R, void* out, hipStream_t s) {
  return launch(stats_kernel, dim3(1), dim3(kBlock), 0, s, counts, E, R,
                static_cast<moe_stats_t*>(out));
}

}  // namespace moe
