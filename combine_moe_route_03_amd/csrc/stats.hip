// stats.hip -- the standalone statistics kernel: one block, one thread per
// expert, counts staged in LDS, then block_stats().
#include "block_stats.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxE = 1024;

__global__ __launch_bounds__(1024) void stats_kernel(const int32_t* __restrict__ counts, int E,
                                                     int R, moe_stats_t* __restrict__ out) {
  __shared__ int32_t cnt[kMaxE];
  __shared__ StatsScratch sc;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = counts[e];
  __syncthreads();
  block_stats(cnt, E, R, sc, out);
}

}  // namespace

hipError_t launch_stats(const int32_t* counts, int E, int R, void* out, hipStream_t s) {
  // One thread per expert, rounded up to a power of two and to whole waves
  // (the sorted pair sums hold one element a thread): E <= 1024.
  int threads = kWave;
  while (threads < E) threads <<= 1;
  return launch(stats_kernel, dim3(1), dim3(threads), 0, s, counts, E, R,
                static_cast<moe_stats_t*>(out));
}

}  // namespace moe
