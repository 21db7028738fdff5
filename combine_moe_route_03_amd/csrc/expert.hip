// expert.hip -- identity-scaled experts of the synthetic workloads: expert e
// multiplies its rows by (e + 1). Rows of one expert are contiguous in the send
// buffer (survey section 1.1, EP flow step 3 runs on contiguous same-expert
// rows), so a row's expert is found by binary search over the bucket starts.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxE = 1024;

template <bool kBF16>
__global__ __launch_bounds__(kBlock) void expert_scale_kernel(
    const uint4* __restrict__ in, uint32_t nvec, uint32_t total, int E, int R, int W,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ cnts, uint4* __restrict__ out) {
  __shared__ int32_t start[kMaxE];  // bucket starts in (wave, rank, slot) order
  __shared__ int32_t bexp[kMaxE];   // expert of each bucket
  const int L = E / R, LW = L / W;
  for (int j = threadIdx.x; j < E; j += kBlock) {
    const int e = bucket_expert(j, R, L, LW);
    start[j] = offs[e];
    bexp[j] = e;
  }
  __syncthreads();
  const uint32_t q = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
  if (q >= total) return;
  const int n = (int)(q / nvec);
  int lo = 0, hi = E - 1;  // last bucket whose start is <= n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= n) lo = mid;
    else hi = mid - 1;
  }
  const int e = bexp[lo];
  if (n < start[lo] || n >= start[lo] + cnts[e]) return;  // row outside every bucket
  const float sc = (float)(e + 1);
  const uint4 v = in[q];
  uint4 o;
  if constexpr (kBF16) {
    o.x = pack_bf16x2(sc * bf16_lo(v.x), sc * bf16_hi(v.x));
    o.y = pack_bf16x2(sc * bf16_lo(v.y), sc * bf16_hi(v.y));
    o.z = pack_bf16x2(sc * bf16_lo(v.z), sc * bf16_hi(v.z));
    o.w = pack_bf16x2(sc * bf16_lo(v.w), sc * bf16_hi(v.w));
  } else {
    o.x = __float_as_uint(sc * __uint_as_float(v.x));
    o.y = __float_as_uint(sc * __uint_as_float(v.y));
    o.z = __float_as_uint(sc * __uint_as_float(v.z));
    o.w = __float_as_uint(sc * __uint_as_float(v.w));
  }
  out[q] = o;
}

}  // namespace

hipError_t launch_expert_scale(const void* in, int dtype, int64_t rows, int64_t H, int E, int R,
                               int W, const int32_t* expert_offsets,
                               const int32_t* expert_counts, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const bool bf16 = dtype == 1;
  const uint32_t nvec = (uint32_t)(H * (bf16 ? 2 : 4) / 16);
  const uint32_t total = (uint32_t)rows * nvec;
  const unsigned grid = (total + kBlock - 1) / kBlock;
  if (bf16)
    hipLaunchKernelGGL((expert_scale_kernel<true>), dim3(grid), dim3(kBlock), 0, s,
                       static_cast<const uint4*>(in), nvec, total, E, R, W, expert_offsets,
                       expert_counts, static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL((expert_scale_kernel<false>), dim3(grid), dim3(kBlock), 0, s,
                       static_cast<const uint4*>(in), nvec, total, E, R, W, expert_offsets,
                       expert_counts, static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
