// combine.hip -- gate-weighted combine back to token order (MoE systems
// survey, crad.ict.ac.cn, section 1.1, eq. (1) y = sum_i G(x)_i E_i(x), and EP
// flow step 4: restore the original order, weight by the gate confidence).
//
// Flat over (token, 16-byte column): each thread gathers its column from the k
// expert rows of its token (each expert row is read exactly once; through the
// caches when the expert rows fit the cache-reuse budget, as the expert stage
// has just written them there, streaming otherwise), runs the
// fp32 fused multiply-add chain in pick order (seeded with -0, the additive
// identity, so an all -0 sum stays -0), rounds once to the output dtype
// and writes one 16-byte vector. Lanes of a wave cover consecutive columns of
// one row, so every gather and the store are contiguous 1 KiB segments; with
// rows a multiple of 64 vectors (kUniform) the wave's token is uniform and its
// k positions and weights can come through the scalar cache.
#include <type_traits>

#include "combine_column.h"
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

// 128-thread blocks: dirichlet_waves (streamed rows) 350-353 -> 341-343 us
// against 256 (512: 349-350, 1024: 346-347, 64: 348-350); the cached-row
// workloads measured the same with either.
constexpr int kBlock = 128;

template <int KMAX, bool kBF16, bool kCacheIn, bool kUniform>
__global__ __launch_bounds__(kBlock) void combine_kernel(const v4u* __restrict__ eo,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ pos, int k,
                                                         uint32_t nvec, uint32_t total,
                                                         uint32_t nrows, v4u* __restrict__ y) {
  const uint32_t q = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
  if (q >= total) return;
  if (nrows == 0) {  // no expert rows: every output is the empty sum, -0
    store_stream(y + q, kBF16 ? v4u{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                              : v4u{0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u});
    return;
  }
  uint32_t t = q / nvec;
  if constexpr (kUniform) t = __builtin_amdgcn_readfirstlane(t);  // whole waves: total % 64 == 0
  const uint32_t col = q - t * nvec;
  store_stream(y + q, combine_column<KMAX, kBF16, kCacheIn>(eo, w + (size_t)t * k,
                                                            pos + (size_t)t * k, k, nvec, col,
                                                            nrows));
}

template <int KMAX>
hipError_t go(const void* eo, bool bf16, const float* w, const int32_t* pos, int k,
              uint32_t nvec, uint32_t total, uint32_t nrows, void* y, hipStream_t s) {
  const unsigned grid = (total + kBlock - 1) / kBlock;
  const v4u* in = static_cast<const v4u*>(eo);
  v4u* out = static_cast<v4u*>(y);
  // the expert rows (nrows x nvec vectors) decide the policy, as in the expert stage
  const bool cache = (int64_t)nrows * nvec * 16 <= kCacheReuseBytes;
  const bool uniform = kCombineUniform && nvec % kWave == 0 && (cache || kStreamUniform);
  auto run = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kBlock), 0, s, in, w, pos, k, nvec, total, nrows, out);
  };
  auto pick = [&](auto bf, auto ca) {
    constexpr bool B = decltype(bf)::value, C = decltype(ca)::value;
    return uniform ? run(combine_kernel<KMAX, B, C, true>) : run(combine_kernel<KMAX, B, C, false>);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (bf16) return cache ? pick(T_{}, T_{}) : pick(T_{}, F_{});
  return cache ? pick(F_{}, T_{}) : pick(F_{}, F_{});
}

}  // namespace

hipError_t launch_combine(const void* expert_out, int dtype, const float* w, const int32_t* pos,
                          int T, int k, int64_t H, int64_t eo_rows, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool bf16 = dtype == 1;
  const uint32_t nvec = (uint32_t)(H * (bf16 ? 2 : 4) / 16);
  const uint32_t total = (uint32_t)T * nvec;
  const uint32_t nrows = (uint32_t)eo_rows;
  if (k <= 2) return go<2>(expert_out, bf16, w, pos, k, nvec, total, nrows, y, s);
  if (k <= 4) return go<4>(expert_out, bf16, w, pos, k, nvec, total, nrows, y, s);
  if (k <= 8) return go<8>(expert_out, bf16, w, pos, k, nvec, total, nrows, y, s);
  if (k <= 16) return go<16>(expert_out, bf16, w, pos, k, nvec, total, nrows, y, s);
  return go<32>(expert_out, bf16, w, pos, k, nvec, total, nrows, y, s);
}

}  // namespace moe
