// combine.hip -- gate-weighted combine back to token order (MoE systems
// survey, crad.ict.ac.cn, section 1.1, eq. (1) y = sum_i G(x)_i E_i(x), and EP
// flow step 4: restore the original order, weight by the gate confidence).
//
// Flat over (token, 16-byte column): each thread gathers its column from the k
// expert rows of its token (all k loads issued before any arithmetic; each
// expert row is read exactly once; through the caches when the expert rows fit
// the cache-reuse budget, as the expert stage has just written them there,
// streaming otherwise), runs the
// fp32 fused multiply-add chain in pick order (seeded with -0, the additive
// identity, so an all -0 sum stays -0), rounds once to the output dtype
// and writes one 16-byte vector. Lanes of a wave cover consecutive columns of
// one row, so every gather and the store are contiguous 1 KiB segments.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 256;

template <int KMAX, bool kBF16, bool kCacheIn>
__global__ __launch_bounds__(kBlock) void combine_kernel(const v4u* __restrict__ eo,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ pos, int k,
                                                         uint32_t nvec, uint32_t total,
                                                         uint32_t nrows, v4u* __restrict__ y) {
  const uint32_t q = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
  if (q >= total) return;
  const uint32_t t = q / nvec, col = q - t * nvec;
  const int32_t* pp = pos + (size_t)t * k;
  const float* ww = w + (size_t)t * k;

  v4u v[KMAX];
  float wt[KMAX];
  bool ok[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    ok[i] = false;
    wt[i] = 0.f;
    v[i] = v4u{0u, 0u, 0u, 0u};
    if (i < k) {
      const int32_t P = pp[i];
      wt[i] = ww[i];
      ok[i] = (uint32_t)P < nrows;
      if (ok[i]) {
        const v4u* src = eo + (size_t)P * nvec + col;
        v[i] = kCacheIn ? *src : load_stream(src);
      }
    }
  }

  v4u out;
  if constexpr (kBF16) {
    float a[8] = {-0.f, -0.f, -0.f, -0.f, -0.f, -0.f, -0.f, -0.f};  // -0: additive identity
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k && ok[i]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[2 * j] = fmaf(wt[i], bf16_lo(v[i][j]), a[2 * j]);
          a[2 * j + 1] = fmaf(wt[i], bf16_hi(v[i][j]), a[2 * j + 1]);
        }
      }
    }
    out = v4u{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
              pack_bf16x2(a[6], a[7])};
  } else {
    float a[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k && ok[i]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = fmaf(wt[i], __uint_as_float(v[i][j]), a[j]);
      }
    }
    out = v4u{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
              __float_as_uint(a[3])};
  }
  store_stream(y + q, out);
}

template <int KMAX>
hipError_t go(const void* eo, bool bf16, const float* w, const int32_t* pos, int k,
              uint32_t nvec, uint32_t total, uint32_t nrows, void* y, hipStream_t s) {
  const unsigned grid = (total + kBlock - 1) / kBlock;
  const v4u* in = static_cast<const v4u*>(eo);
  v4u* out = static_cast<v4u*>(y);
  // the expert rows (nrows x nvec vectors) decide the policy, as in the expert stage
  const bool cache = (int64_t)nrows * nvec * 16 <= kCacheReuseBytes;
  auto run = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kBlock), 0, s, in, w, pos, k, nvec, total, nrows, out);
  };
  if (bf16) return cache ? run(combine_kernel<KMAX, true, true>) : run(combine_kernel<KMAX, true, false>);
  return cache ? run(combine_kernel<KMAX, false, true>) : run(combine_kernel<KMAX, false, false>);
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
