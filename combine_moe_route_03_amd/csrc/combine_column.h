// combine_column.h -- one 16-byte column of one token's gate-weighted sum
// (MoE systems survey, crad.ict.ac.cn, section 1.1, eq. (1) y = sum_i
// G(x)_i E_i(x)): the column gathered from the token's k expert rows, an fp32
// fused multiply-add chain in pick order seeded with -0 (the additive
// identity, so an all -0 sum stays -0), rounded once to the output dtype.
// Shared by the one-pass combine and the per-wave combine, which therefore
// produce the same bits for a token.
#pragma once

#include "device.h"

namespace moe {

// Token-uniform waves (rows a multiple of 64 vectors, so a wave's 64 columns
// share one token): its k positions and weights come through the scalar
// cache. Used for cached rows; on streamed rows the vector path measured
// faster (351 against 357 us on k = 8 over 14 KiB rows).
constexpr bool kCombineUniform = true;
constexpr bool kStreamUniform = false;

// Gathers in flight per thread on streamed rows (rows read once, bypassing
// the caches): one, with the positions through the vector path; on k = 8 over
// 14 KiB rows that measured 351 us against 357 (scalar positions) and 365-368
// (all eight in flight), and on k = 2 the same or better.
constexpr int kStreamGroup = 1;

// pp, ww: the token's k positions and weights. Picks whose position is
// outside [0, nrows) contribute nothing. kCacheIn: rows read through the
// caches (the expert stage has just written them there), all k gathers in
// flight; otherwise streamed, kStreamGroup at a time.
template <int KMAX, bool kBF16, bool kCacheIn>
__device__ __forceinline__ v4u combine_column(const v4u* __restrict__ eo,
                                              const float* __restrict__ ww,
                                              const int32_t* __restrict__ pp, int k,
                                              uint32_t nvec, uint32_t col, uint32_t nrows) {
  // every position and weight first (one wait), then the gathers in groups of
  // kGroup, each group issued back to back and then accumulated (pick order is
  // kept). A pick without a row loads row 0 (discarded) instead of branching
  // around the load, so no gather result has to land before the next issue.
  int32_t P[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    P[i] = (i < k) ? pp[i] : -1;
    wt[i] = (i < k) ? ww[i] : 0.f;
  }
  constexpr int kGroup = kCacheIn ? KMAX : kStreamGroup;
  constexpr int G = kGroup < KMAX ? kGroup : KMAX;
  float a[8] = {-0.f, -0.f, -0.f, -0.f, -0.f, -0.f, -0.f, -0.f};  // -0: additive identity
#pragma unroll
  for (int g0 = 0; g0 < KMAX; g0 += G) {
    v4u v[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = g0 + j;
      if (i < k) {
        const bool ok = (uint32_t)P[i] < nrows;
        const v4u* src = eo + (ok ? (size_t)P[i] * nvec : 0) + col;
        v[j] = kCacheIn ? *src : load_stream(src);
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = g0 + j;
      if (i < k && (uint32_t)P[i] < nrows) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (kBF16) {
            a[2 * c] = fmaf(wt[i], bf16_lo(v[j][c]), a[2 * c]);
            a[2 * c + 1] = fmaf(wt[i], bf16_hi(v[j][c]), a[2 * c + 1]);
          } else {
            a[c] = fmaf(wt[i], __uint_as_float(v[j][c]), a[c]);
          }
        }
      }
    }
  }
  return kBF16 ? v4u{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                     pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])}
               : v4u{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                     __float_as_uint(a[3])};
}

}  // namespace moe
