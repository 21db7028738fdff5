// dispatch_small.hip -- the whole dispatch (counts, offsets, stable positions,
// the optional skew statistics and the permute copy) in one launch for small
// batches: at most one 1024-pick batch, the decode regime, where each separate
// launch costs more than its work.
//
// The steps are those of the separate kernels: the counts of S, the
// bucket-order scan and the stable positions (MoE systems survey section 4.1:
// count + scan + index; irregular AllToAll page: Alltoallv counts and
// displacements), the per-rank and per-expert skew statistics (DODOCO summary,
// "metrics"), then the permute copy (explainer section 3 item 5). With all
// picks in one block no step needs a device-wide ordering point: every block
// reads all T*k expert ids (4 KiB at most, from L2 after the first block) and
// places all picks itself (integer arithmetic, a fixed order: the same result
// in every block), then copies its own share of the (token, 16-byte column)
// vectors, whose loads are issued before the placing work so that their
// latency is hidden under it. Block 0 writes the index outputs; the
// statistics come from one extra block that does not copy.
#include <type_traits>

#include "block_stats.h"
#include "device.h"
#include "index_tables.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kNT = kIndexBlock;  // 1024 threads: one pick of the batch each
constexpr int kNW = kNT / kWave;
// x vectors a thread loads up front: one, so the copy spreads over twice the
// blocks of two (decode: 64 compute units instead of 32; dispatch 10.0-10.1
// -> 9.0-9.3 us; 255 blocks of a quarter vector a thread measured the same)
constexpr int kVecs = 1;

template <int KMAX>
__global__ __launch_bounds__(kNT) void dispatch_small_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int k, int R, int W,
    const v4u* __restrict__ x, uint32_t nvec, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ wave_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token, moe_stats_t* __restrict__ stats,
    v4u* __restrict__ send) {
  __shared__ int32_t s_row[kNT];  // send row of each pick, -1 when dropped
  __shared__ int32_t hist[kIndexMaxE];
  __shared__ int32_t zero[kIndexMaxE];
  __shared__ int32_t cnt[kIndexMaxE];
  __shared__ int32_t off[kIndexMaxE];
  __shared__ int32_t run[kIndexMaxE];
  __shared__ __attribute__((aligned(16))) int32_t wcnt[kNW][kIndexMaxE];
  __shared__ int32_t part[kNW];
  static_assert(sizeof(wcnt) >= sizeof(StatsScratch), "statistics scratch lives in wcnt");

  const int tid = threadIdx.x;
  const int npicks = T * k;  // <= kNT
  const bool stats_block = stats != nullptr && blockIdx.x == gridDim.x - 1;
  const int ncopy = gridDim.x - (stats != nullptr ? 1 : 0);  // blocks that copy

  // This block's first x vectors, loaded before the placing work (their
  // latency overlaps it); further vectors, if any, are loaded in the copy loop.
  const uint32_t nv = (uint32_t)T * nvec;
  const uint32_t stride = (uint32_t)ncopy * kNT;
  v4u xv[kVecs];
#pragma unroll
  for (int u = 0; u < kVecs; ++u) {
    const uint32_t q = blockIdx.x * (uint32_t)kNT + tid + u * stride;
    if (!stats_block && q < nv) xv[u] = load_stream(x + q);
  }

  const bool in_batch = tid < npicks;
  const int e = in_batch ? topk_idx[tid] : -1;
  const bool valid = in_batch && (unsigned)e < (unsigned)E;
  if (tid < E) {
    hist[tid] = 0;
    zero[tid] = 0;
#pragma unroll
    for (int q = 0; q < kNW; ++q) wcnt[q][tid] = 0;
  }
  __syncthreads();

  // Counts (LDS integer atomics: order-free), the bucket scan in (wave, rank,
  // slot) order, the published tables.
  if (valid) atomicAdd(&hist[e], 1);
  __syncthreads();
  const int total = bucket_scan<kNT>(zero, hist, 1, E, E, R, W, -1, 0, cnt, off, run, part);
  if (stats_block) {
    block_stats(cnt, E, R, *reinterpret_cast<StatsScratch*>(&wcnt[0][0]), stats);
    return;
  }
  if (blockIdx.x == 0)
    publish_index<kNT>(cnt, off, total, E, R, W, -1, 0, expert_counts, expert_offsets,
                       rank_counts, rank_offsets, wave_offsets);

  // Stable positions: the whole batch in one pass.
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const int row = batch_rank(e, valid, nbits, wcnt, run, true);
  if (in_batch) {
    s_row[tid] = valid ? row : -1;
    if (blockIdx.x == 0) {
      pos[tid] = valid ? row : -1;
      if (valid) row_token[row] = tid / k;
    }
  }
  __syncthreads();

  // This block's share of the copy: k stores of each x vector.
  uint32_t q = blockIdx.x * (uint32_t)kNT + tid;
  for (int u = 0; q < nv; ++u, q += stride) {
    v4u v;
    if (u < kVecs) {
#pragma unroll
      for (int j = 0; j < kVecs; ++j)
        if (j == u) v = xv[j];
    } else {
      v = load_stream(x + q);
    }
    const uint32_t t = q / nvec, col = q - t * nvec;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const int P = (i < k) ? s_row[t * k + i] : -1;
      if (P >= 0) send[(size_t)P * nvec + col] = v;
    }
  }
}

}  // namespace

bool dispatch_one_launch(int64_t npicks, int E) { return npicks > 0 && npicks <= kNT && E <= kIndexMaxE; }

hipError_t launch_dispatch_small(const int32_t* topk_idx, int T, int E, int k, int R, int W,
                                 const void* x, int64_t row_bytes, int32_t* expert_counts,
                                 int32_t* expert_offsets, int32_t* rank_counts,
                                 int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                                 int32_t* row_token, moe_stats_t* stats, void* send,
                                 hipStream_t s) {
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  // copy blocks: kVecs vectors a thread, at most one block per compute unit
  // (~90 KiB of LDS each), plus the statistics block
  const int64_t nv = (int64_t)T * nvec;
  int64_t blocks = (nv + (int64_t)kNT * kVecs - 1) / ((int64_t)kNT * kVecs);
  blocks = blocks < 1 ? 1 : (blocks > 255 ? 255 : blocks);
  if (stats != nullptr) ++blocks;
  auto run = [&](auto kernel) {
    return launch(kernel, dim3((unsigned)blocks), dim3(kNT), 0, s, topk_idx, T, E, k, R, W,
                  static_cast<const v4u*>(x), nvec, expert_counts, expert_offsets, rank_counts,
                  rank_offsets, wave_offsets, pos, row_token, stats, static_cast<v4u*>(send));
  };
  if (k <= 2) return run(dispatch_small_kernel<2>);
  if (k <= 8) return run(dispatch_small_kernel<8>);
  return run(dispatch_small_kernel<32>);
}

}  // namespace moe
