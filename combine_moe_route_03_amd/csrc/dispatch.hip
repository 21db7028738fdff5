// dispatch.hip -- counts, offsets, stable positions and the permute copy.
//
// The top-k index set is the send-count matrix of the all-to-all (irregular
// AllToAll page, "link to other primitives"); dispatch replaces one-hot matrix
// products by count + scan + index (MoE systems survey section 4.1) and places
// same-expert rows contiguously (survey section 1.1, EP flow step 2).
//
// Four kernels, all on the caller's stream:
//   count_kernel  one 1024-thread block per chunk of picks: LDS histogram ->
//                 hist[chunk][E] (LDS integer atomics: order-free, exact).
//   place_kernel  one block (256 to 1024 threads) per chunk. Each block
//                 re-derives what it
//                 needs from the small hist matrix instead of waiting for a
//                 separate scan launch: the prefix of earlier chunks and the
//                 totals (threads laid out as (row slice, expert) so all loads
//                 are independent), then the bucket-order exclusive scan (one
//                 bucket per thread). Block 0 publishes counts and offsets.
//                 Stable in-chunk ranks come from wave64 ballots (bit-sliced
//                 match on the expert id, popcount of lower lanes) and an LDS
//                 prefix across the block's waves; the next batch of ids is
//                 prefetched while the current one is placed.
//                 The optional statistics come from one extra block, or from
//                 the last placing block when the placing blocks fill the chip.
//   copy_kernel   flat over (token, 16-byte column): one streaming load of x,
//                 k stores; a wave's k positions through the scalar cache.
//   pad_kernel    capacity layout: zero rows past each bucket's kept picks.
//
// Source shards: count and place also run over nsrc equal shards of the picks
// at once (the virtual source ranks of the emulated exchange). Shard s owns
// spc consecutive chunks and hist rows, its own buckets at rows
// [s*src_picks, (s+1)*src_picks), and its own slice of every count and offset
// output; with one shard this is the plain single-rank dispatch.
#include <type_traits>

#include "block_stats.h"
#include "device.h"
#include "index_tables.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kB = kIndexBlock;  // counting block: 1024 threads, 16 waves
constexpr int kMaxE = kIndexMaxE;
// placing blocks resident at once: one per compute unit (1024 threads, ~86 KiB
// LDS; smaller blocks are chosen only for grids far below this)
constexpr int kPlaceResident = 256;

// Picks [p0, p1) of block b: chunk b - src*spc of shard src.
__device__ __forceinline__ void chunk_range(int b, int spc, int nsrc, int64_t chunk,
                                            int64_t src_picks, int& src, int64_t& p0,
                                            int64_t& p1) {
  src = spc > 0 ? b / spc : 0;
  if (src > nsrc - 1) src = nsrc - 1;
  const int64_t end = (int64_t)(src + 1) * src_picks;
  p0 = (int64_t)src * src_picks + (int64_t)(b - src * spc) * chunk;
  p1 = p0 + chunk < end ? p0 + chunk : end;
}

__global__ __launch_bounds__(kB) void count_kernel(const int32_t* __restrict__ idx, int nsrc,
                                                   int spc, int64_t src_picks, int64_t chunk,
                                                   int E, int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxE];
  const int tid = threadIdx.x;
  if (tid < E) h[tid] = 0;
  __syncthreads();
  int src;
  int64_t p0, p1;
  chunk_range(blockIdx.x, spc, nsrc, chunk, src_picks, src, p0, p1);
  for (int64_t base = p0; base < p1; base += 4 * kB) {
    int ev[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t p = base + u * kB + tid;
      ev[u] = (p < p1) ? idx[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&h[ev[u]], 1);
  }
  __syncthreads();
  if (tid < E) hist[(int64_t)blockIdx.x * E + tid] = h[tid];
}

template <int NT>
__global__ __launch_bounds__(NT) void place_kernel(
    const int32_t* __restrict__ idx, int64_t npicks, int nsrc, int spc, int64_t src_picks,
    int64_t chunk, int k, int E, int elog, int R, int W, const int32_t* __restrict__ hist,
    int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ wave_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token, moe_stats_t* __restrict__ stats,
    int sblock, int cap) {
  // cap >= 0: capacity-factor layout (every bucket exactly cap rows, an expert
  // keeps its first cap picks in token order, later ones are dropped);
  // cap < 0: buckets sized by the counts. Capacity runs with one shard only.
  __shared__ int32_t run[kMaxE];           // next free row per expert for this block
  __shared__ int32_t cnt[kMaxE];           // total picks per expert
  __shared__ int32_t off[kMaxE];           // first row of each expert's bucket
  constexpr int NW = NT / kWave;           // waves of the block
  __shared__ int32_t ppre[NT];             // (slice, expert) partial prefix
  __shared__ int32_t pall[NT];             // (slice, expert) partial total
  __shared__ __attribute__((aligned(16))) int32_t wcnt[NW][kMaxE];  // per-wave counts of a batch
  __shared__ int32_t part[NW];
  static_assert(sizeof(wcnt) >= sizeof(StatsScratch), "statistics scratch lives in wcnt");

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = blockIdx.x;
  const int L = E / R, LW = L / W;
  const int ep = 1 << elog;        // E rounded up to a power of two
  const int64_t rows = cap < 0 ? npicks : (int64_t)E * cap;  // rows of the send buffer
  const int nslice = NT >> elog;   // row slices of the hist matrix
  // This block's shard: hist rows [h0, h1), rows from base, outputs at slice src.
  int src;
  int64_t p0, p1;
  chunk_range(b, spc, nsrc, chunk, src_picks, src, p0, p1);
  const int h0 = src * spc, h1 = h0 + spc;
  const int64_t base = (int64_t)src * src_picks;
  // This chunk's first batch of ids, loaded now so that its latency overlaps
  // the histogram read and the scans below.
  int e_next = (p0 + tid < p1) ? idx[p0 + tid] : -1;

  if (tid < E) {
#pragma unroll
    for (int q = 0; q < NW; ++q) wcnt[q][tid] = 0;
  }

  // 1. Picks of each expert in the shard's earlier chunks and in all its
  //    chunks. Thread (s, e) = (tid >> elog, tid & (ep-1)) sums rows h0+s,
  //    h0+s+nslice, ...
  {
    const int e = tid & (ep - 1), s = tid >> elog;
    int pre = 0, all = 0;
    if (e < E) {
      for (int r0 = h0 + s; r0 < h1; r0 += 4 * nslice) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = r0 + u * nslice;
          v[u] = (r < h1) ? hist[(int64_t)r * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          all += v[u];
          pre += (r0 + u * nslice < b) ? v[u] : 0;
        }
      }
    }
    if (ep < kWave) {
      // the 64 / ep slices of a wave hold the same experts: fold them by lane
      // exchanges, then the wave's sums are its row of the partials (16 rows
      // left to add instead of 1024 / ep; local layer index 8.9 -> 8.0 us)
      for (int o = ep; o < kWave; o <<= 1) {
        pre += __shfl_xor(pre, o);
        all += __shfl_xor(all, o);
      }
      if (lane < ep) {
        ppre[wid * ep + lane] = pre;
        pall[wid * ep + lane] = all;
      }
    } else {
      ppre[tid] = pre;
      pall[tid] = all;
    }
  }
  __syncthreads();
  const int nrow = ep < kWave ? NW : nslice;  // partial rows
  // The statistics: an extra block past the placing ones computes them and
  // leaves, or (when the placing blocks already fill the chip) placing block
  // sblock computes them after its own placement.
  const bool stats_here = stats != nullptr && b == sblock;
  if (stats_here && sblock >= nsrc * spc) {
    if (tid < E) {
      int A = 0;
      for (int s = 0; s < nrow; ++s) A += pall[s * ep + tid];
      cnt[tid] = A;
    }
    __syncthreads();
    block_stats(cnt, E, R, *reinterpret_cast<StatsScratch*>(&wcnt[0][0]), stats);
    return;
  }

  // 2. Totals, bucket offsets in (wave, rank, slot) order (with a capacity
  //    every bucket is cap rows long) and this block's first free row of each
  //    bucket, one bucket per thread. The shard's first block publishes its
  //    counts and offsets.
  const int total =
      bucket_scan<NT>(ppre, pall, nrow, ep, E, R, W, cap, base, cnt, off, run, part);
  if (b == h0)
    publish_index<NT>(cnt, off, total, E, R, W, cap, base, expert_counts + (int64_t)src * E,
                  expert_offsets + (int64_t)src * E, rank_counts + (int64_t)src * W * R,
                  rank_offsets + (int64_t)src * W * R, wave_offsets + (int64_t)src * (W + 1));

  // 3. Stable ranks inside the chunk, NT picks per batch.
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  for (int64_t base_p = p0; base_p < p1; base_p += NT) {
    const int64_t p = base_p + tid;
    const int e = e_next;
    e_next = (p + NT < p1) ? idx[p + NT] : -1;  // prefetch the next batch
    const bool valid = (p < p1) && ((unsigned)e < (unsigned)E);
    const int rel = batch_rank(e, valid, nbits, wcnt, run, base_p + NT >= p1);
    if (valid) {
      const int P = cap < 0 ? rel : (rel < cap ? off[e] + rel : -1);
      pos[p] = P;
      if (row_token && P >= 0 && (int64_t)P < rows) row_token[P] = (int32_t)(p / k);
    } else if (p < p1) {
      pos[p] = -1;
    }
  }
  if (stats_here) {
    __syncthreads();  // wcnt, the statistics scratch, is free again
    block_stats(cnt, E, R, *reinterpret_cast<StatsScratch*>(&wcnt[0][0]), stats);
  }
}

// send[pos[t][i]][c] = x[t][c] for 16-byte columns c: each x vector is loaded
// once (streaming load) and stored k times. A block covers U * kCopyBlock
// consecutive (token, column) vectors, U per thread, all loads issued before
// the stores. With rows a multiple of 64 vectors (kUniform) the 64 lanes of a
// wave share one token, so the token and its k positions are wave-uniform and
// come through the scalar cache, all k read before the first store.
constexpr int kCopyBlock = 256;
constexpr bool kCopyTwo = true;
// Blocks of kCopyBlock threads resident at once on the chip (256 compute
// units, 32 waves each).
constexpr int64_t kCopyResident = 256 * 32 / (kCopyBlock / kWave);

template <int KMAX, bool kUniform, int U>
__global__ __launch_bounds__(kCopyBlock) void copy_kernel(const v4u* __restrict__ x,
                                                          const int32_t* __restrict__ pos, int k,
                                                          uint32_t nvec, uint32_t total,
                                                          uint32_t nrows, v4u* __restrict__ send) {
  const uint32_t q0 = blockIdx.x * (uint32_t)(kCopyBlock * U) + threadIdx.x;
  v4u v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t q = q0 + u * kCopyBlock;
    if (q < total) v[u] = load_stream(x + q);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t q = q0 + u * kCopyBlock;
    if (q >= total) continue;  // with kUniform, whole waves (total % 64 == 0)
    uint32_t t = q / nvec;
    if constexpr (kUniform) t = __builtin_amdgcn_readfirstlane(t);
    const uint32_t col = q - t * nvec;
    const int32_t* pp = pos + (size_t)t * k;
    int32_t P[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) P[i] = (i < k) ? pp[i] : -1;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if ((uint32_t)P[i] < nrows) send[(size_t)P[i] * nvec + col] = v[u];
  }
}

// Zero padding of the capacity layout: the gridDim.y blocks of column j fill
// bucket j's rows past the kept ones with zero vectors (interleaved by block)
// and mark them row_token = -1.
__global__ __launch_bounds__(kCopyBlock) void pad_kernel(int E, int R, int W, int cap,
                                                         const int32_t* __restrict__ kept,
                                                         uint32_t nvec, v4u* __restrict__ send,
                                                         int32_t* __restrict__ row_token) {
  const int j = blockIdx.x, L = E / R, LW = L / W;
  const int e = bucket_expert(j, R, L, LW);
  const int64_t r0 = (int64_t)j * cap + kept[e], r1 = (int64_t)(j + 1) * cap;
  const int64_t first = (int64_t)blockIdx.y * kCopyBlock + threadIdx.x;
  const int64_t step = (int64_t)gridDim.y * kCopyBlock;
  for (int64_t r = r0 + first; r < r1; r += step) row_token[r] = -1;
  const int64_t n = (r1 - r0) * nvec;
  for (int64_t q = first; q < n; q += step) send[r0 * nvec + q] = v4u{0u, 0u, 0u, 0u};
}

// Threads of a placing block: 1024, or fewer (a power of two from 256) when
// that still holds one bucket per thread, the whole chunk in one batch and the
// block's read of the nb x E histogram in one round of four loads a thread,
// and (with statistics) leaves at least eight threads per value for the pair
// sums; the block's barriers then span fewer waves (local layer index 7.4-7.7
// -> 6.7-6.8 us). Measured no better or slower otherwise: zipf (larger
// histogram), dirichlet_waves (19.2 -> 26.0 us: more load rounds a block),
// decode_hot (statistics block with four threads per value, 6.4 -> 6.8 us).
int place_threads(int E, int64_t chunk, int64_t nb, bool stats) {
  const int64_t ep = pow2_at_least(E);
  int nt = 256;
  while (nt < kIndexBlock &&
         (nt < ep || nt < chunk || nb * ep > 4 * nt || (stats && nt < 8 * ep)))
    nt <<= 1;
  return nt;
}

template <typename... A>
hipError_t launch_place_kernel(int nt, unsigned grid, hipStream_t s, A... a) {
  switch (nt) {
    case 256: return launch(place_kernel<256>, dim3(grid), dim3(256), 0, s, a...);
    case 512: return launch(place_kernel<512>, dim3(grid), dim3(512), 0, s, a...);
    default: return launch(place_kernel<kIndexBlock>, dim3(grid), dim3(kIndexBlock), 0, s, a...);
  }
}

int ilog2_ceil(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

}  // namespace

hipError_t launch_count(const int32_t* idx, int64_t npicks, int E, int32_t* hist,
                        hipStream_t s) {
  const int64_t nb = num_chunks(npicks, E);
  if (nb == 0) return hipSuccess;
  return launch(count_kernel, dim3((unsigned)nb), dim3(kB), 0, s, idx, 1, (int)nb, npicks,
                chunk_picks(npicks, E), E, hist);
}

hipError_t launch_place_chunks(const int32_t* idx, int64_t npicks, int64_t chunk, int nb, int k,
                               int E, int R, int W, const int32_t* hist, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* rank_counts,
                               int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                               int32_t* row_token, moe_stats_t* stats, int cap, hipStream_t s) {
  // With no picks one block still runs to publish zero counts and offsets. The
  // statistics come from one extra block after the placing blocks, unless
  // those already take every compute unit (one 1024-thread block each): the
  // extra block would then wait for a second round (dirichlet_waves, 256
  // chunks: 26.5 us against 13.6 without statistics), so the last placing
  // block computes them after its placement (19.1 us; block 0, which also
  // publishes the tables, 20.4).
  const int nplace = nb == 0 ? 1 : nb;
  const bool in_place = stats != nullptr && nplace >= kPlaceResident;
  const int sblock = in_place ? nplace - 1 : nplace;
  const unsigned grid = (unsigned)nplace + (stats != nullptr && !in_place ? 1u : 0u);
  const int nt = place_threads(E, chunk, nplace, stats != nullptr);
  return launch_place_kernel(nt, grid, s, idx, npicks, 1, nb, npicks, chunk, k, E, ilog2_ceil(E),
                             R, W, hist, expert_counts, expert_offsets, rank_counts, rank_offsets,
                             wave_offsets, pos, row_token, stats, sblock, cap);
}

hipError_t launch_place(const int32_t* idx, int64_t npicks, int k, int E, int R, int W,
                        const int32_t* hist, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                        int32_t* pos, int32_t* row_token, hipStream_t s) {
  return launch_place_chunks(idx, npicks, chunk_picks(npicks, E), (int)num_chunks(npicks, E), k,
                             E, R, W, hist, expert_counts, expert_offsets, rank_counts,
                             rank_offsets, wave_offsets, pos, row_token, nullptr, -1, s);
}

hipError_t launch_copy(const void* x, const int32_t* pos, int T, int k, int64_t row_bytes,
                       int64_t send_rows, void* send, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  const uint32_t total = (uint32_t)T * nvec;
  const uint32_t nrows = (uint32_t)send_rows;
  const bool uniform = nvec % kWave == 0;
  // Two vectors a thread when one a thread would need between one and two
  // rounds of resident blocks: the launch then fits one round (zipf-sized
  // copies measured 10% faster); larger copies measured best at one.
  const int64_t blocks1 = ((int64_t)total + kCopyBlock - 1) / kCopyBlock;
  const bool two = kCopyTwo && blocks1 > kCopyResident && blocks1 <= 2 * kCopyResident;
  auto go = [&](auto kmax) {
    constexpr int KM = decltype(kmax)::value;
    auto run = [&](auto kernel, int u) {
      const unsigned grid = (unsigned)((total + kCopyBlock * u - 1) / (kCopyBlock * u));
      return launch(kernel, dim3(grid), dim3(kCopyBlock), 0, s, static_cast<const v4u*>(x), pos,
                    k, nvec, total, nrows, static_cast<v4u*>(send));
    };
    if (two) return uniform ? run(copy_kernel<KM, true, 2>, 2) : run(copy_kernel<KM, false, 2>, 2);
    return uniform ? run(copy_kernel<KM, true, 1>, 1) : run(copy_kernel<KM, false, 1>, 1);
  };
  if (k <= 2) return go(std::integral_constant<int, 2>{});
  if (k <= 4) return go(std::integral_constant<int, 4>{});
  if (k <= 8) return go(std::integral_constant<int, 8>{});
  if (k <= 16) return go(std::integral_constant<int, 16>{});
  return go(std::integral_constant<int, 32>{});
}

hipError_t launch_pad(int E, int R, int W, int cap, const int32_t* kept, int64_t row_bytes,
                      void* send, int32_t* row_token, hipStream_t s) {
  if (cap == 0) return hipSuccess;
  // enough blocks per bucket for ~4096 in all (a bucket's padding is at most
  // cap rows), so that the fill is not limited to E blocks
  const int64_t vecs = (int64_t)cap * (row_bytes / 16);
  int64_t per = (vecs + kCopyBlock - 1) / kCopyBlock;
  const int64_t want = (4096 + E - 1) / E;
  if (per > want) per = want;
  if (per < 1) per = 1;
  return launch(pad_kernel, dim3((unsigned)E, (unsigned)per), dim3(kCopyBlock), 0, s, E, R, W,
                cap, kept, (uint32_t)(row_bytes / 16), static_cast<v4u*>(send), row_token);
}

// Source shards: nsrc shards of src_picks picks, spc chunks each (spc >= 1).
void source_chunks(int64_t src_picks, int E, int64_t& chunk, int& spc) {
  const int64_t n = num_chunks(src_picks, E);
  spc = n < 1 ? 1 : (int)n;
  chunk = chunk_picks(src_picks, E);
}

hipError_t launch_count_sources(const int32_t* idx, int nsrc, int64_t src_picks, int E,
                                int32_t* hist, hipStream_t s) {
  int64_t chunk;
  int spc;
  source_chunks(src_picks, E, chunk, spc);
  return launch(count_kernel, dim3((unsigned)(nsrc * spc)), dim3(kB), 0, s, idx, nsrc, spc,
                src_picks, chunk, E, hist);
}

hipError_t launch_place_sources(const int32_t* idx, int nsrc, int64_t src_picks, int k, int E,
                                int R, int W, const int32_t* hist, int32_t* expert_counts,
                                int32_t* expert_offsets, int32_t* rank_counts,
                                int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                                hipStream_t s) {
  int64_t chunk;
  int spc;
  source_chunks(src_picks, E, chunk, spc);
  return launch_place_kernel(kIndexBlock, (unsigned)(nsrc * spc), s, idx,
                (int64_t)nsrc * src_picks, nsrc, spc, src_picks, chunk, k, E, ilog2_ceil(E), R, W,
                hist, expert_counts, expert_offsets, rank_counts, rank_offsets, wave_offsets, pos,
                (int32_t*)nullptr, (moe_stats_t*)nullptr, -1, -1);
}

}  // namespace moe
