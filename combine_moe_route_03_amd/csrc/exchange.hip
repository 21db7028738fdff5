// exchange.hip -- the expert-parallel exchange of R ranks emulated on one
// device (MoE systems survey, crad.ict.ac.cn, section 1.1, EP flow steps 2-4;
// irregular AllToAll page, "sources of irregular a2a": each (source,
// destination) pair has its own row count, possibly zero, as Alltoallv takes).
//
// Layouts (rows; offsets absolute in the concatenated buffers):
//   send   source s at rows [s*P, (s+1)*P), P = picks per source, buckets in
//          (wave, destination, slot) order;
//   recv   (destination, wave, source) messages back to back;
//   grouped (expert, source) segments back to back: every destination's rows
//          by local expert, then source; over all destinations plain expert
//          order, token order inside an expert.
//
// Kernels:
//   vsrc_plan_kernel     one block: recv_counts = the (source, wave, dest)
//                        send counts transposed, recv_offsets their exclusive
//                        scan, expert counts (column sums of the per-source
//                        counts) and the grouped expert offsets.
//   regroup_plan_kernel  per (expert, source) segment of the grouped layout:
//                        its first grouped row, its length, and its first row in
//                        recv (the destination's message of that source and
//                        wave, past the earlier slots of the wave).
//   segcopy_kernel       moves whole rows between two layouts described by a
//                        segment table. One side ("key") is the concatenation
//                        of the segments in table order; a block takes 2048
//                        16-byte vectors of it, two waves find its first and
//                        last segment with a 64-way search (three probes for
//                        8192 segments), the segments in between go to LDS,
//                        and each thread walks them while it moves 4 vectors
//                        at a time (all loads before the stores). Forward
//                        writes the key side, back reads it. Loads stream;
//                        stores go through the caches when the output fits
//                        the cache-reuse budget (the next stage reads it).
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kPlanBlock = 1024;

// sum of p[i * stride] for i in [0, n): eight independent loads in flight per
// round instead of one load-add dependence per element.
__device__ __forceinline__ int64_t sum_strided(const int32_t* __restrict__ p, int n,
                                               int64_t stride) {
  int64_t acc = 0;
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(i + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; i < n; ++i) acc += p[(int64_t)i * stride];
  return acc;
}
constexpr int kPlanWaves = kPlanBlock / kWave;

// Exclusive scan of v over the block (kPlanBlock threads), carried through
// part[]; returns this thread's exclusive prefix and the block total in *tot.
__device__ int64_t block_excl_scan(int64_t v, int64_t* part, int64_t* tot) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  int64_t incl = v;
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) part[wid] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int q = 0; q < kPlanWaves; ++q) {
    before += q < wid ? part[q] : 0;
    all += part[q];
  }
  __syncthreads();  // part is reused by the next call
  *tot = all;
  return before + incl - v;
}

__global__ __launch_bounds__(kPlanBlock) void vsrc_plan_kernel(
    int R, int W, int E, const int32_t* __restrict__ src_counts,
    const int32_t* __restrict__ send_counts, int32_t* __restrict__ recv_counts,
    int32_t* __restrict__ recv_offsets, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets) {
  __shared__ int64_t part[kPlanWaves];
  const int tid = threadIdx.x;
  const int n3 = R * W * R;
  // recv entry i = (d*W + w)*R + s is send entry (s*W + w)*R + d. Thread tid
  // owns entries [tid*per, (tid+1)*per): their sum goes through one block
  // scan, then a second pass (L2 hits) writes counts and offsets.
  const int per = (n3 + kPlanBlock - 1) / kPlanBlock;
  const int i0 = tid * per < n3 ? tid * per : n3;
  const int i1 = i0 + per < n3 ? i0 + per : n3;
  const auto sent = [&](int i) -> int32_t {
    const int s = i % R, w = (i / R) % W, d = i / (R * W);
    return send_counts[((int64_t)s * W + w) * R + d];
  };
  int64_t mine = 0;
  for (int i = i0; i < i1; i += 8) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i + u < i1 ? sent(i + u) : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) mine += v[u];
  }
  int64_t tot;
  int64_t run = block_excl_scan(mine, part, &tot);
  for (int i = i0; i < i1; i += 8) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i + u < i1 ? sent(i + u) : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i + u < i1) {
        recv_counts[i + u] = v[u];
        recv_offsets[i + u] = (int32_t)run;
        run += v[u];
      }
    }
  }
  int64_t carry = 0;
  for (int e0 = 0; e0 < E; e0 += kPlanBlock) {
    const int e = e0 + tid;
    const int64_t c = e < E ? sum_strided(src_counts + e, R, E) : 0;
    int64_t tot;
    const int64_t ex = block_excl_scan(c, part, &tot);
    if (e < E) {
      expert_counts[e] = (int32_t)c;
      expert_offsets[e] = (int32_t)(carry + ex);
    }
    carry += tot;
  }
}

// Segment t = e*R + s, one thread each: its first grouped row (the expert's
// offset plus the counts of the earlier sources for that expert) and the first
// row of the other side: in recv, the source's message of that destination and
// wave plus the counts of the wave's earlier slots; or, for the direct
// exchange (src_offsets non-null), the source's own bucket of expert e in send.
__global__ __launch_bounds__(256) void regroup_plan_kernel(
    int R, int W, int E, const int32_t* __restrict__ src_counts,
    const int32_t* __restrict__ recv_offsets, const int32_t* __restrict__ src_offsets,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ grp_start,
    int32_t* __restrict__ seg_count, int32_t* __restrict__ other) {
  const int L = E / R, LW = L / W;
  const int64_t nseg = (int64_t)E * R;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nseg; t += stride) {
    const int e = (int)(t / R), s = (int)(t % R);
    const int d = e / L, j = e % L, w = j / LW;
    grp_start[t] = (int32_t)(expert_offsets[e] + sum_strided(src_counts + e, s, E));
    seg_count[t] = src_counts[(int64_t)s * E + e];
    if (src_offsets != nullptr) {
      other[t] = src_offsets[(int64_t)s * E + e];
    } else {
      const int32_t* row = src_counts + (int64_t)s * E + (int64_t)d * L;
      other[t] = (int32_t)(recv_offsets[((int64_t)d * W + w) * R + s] +
                           sum_strided(row + w * LW, j - w * LW, 1));
    }
  }
}

constexpr int kSegBlock = 256;
constexpr int kSegU = 4;      // vectors per thread in flight
constexpr int kSegIters = 2;  // batches per block (at most)
constexpr int kSegVecs = kSegBlock * kSegU * kSegIters;
constexpr int kSpan = 512;    // segments of one block staged in LDS

// Largest i in [0, nseg) with key[i] <= r, by one full wave (uniform result).
// Each round probes 64 evenly spaced entries; the probes at or below r form a
// prefix of the lanes (key is non-decreasing), whose length picks the
// sub-range.
__device__ int find_segment(const int32_t* __restrict__ key, int nseg, int64_t r) {
  const int lane = threadIdx.x & (kWave - 1);
  int lo = 0, hi = nseg;
  while (hi - lo > 1) {
    const int step = (hi - lo + kWave - 1) / kWave;
    const int p = lo + lane * step;
    const bool ok = p < hi && (int64_t)key[p] <= r;
    int c = __popcll(__ballot(ok));
    c = c < 1 ? 1 : c;
    lo += (c - 1) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

// The other side's entry of segment i: the same index, or for the exchange
// the (source, wave, destination) entry of the (destination, wave, source)
// segment i.
template <bool kTranspose>
__device__ __forceinline__ int64_t other_index(int i, int R, int W) {
  if constexpr (kTranspose) {
    const int s = i % R, w = (i / R) % W, d = i / (R * W);
    return ((int64_t)s * W + w) * R + d;
  } else {
    return i;
  }
}

// Block b moves key-side vectors [b*vpb, (b+1)*vpb). Waves 0 and 1
// find the segments of its first and last row; the segments in between
// (their key-side begin and end and other-side begin) are staged in LDS, so
// each thread's walk from segment to segment reads LDS. A block spanning more
// than kSpan segments (many empty ones) binary-searches the tables in memory.
template <bool kBack, bool kTranspose, bool kCacheOut>
__global__ __launch_bounds__(kSegBlock) void segcopy_kernel(
    const v4u* __restrict__ in, v4u* __restrict__ out, const int32_t* __restrict__ key,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ other, int nseg, int R, int W,
    uint32_t nvec, int64_t key_rows, int64_t other_rows, int vpb) {
  __shared__ int32_t s_beg[kSpan], s_end[kSpan], s_oth[kSpan];
  __shared__ int s_seg[2];
  // rows of the key side in use: the end of the last segment
  int64_t total = (int64_t)key[nseg - 1] + cnt[nseg - 1];
  total = total < key_rows ? total : key_rows;
  const int64_t nq = total * nvec;
  const int64_t q0 = (int64_t)blockIdx.x * vpb;
  if (q0 >= nq) return;
  const int64_t qe = q0 + vpb < nq ? q0 + vpb : nq;
  const int tid = threadIdx.x, wid = tid / kWave;
  if (wid < 2) {
    const int f = find_segment(key, nseg, (wid == 0 ? q0 : qe - 1) / nvec);
    if ((tid & (kWave - 1)) == 0) s_seg[wid] = f;
  }
  __syncthreads();
  const int seg0 = s_seg[0];
  const int span = s_seg[1] - seg0 + 1;
  const bool staged = span <= kSpan;  // uniform over the block
  if (staged) {
    for (int i = tid; i < span; i += kSegBlock) {
      const int g = seg0 + i;
      const int32_t b = key[g];
      s_beg[i] = b;
      s_end[i] = b + cnt[g];
      s_oth[i] = other[other_index<kTranspose>(g, R, W)];
    }
    __syncthreads();
  }
  const auto seg_beg = [&](int i) -> int64_t { return staged ? s_beg[i] : key[seg0 + i]; };
  const auto seg_end = [&](int i) -> int64_t {
    return staged ? s_end[i] : (int64_t)key[seg0 + i] + cnt[seg0 + i];
  };
  const auto seg_oth = [&](int i) -> int64_t {
    return staged ? s_oth[i] : other[other_index<kTranspose>(seg0 + i, R, W)];
  };

  int seg = 0;  // relative to seg0; items of a thread come in increasing order
#pragma unroll 1
  for (int it = 0; it * kSegU * kSegBlock < vpb; ++it) {
    int64_t src[kSegU], dst[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
      // the vector index space is below 2^31 (checked by the entry points)
      const uint32_t q = (uint32_t)q0 + (it * kSegU + u) * kSegBlock + tid;
      src[u] = -1;
      dst[u] = -1;
      if ((int64_t)q >= qe) continue;
      const uint32_t rq = q / nvec;
      const int64_t r = rq, col = q - rq * nvec;
      if (staged) {
        while (seg + 1 < span && r >= seg_end(seg)) ++seg;
      } else {
        // many (mostly empty) segments: binary search for the last one that
        // begins at or before r, from the thread's current one
        int lo = seg, hi = span - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (seg_beg(mid) <= r) lo = mid;
          else hi = mid - 1;
        }
        seg = lo;
      }
      const int64_t b = seg_beg(seg), o = seg_oth(seg) + (r - b);
      if (r < b || r >= seg_end(seg) || o < 0 || o >= other_rows) continue;  // inconsistent tables
      src[u] = (kBack ? r : o) * nvec + col;
      dst[u] = (kBack ? o : r) * nvec + col;
    }
    v4u v[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u)
      if (src[u] >= 0) v[u] = load_stream(in + src[u]);
#pragma unroll
    for (int u = 0; u < kSegU; ++u)
      if (dst[u] >= 0) {
        if constexpr (kCacheOut) out[dst[u]] = v[u];
        else store_stream(out + dst[u], v[u]);
      }
  }
}

template <bool kTranspose>
hipError_t segcopy(const void* in, void* out, const int32_t* key, const int32_t* cnt,
                   const int32_t* other, int nseg, int R, int W, int64_t row_bytes,
                   int64_t key_rows, int64_t other_rows, bool back, hipStream_t s) {
  if (key_rows == 0 || nseg == 0) return hipSuccess;
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  const int64_t nq = key_rows * nvec;
  // vectors per block: kSegVecs, or fewer (down to one per thread) while the
  // grid would stay under 2048 blocks (8 per compute unit)
  int vpb = kSegVecs;
  while (vpb > kSegBlock && (nq + vpb - 1) / vpb < 2048) vpb >>= 1;
  const unsigned grid = (unsigned)((nq + vpb - 1) / vpb);
  const v4u* i = static_cast<const v4u*>(in);
  v4u* o = static_cast<v4u*>(out);
  // loads stream (each row is read once)
  auto go = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kSegBlock), 0, s, i, o, key, cnt, other, nseg, R, W,
                  nvec, key_rows, other_rows, vpb);
  };
  // Outputs that fit the cache-reuse budget are stored through the caches: the
  // next stage reads them right after, from the Infinity Cache (zipf, 8 ranks:
  // each copy 37.5 -> 33.5 us, and the stages reading their output faster too;
  // step 259 -> 235 us).
  const int64_t out_rows = back ? other_rows : key_rows;
  const bool cache = out_rows * row_bytes <= kCacheReuseBytes;
  if (cache)
    return back ? go(segcopy_kernel<true, kTranspose, true>)
                : go(segcopy_kernel<false, kTranspose, true>);
  return back ? go(segcopy_kernel<true, kTranspose, false>)
              : go(segcopy_kernel<false, kTranspose, false>);
}

}  // namespace

hipError_t launch_vsrc_plan(int R, int W, int E, const int32_t* src_counts,
                            const int32_t* send_counts, int32_t* recv_counts,
                            int32_t* recv_offsets, int32_t* expert_counts,
                            int32_t* expert_offsets, hipStream_t s) {
  return launch(vsrc_plan_kernel, dim3(1), dim3(kPlanBlock), 0, s, R, W, E, src_counts,
                send_counts, recv_counts, recv_offsets, expert_counts, expert_offsets);
}

hipError_t launch_vsrc_exchange(const void* in, void* out, int64_t row_bytes, int64_t rows, int R,
                                int W, const int32_t* send_offsets, const int32_t* recv_counts,
                                const int32_t* recv_offsets, bool back, hipStream_t s) {
  // key side: recv (segments (d, w, s) in table order); other side: send
  return segcopy<true>(in, out, recv_offsets, recv_counts, send_offsets, R * W * R, R, W,
                       row_bytes, rows, rows, back, s);
}

// Grouped layout against recv (regroup) or against send (direct exchange).
static hipError_t grouped_copy(const void* in, void* out, int64_t row_bytes, int64_t rows, int E, int R,
                        int W, const int32_t* src_counts, const int32_t* recv_offsets,
                        const int32_t* src_offsets, const int32_t* expert_offsets,
                        int32_t* tables, bool back, hipStream_t s) {
  const int64_t nseg = (int64_t)E * R;
  int32_t* grp_start = tables;
  int32_t* seg_count = tables + nseg;
  int32_t* other = tables + 2 * nseg;
  const int64_t want = (nseg + 255) / 256;
  const unsigned grid = (unsigned)(want < 1024 ? want : 1024);
  hipError_t e = launch(regroup_plan_kernel, dim3(grid), dim3(256), 0, s, R, W, E, src_counts,
                        recv_offsets, src_offsets, expert_offsets, grp_start, seg_count, other);
  if (e != hipSuccess) return e;
  // key side: grouped
  return segcopy<false>(in, out, grp_start, seg_count, other, (int)nseg, R, W, row_bytes, rows,
                        rows, back, s);
}

hipError_t launch_vsrc_regroup(const void* in, void* out, int64_t row_bytes, int64_t rows, int E,
                               int R, int W, const int32_t* src_counts,
                               const int32_t* recv_offsets, const int32_t* expert_offsets,
                               int32_t* tables, bool back, hipStream_t s) {
  return grouped_copy(in, out, row_bytes, rows, E, R, W, src_counts, recv_offsets, nullptr,
                      expert_offsets, tables, back, s);
}

hipError_t launch_vsrc_direct(const void* in, void* out, int64_t row_bytes, int64_t rows, int E,
                              int R, int W, const int32_t* src_counts, const int32_t* src_offsets,
                              const int32_t* expert_offsets, int32_t* tables, bool back,
                              hipStream_t s) {
  return grouped_copy(in, out, row_bytes, rows, E, R, W, src_counts, nullptr, src_offsets,
                      expert_offsets, tables, back, s);
}

}  // namespace moe
