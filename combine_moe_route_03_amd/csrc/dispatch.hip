// dispatch.hip -- counts, offsets, stable positions and the permute copy.
//
// The top-k index set is the send-count matrix of the all-to-all (irregular
// AllToAll page, "link to other primitives"); dispatch replaces one-hot matrix
// products by count + scan + index (MoE systems survey section 4.1) and places
// same-expert rows contiguously (survey section 1.1, EP flow step 2).
//
// Three kernels, all on the caller's stream:
//   count_kernel  one block per chunk of picks: LDS histogram -> hist[chunk][E]
//   place_kernel  one block per chunk: prefix of earlier chunks + bucket-order
//                 exclusive scan (every block redoes the E-long scan in LDS, so
//                 no separate scan launch is needed); block 0 publishes counts
//                 and offsets; then stable in-chunk ranks from wave64 ballots
//                 (bit-sliced match on the expert id, popcount of lower lanes)
//                 and an LDS prefix across the block's four waves.
//   copy_kernel   flat over (token, 16-byte column): one load of x, k stores.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kMaxE = 1024;

__global__ __launch_bounds__(kBlock) void count_kernel(const int32_t* __restrict__ idx,
                                                       int64_t npicks, int64_t chunk, int E,
                                                       int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxE];
  for (int e = threadIdx.x; e < E; e += kBlock) h[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * chunk;
  const int64_t p1 = (p0 + chunk < npicks) ? p0 + chunk : npicks;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += kBlock) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBlock) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(kBlock) void place_kernel(
    const int32_t* __restrict__ idx, int64_t npicks, int64_t chunk, int nb, int k, int E, int R,
    int W, const int32_t* __restrict__ hist, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ wave_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token) {
  __shared__ int32_t run[kMaxE];      // next free row per expert for this block
  __shared__ int32_t cnt[kMaxE];      // total picks per expert
  __shared__ int32_t off[kMaxE];      // first row of each expert's bucket
  __shared__ int32_t wcnt[4][kMaxE];  // per-wave counts inside one 256-pick batch
  __shared__ int32_t part[4];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid >> 6;
  const int b = blockIdx.x;
  const int L = E / R, LW = L / W;

  for (int e = tid; e < E; e += kBlock) {
    wcnt[0][e] = 0;
    wcnt[1][e] = 0;
    wcnt[2][e] = 0;
    wcnt[3][e] = 0;
  }
  // 1. Picks of expert e in earlier chunks (run) and in all chunks (cnt).
  for (int e = tid; e < E; e += kBlock) {
    int pre = 0, all = 0;
    for (int bb = 0; bb < nb; ++bb) {
      const int v = hist[(int64_t)bb * E + e];
      all += v;
      pre += (bb < b) ? v : 0;
    }
    run[e] = pre;
    cnt[e] = all;
  }
  __syncthreads();

  // 2. Exclusive scan of cnt over buckets in (wave, rank, slot) order; thread
  //    tid owns buckets 4*tid .. 4*tid+3 (E <= 1024 = 4 * 256).
  int c[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 4 * tid + q;
    c[q] = (j < E) ? cnt[bucket_expert(j, R, L, LW)] : 0;
    sum += c[q];
  }
  int incl = sum;
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) part[wid] = incl;
  __syncthreads();
  int excl = incl - sum, total = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    excl += (q < wid) ? part[q] : 0;
    total += part[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 4 * tid + q;
    if (j < E) off[bucket_expert(j, R, L, LW)] = excl;
    excl += c[q];
  }
  __syncthreads();

  if (b == 0) {
    for (int e = tid; e < E; e += kBlock) {
      expert_counts[e] = cnt[e];
      expert_offsets[e] = off[e];
    }
    for (int q = tid; q < W * R; q += kBlock) {  // q = w * R + r: buckets q*LW .. q*LW+LW-1
      int s = 0;
      for (int j = q * LW; j < q * LW + LW; ++j) s += cnt[bucket_expert(j, R, L, LW)];
      rank_counts[q] = s;
      rank_offsets[q] = off[bucket_expert(q * LW, R, L, LW)];
    }
    for (int w = tid; w <= W; w += kBlock)
      wave_offsets[w] = (w < W) ? off[bucket_expert(w * R * LW, R, L, LW)] : total;
  }
  for (int e = tid; e < E; e += kBlock) run[e] += off[e];
  __syncthreads();

  // 3. Stable ranks inside the chunk, 256 picks per batch.
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const int64_t p0 = (int64_t)b * chunk;
  const int64_t p1 = (p0 + chunk < npicks) ? p0 + chunk : npicks;
  for (int64_t base = p0; base < p1; base += kBlock) {
    const int64_t p = base + tid;
    const int e = (p < p1) ? idx[p] : -1;
    const bool valid = (p < p1) && ((unsigned)e < (unsigned)E);
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t bal = __ballot(valid && set);
      peers &= set ? bal : ~bal;
    }
    const int rk = __popcll(peers & lanemask_lt());
    const int nw = __popcll(peers);
    const bool leader = valid && (rk == nw - 1);
    if (leader) wcnt[wid][e] = nw;
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int q = 0; q < wid; ++q) before += wcnt[q][e];
      const int P = run[e] + before + rk;
      pos[p] = P;
      if ((uint64_t)P < (uint64_t)npicks) row_token[P] = (int32_t)(p / k);
    } else if (p < p1) {
      pos[p] = -1;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&run[e], nw);
      wcnt[wid][e] = 0;
    }
    __syncthreads();
  }
}

// send[pos[t][i]][c] = x[t][c] for 16-byte columns c; each x vector loaded once.
template <int U>
__global__ __launch_bounds__(kBlock) void copy_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ pos, int k,
                                                      uint32_t nvec, uint32_t total,
                                                      uint32_t nrows, uint4* __restrict__ send) {
  const uint32_t q0 = blockIdx.x * (uint32_t)(kBlock * U) + threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t q = q0 + u * kBlock;
    v[u] = (q < total) ? x[q] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t q = q0 + u * kBlock;
    if (q < total) {
      const uint32_t t = q / nvec, col = q - t * nvec;
      const int32_t* pp = pos + (size_t)t * k;
      for (int i = 0; i < k; ++i) {
        const int32_t P = pp[i];
        if ((uint32_t)P < nrows) send[(size_t)P * nvec + col] = v[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_count(const int32_t* idx, int64_t npicks, int E, int32_t* hist,
                        hipStream_t s) {
  const int64_t nb = num_chunks(npicks);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(count_kernel, dim3((unsigned)nb), dim3(kBlock), 0, s, idx, npicks,
                     chunk_picks(npicks), E, hist);
  return hipGetLastError();
}

hipError_t launch_place(const int32_t* idx, int64_t npicks, int k, int E, int R, int W,
                        const int32_t* hist, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                        int32_t* pos, int32_t* row_token, hipStream_t s) {
  const int64_t nb = num_chunks(npicks);
  // With no picks one block still runs to publish zero counts and offsets.
  const unsigned grid = nb == 0 ? 1u : (unsigned)nb;
  hipLaunchKernelGGL(place_kernel, dim3(grid), dim3(kBlock), 0, s, idx, npicks,
                     chunk_picks(npicks), (int)nb, k, E, R, W, hist, expert_counts,
                     expert_offsets, rank_counts, rank_offsets, wave_offsets, pos, row_token);
  return hipGetLastError();
}

hipError_t launch_copy(const void* x, const int32_t* pos, int T, int k, int64_t row_bytes,
                       void* send, hipStream_t s) {
  if (T == 0) return hipSuccess;
  constexpr int U = 4;
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  const uint32_t total = (uint32_t)T * nvec;
  const uint32_t nrows = (uint32_t)T * (uint32_t)k;
  const unsigned grid = (unsigned)((total + kBlock * U - 1) / (kBlock * U));
  hipLaunchKernelGGL((copy_kernel<U>), dim3(grid), dim3(kBlock), 0, s,
                     static_cast<const uint4*>(x), pos, k, nvec, total, nrows,
                     static_cast<uint4*>(send));
  return hipGetLastError();
}

}  // namespace moe
