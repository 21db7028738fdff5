// index_tables.h -- block-level pieces of the placing kernel's index stage
// (blocks of NT <= 1024 threads, E <= NT, so thread j owns bucket j and expert j): the
// bucket scan, the published tables, the stable in-batch rank.
//
// The send buffer holds one bucket per expert in (wave, rank, slot) order
// (bucket_expert); the Alltoallv tables are the per-(wave, rank) sums and the
// first rows of those buckets (irregular AllToAll page, Alltoallv counts and
// displacements in rows).
#pragma once

#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kIndexMaxE = 1024;

// Inclusive prefix sum over the 64 lanes of a wave by DPP (the whole wave must
// be active): row_shr 1, 2, 4, 8 inside each row of 16 lanes (lanes shifted in
// from outside the row read 0), then row_bcast 15 (last lane of rows 0 and 2
// into rows 1 and 3) and row_bcast 31 (lane 31 into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Thread j < E owns bucket j of the (wave, rank, slot) order and its expert
// e = bucket_expert(j). It sums e's nrow partial rows (row stride ep) of the
// picks before this block (ppre) and of all picks (pall); the bucket sizes
// (that total, or cap for every bucket when cap >= 0) are scanned in bucket
// order, and the thread writes cnt[e] (total), off[e] (first row of the
// bucket, relative) and run[e] (next free row: picks before this block, plus
// base + off[e] without a capacity; with one the rank inside the bucket
// decides between a row and a drop, so it stays relative). Returns the total.
// Called by every thread of the NT-thread block (E <= NT); part holds NT / 64
// ints of LDS. Two barriers, the last at the end.
template <int NT>
__device__ __forceinline__ int bucket_scan(const int32_t* ppre, const int32_t* pall, int nrow,
                                           int ep, int E, int R, int W, int cap, int64_t base,
                                           int32_t* cnt, int32_t* off, int32_t* run,
                                           int32_t* part) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int L = E / R, LW = L / W;
  const int e = (tid < E) ? bucket_expert(tid, R, L, LW) : 0;
  int P = 0, A = 0;
  if (tid < E) {
    for (int s = 0; s < nrow; ++s) {
      P += ppre[s * ep + e];
      A += pall[s * ep + e];
    }
  }
  const int cj = (tid < E) ? (cap >= 0 ? cap : A) : 0;
  const int incl = wave_incl_scan(cj);  // DPP: no LDS round trips (local layer index 8.6 vs 8.9 us)
  if (lane == kWave - 1) part[wid] = incl;
  __syncthreads();
  int excl = incl - cj, total = 0;
#pragma unroll
  for (int q = 0; q < NT / kWave; ++q) {
    excl += (q < wid) ? part[q] : 0;
    total += part[q];
  }
  if (tid < E) {
    cnt[e] = A;
    off[e] = excl;
    run[e] = cap < 0 ? (int32_t)base + excl + P : P;
  }
  __syncthreads();
  return total;
}

// Counts and offsets of one dispatch (rows from `base`): expert_counts (kept
// rows: min(c, cap) with a capacity), expert_offsets, per-(wave, rank)
// rank_counts / rank_offsets (whole buckets) and wave_offsets[W+1], written by
// the NT threads of one block (E <= NT).
template <int NT>
__device__ __forceinline__ void publish_index(const int32_t* cnt, const int32_t* off, int total,
                                              int E, int R, int W, int cap, int64_t base,
                                              int32_t* ec, int32_t* eo, int32_t* rc, int32_t* ro,
                                              int32_t* wo) {
  const int tid = threadIdx.x;
  const int L = E / R, LW = L / W;
  if (tid < E) {
    ec[tid] = (cap >= 0 && cnt[tid] > cap) ? cap : cnt[tid];
    eo[tid] = (int32_t)(base + off[tid]);
  }
  for (int q = tid; q < W * R; q += NT) {  // q = w * R + r: buckets q*LW .. q*LW+LW-1
    int s = 0;
    for (int j = q * LW; j < q * LW + LW; ++j) s += cap >= 0 ? cap : cnt[bucket_expert(j, R, L, LW)];
    rc[q] = s;
    ro[q] = (int32_t)(base + off[bucket_expert(q * LW, R, L, LW)]);
  }
  for (int w = tid; w <= W; w += NT)
    wo[w] = (int32_t)(base + ((w < W) ? off[bucket_expert(w * R * LW, R, L, LW)] : total));
}

// Stable rank of this thread's pick (expert e, valid) among the block's picks
// of e so far: run[e] (earlier batches) + picks of e in lower waves of this
// batch + lower lanes of this wave (bit-sliced ballot match on the id,
// popcount of the lower peers). Then run[] advances by the batch's counts.
// wcnt must be zero for the experts used; it is left zero. Every thread of
// the block calls it (three barriers). After the block's last batch (`last`,
// uniform) nothing reads run or wcnt again: one barrier, neither is updated.
__device__ __forceinline__ int batch_rank(int e, bool valid, int nbits,
                                          int32_t (*wcnt)[kIndexMaxE], int32_t* run, bool last) {
  const int wid = threadIdx.x / kWave;
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
  int rel = 0;
  if (valid) {
    int before = 0;
    for (int q = 0; q < wid; ++q) before += wcnt[q][e];
    rel = run[e] + before + rk;
  }
  if (last) return rel;
  __syncthreads();
  if (leader) {
    atomicAdd(&run[e], nw);
    wcnt[wid][e] = 0;
  }
  __syncthreads();
  return rel;
}

}  // namespace moe
