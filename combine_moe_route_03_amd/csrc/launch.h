// launch.h -- internal host-side launchers, one per kernel family. The C ABI
// (abi.hip) validates arguments and then calls these; they only size grids and
// launch on the given stream. Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_ext.h>

#include "../../include/moe_route.h"
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- chunking
// Counting and placing cut the T*k picks into chunks of whole 1024-pick
// batches (one 1024-thread block per chunk). Every place block re-reads all
// chunk histograms (chunks x E int32), so the chunk count is capped at
// 65536 / pow2(E) (and 512) to keep that read at most 256 KiB per block.
constexpr int kIndexBlock = 1024;

inline int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Most chunks (hist rows) a placing pass reads for E experts.
inline int64_t max_index_chunks(int E) {
  const int64_t m = 65536 / pow2_at_least(E);
  return m > 512 ? 512 : m;
}

inline int64_t chunk_picks(int64_t npicks, int E) {
  const int64_t max_chunks = max_index_chunks(E);
  int64_t c = (npicks + max_chunks - 1) / max_chunks;
  c = (c + kIndexBlock - 1) / kIndexBlock * kIndexBlock;
  return c < kIndexBlock ? kIndexBlock : c;
}

inline int64_t num_chunks(int64_t npicks, int E) {
  if (npicks == 0) return 0;
  const int64_t c = chunk_picks(npicks, E);
  return (npicks + c - 1) / c;
}

// ----------------------------------------------------------- cache policy
// The expert rows are written by one kernel and gathered by the combine right
// after. While that buffer fits comfortably in the 256 MB Infinity Cache (at
// most half of it) both sides go through the caches and the combine reads it
// from there; beyond that both stream (non-temporal), which measured faster
// for buffers of a few GB.
constexpr int64_t kCacheReuseBytes = int64_t(128) << 20;

// ------------------------------------------------------------ kernel timing
// Optional per-thread timing events (benchmark hook; see
// moe_set_timing_events): while armed, the i-th kernel launched (i < n) records
// start[i] when it begins executing and stop[i] when it ends.
constexpr int kMaxTimedLaunches = 8;
struct LaunchTiming {
  hipEvent_t start[kMaxTimedLaunches] = {};
  hipEvent_t stop[kMaxTimedLaunches] = {};
  int n = 0;         // armed pairs
  int launched = 0;  // kernels launched since arming
};
LaunchTiming& launch_timing();

template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t shmem,
                  hipStream_t s, Args... args) {
  LaunchTiming& tm = launch_timing();
  if (tm.n > 0) {
    const int i = tm.launched++;
    hipEvent_t a = i < tm.n ? tm.start[i] : nullptr;
    hipEvent_t b = i < tm.n ? tm.stop[i] : nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, a, b, 0u, static_cast<Params>(args)...);
  } else {
    kernel<<<grid, block, shmem, s>>>(static_cast<Params>(args)...);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s);

// hist: [num_chunks][E] int32 workspace.
hipError_t launch_count(const int32_t* idx, int64_t npicks, int E, int32_t* hist, hipStream_t s);

hipError_t launch_place(const int32_t* idx, int64_t npicks, int k, int E, int R, int W,
                        const int32_t* hist, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                        int32_t* pos, int32_t* row_token, hipStream_t s);

// Routing fused with counting: hist[b][E] for blocks of
// route_count_tokens_per_block(T, E, k) tokens (at most max_index_chunks(E)
// blocks), then placing with chunks of that many tokens' picks; with `stats`
// non-null one extra place block writes the skew statistics.
int route_count_tokens_per_block(int T, int E, int k);
hipError_t launch_route_count(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                              int32_t* hist, hipStream_t s);
hipError_t launch_place_chunks(const int32_t* idx, int64_t npicks, int64_t chunk, int nb, int k,
                               int E, int R, int W, const int32_t* hist, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* rank_counts,
                               int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                               int32_t* row_token, moe_stats_t* stats, int cap, hipStream_t s);

// Counts, offsets, positions, the statistics (stats may be null) and the
// dispatch copy in one launch; only for dispatch_one_launch(T*k, E) (all picks
// in one 1024-pick batch). Ids outside [0, E) are dropped picks.
bool dispatch_one_launch(int64_t npicks, int E);
hipError_t launch_dispatch_small(const int32_t* topk_idx, int T, int E, int k, int R, int W,
                                 const void* x, int64_t row_bytes, int32_t* expert_counts,
                                 int32_t* expert_offsets, int32_t* rank_counts,
                                 int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                                 int32_t* row_token, moe_stats_t* stats, void* send,
                                 hipStream_t s);

// Row copies; row_bytes is a multiple of 16.
hipError_t launch_copy(const void* x, const int32_t* pos, int T, int k, int64_t row_bytes,
                       int64_t send_rows, void* send, hipStream_t s);
// Capacity layout: zero rows and row_token = -1 past each bucket's kept rows.
hipError_t launch_pad(int E, int R, int W, int cap, const int32_t* kept, int64_t row_bytes,
                      void* send, int32_t* row_token, hipStream_t s);

hipError_t launch_expert_scale(const void* in, int dtype, int64_t rows, int64_t H, int E, int R,
                               int W, const int32_t* expert_offsets,
                               const int32_t* expert_counts, void* out, hipStream_t s);

// The identity-scaled experts on the rows of one expert wave w (bounds read
// from wave_offsets on the device).
hipError_t launch_expert_scale_wave(const void* in, int dtype, int64_t rows_max, int64_t H, int E,
                                    int R, int W, const int32_t* expert_offsets,
                                    const int32_t* expert_counts, const int32_t* wave_offsets,
                                    int w, void* out, hipStream_t s);

// expert_out has eo_rows rows; picks with pos outside [0, eo_rows) are skipped.
hipError_t launch_combine(const void* expert_out, int dtype, const float* w, const int32_t* pos,
                          int T, int k, int64_t H, int64_t eo_rows, void* y, hipStream_t s);

hipError_t launch_stats(const int32_t* counts, int E, int R, void* out, hipStream_t s);

// The wave schedule's combine: the tokens listed by completion wave (a count
// and a place launch of nb blocks of tpb tokens; hist: [nb][W] int32
// workspace), then the combine of the tokens of completion waves [w0, w1)
// (the one-pass combine's arithmetic; rows are the T*k of the plain layout).
void combine_order_blocks(int64_t T, int W, int64_t& tpb, int64_t& nb);
hipError_t launch_combine_order(const int32_t* pos, int T, int k, const int32_t* wave_offsets,
                                int W, int32_t* token_wave_offsets, int32_t* token_order,
                                int32_t* hist, hipStream_t s);
hipError_t launch_combine_waves(const void* expert_out, int dtype, const float* w,
                                const int32_t* pos, int T, int k, int64_t H,
                                const int32_t* token_order, const int32_t* token_wave_offsets,
                                int w0, int w1, void* y, hipStream_t s);
// What the wave pipelines need to combine each wave's completed tokens (y
// null: no combine in the pipeline), and the stream for those combines (null:
// the copy stream).
struct WaveCombine {
  const float* w = nullptr;
  const int32_t* pos = nullptr;
  const int32_t* token_order = nullptr;
  const int32_t* token_wave_offsets = nullptr;
  void* y = nullptr;
  hipStream_t stream = nullptr;
};

// Virtual source shards (the emulated exchange): nsrc shards of src_picks
// picks; hist holds nsrc * source_chunks rows of E. Each shard's counts and
// offsets go to its own slice ([nsrc][E], [nsrc][W*R], [nsrc][W+1]); positions
// are absolute rows with shard s at [s*src_picks, (s+1)*src_picks).
void source_chunks(int64_t src_picks, int E, int64_t& chunk, int& spc);
hipError_t launch_count_sources(const int32_t* idx, int nsrc, int64_t src_picks, int E,
                                int32_t* hist, hipStream_t s);
hipError_t launch_place_sources(const int32_t* idx, int nsrc, int64_t src_picks, int k, int E,
                                int R, int W, const int32_t* hist, int32_t* expert_counts,
                                int32_t* expert_offsets, int32_t* rank_counts,
                                int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                                hipStream_t s);
// Receive side of the exchange and the grouped expert layout from the
// per-source counts ([R][E]) and send counts ([R][W][R]).
hipError_t launch_vsrc_plan(int R, int W, int E, const int32_t* src_counts,
                            const int32_t* send_counts, int32_t* recv_counts,
                            int32_t* recv_offsets, int32_t* expert_counts,
                            int32_t* expert_offsets, hipStream_t s);
// Block transpose send -> recv (back: recv -> send); rows = buffer rows.
hipError_t launch_vsrc_exchange(const void* in, void* out, int64_t row_bytes, int64_t rows, int R,
                                int W, const int32_t* send_offsets, const int32_t* recv_counts,
                                const int32_t* recv_offsets, bool back, hipStream_t s);
// Direct exchange send -> grouped (back: grouped -> send): each (expert,
// source) segment straight from the source's bucket; tables as the regroup.
hipError_t launch_vsrc_direct(const void* in, void* out, int64_t row_bytes, int64_t rows, int E,
                              int R, int W, const int32_t* src_counts, const int32_t* src_offsets,
                              const int32_t* expert_offsets, int32_t* tables, bool back,
                              hipStream_t s);
// Receive-side regroup recv -> grouped (back: grouped -> recv); tables holds
// 3 * E * R int32.
hipError_t launch_vsrc_regroup(const void* in, void* out, int64_t row_bytes, int64_t rows, int E,
                               int R, int W, const int32_t* src_counts,
                               const int32_t* recv_offsets, const int32_t* expert_offsets,
                               int32_t* tables, bool back, hipStream_t s);

// Fitted symmetric Dirichlet alpha of E <= 1024 counts into one device double.
hipError_t launch_dirichlet_alpha(const int32_t* counts, int E, double* out, hipStream_t s);

// Grouped SwiGLU FFN (bf16): gate/up GEMM with fused SiLU*up into hbuf
// [rows][I], then the down GEMM into out [rows][H]. Needs I % 64 == 0 and
// H % 128 == 0.
// With a side stream the odd-id experts run there, forked from s by the event
// `fork` and joined back by `join` (both caller-owned); without, one chain.
hipError_t launch_expert_swiglu(const void* send, int64_t rows, int H, int I, int E,
                                const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                                const void* w_down, void* hbuf, void* out, hipStream_t s,
                                hipStream_t side, hipEvent_t fork, hipEvent_t join);

// The FFN on a subset of n experts: the i-th is expert (i / sg) * sstride +
// sbase + i % sg (all E experts: n = sg = E, sstride = sbase = 0).
hipError_t launch_expert_swiglu_subset(const void* send, int64_t rows, int H, int I, int n,
                                       int sg, int sstride, int sbase, const int32_t* offs,
                                       const int32_t* cnts, const void* w_gate_up,
                                       const void* w_down, void* hbuf, void* out, hipStream_t s);

// The gather dispatch of wave w's rows: send[r] = x[row_token[r]] for r in
// [wave_offsets[w], wave_offsets[w+1]) (read on the device).
hipError_t launch_gather_wave(const void* x, const int32_t* row_token, const int32_t* wave_offsets,
                              int w, int T, int64_t rows_max, int64_t row_bytes, void* send,
                              hipStream_t s);
// Wave-pipelined identity-scaled experts: per wave, gather dispatch of its rows
// on `copy`, then the experts of the wave on `compute` after an event, and
// (with wc.y) the combine of the wave's completed tokens on wc.stream, or on
// `copy` once the next wave's gather is queued; events holds at least 2 + 2W
// caller-owned events when a second stream is used.
hipError_t launch_scale_waves(const void* x, int T, int k, int64_t row_bytes, int dtype, int64_t H,
                              int E, int R, int W, const int32_t* row_token,
                              const int32_t* wave_offsets, const int32_t* offs,
                              const int32_t* cnts, void* send, void* out, const WaveCombine& wc,
                              hipStream_t compute, hipStream_t copy, const hipEvent_t* events);
// The same with the SwiGLU experts (copy == compute: the same work,
// serialised); `side` (may be null) carries the second chain of a wave's
// experts; events holds at least 2 + 4W caller-owned events when copy !=
// compute, side is non-null or wc.stream is a stream of its own.
hipError_t launch_swiglu_waves(const void* x, int T, int k, int H, int I, int E, int R, int W,
                               const int32_t* row_token, const int32_t* wave_offsets,
                               const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                               const void* w_down, void* send, void* hbuf, void* out,
                               const WaveCombine& wc, hipStream_t compute, hipStream_t copy,
                               hipStream_t side, const hipEvent_t* events);

// Expert id of the j-th bucket when buckets run in (wave, rank, slot) order:
// L = E / R slots per rank, LW = L / W slots per wave.
__host__ __device__ __forceinline__ int bucket_expert(int j, int R, int L, int LW) {
  const int per_wave = R * LW;
  const int w = j / per_wave;
  const int rem = j - w * per_wave;
  const int r = rem / LW;
  return r * L + w * LW + (rem - r * LW);
}

}  // namespace moe
