// launch.h -- internal host-side launchers, one per kernel family. The C ABI
// (abi.hip) validates arguments and then calls these; they only size grids and
// launch on the given stream. Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// The T*k picks are cut into chunks for counting and placing: at least
// kMinChunkPicks picks each, at most kMaxChunks chunks, multiples of 256.
constexpr int64_t kMinChunkPicks = 2048;
constexpr int64_t kMaxChunks = 512;

inline int64_t chunk_picks(int64_t npicks) {
  int64_t c = (npicks + kMaxChunks - 1) / kMaxChunks;
  c = (c + 255) / 256 * 256;
  return c < kMinChunkPicks ? kMinChunkPicks : c;
}

inline int64_t num_chunks(int64_t npicks) {
  return npicks == 0 ? 0 : (npicks + chunk_picks(npicks) - 1) / chunk_picks(npicks);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s);

// hist: [num_chunks][E] int32 workspace.
hipError_t launch_count(const int32_t* idx, int64_t npicks, int E, int32_t* hist, hipStream_t s);

hipError_t launch_place(const int32_t* idx, int64_t npicks, int k, int E, int R, int W,
                        const int32_t* hist, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                        int32_t* pos, int32_t* row_token, hipStream_t s);

// Row copies; row_bytes is a multiple of 16.
hipError_t launch_copy(const void* x, const int32_t* pos, int T, int k, int64_t row_bytes,
                       void* send, hipStream_t s);

hipError_t launch_expert_scale(const void* in, int dtype, int64_t rows, int64_t H, int E, int R,
                               int W, const int32_t* expert_offsets,
                               const int32_t* expert_counts, void* out, hipStream_t s);

hipError_t launch_combine(const void* expert_out, int dtype, const float* w, const int32_t* pos,
                          int T, int k, int64_t H, void* y, hipStream_t s);

hipError_t launch_stats(const int32_t* counts, int E, int R, void* out, hipStream_t s);

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
