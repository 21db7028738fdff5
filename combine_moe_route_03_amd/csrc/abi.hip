// abi.hip -- the extern "C" entry points declared in include/moe_route.h.
// Every call validates its arguments on the host before touching the HIP
// runtime; on error it returns a negative moe_status and launches nothing.
#include "../../include/moe_route.h"
#include "launch.h"

#include <cmath>
#include <mutex>

namespace {

constexpr int64_t kIndexLimit = int64_t(1) << 31;  // flat 32-bit index spaces of the row kernels

int elem_bytes(int32_t dtype) {
  return dtype == MOE_F32 ? 4 : (dtype == MOE_BF16 ? 2 : 0);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const moe_shape* sh) {
  if (!sh) return MOE_ERR_ARG;
  if (sh->dtype != MOE_F32 && sh->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (sh->T < 0 || sh->H < 1 || sh->E < 1 || sh->E > 1024 || sh->k < 1 || sh->k > 32 ||
      sh->k > sh->E || sh->R < 1 || sh->W < 1)
    return MOE_ERR_ARG;
  if (sh->E % sh->R != 0) return MOE_ERR_ARG;
  if ((sh->E / sh->R) % sh->W != 0) return MOE_ERR_ARG;
  const int64_t row_bytes = int64_t(sh->H) * elem_bytes(sh->dtype);
  if (row_bytes % 16 != 0) return MOE_ERR_ALIGN;
  const int64_t picks = int64_t(sh->T) * sh->k;
  if (picks >= kIndexLimit) return MOE_ERR_ARG;
  if (picks * (row_bytes / 16) >= kIndexLimit) return MOE_ERR_ARG;
  return MOE_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Histogram rows of the fused routing + counting pass (one per routing block).
int64_t route_index_blocks(const moe_shape* sh) {
  if (sh->T == 0) return 0;
  const int64_t tpb = moe::route_count_tokens_per_block(sh->T, sh->E, sh->k);
  return (sh->T + tpb - 1) / tpb;
}

size_t workspace_bytes(const moe_shape* sh) {
  int64_t nb = moe::num_chunks(int64_t(sh->T) * sh->k, sh->E);
  const int64_t nr = route_index_blocks(sh);
  if (nr > nb) nb = nr;
  const int64_t bytes = (nb < 1 ? 1 : nb) * int64_t(sh->E) * 4;
  return size_t((bytes + 255) / 256 * 256);
}

// The index outputs (everything but the workspace).
int check_index_ptrs(const moe_shape* sh, const int32_t* topk_idx, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                     int32_t* wave_offsets, int32_t* pos, int32_t* row_token) {
  if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets || !wave_offsets)
    return MOE_ERR_ARG;
  if (sh->T > 0 && (!topk_idx || !pos || !row_token)) return MOE_ERR_ARG;
  const void* ptrs[] = {topk_idx, expert_counts, expert_offsets, rank_counts, rank_offsets,
                        wave_offsets, pos, row_token};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int check_index_args(const moe_shape* sh, const int32_t* topk_idx, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                     int32_t* wave_offsets, int32_t* pos, int32_t* row_token, void* workspace,
                     size_t workspace_bytes_given) {
  const int st = check_index_ptrs(sh, topk_idx, expert_counts, expert_offsets, rank_counts,
                                  rank_offsets, wave_offsets, pos, row_token);
  if (st != MOE_OK) return st;
  if (!workspace) return MOE_ERR_ARG;
  if (!aligned(workspace, 4)) return MOE_ERR_ALIGN;
  if (workspace_bytes_given < workspace_bytes(sh)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int check_copy_args(const moe_shape* sh, const void* x, const int32_t* pos, void* send_buf) {
  if (sh->T > 0 && (!x || !pos || !send_buf)) return MOE_ERR_ARG;
  if (!aligned(x, 16) || !aligned(send_buf, 16) || !aligned(pos, 4)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// Virtual-source exchange: equal source shards.
int check_vsrc_shape(const moe_shape* sh) {
  const int st = check_shape(sh);
  if (st != MOE_OK) return st;
  if (sh->T % sh->R != 0) return MOE_ERR_ARG;
  return MOE_OK;
}

// Per-source hist rows and wave offsets (dispatch), or the 3 * E * R segment
// table (regroup, direct exchange).
size_t vsrc_workspace_bytes(const moe_shape* sh) {
  int64_t chunk;
  int spc;
  moe::source_chunks(int64_t(sh->T / sh->R) * sh->k, sh->E, chunk, spc);
  const int64_t R = sh->R, E = sh->E;
  const int64_t disp = (R * spc * E + R * (sh->W + 1)) * 4;
  const int64_t regroup = 3 * E * R * 4;
  const int64_t bytes = disp > regroup ? disp : regroup;
  return size_t((bytes + 255) / 256 * 256);
}

// The per-wave combine's tables and the combine inputs; y == NULL means no
// combine (then the rest may be NULL too).
int check_wave_combine(const moe_shape* sh, const float* topk_w, const int32_t* pos,
                       const int32_t* token_order, const int32_t* token_wave_offsets,
                       const void* y) {
  if (!y) return MOE_OK;
  if (!token_wave_offsets) return MOE_ERR_ARG;
  if (sh->T > 0 && (!topk_w || !pos || !token_order)) return MOE_ERR_ARG;
  if (!aligned(y, 16) || !aligned(topk_w, 4) || !aligned(pos, 4) || !aligned(token_order, 4) ||
      !aligned(token_wave_offsets, 4))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

// A per-wave combine on a stream other than the compute stream (it then
// needs the events).
bool own_combine_stream(const void* y, moe_stream_t combine_stream, moe_stream_t compute_stream) {
  return y && combine_stream && combine_stream != compute_stream;
}

int check_events(void* const* events, int32_t n_events, int32_t need) {
  if (!events || n_events < need) return MOE_ERR_ARG;
  for (int32_t i = 0; i < need; ++i)
    if (!events[i]) return MOE_ERR_ARG;
  return MOE_OK;
}

int check_vsrc_move(const moe_shape* sh, int32_t direction, const void* in, const void* out) {
  if (direction != 0 && direction != 1) return MOE_ERR_ARG;
  if (sh->T > 0 && (!in || !out)) return MOE_ERR_ARG;
  if (!aligned(in, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

}  // namespace

namespace moe {
LaunchTiming& launch_timing() {
  thread_local LaunchTiming t;
  return t;
}
}  // namespace moe

extern "C" {

int moe_set_timing_events(void* const* start_events, void* const* stop_events, int32_t n) {
  moe::LaunchTiming& t = moe::launch_timing();
  if (n < 0 || n > moe::kMaxTimedLaunches) return MOE_ERR_ARG;
  if (n > 0 && (!start_events || !stop_events)) return MOE_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    t.start[i] = reinterpret_cast<hipEvent_t>(start_events[i]);
    t.stop[i] = reinterpret_cast<hipEvent_t>(stop_events[i]);
  }
  t.n = n;
  t.launched = 0;
  return MOE_OK;
}

int moe_timed_launches(void) { return moe::launch_timing().launched; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: null pointer or size/shape outside the limits";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: pointer or row size breaks the alignment rules";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unknown dtype";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: the HIP runtime rejected a launch";
    default: return "unknown moe_status";
  }
}

int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
              float* topk_w, moe_stream_t stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return MOE_ERR_ARG;
  if (int64_t(T) * k >= kIndexLimit || int64_t(T) * E >= (int64_t(1) << 40)) return MOE_ERR_ARG;
  if (T > 0 && (!logits || !topk_idx || !topk_w)) return MOE_ERR_ARG;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_ERR_ALIGN;
  return status_of(moe::launch_route(logits, T, E, k, topk_idx, topk_w, as_stream(stream)));
}

size_t moe_dispatch_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return workspace_bytes(shape);
}

int moe_dispatch_index(const moe_shape* shape, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                       int32_t* wave_offsets, int32_t* pos, int32_t* row_token, void* workspace,
                       size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  st = check_index_args(shape, topk_idx, expert_counts, expert_offsets, rank_counts,
                        rank_offsets, wave_offsets, pos, row_token, workspace,
                        workspace_bytes_given);
  if (st != MOE_OK) return st;
  const int64_t npicks = int64_t(shape->T) * shape->k;
  hipStream_t s = as_stream(stream);
  int32_t* hist = static_cast<int32_t*>(workspace);
  st = status_of(moe::launch_count(topk_idx, npicks, shape->E, hist, s));
  if (st != MOE_OK) return st;
  return status_of(moe::launch_place(topk_idx, npicks, shape->k, shape->E, shape->R, shape->W,
                                     hist, expert_counts, expert_offsets, rank_counts,
                                     rank_offsets, wave_offsets, pos, row_token, s));
}

int moe_route_index(const moe_shape* shape, const float* logits, int32_t* topk_idx,
                    float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                    int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                    int32_t* pos, int32_t* row_token, moe_stats_t* stats, void* workspace,
                    size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (int64_t(shape->T) * shape->E >= (int64_t(1) << 40)) return MOE_ERR_ARG;
  if (shape->T > 0 && (!logits || !topk_w)) return MOE_ERR_ARG;
  if (!aligned(logits, 4) || !aligned(topk_w, 4) || !aligned(stats, 8)) return MOE_ERR_ALIGN;
  st = check_index_args(shape, topk_idx, expert_counts, expert_offsets, rank_counts,
                        rank_offsets, wave_offsets, pos, row_token, workspace,
                        workspace_bytes_given);
  if (st != MOE_OK) return st;
  const int64_t npicks = int64_t(shape->T) * shape->k;
  const int64_t tpb = moe::route_count_tokens_per_block(shape->T, shape->E, shape->k);
  hipStream_t s = as_stream(stream);
  int32_t* hist = static_cast<int32_t*>(workspace);
  st = status_of(moe::launch_route_count(logits, shape->T, shape->E, shape->k, topk_idx, topk_w,
                                         hist, s));
  if (st != MOE_OK) return st;
  return status_of(moe::launch_place_chunks(
      topk_idx, npicks, tpb * shape->k, (int)route_index_blocks(shape), shape->k, shape->E,
      shape->R, shape->W, hist, expert_counts, expert_offsets, rank_counts, rank_offsets,
      wave_offsets, pos, row_token, stats, -1, s));
}

int moe_route_dispatch(const moe_shape* shape, const float* logits, const void* x,
                       int32_t* topk_idx, float* topk_w, void* send_buf, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                       int32_t* wave_offsets, int32_t* pos, int32_t* row_token,
                       moe_stats_t* stats, void* workspace, size_t workspace_bytes_given,
                       moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (int64_t(shape->T) * shape->E >= (int64_t(1) << 40)) return MOE_ERR_ARG;
  if (shape->T > 0 && (!logits || !topk_w)) return MOE_ERR_ARG;
  if (!aligned(logits, 4) || !aligned(topk_w, 4) || !aligned(stats, 8)) return MOE_ERR_ALIGN;
  st = check_index_args(shape, topk_idx, expert_counts, expert_offsets, rank_counts,
                        rank_offsets, wave_offsets, pos, row_token, workspace,
                        workspace_bytes_given);
  if (st != MOE_OK) return st;
  st = check_copy_args(shape, x, pos, send_buf);
  if (st != MOE_OK) return st;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  if (moe::dispatch_one_launch(int64_t(shape->T) * shape->k, shape->E)) {
    hipStream_t s = as_stream(stream);
    st = status_of(moe::launch_route(logits, shape->T, shape->E, shape->k, topk_idx, topk_w, s));
    if (st != MOE_OK) return st;
    return status_of(moe::launch_dispatch_small(
        topk_idx, shape->T, shape->E, shape->k, shape->R, shape->W, x, row_bytes, expert_counts,
        expert_offsets, rank_counts, rank_offsets, wave_offsets, pos, row_token, stats, send_buf,
        s));
  }
  st = moe_route_index(shape, logits, topk_idx, topk_w, expert_counts, expert_offsets,
                       rank_counts, rank_offsets, wave_offsets, pos, row_token, stats, workspace,
                       workspace_bytes_given, stream);
  if (st != MOE_OK) return st;
  return moe_dispatch_copy(shape, x, pos, send_buf, stream);
}

int moe_dispatch_copy(const moe_shape* shape, const void* x, const int32_t* pos, void* send_buf,
                      moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  st = check_copy_args(shape, x, pos, send_buf);
  if (st != MOE_OK) return st;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  return status_of(
      moe::launch_copy(x, pos, shape->T, shape->k, row_bytes, int64_t(shape->T) * shape->k,
                       send_buf, as_stream(stream)));
}

int moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_idx, void* send_buf,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* rank_counts,
                 int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos, int32_t* row_token,
                 void* workspace, size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  st = check_index_args(shape, topk_idx, expert_counts, expert_offsets, rank_counts,
                        rank_offsets, wave_offsets, pos, row_token, workspace,
                        workspace_bytes_given);
  if (st != MOE_OK) return st;
  st = check_copy_args(shape, x, pos, send_buf);
  if (st != MOE_OK) return st;
  if (moe::dispatch_one_launch(int64_t(shape->T) * shape->k, shape->E))
    return status_of(moe::launch_dispatch_small(
        topk_idx, shape->T, shape->E, shape->k, shape->R, shape->W, x,
        int64_t(shape->H) * elem_bytes(shape->dtype), expert_counts, expert_offsets, rank_counts,
        rank_offsets, wave_offsets, pos, row_token, nullptr, send_buf, as_stream(stream)));
  st = moe_dispatch_index(shape, topk_idx, expert_counts, expert_offsets, rank_counts,
                          rank_offsets, wave_offsets, pos, row_token, workspace,
                          workspace_bytes_given, stream);
  if (st != MOE_OK) return st;
  return moe_dispatch_copy(shape, x, pos, send_buf, stream);
}

int moe_expert_scale_rows(const moe_shape* shape, int64_t rows, const void* send_buf,
                          const int32_t* expert_offsets, const int32_t* expert_counts,
                          void* expert_out, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (rows < 0 || rows * (int64_t(shape->H) * elem_bytes(shape->dtype) / 16) >= kIndexLimit)
    return MOE_ERR_ARG;
  if (!expert_offsets || !expert_counts) return MOE_ERR_ARG;
  if (rows > 0 && (!send_buf || !expert_out)) return MOE_ERR_ARG;
  if (!aligned(send_buf, 16) || !aligned(expert_out, 16) || !aligned(expert_offsets, 4) ||
      !aligned(expert_counts, 4))
    return MOE_ERR_ALIGN;
  return status_of(moe::launch_expert_scale(send_buf, shape->dtype, rows, shape->H, shape->E,
                                            shape->R, shape->W, expert_offsets, expert_counts,
                                            expert_out, as_stream(stream)));
}

int moe_expert_scale(const moe_shape* shape, const void* send_buf, const int32_t* expert_offsets,
                     const int32_t* expert_counts, void* expert_out, moe_stream_t stream) {
  if (!shape) return MOE_ERR_ARG;
  return moe_expert_scale_rows(shape, int64_t(shape->T) * shape->k, send_buf, expert_offsets,
                               expert_counts, expert_out, stream);
}

size_t moe_expert_swiglu_workspace_bytes(const moe_shape* shape, int32_t I) {
  if (check_shape(shape) != MOE_OK || I < 64 || I % 64 != 0) return 0;
  const int64_t bytes = int64_t(shape->T) * shape->k * I * 2;
  return size_t((bytes < 256 ? 256 : bytes + 255) / 256 * 256);
}

}  // extern "C"

namespace {
int check_swiglu_args(const moe_shape* shape, int32_t I, const void* send_buf,
                      const int32_t* expert_offsets, const int32_t* expert_counts,
                      const void* w_gate_up, const void* w_down, const void* expert_out,
                      const void* workspace, size_t workspace_bytes_given) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (I < 64 || I % 64 != 0 || shape->H % 128 != 0) return MOE_ERR_ARG;
  if (int64_t(shape->E) * 2 * I * shape->H >= (int64_t(1) << 40)) return MOE_ERR_ARG;
  // the kernels address one expert's weights and one 256-row tile through
  // buffer descriptors with a 31-bit byte range
  if (int64_t(4) * I * shape->H >= (int64_t(1) << 31) || int64_t(512) * shape->H >= (int64_t(1) << 31))
    return MOE_ERR_ARG;
  if (!expert_offsets || !expert_counts || !w_gate_up || !w_down || !workspace) return MOE_ERR_ARG;
  if (shape->T > 0 && (!send_buf || !expert_out)) return MOE_ERR_ARG;
  if (!aligned(send_buf, 16) || !aligned(expert_out, 16) || !aligned(w_gate_up, 16) ||
      !aligned(w_down, 16) || !aligned(workspace, 16) || !aligned(expert_offsets, 4) ||
      !aligned(expert_counts, 4))
    return MOE_ERR_ALIGN;
  if (int64_t(shape->T) * shape->k * I >= kIndexLimit) return MOE_ERR_ARG;
  if (workspace_bytes_given < moe_expert_swiglu_workspace_bytes(shape, I)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_expert_swiglu(const moe_shape* shape, int32_t I, const void* send_buf,
                      const int32_t* expert_offsets, const int32_t* expert_counts,
                      const void* w_gate_up, const void* w_down, void* expert_out,
                      void* workspace, size_t workspace_bytes_given, moe_stream_t stream,
                      moe_stream_t side_stream, void* fork_event, void* join_event) {
  const int st = check_swiglu_args(shape, I, send_buf, expert_offsets, expert_counts, w_gate_up,
                                   w_down, expert_out, workspace, workspace_bytes_given);
  if (st != MOE_OK) return st;
  if (side_stream && (!fork_event || !join_event)) return MOE_ERR_ARG;
  const int64_t rows = int64_t(shape->T) * shape->k;
  return status_of(moe::launch_expert_swiglu(
      send_buf, rows, shape->H, I, shape->E, expert_offsets, expert_counts, w_gate_up, w_down,
      workspace, expert_out, as_stream(stream), as_stream(side_stream),
      static_cast<hipEvent_t>(fork_event), static_cast<hipEvent_t>(join_event)));
}

int32_t moe_scale_waves_events(int32_t W) { return W < 1 || W > (1 << 20) ? -1 : 2 + 2 * W; }

int moe_scale_waves(const moe_shape* shape, const void* x, const int32_t* row_token,
                    const int32_t* wave_offsets, const int32_t* expert_offsets,
                    const int32_t* expert_counts, void* send_buf, void* expert_out,
                    const float* topk_w, const int32_t* pos, const int32_t* token_order,
                    const int32_t* token_wave_offsets, void* y, moe_stream_t compute_stream,
                    moe_stream_t copy_stream, moe_stream_t combine_stream, void* const* events,
                    int32_t n_events) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!wave_offsets || !expert_offsets || !expert_counts) return MOE_ERR_ARG;
  if (shape->T > 0 && (!x || !row_token || !send_buf || !expert_out)) return MOE_ERR_ARG;
  if (!aligned(x, 16) || !aligned(send_buf, 16) || !aligned(expert_out, 16) ||
      !aligned(row_token, 4) || !aligned(wave_offsets, 4) || !aligned(expert_offsets, 4) ||
      !aligned(expert_counts, 4))
    return MOE_ERR_ALIGN;
  if ((st = check_wave_combine(shape, topk_w, pos, token_order, token_wave_offsets, y)) != MOE_OK)
    return st;
  if ((copy_stream != compute_stream || own_combine_stream(y, combine_stream, compute_stream)) &&
      (st = check_events(events, n_events, moe_scale_waves_events(shape->W))) != MOE_OK)
    return st;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  moe::WaveCombine wc;
  if (y) wc = {topk_w, pos, token_order, token_wave_offsets, y, as_stream(combine_stream)};
  return status_of(moe::launch_scale_waves(
      x, shape->T, shape->k, row_bytes, shape->dtype, shape->H, shape->E, shape->R, shape->W,
      row_token, wave_offsets, expert_offsets, expert_counts, send_buf, expert_out, wc,
      as_stream(compute_stream), as_stream(copy_stream),
      reinterpret_cast<const hipEvent_t*>(events)));
}

int32_t moe_swiglu_waves_events(int32_t W) { return W < 1 || W > (1 << 20) ? -1 : 2 + 4 * W; }

int moe_swiglu_waves(const moe_shape* shape, int32_t I, const void* x, const int32_t* row_token,
                     const int32_t* wave_offsets, const int32_t* expert_offsets,
                     const int32_t* expert_counts, const void* w_gate_up, const void* w_down,
                     void* send_buf, void* expert_out, void* workspace,
                     size_t workspace_bytes_given, const float* topk_w, const int32_t* pos,
                     const int32_t* token_order, const int32_t* token_wave_offsets, void* y,
                     moe_stream_t compute_stream, moe_stream_t copy_stream,
                     moe_stream_t side_stream, moe_stream_t combine_stream, void* const* events,
                     int32_t n_events) {
  int st = check_swiglu_args(shape, I, send_buf, expert_offsets, expert_counts, w_gate_up,
                             w_down, expert_out, workspace, workspace_bytes_given);
  if (st != MOE_OK) return st;
  if (!wave_offsets) return MOE_ERR_ARG;
  if (shape->T > 0 && (!x || !row_token)) return MOE_ERR_ARG;
  if (!aligned(x, 16) || !aligned(row_token, 4) || !aligned(wave_offsets, 4)) return MOE_ERR_ALIGN;
  if ((st = check_wave_combine(shape, topk_w, pos, token_order, token_wave_offsets, y)) != MOE_OK)
    return st;
  if ((copy_stream != compute_stream || side_stream ||
       own_combine_stream(y, combine_stream, compute_stream)) &&
      (st = check_events(events, n_events, moe_swiglu_waves_events(shape->W))) != MOE_OK)
    return st;
  moe::WaveCombine wc;
  if (y) wc = {topk_w, pos, token_order, token_wave_offsets, y, as_stream(combine_stream)};
  return status_of(moe::launch_swiglu_waves(
      x, shape->T, shape->k, shape->H, I, shape->E, shape->R, shape->W, row_token, wave_offsets,
      expert_offsets, expert_counts, w_gate_up, w_down, send_buf, workspace, expert_out, wc,
      as_stream(compute_stream), as_stream(copy_stream), as_stream(side_stream),
      reinterpret_cast<const hipEvent_t*>(events)));
}

size_t moe_combine_order_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  int64_t tpb, nb;
  moe::combine_order_blocks(shape->T, shape->W, tpb, nb);
  const int64_t bytes = nb * int64_t(shape->W) * 4;
  return size_t((bytes + 255) / 256 * 256);
}

int moe_combine_order(const moe_shape* shape, const int32_t* pos, const int32_t* wave_offsets,
                      int32_t* token_wave_offsets, int32_t* token_order, void* workspace,
                      size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!wave_offsets || !token_wave_offsets || !workspace) return MOE_ERR_ARG;
  if (shape->T > 0 && (!pos || !token_order)) return MOE_ERR_ARG;
  if (!aligned(pos, 4) || !aligned(wave_offsets, 4) || !aligned(token_wave_offsets, 4) ||
      !aligned(token_order, 4) || !aligned(workspace, 4))
    return MOE_ERR_ALIGN;
  if (workspace_bytes_given < moe_combine_order_workspace_bytes(shape)) return MOE_ERR_WORKSPACE;
  return status_of(moe::launch_combine_order(pos, shape->T, shape->k, wave_offsets, shape->W,
                                             token_wave_offsets, token_order,
                                             static_cast<int32_t*>(workspace),
                                             as_stream(stream)));
}

int moe_combine_waves(const moe_shape* shape, const void* expert_out, const float* topk_w,
                      const int32_t* pos, const int32_t* token_order,
                      const int32_t* token_wave_offsets, int32_t w0, int32_t w1, void* y,
                      moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (w0 < 0 || w1 < w0 || w1 > shape->W) return MOE_ERR_ARG;
  if (!y) return MOE_ERR_ARG;
  if ((st = check_wave_combine(shape, topk_w, pos, token_order, token_wave_offsets, y)) != MOE_OK)
    return st;
  if (shape->T > 0 && !expert_out) return MOE_ERR_ARG;
  if (!aligned(expert_out, 16)) return MOE_ERR_ALIGN;
  return status_of(moe::launch_combine_waves(expert_out, shape->dtype, topk_w, pos, shape->T,
                                             shape->k, shape->H, token_order, token_wave_offsets,
                                             w0, w1, y, as_stream(stream)));
}

int moe_combine_rows(const moe_shape* shape, int64_t rows, const void* expert_out,
                     const float* topk_w, const int32_t* pos, void* y, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (rows < 0 || rows * (int64_t(shape->H) * elem_bytes(shape->dtype) / 16) >= kIndexLimit)
    return MOE_ERR_ARG;
  if (shape->T > 0 && (!expert_out || !topk_w || !pos || !y)) return MOE_ERR_ARG;
  if (!aligned(expert_out, 16) || !aligned(y, 16) || !aligned(topk_w, 4) || !aligned(pos, 4))
    return MOE_ERR_ALIGN;
  return status_of(moe::launch_combine(expert_out, shape->dtype, topk_w, pos, shape->T, shape->k,
                                       shape->H, rows, y, as_stream(stream)));
}

int moe_combine(const moe_shape* shape, const void* expert_out, const float* topk_w,
                const int32_t* pos, void* y, moe_stream_t stream) {
  if (!shape) return MOE_ERR_ARG;
  return moe_combine_rows(shape, int64_t(shape->T) * shape->k, expert_out, topk_w, pos, y,
                          stream);
}

double moe_wave_time(double message_bytes, double alpha_s, double beta_bytes_per_s, int32_t W) {
  if (W < 1 || !(alpha_s >= 0.0) || !(beta_bytes_per_s > 0.0) || !(message_bytes >= 0.0))
    return -1.0;
  return W * alpha_s + message_bytes / beta_bytes_per_s + message_bytes / (W * beta_bytes_per_s);
}

int32_t moe_plan_waves(double message_bytes, double alpha_s, double beta_bytes_per_s, int32_t L,
                       double* time_out) {
  if (L < 1 || moe_wave_time(message_bytes, alpha_s, beta_bytes_per_s, 1) < 0.0) return -1;
  // T(W) is convex in W with its real minimum at sqrt(M / (alpha beta)); the
  // layout needs W | L, so the best feasible W is a divisor of L on either side.
  int32_t best = 1;
  double tbest = moe_wave_time(message_bytes, alpha_s, beta_bytes_per_s, 1);
  for (int32_t d = 1; (int64_t)d * d <= L; ++d) {
    if (L % d != 0) continue;
    for (int32_t W : {d, L / d}) {
      const double t = moe_wave_time(message_bytes, alpha_s, beta_bytes_per_s, W);
      if (t < tbest || (t == tbest && W < best)) {
        tbest = t;
        best = W;
      }
    }
  }
  if (time_out) *time_out = tbest;
  return best;
}

double moe_link_p95(double mean_bytes, double tokens, int32_t destinations) {
  if (destinations < 1 || !(tokens > 0.0) || !(mean_bytes >= 0.0)) return -1.0;
  return mean_bytes * (1.0 + 1.645 * std::sqrt(destinations / tokens));
}

int32_t moe_expert_capacity(int32_t k, double f, int32_t T, int32_t E) {
  if (k < 1 || T < 0 || E < 1 || !(f >= 0.0)) return -1;
  const double ec = std::ceil(double(k) * f * double(T) / double(E));
  return ec > 2147483647.0 ? -1 : int32_t(ec);
}

int moe_dispatch_capacity(const moe_shape* shape, int32_t capacity, const void* x,
                          const int32_t* topk_idx, void* send_buf, int32_t* kept_counts,
                          int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                          int32_t* wave_offsets, int32_t* pos, int32_t* row_token,
                          void* workspace, size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const int64_t nvec = int64_t(shape->H) * elem_bytes(shape->dtype) / 16;
  const int64_t rows = int64_t(shape->E) * capacity;
  if (capacity < 0 || rows * nvec >= kIndexLimit) return MOE_ERR_ARG;
  if (!kept_counts || !expert_offsets || !rank_counts || !rank_offsets || !wave_offsets ||
      !workspace)
    return MOE_ERR_ARG;
  if (shape->T > 0 && (!topk_idx || !pos || !x)) return MOE_ERR_ARG;
  if (rows > 0 && (!send_buf || !row_token)) return MOE_ERR_ARG;
  const void* ptrs[] = {topk_idx, kept_counts, expert_offsets, rank_counts, rank_offsets,
                        wave_offsets, pos, workspace};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return MOE_ERR_ALIGN;
  if (workspace_bytes_given < workspace_bytes(shape)) return MOE_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(send_buf, 16) || !aligned(row_token, 4)) return MOE_ERR_ALIGN;
  const int64_t npicks = int64_t(shape->T) * shape->k;
  hipStream_t s = as_stream(stream);
  int32_t* hist = static_cast<int32_t*>(workspace);
  st = status_of(moe::launch_count(topk_idx, npicks, shape->E, hist, s));
  if (st != MOE_OK) return st;
  st = status_of(moe::launch_place_chunks(
      topk_idx, npicks, moe::chunk_picks(npicks, shape->E), (int)moe::num_chunks(npicks, shape->E),
      shape->k, shape->E, shape->R, shape->W, hist, kept_counts, expert_offsets, rank_counts,
      rank_offsets, wave_offsets, pos, row_token, nullptr, capacity, s));
  if (st != MOE_OK) return st;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  st = status_of(moe::launch_copy(x, pos, shape->T, shape->k, row_bytes, rows, send_buf, s));
  if (st != MOE_OK) return st;
  return status_of(moe::launch_pad(shape->E, shape->R, shape->W, capacity, kept_counts, row_bytes,
                                   send_buf, row_token, s));
}

int moe_dirichlet_alpha(const int32_t* expert_counts, int32_t E, double* alpha_out,
                        moe_stream_t stream) {
  if (!expert_counts || !alpha_out || E < 1 || E > 1024) return MOE_ERR_ARG;
  if (!aligned(expert_counts, 4) || !aligned(alpha_out, 8)) return MOE_ERR_ALIGN;
  return status_of(moe::launch_dirichlet_alpha(expert_counts, E, alpha_out, as_stream(stream)));
}

int moe_stats(const int32_t* expert_counts, int32_t E, int32_t R, moe_stats_t* out,
              moe_stream_t stream) {
  if (!expert_counts || !out) return MOE_ERR_ARG;
  if (E < 1 || E > 1024 || R < 1 || E % R != 0) return MOE_ERR_ARG;
  if (!aligned(expert_counts, 4) || !aligned(out, 8)) return MOE_ERR_ALIGN;
  return status_of(moe::launch_stats(expert_counts, E, R, out, as_stream(stream)));
}

// ------------------------------------------------ virtual-source exchange

size_t moe_vsrc_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return vsrc_workspace_bytes(shape);
}

int moe_vsrc_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                      void* send_buf, int32_t* src_counts, int32_t* src_offsets,
                      int32_t* send_counts, int32_t* send_offsets, int32_t* recv_counts,
                      int32_t* recv_offsets,
                      int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                      void* workspace, size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_vsrc_shape(shape);
  if (st != MOE_OK) return st;
  if (!src_counts || !src_offsets || !send_counts || !send_offsets || !recv_counts ||
      !recv_offsets || !expert_counts || !expert_offsets || !workspace)
    return MOE_ERR_ARG;
  if (shape->T > 0 && (!topk_idx || !pos)) return MOE_ERR_ARG;
  const void* p4[] = {topk_idx, src_counts, src_offsets, send_counts, send_offsets, recv_counts,
                      recv_offsets, expert_counts, expert_offsets, pos, workspace};
  for (const void* p : p4)
    if (!aligned(p, 4)) return MOE_ERR_ALIGN;
  st = check_copy_args(shape, x, pos, send_buf);
  if (st != MOE_OK) return st;
  if (workspace_bytes_given < vsrc_workspace_bytes(shape)) return MOE_ERR_WORKSPACE;
  const int R = shape->R, W = shape->W, E = shape->E, k = shape->k;
  const int64_t src_picks = int64_t(shape->T / R) * k;
  int64_t chunk;
  int spc;
  moe::source_chunks(src_picks, E, chunk, spc);
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* wave_offsets = hist + int64_t(R) * spc * E;
  hipStream_t s = as_stream(stream);
  st = status_of(moe::launch_count_sources(topk_idx, R, src_picks, E, hist, s));
  if (st != MOE_OK) return st;
  st = status_of(moe::launch_place_sources(topk_idx, R, src_picks, k, E, R, W, hist, src_counts,
                                           src_offsets, send_counts, send_offsets, wave_offsets,
                                           pos, s));
  if (st != MOE_OK) return st;
  st = status_of(moe::launch_vsrc_plan(R, W, E, src_counts, send_counts, recv_counts,
                                       recv_offsets, expert_counts, expert_offsets, s));
  if (st != MOE_OK) return st;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  return status_of(moe::launch_copy(x, pos, shape->T, k, row_bytes, int64_t(shape->T) * k,
                                    send_buf, s));
}

int moe_vsrc_exchange(const moe_shape* shape, int32_t direction, const void* in, void* out,
                      const int32_t* send_offsets, const int32_t* recv_counts,
                      const int32_t* recv_offsets, moe_stream_t stream) {
  int st = check_vsrc_shape(shape);
  if (st != MOE_OK) return st;
  st = check_vsrc_move(shape, direction, in, out);
  if (st != MOE_OK) return st;
  if (!send_offsets || !recv_counts || !recv_offsets) return MOE_ERR_ARG;
  if (!aligned(send_offsets, 4) || !aligned(recv_counts, 4) || !aligned(recv_offsets, 4))
    return MOE_ERR_ALIGN;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  return status_of(moe::launch_vsrc_exchange(in, out, row_bytes, int64_t(shape->T) * shape->k,
                                             shape->R, shape->W, send_offsets, recv_counts,
                                             recv_offsets, direction == 1, as_stream(stream)));
}

int moe_vsrc_exchange_direct(const moe_shape* shape, int32_t direction, const void* in,
                             void* out, const int32_t* src_counts, const int32_t* src_offsets,
                             const int32_t* expert_offsets, void* workspace,
                             size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_vsrc_shape(shape);
  if (st != MOE_OK) return st;
  st = check_vsrc_move(shape, direction, in, out);
  if (st != MOE_OK) return st;
  if (!src_counts || !src_offsets || !expert_offsets || !workspace) return MOE_ERR_ARG;
  if (!aligned(src_counts, 4) || !aligned(src_offsets, 4) || !aligned(expert_offsets, 4) ||
      !aligned(workspace, 4))
    return MOE_ERR_ALIGN;
  if (workspace_bytes_given < vsrc_workspace_bytes(shape)) return MOE_ERR_WORKSPACE;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  return status_of(moe::launch_vsrc_direct(
      in, out, row_bytes, int64_t(shape->T) * shape->k, shape->E, shape->R, shape->W, src_counts,
      src_offsets, expert_offsets, static_cast<int32_t*>(workspace), direction == 1,
      as_stream(stream)));
}

int moe_vsrc_regroup(const moe_shape* shape, int32_t direction, const void* in, void* out,
                     const int32_t* src_counts, const int32_t* recv_offsets,
                     const int32_t* expert_offsets, void* workspace,
                     size_t workspace_bytes_given, moe_stream_t stream) {
  int st = check_vsrc_shape(shape);
  if (st != MOE_OK) return st;
  st = check_vsrc_move(shape, direction, in, out);
  if (st != MOE_OK) return st;
  if (!src_counts || !recv_offsets || !expert_offsets || !workspace) return MOE_ERR_ARG;
  if (!aligned(src_counts, 4) || !aligned(recv_offsets, 4) || !aligned(expert_offsets, 4) ||
      !aligned(workspace, 4))
    return MOE_ERR_ALIGN;
  if (workspace_bytes_given < vsrc_workspace_bytes(shape)) return MOE_ERR_WORKSPACE;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  return status_of(moe::launch_vsrc_regroup(
      in, out, row_bytes, int64_t(shape->T) * shape->k, shape->E, shape->R, shape->W, src_counts,
      recv_offsets, expert_offsets, static_cast<int32_t*>(workspace), direction == 1,
      as_stream(stream)));
}

}  // extern "C"

// ------------------------------------------------- allocation-free dispatch
// moe_dispatch_noalloc keeps the index stage's histogram rows in a file-scope
// device array instead of a caller workspace, for callers that cannot
// allocate. In host code `scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device (with that device
// current) and only that address is handed to kernels.
namespace {

constexpr size_t kScratchBytes = size_t(256) << 10;  // the index workspace's largest size
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxScratchDevices] = {};

// The device address of this device's copy of `scratch` (looked up on the
// first call made with the device current), or null on failure.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_dispatch_noalloc(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                         void* send_buf, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                         int32_t* pos, int32_t* row_token, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  st = check_index_ptrs(shape, topk_idx, expert_counts, expert_offsets, rank_counts,
                        rank_offsets, wave_offsets, pos, row_token);
  if (st != MOE_OK) return st;
  st = check_copy_args(shape, x, pos, send_buf);
  if (st != MOE_OK) return st;
  const int64_t npicks = int64_t(shape->T) * shape->k;
  const int64_t row_bytes = int64_t(shape->H) * elem_bytes(shape->dtype);
  if (moe::dispatch_one_launch(npicks, shape->E))  // one launch, no histogram workspace
    return status_of(moe::launch_dispatch_small(
        topk_idx, shape->T, shape->E, shape->k, shape->R, shape->W, x, row_bytes, expert_counts,
        expert_offsets, rank_counts, rank_offsets, wave_offsets, pos, row_token, nullptr,
        send_buf, as_stream(stream)));
  // the count pass writes every row of its histogram, so nothing needs clearing
  const int64_t need = moe::num_chunks(npicks, shape->E) * int64_t(shape->E) * 4;
  if (need > int64_t(kScratchBytes)) return MOE_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_DEVICE;
  hipStream_t s = as_stream(stream);
  int32_t* hist = static_cast<int32_t*>(ws);
  st = status_of(moe::launch_count(topk_idx, npicks, shape->E, hist, s));
  if (st != MOE_OK) return st;
  st = status_of(moe::launch_place(topk_idx, npicks, shape->k, shape->E, shape->R, shape->W,
                                   hist, expert_counts, expert_offsets, rank_counts,
                                   rank_offsets, wave_offsets, pos, row_token, s));
  if (st != MOE_OK) return st;
  return status_of(moe::launch_copy(x, pos, shape->T, shape->k, row_bytes, npicks, send_buf, s));
}

}  // extern "C"
