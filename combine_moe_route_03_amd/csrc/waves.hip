// waves.hip -- wave-pipelined execution of the local expert layer (irregular
// AllToAll page, "Wave-Scheduled pipelining": the experts split into W waves,
// each wave runs dispatch -> compute while the next wave's dispatch is already
// under way; the pipeline's cost model is the page's T(W)).
//
// Wave w owns local slots [w*L/W, (w+1)*L/W) of every rank, i.e. the rows
// [wave_offsets[w], wave_offsets[w+1]) of the wave-ordered send buffer. Per
// wave: a gather dispatch of exactly those rows (send[r] = x[row_token[r]]) on
// a copy stream, an event, and the SwiGLU FFN of that wave's experts on the
// compute stream once the event has fired; so the gather of wave w+1 (HBM
// bound) runs under the FFN of wave w (MFMA bound). Where the wave's experts
// split into even and odd slots, the odd ones run on the caller's side stream
// forked from the compute stream and joined back, as the unpipelined FFN does;
// every stream and event is the caller's (the library keeps none). With a
// combine in the pipeline, the tokens completed by wave w (all their experts
// in waves <= w) are combined after wave w's experts: on a combine stream of
// their own at once, or on the copy stream behind the gather of wave w+1 (the
// page asks that a wave's dispatch never wait behind a combine); the tokens'
// bits equal the one-pass combine's.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kU = 4;  // vectors per thread in flight

// Rows [wave_offsets[w], wave_offsets[w+1]) of send <- x[row_token[r]], read
// on the device; a grid-stride loop over the wave's (row, 16-byte column)
// pairs. Rows whose token is outside [0, T) are skipped. kCache: the stores
// go through the caches (the wave's experts read the rows next); otherwise
// they stream (the whole send buffer past the cache budget).
template <bool kCache>
__global__ __launch_bounds__(kBlock) void gather_wave_kernel(
    const v4u* __restrict__ x, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ wave_offsets, int w, int T, int64_t rows_max, uint32_t nvec,
    v4u* __restrict__ send) {
  int64_t a = wave_offsets[w], b = wave_offsets[w + 1];
  a = a < 0 ? 0 : a;
  b = b < rows_max ? b : rows_max;
  const int64_t n = b > a ? (b - a) * nvec : 0;
  const int64_t step = (int64_t)gridDim.x * kBlock * kU;
  for (int64_t q0 = (int64_t)blockIdx.x * kBlock * kU; q0 < n; q0 += step) {
    int64_t src[kU], dst[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t q = q0 + u * kBlock + threadIdx.x;
      src[u] = dst[u] = -1;
      if (q >= n) continue;
      const int64_t r = a + q / nvec, col = q % nvec;
      const int32_t t = row_token[r];
      if ((uint32_t)t >= (uint32_t)T) continue;
      src[u] = (int64_t)t * nvec + col;
      dst[u] = r * nvec + col;
    }
    v4u v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (src[u] >= 0) v[u] = x[src[u]];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (dst[u] >= 0) {
        if constexpr (kCache) send[dst[u]] = v[u];
        else store_stream(send + dst[u], v[u]);
      }
  }
}

}  // namespace

hipError_t launch_gather_wave(const void* x, const int32_t* row_token, const int32_t* wave_offsets,
                              int w, int T, int64_t rows_max, int64_t row_bytes, void* send,
                              hipStream_t s) {
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  const int64_t want = (rows_max * nvec + kBlock * kU - 1) / (kBlock * kU);
  const unsigned grid = (unsigned)(want < 2048 ? (want < 1 ? 1 : want) : 2048);
  // the expert stage's policy for the same buffer: streaming stores past the
  // budget (dirichlet_waves, 1.9 GB: gather 590 -> 540 us at W = 1, step at
  // W = 8 1.638 -> 1.567 ms with two streams; the x rows re-read for each
  // copy come from HBM either way)
  auto go = [&](auto kernel) {
    return launch(kernel, dim3(grid), dim3(kBlock), 0, s, static_cast<const v4u*>(x), row_token,
                  wave_offsets, w, T, rows_max, nvec, static_cast<v4u*>(send));
  };
  return rows_max * row_bytes <= kCacheReuseBytes ? go(gather_wave_kernel<true>)
                                                  : go(gather_wave_kernel<false>);
}

namespace {

// The combine of the tokens completed by wave w on `cs`, once the event
// `done` (wave w's experts, recorded on the compute stream) has fired.
hipError_t combine_wave(const WaveCombine& wc, const void* out, int dtype, int T, int k, int64_t H,
                        int w, bool sep, hipEvent_t done, hipStream_t cs) {
  if (sep) {
    const hipError_t e = hipStreamWaitEvent(cs, done, 0);
    if (e != hipSuccess) return e;
  }
  return launch_combine_waves(out, dtype, wc.w, wc.pos, T, k, H, wc.token_order,
                              wc.token_wave_offsets, w, w + 1, wc.y, cs);
}

// Wave w's experts are queued on `compute`: record `done` there. On a
// combine stream of its own, the tokens completed by wave w are combined at
// once; on the copy stream, the tokens completed by wave w - 1 (done_prev),
// behind the gather of wave w already queued there, so a gather never waits
// behind a combine of a later wave.
hipError_t after_experts(const WaveCombine& wc, const void* out, int dtype, int T, int k,
                         int64_t H, int w, hipEvent_t done, hipEvent_t done_prev,
                         hipStream_t compute, hipStream_t copy) {
  if (wc.y == nullptr) return hipSuccess;
  const hipStream_t cs = wc.stream ? wc.stream : copy;
  const bool sep = cs != compute;
  if (sep) {
    const hipError_t e = hipEventRecord(done, compute);
    if (e != hipSuccess) return e;
  }
  if (cs != copy) return combine_wave(wc, out, dtype, T, k, H, w, sep, done, cs);
  if (w == 0) return hipSuccess;
  return combine_wave(wc, out, dtype, T, k, H, w - 1, sep, done_prev, cs);
}

// On the copy stream, the last wave's completed tokens; then the compute
// stream joins the combine stream (everything of the call is on `compute`
// when it returns).
hipError_t finish_combine(const WaveCombine& wc, const void* out, int dtype, int T, int k,
                          int64_t H, int W, hipEvent_t done_last, hipEvent_t join,
                          hipStream_t compute, hipStream_t copy) {
  if (wc.y == nullptr) return hipSuccess;
  const hipStream_t cs = wc.stream ? wc.stream : copy;
  const bool sep = cs != compute;
  hipError_t e = hipSuccess;
  if (cs == copy && (e = combine_wave(wc, out, dtype, T, k, H, W - 1, sep, done_last, cs)) !=
                        hipSuccess)
    return e;
  if (!sep) return hipSuccess;
  if ((e = hipEventRecord(join, cs)) != hipSuccess) return e;
  return hipStreamWaitEvent(compute, join, 0);
}

}  // namespace

// The identity-scaled experts of the synthetic workloads in the same
// schedule: per wave its gather dispatch on the copy stream, an event, and
// the wave's experts on the compute stream (bit-identical to the one-pass copy
// and expert stage: both are bit copies and the same per-element product).
// events: [0] copy start, [1..W] gathers, [1+W+w] wave w's experts done,
// [1+2W] the final join.
hipError_t launch_scale_waves(const void* x, int T, int k, int64_t row_bytes, int dtype, int64_t H,
                              int E, int R, int W, const int32_t* row_token,
                              const int32_t* wave_offsets, const int32_t* offs,
                              const int32_t* cnts, void* send, void* out, const WaveCombine& wc,
                              hipStream_t compute, hipStream_t copy, const hipEvent_t* events) {
  const int64_t rows = (int64_t)T * k;
  if (rows == 0) return hipSuccess;
  const bool two = copy != compute;
  // the events a combine on a stream of its own uses (null when none is needed)
  const auto ev = [&](int i) { return events ? events[i] : nullptr; };
  hipError_t e = hipSuccess;
  if (two) {
    if ((e = hipEventRecord(events[0], compute)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(copy, events[0], 0)) != hipSuccess) return e;
  }
  for (int w = 0; w < W; ++w) {
    e = launch_gather_wave(x, row_token, wave_offsets, w, T, rows, row_bytes, send, copy);
    if (e != hipSuccess) return e;
    if (two) {
      if ((e = hipEventRecord(events[w + 1], copy)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(compute, events[w + 1], 0)) != hipSuccess) return e;
    }
    e = launch_expert_scale_wave(send, dtype, rows, H, E, R, W, offs, cnts, wave_offsets, w, out,
                                 compute);
    if (e != hipSuccess) return e;
    e = after_experts(wc, out, dtype, T, k, H, w, ev(1 + W + w), ev(W + w), compute, copy);
    if (e != hipSuccess) return e;
  }
  return finish_combine(wc, out, dtype, T, k, H, W, ev(2 * W), ev(1 + 2 * W), compute, copy);
}

// events: [0] copy start, [1..W] gathers, [1+W+2w] / [2+W+2w] wave w's fork
// and join, [1+3W+w] wave w's experts done, [1+4W] the final join.
hipError_t launch_swiglu_waves(const void* x, int T, int k, int H, int I, int E, int R, int W,
                               const int32_t* row_token, const int32_t* wave_offsets,
                               const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                               const void* w_down, void* send, void* hbuf, void* out,
                               const WaveCombine& wc, hipStream_t compute, hipStream_t copy,
                               hipStream_t side, const hipEvent_t* events) {
  const int64_t rows = (int64_t)T * k;
  if (rows == 0) return hipSuccess;
  const int L = E / R, LW = L / W;
  const int64_t row_bytes = (int64_t)H * 2;
  const bool two = copy != compute;
  // A wave's experts run as two chains (even and odd slots, the second on the
  // side stream) when the caller gives one, that split is one stride-2 run of
  // expert ids (one rank, or one wave: all experts) and the wave has at least
  // eight experts. Local layer, one stream: W = 1 776 -> 741 us, W = 2 867 ->
  // 842; with chains of one or two experts W = 4 1011 -> 1019, W = 8 1446 ->
  // 1632 (the fork and join cost more than the overlap gives). Otherwise one
  // chain.
  const bool chains = side != nullptr && R * LW >= 8 && (R == 1 || W == 1);
  const auto ev = [&](int i) { return events ? events[i] : nullptr; };
  hipError_t e = hipSuccess;
  if (two) {
    // the copy stream starts after everything already queued on the compute
    // stream (the index stage that wrote row_token and wave_offsets)
    if ((e = hipEventRecord(events[0], compute)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(copy, events[0], 0)) != hipSuccess) return e;
  }
  for (int w = 0; w < W; ++w) {
    e = launch_gather_wave(x, row_token, wave_offsets, w, T, rows, row_bytes, send, copy);
    if (e != hipSuccess) return e;
    if (two) {
      if ((e = hipEventRecord(events[w + 1], copy)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(compute, events[w + 1], 0)) != hipSuccess) return e;
    }
    if (!chains) {
      // the R*LW experts of wave w: slots w*LW .. w*LW+LW-1 of every rank
      e = launch_expert_swiglu_subset(send, rows, H, I, R * LW, LW, L, w * LW, offs, cnts,
                                      w_gate_up, w_down, hbuf, out, compute);
      if (e != hipSuccess) return e;
    } else {
      // the wave's experts w*LW + 2i + c (R == 1), or 2i + c (W == 1), as two
      // chains: c = 0 on the compute stream, c = 1 on the side stream
      hipEvent_t fork = events[1 + W + 2 * w], join = events[2 + W + 2 * w];
      if ((e = hipEventRecord(fork, compute)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return e;
      const int n = R * LW;
      for (int c = 0; c < 2; ++c) {
        e = launch_expert_swiglu_subset(send, rows, H, I, (n - c + 1) / 2, 1, 2, w * LW + c, offs,
                                        cnts, w_gate_up, w_down, hbuf, out, c ? side : compute);
        if (e != hipSuccess) return e;
      }
      if ((e = hipEventRecord(join, side)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(compute, join, 0)) != hipSuccess) return e;
    }
    e = after_experts(wc, out, 1, T, k, H, w, ev(1 + 3 * W + w), ev(3 * W + w), compute, copy);
    if (e != hipSuccess) return e;
  }
  return finish_combine(wc, out, 1, T, k, H, W, ev(4 * W), ev(1 + 4 * W), compute, copy);
}

}  // namespace moe
