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
// split into even and odd slots, the odd ones run on a side stream forked
// from the compute stream and joined back, as the unpipelined FFN does. The
// combine runs once, after the last wave, with the same arithmetic as the
// unpipelined path.
#include <vector>

#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kU = 4;  // vectors per thread in flight

// Rows [wave_offsets[w], wave_offsets[w+1]) of send <- x[row_token[r]], read
// on the device; a grid-stride loop over the wave's (row, 16-byte column)
// pairs. Rows whose token is outside [0, T) are skipped.
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
      if (dst[u] >= 0) send[dst[u]] = v[u];  // through the caches: the FFN reads it next
  }
}

// Events of the pipeline, created once per host thread and device (an event
// belongs to the device current when it was created) and reused by later calls
// (a wait takes the event's most recent record at the time it is enqueued).
constexpr int kMaxDevices = 64;

// A side stream for the second chain of a wave's experts, one per host thread
// and device like the events.
hipError_t side_stream(hipStream_t& out) {
  thread_local hipStream_t pool[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!pool[dev]) {
    hipStream_t st = nullptr;
    if ((err = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return err;
    pool[dev] = st;
  }
  out = pool[dev];
  return hipSuccess;
}

hipError_t wave_events(int n, std::vector<hipEvent_t>*& out) {
  thread_local std::vector<hipEvent_t> pool[kMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::vector<hipEvent_t>& p = pool[dev];
  while ((int)p.size() < n) {
    hipEvent_t e;
    err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (err != hipSuccess) return err;
    p.push_back(e);
  }
  out = &p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_gather_wave(const void* x, const int32_t* row_token, const int32_t* wave_offsets,
                              int w, int T, int64_t rows_max, int64_t row_bytes, void* send,
                              hipStream_t s) {
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  const int64_t want = (rows_max * nvec + kBlock * kU - 1) / (kBlock * kU);
  const unsigned grid = (unsigned)(want < 2048 ? (want < 1 ? 1 : want) : 2048);
  return launch(gather_wave_kernel, dim3(grid), dim3(kBlock), 0, s, static_cast<const v4u*>(x),
                row_token, wave_offsets, w, T, rows_max, nvec, static_cast<v4u*>(send));
}

hipError_t launch_swiglu_waves(const void* x, int T, int k, int H, int I, int E, int R, int W,
                               const int32_t* row_token, const int32_t* wave_offsets,
                               const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                               const void* w_down, void* send, void* hbuf, void* out,
                               hipStream_t compute, hipStream_t copy) {
  const int64_t rows = (int64_t)T * k;
  if (rows == 0) return hipSuccess;
  const int L = E / R, LW = L / W;
  const int64_t row_bytes = (int64_t)H * 2;
  const bool two = copy != compute;
  // A wave's experts run as two chains (even and odd slots, the second on a
  // side stream) when that split is one stride-2 run of expert ids (one rank,
  // or one wave: all experts) and the wave has at least eight experts. Local
  // layer, one stream: W = 1 776 -> 741 us, W = 2 867 -> 842; with chains of
  // one or two experts W = 4 1011 -> 1019, W = 8 1446 -> 1632 (the fork and
  // join cost more than the overlap gives). Otherwise one chain.
  const bool chains = R * LW >= 8 && (R == 1 || W == 1);
  std::vector<hipEvent_t>* ev = nullptr;
  hipStream_t side = nullptr;
  hipError_t e = hipSuccess;
  // events: [0] copy start, [1..W] gathers, then a fork and a join per wave
  if ((e = wave_events(1 + W + (chains ? 2 * W : 0), ev)) != hipSuccess) return e;
  if (chains && (e = side_stream(side)) != hipSuccess) return e;
  if (two) {
    // the copy stream starts after everything already queued on the compute
    // stream (the index stage that wrote row_token and wave_offsets)
    if ((e = hipEventRecord((*ev)[0], compute)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(copy, (*ev)[0], 0)) != hipSuccess) return e;
  }
  for (int w = 0; w < W; ++w) {
    e = launch_gather_wave(x, row_token, wave_offsets, w, T, rows, row_bytes, send, copy);
    if (e != hipSuccess) return e;
    if (two) {
      if ((e = hipEventRecord((*ev)[w + 1], copy)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(compute, (*ev)[w + 1], 0)) != hipSuccess) return e;
    }
    if (!chains) {
      // the R*LW experts of wave w: slots w*LW .. w*LW+LW-1 of every rank
      e = launch_expert_swiglu_subset(send, rows, H, I, R * LW, LW, L, w * LW, offs, cnts,
                                      w_gate_up, w_down, hbuf, out, compute);
      if (e != hipSuccess) return e;
      continue;
    }
    // the wave's experts w*LW + 2i + c (R == 1), or 2i + c (W == 1), as two
    // chains: c = 0 on the compute stream, c = 1 on the side stream
    hipEvent_t fork = (*ev)[1 + W + 2 * w], join = (*ev)[2 + W + 2 * w];
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
  return hipSuccess;
}

}  // namespace moe
