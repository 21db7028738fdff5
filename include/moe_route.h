/*
 * moe_route.h -- C ABI of the gfx950 (MI355X) library for the one-GPU share of
 * the Mixture-of-Experts expert-parallel exchange: top-k gating, send-count
 * matrix S with Alltoallv-style counts and offsets, stable permutation of token
 * rows into expert/rank/wave-contiguous send buffers, gate-weighted combine,
 * and S's skew statistics.
 *
 * The steps follow the MoE-layer flow of the cross-card communication
 * explainer (cloud.baidu.com, section 4: gating -> permute by device ->
 * all-to-all -> local experts -> all-to-all -> combine) and the EP flow of the
 * MoE systems survey (crad.ict.ac.cn, section 1.1, steps 1-4). The all-to-all
 * itself is not performed: the rank-bucketed send buffer is what one GPU would
 * hand to it.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers unless stated otherwise. The
 *     caller owns every buffer, stream and event; the library never allocates,
 *     frees, creates or keeps them past the call. The one piece of mutable
 *     library state is the benchmark timing hook (moe_set_timing_events): per
 *     host thread, inert unless armed, and not part of the path.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream). Results are ready when the stream reaches that point.
 *   - Arguments are validated on the host before anything is launched. On any
 *     error nothing is launched and nothing is written; the return value is a
 *     negative moe_status. A failed launch returns MOE_ERR_DEVICE; a fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - Layouts are row-major: logits[T][E] fp32, x and y [T][H], topk_idx,
 *     topk_w and pos [T][k]; send buffers and expert outputs [T*k][H].
 *   - Expert e lives on virtual rank r = e / L (L = E / R local experts per
 *     rank, contiguous blocks; experts are split evenly over devices,
 *     explainer section 3 item 1) in local slot s = e % L. Its wave is
 *     floor(s * W / L): W waves of E / W experts each (irregular AllToAll
 *     page, "Wave-Scheduled"), each wave reaching every rank.
 *   - Send-buffer rows are grouped in buckets ordered by (wave, rank, slot);
 *     inside a bucket rows follow ascending token index (stable). With W = 1
 *     this is plain expert-id order. Counts and offsets are in ROWS; the byte
 *     displacement of a row is rows * H * element size.
 *   - Limits: 1 <= E <= 1024, 1 <= k <= min(E, 32), E % R == 0, L % W == 0,
 *     T >= 0, H >= 1, R >= 1, W >= 1, T * k < 2^31, H * element size a
 *     multiple of 16 bytes and T * k * H * element size / 16 < 2^31 (the row
 *     kernels index 16-byte vectors in 32 bits), hidden-state pointers 16-byte
 *     aligned, index/weight pointers 4-byte aligned.
 *   - T == 0 is valid: counts and offsets are written as zeros, nothing else.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* null pointer, or a size/shape outside the limits */
  MOE_ERR_ALIGN = -2,       /* a pointer or the row size breaks the alignment rules */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_dispatch_workspace_bytes() */
  MOE_ERR_UNSUPPORTED = -4, /* unknown dtype */
  MOE_ERR_DEVICE = -5       /* the HIP runtime rejected a launch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Problem shape shared by the dispatch, expert and combine calls. */
typedef struct {
  int32_t T;     /* tokens held by this GPU */
  int32_t H;     /* hidden size (elements per token row) */
  int32_t E;     /* experts */
  int32_t k;     /* experts per token */
  int32_t R;     /* virtual destination ranks (E % R == 0) */
  int32_t W;     /* expert waves (L % W == 0) */
  int32_t dtype; /* moe_dtype of x, send buffers, expert outputs and y */
} moe_shape;

/* Skew statistics of the send-count matrix (DODOCO summary, "metrics"). */
typedef struct {
  double expert_max_over_mean; /* max_e c[e] / (total / E) */
  double expert_gini;          /* Gini of the E per-expert loads */
  double rank_max_over_mean;   /* max_r l[r] / (total / R), l = row sums of S */
  double rank_gini;            /* Gini of the R per-rank loads */
  int64_t total;               /* sum of S */
  int32_t expert_max, expert_min, rank_max, rank_min;
} moe_stats_t;

/* Top-k gating, MoE systems survey section 1.1 eq. (2):
 *   G(x) = softmax(TopK(x W_gate, k)), the non-kept logits acting as -inf.
 * logits   [T][E] fp32 (the router GEMM output x W_gate; finite values).
 * topk_idx [T][k] int32 out: experts by descending logit; equal logits (and
 *          +0 / -0) are ordered by ascending expert id.
 * topk_w   [T][k] fp32 out: exp(l_i - l_0) / sum_j exp(l_j - l_0), evaluated
 *          in double and rounded once to fp32.
 * Errors: MOE_ERR_ARG (null pointer with T > 0, E or k outside the limits),
 *         MOE_ERR_ALIGN (a pointer not 4-byte aligned), MOE_ERR_DEVICE. */
int moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
              int32_t* topk_idx, float* topk_w, moe_stream_t stream);

/* Bytes of device workspace moe_dispatch / moe_dispatch_index need for this
 * shape (host-only, pure; 0 for an invalid shape). */
size_t moe_dispatch_workspace_bytes(const moe_shape* shape);

/* Counts, offsets and positions: everything the Alltoallv needs before the
 * payload moves (irregular AllToAll page: the top-k index set is the a2a
 * send-count matrix, passed in full as Alltoallv counts; survey section 4.1:
 * sort/count/index dispatch instead of one-hot matrix products).
 * topk_idx       [T][k] int32 in: entries outside [0, E) are dropped picks
 *                (not counted, pos = -1, no row).
 * expert_counts  [E]   out: c[e]; viewed as R x L (row = destination rank,
 *                column = local slot) it is S.
 * expert_offsets [E]   out: first row of expert e's bucket.
 * rank_counts    [W*R] out: rows wave w sends to rank r (Alltoallv sendcounts).
 * rank_offsets   [W*R] out: absolute first row of (w, r); the wave-local
 *                sdispls are rank_offsets[w*R + r] - wave_offsets[w].
 * wave_offsets   [W+1] out: first row of each wave; wave_offsets[W] = rows.
 * pos            [T][k] out: send-buffer row of pick (t, i).
 * row_token      [T*k] out: token of each row (rows >= sum c are untouched).
 * workspace      device scratch of moe_dispatch_workspace_bytes(shape) bytes
 *                (contents need not be initialised; clobbered by the call).
 * Errors: MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED,
 *         MOE_ERR_DEVICE. */
int moe_dispatch_index(const moe_shape* shape, const int32_t* topk_idx,
                       int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* rank_counts, int32_t* rank_offsets,
                       int32_t* wave_offsets, int32_t* pos, int32_t* row_token,
                       void* workspace, size_t workspace_bytes,
                       moe_stream_t stream);

/* Routing, the index stage and (optionally) the skew statistics in two
 * launches: moe_route, then moe_dispatch_index, then moe_stats on the counts
 * when stats is non-NULL, with identical results, but the counting pass runs
 * inside the routing kernel (each routing block histograms its own picks) and
 * the statistics come from one extra block of the placing kernel.
 * logits [T][E] fp32 in; topk_idx, topk_w [T][k] out (as moe_route); the
 * index outputs as moe_dispatch_index; stats: NULL or one device moe_stats_t
 * (8-byte aligned). workspace: moe_dispatch_workspace_bytes(shape) bytes.
 * Errors: as moe_route and moe_dispatch_index. */
int moe_route_index(const moe_shape* shape, const float* logits, int32_t* topk_idx,
                    float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                    int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                    int32_t* pos, int32_t* row_token, moe_stats_t* stats, void* workspace,
                    size_t workspace_bytes, moe_stream_t stream);

/* moe_route_index followed by moe_dispatch_copy (routing, counts, offsets,
 * positions, the optional statistics and the permute copy) with identical
 * results. When all T * k picks fit one 1024-pick batch (the decode regime)
 * it is TWO launches: the routing kernel, then the one-launch dispatch of
 * moe_dispatch with one extra block for the statistics. Otherwise the three
 * launches of the two calls (routing with the counting pass, placing with the
 * statistics block, copy). Arguments as those two calls (logits [T][E] fp32,
 * x [T][H], send_buf [T*k][H]; stats NULL or one device moe_stats_t;
 * workspace of moe_dispatch_workspace_bytes(shape) bytes, unused by the
 * one-launch dispatch). Errors: as moe_route_index and moe_dispatch_copy. */
int moe_route_dispatch(const moe_shape* shape, const float* logits, const void* x,
                       int32_t* topk_idx, float* topk_w, void* send_buf, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                       int32_t* wave_offsets, int32_t* pos, int32_t* row_token,
                       moe_stats_t* stats, void* workspace, size_t workspace_bytes,
                       moe_stream_t stream);

/* The permute copy (explainer section 3 item 5: rows are reordered by
 * destination and packed before sending): send_buf[pos[t][i]][:] = x[t][:],
 * a bit copy. Each x row is read once and written k times; picks with
 * pos outside [0, T*k) are skipped.
 * x [T][H], send_buf [T*k][H] (dtype of shape). */
int moe_dispatch_copy(const moe_shape* shape, const void* x, const int32_t* pos,
                      void* send_buf, moe_stream_t stream);

/* moe_dispatch_index followed by moe_dispatch_copy on the same stream, with
 * identical results. When all T * k picks fit one 1024-pick batch (T * k <=
 * 1024, E <= 1024: the decode regime) it is ONE launch: every block reads all
 * expert ids and places all picks itself (no device-wide ordering point is
 * needed), then copies its share of the rows; block 0 writes the index tables
 * (the workspace is then unused). Otherwise count, place and copy launches. */
int moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                 void* send_buf, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* rank_counts,
                 int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                 int32_t* row_token, void* workspace, size_t workspace_bytes,
                 moe_stream_t stream);

/* moe_dispatch without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The index stage's per-chunk histograms live in a
 * static device array of moe_noalloc_scratch_bytes() = 256 KiB that the
 * library holds on each device it runs on until the process ends (its device
 * address is looked up on the first call made with that device current).
 * Same arguments, results and launches as moe_dispatch (whose one-launch form
 * for T * k <= 1024 needs no histogram at all); nothing is allocated or freed. Every call on one device shares that device's array: calls that
 * overlap on one device (concurrent streams, or several host threads) race
 * and must be serialised by the caller. The array's contents need no
 * initialisation (each call writes every histogram row it reads).
 * Errors: as moe_dispatch; MOE_ERR_WORKSPACE when the shape's histogram
 * (chunks x E int32) exceeds the array (no valid shape does: at most
 * 65536 / pow2(E) chunks of E counts); MOE_ERR_DEVICE when the array's device
 * address cannot be found or a launch fails. */
int moe_dispatch_noalloc(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                         void* send_buf, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* rank_counts, int32_t* rank_offsets, int32_t* wave_offsets,
                         int32_t* pos, int32_t* row_token, moe_stream_t stream);

/* Bytes of the static device array moe_dispatch_noalloc uses (host-only). */
size_t moe_noalloc_scratch_bytes(void);

/* Expert capacity (MoE systems survey section 1.2 item 2, eq. (3)): rows per
 * expert for capacity factor f, ceil(k * f * T / E) evaluated in double in
 * that order. Host-only, pure; -1 for k < 1, T < 0, E < 1, f < 0 (or NaN) or a
 * result beyond int32. */
int32_t moe_expert_capacity(int32_t k, double f, int32_t T, int32_t E);

/* Wave-scheduled exchange model (irregular AllToAll page, "optimal wave
 * count"; host-only, pure): the end-to-end time of W expert waves
 *   T(W) = W alpha + M / beta + M / (W beta)
 * with alpha the start latency of one wave (s), beta one link's bandwidth
 * (bytes/s) and M the bytes the most loaded link carries. -1 for W < 1,
 * alpha < 0, beta <= 0 or M < 0. */
double moe_wave_time(double message_bytes, double alpha_s, double beta_bytes_per_s, int32_t W);

/* The wave count for this layout: the divisor W of L (the local experts per
 * rank; waves split them, so L mod W = 0) with the smallest T(W), ties to the
 * smaller W (the real optimum is sqrt(M / (alpha beta)); the page's NVLink 5.0
 * example, 16 MB at 1 us and 50 GB/s, gives about 18). Writes T(W) to
 * *time_out when non-NULL. -1 for L < 1 or invalid model parameters. */
int32_t moe_plan_waves(double message_bytes, double alpha_s, double beta_bytes_per_s, int32_t L,
                       double* time_out);

/* 95th-percentile bytes on one link when `tokens` tokens pick among
 * `destinations` equally likely destinations (irregular AllToAll page,
 * "long-tail latency"; normal approximation of the multinomial, valid for
 * tokens / destinations >= 10): mean (1 + 1.645 sqrt(destinations / tokens)).
 * -1 for destinations < 1, tokens <= 0 or mean < 0. */
double moe_link_p95(double mean_bytes, double tokens, int32_t destinations);

/* Capacity-factor dispatch (survey section 1.2 eq. (3) and section 1.1 EP flow
 * step 2: samples beyond an expert's capacity are dropped, unused capacity is
 * padded with zeros). Every bucket holds exactly `capacity` rows; bucket j of
 * the (wave, rank, slot) order starts at row j * capacity; an expert keeps its
 * first `capacity` picks in (token, pick) order and drops the rest (pos = -1),
 * as it drops ids outside [0, E).
 * send_buf       [E*capacity][H] out: kept rows, zero rows for padding.
 * kept_counts    [E] out: min(c[e], capacity).
 * expert_offsets [E] out: first row of expert e's bucket (= j * capacity).
 * rank_counts, rank_offsets [W*R], wave_offsets [W+1] out: whole buckets
 *                (padding is part of what each destination receives).
 * pos [T][k] out; row_token [E*capacity] out (-1 on padding rows).
 * workspace: moe_dispatch_workspace_bytes(shape) bytes.
 * Four launches: count, place, copy, pad. Follow with moe_expert_scale_rows /
 * moe_combine_rows with rows = E * capacity.
 * Errors: MOE_ERR_ARG (capacity < 0, E*capacity rows beyond the index limits,
 *         null pointers), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED,
 *         MOE_ERR_DEVICE. */
int moe_dispatch_capacity(const moe_shape* shape, int32_t capacity, const void* x,
                          const int32_t* topk_idx, void* send_buf, int32_t* kept_counts,
                          int32_t* expert_offsets, int32_t* rank_counts,
                          int32_t* rank_offsets, int32_t* wave_offsets, int32_t* pos,
                          int32_t* row_token, void* workspace, size_t workspace_bytes,
                          moe_stream_t stream);

/* Identity-scaled experts (the experts of the synthetic workloads):
 * expert_out[n][:] = round_dtype((e(n) + 1) * send_buf[n][:]) for every row n
 * inside some expert's bucket [expert_offsets[e], + expert_counts[e]); other
 * rows are untouched. Rounding is to nearest, ties to even. The buckets must
 * lie in the (wave, rank, slot) order of the shape's R and W, as every dispatch
 * entry writes them; plain expert order (moe_vsrc_regroup's grouped layout) is
 * that order with W = 1. */
int moe_expert_scale(const moe_shape* shape, const void* send_buf,
                     const int32_t* expert_offsets,
                     const int32_t* expert_counts, void* expert_out,
                     moe_stream_t stream);

/* moe_expert_scale over a send buffer of `rows` rows (the capacity layout has
 * E*capacity rows instead of T*k). */
int moe_expert_scale_rows(const moe_shape* shape, int64_t rows, const void* send_buf,
                          const int32_t* expert_offsets, const int32_t* expert_counts,
                          void* expert_out, moe_stream_t stream);

/* Bytes of device workspace moe_expert_swiglu needs (the bf16 intermediate,
 * T*k x I); 0 for an invalid shape or I. Host-only, pure. */
size_t moe_expert_swiglu_workspace_bytes(const moe_shape* shape, int32_t I);

/* SwiGLU expert FFN on each expert's contiguous rows (expert compute, survey
 * section 1.1 EP flow step 3; per-expert variable-size GEMMs driven by the
 * counts, survey section 4.1), on MFMA:
 *   g = s . Wg[e][j], u = s . Wu[e][j]      (fp32 accumulation over H)
 *   h_j = round_bf16( g / (1 + exp(-g)) * u )   (stored in the workspace)
 *   expert_out[n][c] = round_bf16( sum_j Wd[e][c][j] h_j )  (fp32 accumulation)
 * for every row n in [expert_offsets[e], + expert_counts[e]); other rows are
 * untouched. bf16 only (shape->dtype == MOE_BF16); I % 64 == 0, H % 128 == 0,
 * 4*I*H < 2^31 and 512*H < 2^31 (one expert's weights and one 256-row tile are
 * addressed with 31-bit byte offsets).
 * w_gate_up [E][2I][H] bf16 (rows 0..I-1 gate, I..2I-1 up), w_down [E][H][I]
 * bf16, send_buf and expert_out [T*k][H], all 16-byte aligned. workspace:
 * moe_expert_swiglu_workspace_bytes(shape, I) bytes, clobbered.
 * Two chains: with side_stream non-NULL the odd-id experts run there (their
 * gate/up then down GEMM) while the even-id experts run on `stream`, so one
 * chain's partial last round of tiles is filled by the other's. side_stream
 * is forked from `stream` by recording fork_event on `stream` (after the work
 * already queued there) and joined back by recording join_event on
 * side_stream, which `stream` then waits on: ordering is as one call on
 * `stream`. All three are the caller's (hipStream_t, hipEvent_t handles, on
 * the device of `stream`, default priority); a caller running several FFN
 * calls at once gives each its own side stream and events. side_stream NULL:
 * one chain of all experts on `stream` (the events are then ignored). The
 * call can be captured in a HIP graph (record and wait become graph edges).
 * Errors: MOE_ERR_ARG (also side_stream without both events), MOE_ERR_ALIGN,
 *         MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
int moe_expert_swiglu(const moe_shape* shape, int32_t I, const void* send_buf,
                      const int32_t* expert_offsets, const int32_t* expert_counts,
                      const void* w_gate_up, const void* w_down, void* expert_out,
                      void* workspace, size_t workspace_bytes, moe_stream_t stream,
                      moe_stream_t side_stream, void* fork_event, void* join_event);

/* Combine, MoE systems survey section 1.1 eq. (1) and EP flow step 4 (restore
 * the original token order, weight each expert output by its gate value):
 *   y[t][:] = round_dtype( fma-chain over i = 0..k-1 of
 *             topk_w[t][i] * expert_out[pos[t][i]][:] )
 * accumulated in fp32 in pick order with fused multiply-adds starting from -0
 * (the additive identity, so identity experts return x bit for bit, -0
 * included), rounded once to nearest-even. Picks with pos outside [0, T*k)
 * contribute nothing.
 * expert_out [T*k][H], topk_w [T][k] fp32, pos [T][k], y [T][H]. */
int moe_combine(const moe_shape* shape, const void* expert_out,
                const float* topk_w, const int32_t* pos, void* y,
                moe_stream_t stream);

/* moe_combine over an expert-row buffer of `rows` rows (E*capacity for the
 * capacity layout): picks with pos outside [0, rows) contribute nothing. */
int moe_combine_rows(const moe_shape* shape, int64_t rows, const void* expert_out,
                     const float* topk_w, const int32_t* pos, void* y,
                     moe_stream_t stream);

/* Skew statistics of S from expert_counts [E] (DODOCO summary, "metrics"):
 * per-expert max/mean and the Gini coefficient
 *   G(v) = sum_a sum_b |v_a - v_b| / (2 n sum v)
 * of the per-rank loads (and of the per-expert loads), with exact 64-bit
 * integer numerators and one double division each; 0 when sum v = 0.
 * out: DEVICE pointer to one moe_stats_t.
 * Errors: MOE_ERR_ARG (null pointer, E outside the limits, E % R != 0). */
int moe_stats(const int32_t* expert_counts, int32_t E, int32_t R,
              moe_stats_t* out, moe_stream_t stream);

/* Fitted symmetric Dirichlet alpha of the expert counts (DODOCO summary,
 * "metrics": the third scalar summary of S, resolving near-uniform routings
 * where the Gini coefficient compresses). Reading: the maximum-likelihood
 * alpha of a Dirichlet-multinomial with E equal concentrations, i.e. the root
 * of sum_{c_e > 0} [psi(c_e + a) - psi(a)] - E [psi(N + E a) - psi(E a)],
 * searched on [1e-8, 1e6]: +inf when the score is still positive at 1e6 (as
 * even as multinomial sampling), 0 when negative at 1e-8, NaN for E < 2 or no
 * picks; otherwise to ~1e-12 relative. One block; writes one device double.
 * Errors: MOE_ERR_ARG (null pointer, E outside [1, 1024]), MOE_ERR_ALIGN
 *         (alpha_out not 8-byte aligned), MOE_ERR_DEVICE. */
int moe_dirichlet_alpha(const int32_t* expert_counts, int32_t E, double* alpha_out,
                        moe_stream_t stream);

/* Completion-wave order of the tokens, for the combine of the wave schedule
 * (irregular AllToAll page, "Wave-Scheduled" pipelining: each wave runs
 * dispatch -> compute -> combine). A token's weighted sum needs all its kept
 * picks' expert outputs, so it is complete after the last wave holding one of
 * its rows: the wave of its largest position, where row r is in the largest
 * wave w with wave_offsets[w] <= r (picks with pos outside [0, T*k) do not
 * count; a token with none is complete before any wave, wave 0).
 * pos [T][k], wave_offsets [W+1]: as written by a dispatch-index call with the
 *   same shape (DEVICE, in).
 * token_wave_offsets [W+1] out: first entry of each wave's tokens (last = T).
 * token_order [T] out: the tokens wave by wave, ascending id within a wave.
 * workspace: device scratch of moe_combine_order_workspace_bytes(shape) bytes
 *   (contents need not be initialised; clobbered by the call).
 * Two launches (a count and a place pass over blocks of tokens).
 * Errors: MOE_ERR_ARG (null pointers, shape), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE,
 *         MOE_ERR_DEVICE. */
int moe_combine_order(const moe_shape* shape, const int32_t* pos, const int32_t* wave_offsets,
                      int32_t* token_wave_offsets, int32_t* token_order, void* workspace,
                      size_t workspace_bytes, moe_stream_t stream);

/* Bytes of device workspace moe_combine_order needs for this shape (host-only,
 * pure; 0 for an invalid shape; at most 2 MiB). */
size_t moe_combine_order_workspace_bytes(const moe_shape* shape);

/* The combine of the tokens whose completion wave lies in [w0, w1) (entries
 * token_wave_offsets[w0] .. token_wave_offsets[w1] of token_order, from
 * moe_combine_order): y[t] for those tokens, with moe_combine's arithmetic,
 * so each token's bits equal moe_combine's; other rows of y are untouched.
 * Over w0..w1 = 0..W, in one call or any split, it writes all of y.
 * expert_out [T*k][H] (the plain layout), topk_w [T][k], pos [T][k], y [T][H].
 * Errors: MOE_ERR_ARG (null pointers, 0 <= w0 <= w1 <= W violated),
 *         MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
int moe_combine_waves(const moe_shape* shape, const void* expert_out, const float* topk_w,
                      const int32_t* pos, const int32_t* token_order,
                      const int32_t* token_wave_offsets, int32_t w0, int32_t w1, void* y,
                      moe_stream_t stream);

/* Wave-pipelined local layer (irregular AllToAll page, "Wave-Scheduled"
 * pipelining: the experts in W waves, each wave's dispatch -> compute ->
 * combine, the next wave's dispatch overlapping this wave's compute). Wave w
 * owns local slots [w*L/W, (w+1)*L/W) of every rank, i.e. the send rows
 * [wave_offsets[w], wave_offsets[w+1]) written by a dispatch-index call with
 * the same shape. For each wave, in order: on copy_stream the gather dispatch
 * send_buf[r] = x[row_token[r]] of the wave's rows, an event, and on
 * compute_stream (after that event) the moe_expert_swiglu arithmetic on the
 * wave's R*L/W experts; with y non-NULL, then the combine of the tokens
 * completed by this wave, after an event on compute_stream: on
 * combine_stream when it is non-NULL (at once), else on copy_stream behind
 * the next wave's gather (the page asks that a wave's dispatch never wait
 * behind a combine; a stream of its own keeps the two apart).
 * Results are bit-identical to moe_dispatch_copy + moe_expert_swiglu (+
 * moe_combine). copy_stream first waits for the work already queued on
 * compute_stream; when this call returns, compute_stream carries every wave's
 * FFN and, with y, joins the last combine (without y, follow with moe_combine
 * there). copy_stream == compute_stream runs the same
 * launches serialised. With side_stream non-NULL, a wave whose experts split
 * into even and odd slots as one stride-2 run of ids each (R == 1, or W == 1)
 * and that holds at least eight experts runs the odd ones on side_stream,
 * forked from compute_stream after the wave's event and joined back into it
 * (as in moe_expert_swiglu).
 * y, topk_w, pos, token_order, token_wave_offsets: the per-wave combine
 * (as moe_combine_waves; token tables from moe_combine_order); y NULL: no
 * combine (the others may be NULL then).
 * events: n_events caller-owned hipEvent_t handles, at least
 * moe_swiglu_waves_events(W) = 2 + 4W of them whenever copy_stream !=
 * compute_stream, side_stream is non-NULL, or y and a combine_stream other
 * than compute_stream are given (one to start the copy stream, one per
 * gather, a fork and a join per wave, one per wave's experts and a final
 * join); unused otherwise. Streams and events are the caller's, on one device.
 * Arguments otherwise as moe_expert_swiglu, plus x [T][H], row_token [T*k],
 * wave_offsets [W+1] (DEVICE). W gathers, 2W FFN kernels (4W with the two
 * chains) and W combines with y.
 * Errors: as moe_expert_swiglu; MOE_ERR_ARG also for null x / row_token /
 *         wave_offsets / combine tables with y, and for too few (or null)
 *         events when they are used. */
int moe_swiglu_waves(const moe_shape* shape, int32_t I, const void* x, const int32_t* row_token,
                     const int32_t* wave_offsets, const int32_t* expert_offsets,
                     const int32_t* expert_counts, const void* w_gate_up, const void* w_down,
                     void* send_buf, void* expert_out, void* workspace, size_t workspace_bytes,
                     const float* topk_w, const int32_t* pos, const int32_t* token_order,
                     const int32_t* token_wave_offsets, void* y, moe_stream_t compute_stream,
                     moe_stream_t copy_stream, moe_stream_t side_stream,
                     moe_stream_t combine_stream, void* const* events, int32_t n_events);

/* The same wave schedule with the identity-scaled experts of moe_expert_scale
 * (the experts of the synthetic workloads): for each wave w, on copy_stream
 * the gather dispatch send_buf[r] = x[row_token[r]] of rows [wave_offsets[w],
 * wave_offsets[w+1]), an event, and on compute_stream the (e+1) scaling of
 * those rows into expert_out; with y non-NULL the per-wave combine as in
 * moe_swiglu_waves (on combine_stream, or behind the next gather on
 * copy_stream when it is NULL). Results are bit-identical to moe_dispatch_copy +
 * moe_expert_scale (+ moe_combine; without y follow with moe_combine on
 * compute_stream). copy_stream first waits for the work already queued on
 * compute_stream; copy_stream == compute_stream runs the same launches
 * serialised. events: at least moe_scale_waves_events(W) = 2 + 2W caller-owned
 * hipEvent_t handles when copy_stream != compute_stream, or y and a
 * combine_stream other than compute_stream are given (unused otherwise). 2W launches,
 * 3W with y. row_token, wave_offsets, expert_offsets, expert_counts as
 * written by a dispatch-index call with the same shape (DEVICE).
 * Errors: MOE_ERR_ARG (null pointers, too few or null events), MOE_ERR_ALIGN,
 *         MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
int moe_scale_waves(const moe_shape* shape, const void* x, const int32_t* row_token,
                    const int32_t* wave_offsets, const int32_t* expert_offsets,
                    const int32_t* expert_counts, void* send_buf, void* expert_out,
                    const float* topk_w, const int32_t* pos, const int32_t* token_order,
                    const int32_t* token_wave_offsets, void* y, moe_stream_t compute_stream,
                    moe_stream_t copy_stream, moe_stream_t combine_stream, void* const* events,
                    int32_t n_events);

/* Events moe_swiglu_waves needs for W waves: 2 + 4W (-1 for W outside
 * [1, 2^20]). Host-only, pure. */
int32_t moe_swiglu_waves_events(int32_t W);

/* Events moe_scale_waves needs for W waves: 2 + 2W (-1 for W outside
 * [1, 2^20]). Host-only, pure. */
int32_t moe_scale_waves_events(int32_t W);

/* ---------------------------------------------------------------------------
 * Virtual-source exchange: the expert-parallel exchange of R ranks emulated on
 * one device (MoE systems survey, crad.ict.ac.cn, section 1.1, EP flow steps
 * 2-4; irregular AllToAll page, "sources of irregular a2a": every (source,
 * destination) pair has its own row count, possibly 0, as an Alltoallv takes
 * them). The T tokens split into R equal source shards (T % R == 0): source s
 * holds tokens [s*T/R, (s+1)*T/R). Destination d owns experts d*L .. d*L+L-1,
 * L = E/R; with W waves each (source, wave, destination) triple is one
 * message. All counts and offsets are in rows; offsets are absolute rows of the
 * concatenated buffers below, so a real Alltoallv of rank s would take the
 * rows of its own slice, relative to its own first row. Buffers hold T*k rows
 * of H elements (row layout as in moe_dispatch):
 *   send     source s at rows [s*T/R*k, (s+1)*T/R*k) in the single-rank
 *            dispatch layout of its own tokens (buckets in (wave, destination,
 *            slot) order, token order inside a bucket); rows of dropped ids
 *            (outside [0, E)) stay unused at the end of the source's range.
 *   recv     the (destination, wave, source) messages back to back.
 *   grouped  each destination's rows by local expert, then source, i.e. over
 *            all destinations expert order and token order inside an expert.
 * Rows past the last message or segment are left as they are.
 * One call of each direction at a time per buffer set; all on `stream`. */

/* Workspace bytes of moe_vsrc_dispatch and moe_vsrc_regroup for this shape
 * (0 if the shape is invalid). */
size_t moe_vsrc_workspace_bytes(const moe_shape* shape);

/* Every source's dispatch at once plus the count exchange (one-rank dispatch
 * of each shard, then the receive side's tables).
 * x [T][H] in; topk_idx [T][k] in; send_buf [T*k][H] out.
 * src_counts   [R][E] out: picks of expert e among source s's tokens.
 * src_offsets  [R][E] out: first send row of source s's bucket of expert e.
 * send_counts  [R][W][R] out: rows source s sends in wave w to destination d.
 * send_offsets [R][W][R] out: first send row of that message.
 * recv_counts  [R][W][R] out: rows destination d receives in wave w from
 *              source s (= send_counts transposed).
 * recv_offsets [R][W][R] out: first recv row of that message.
 * expert_counts, expert_offsets [E] out: the grouped layout, buckets in
 *              expert order (for moe_vsrc_regroup, moe_expert_swiglu, and
 *              moe_expert_scale_rows with a shape of W = 1).
 * pos [T][k] out: send row of each pick, -1 for dropped ids (combine input).
 * Four launches: count, place (per shard), plan, copy. All pointers DEVICE.
 * Errors: MOE_ERR_ARG (T % R != 0, shape outside the limits, null pointers),
 *         MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
int moe_vsrc_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                      void* send_buf, int32_t* src_counts, int32_t* src_offsets,
                      int32_t* send_counts,
                      int32_t* send_offsets, int32_t* recv_counts, int32_t* recv_offsets,
                      int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                      void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* The all-to-all as a block transpose of whole messages. direction 0
 * (dispatch): in = send layout, out = recv layout; direction 1 (combine): in =
 * recv layout, out = send layout (the reverse exchange of the expert rows).
 * send_offsets, recv_counts, recv_offsets as written by moe_vsrc_dispatch;
 * entries that do not describe rows inside the buffers are skipped. One launch.
 * Errors: MOE_ERR_ARG (direction not 0/1, null pointers, shape), MOE_ERR_ALIGN
 *         (buffers not 16-byte aligned), MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE. */
int moe_vsrc_exchange(const moe_shape* shape, int32_t direction, const void* in, void* out,
                      const int32_t* send_offsets, const int32_t* recv_counts,
                      const int32_t* recv_offsets, moe_stream_t stream);

/* The exchange written straight into the receivers' grouped layout, one pass:
 * every (expert, source) segment goes from source s's bucket of expert e in the
 * send layout to its rows in the grouped layout (what one-sided stores into
 * peer receive buffers do, with the counts exchanged first), i.e.
 * moe_vsrc_exchange followed by moe_vsrc_regroup in one copy. direction 0:
 * in = send layout, out = grouped layout; direction 1: in = grouped layout,
 * out = send layout. src_counts, src_offsets, expert_offsets as written by
 * moe_vsrc_dispatch. Two launches (segment table into the workspace, then the
 * copy). Errors: as moe_vsrc_regroup. */
int moe_vsrc_exchange_direct(const moe_shape* shape, int32_t direction, const void* in,
                             void* out, const int32_t* src_counts, const int32_t* src_offsets,
                             const int32_t* expert_offsets, void* workspace,
                             size_t workspace_bytes, moe_stream_t stream);

/* Receive-side regroup of every destination from its (wave, source) messages
 * into (local expert, source) order. direction 0: in = recv layout, out =
 * grouped layout; direction 1: in = grouped layout, out = recv layout.
 * src_counts, recv_offsets, expert_offsets as written by moe_vsrc_dispatch.
 * Two launches (segment table into the workspace, then the copy).
 * Errors: as moe_vsrc_exchange, plus MOE_ERR_WORKSPACE. */
int moe_vsrc_regroup(const moe_shape* shape, int32_t direction, const void* in, void* out,
                     const int32_t* src_counts, const int32_t* recv_offsets,
                     const int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                     moe_stream_t stream);

/* Kernel timing hook for benchmarks (not a step of the path). After
 * moe_set_timing_events(starts, stops, n), the kernels this library launches
 * from the calling thread use AMD's extended launch: the i-th one (i < n, at
 * most 8) records starts[i] when it begins executing and stops[i] when it
 * ends, so hipEventElapsedTime(starts[i], stops[i]) is that kernel's execution
 * time. Later launches are not timed. Events are created by the caller
 * (hipEventCreate) and passed as void* hipEvent_t handles. Thread-local;
 * n = 0 turns it off. Errors: MOE_ERR_ARG (n outside [0, 8], NULL arrays). */
int moe_set_timing_events(void* const* start_events, void* const* stop_events,
                          int32_t n);

/* Number of kernels launched from the calling thread since the last
 * moe_set_timing_events call (counted only while n > 0). */
int moe_timed_launches(void);

/* Human-readable name of a moe_status value (static string, never NULL). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ROUTE_H */
