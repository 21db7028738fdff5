/*
 * oracle.h -- plain single-threaded CPU reference of the MoE routing,
 * dispatch, expert, combine and skew-statistics path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this code: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do. It shares no header, helper, table or constant with
 * the HIP library under combine_moe_route_03_amd/csrc.
 *
 * Conventions
 *   - Floating point is IEEE double unless a function says otherwise.
 *   - bf16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   - Token-major row layouts: logits[T][E], x[T][H], idx/w/pos[T][k].
 *   - Expert e lives on rank e / L (L = E / R local experts per rank) in local
 *     slot e % L; its wave is floor(slot * W / L).
 *   - Buckets are ordered by (wave, rank, local slot); inside a bucket, rows
 *     follow ascending token index.
 *   - A pick whose expert id lies outside [0, E) is dropped: it is not counted,
 *     gets pos = -1, and contributes nothing to the combine.
 *
 * Parity status per function is stated in each comment ("pinned by").
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Top-k gating, MoE systems survey (crad.ict.ac.cn) section 1.1, eq. (2):
 * G(x) = softmax(TopK(x W_gate, k)); the logits x W_gate are the input.
 * idx[t][i]: the i-th largest logit of row t (ties -> lower expert id).
 * w[t][i]  : exp(l_i - l_0) / sum_j exp(l_j - l_0) in double. */
void oracle_route(const float* logits, int64_t T, int32_t E, int32_t k,
                  int32_t* idx, double* w);

/* Send-count matrix S (DODOCO summary, "metrics"; irregular AllToAll page,
 * "EP irregular a2a" and "link to other primitives"): expert_counts[e] is the
 * number of picks of expert e; viewed as R x L it is S. rank_counts[w*R+r] is
 * the number of rows wave w sends to rank r (Alltoallv send counts). */
void oracle_counts(const int32_t* idx, int64_t T, int32_t k, int32_t E,
                   int32_t R, int32_t W, int32_t* expert_counts,
                   int32_t* rank_counts);

/* Exclusive prefix sums in bucket order: expert_offsets[E], rank_offsets[W*R]
 * (absolute first row), wave_offsets[W+1]. */
void oracle_offsets(const int32_t* expert_counts, int32_t E, int32_t R,
                    int32_t W, int32_t* expert_offsets, int32_t* rank_offsets,
                    int32_t* wave_offsets);

/* Stable positions (MoE systems survey section 1.1, EP flow step 2: invert
 * token->expert into expert->token and place same-expert tokens contiguously).
 * pos[t][i] = expert_offsets[e] + #{t' < t : e in idx[t']}; row_token[pos] = t.
 * row_token entries past the last placed row are left untouched. */
void oracle_positions(const int32_t* idx, int64_t T, int32_t k, int32_t E,
                      const int32_t* expert_offsets, int32_t* pos,
                      int32_t* row_token);

/* send_buf[n][:] = x[row_token[n]][:] for n < nrows (raw byte copy). */
void oracle_dispatch_copy(const void* x, int64_t row_bytes,
                          const int32_t* row_token, int64_t nrows,
                          void* send_buf);

/* Expert capacity, MoE systems survey section 1.2 item 2), eq. (3): the rows
 * one expert may take, k * f * T / E for capacity factor f, rounded up to a
 * whole row (the equation is garbled in extraction; the fraction bar is read
 * under T / E). Evaluated in double in the order ((k * f) * T) / E. Returns -1
 * for f < 0 or a result that does not fit int32. */
int32_t oracle_expert_capacity(int32_t k, double f, int64_t T, int32_t E);

/* Capacity-factor dispatch (survey section 1.2 eq. (3) and EP flow step 2:
 * samples beyond an expert's capacity are dropped, unused capacity is padded
 * with zeros). Every expert bucket has exactly cap rows; bucket j of the
 * (wave, rank, slot) order starts at row j * cap. An expert keeps its first
 * cap picks in (token, pick) order; later picks are dropped (pos = -1), as are
 * picks with ids outside [0, E). Outputs:
 *   kept_counts[e] = min(c[e], cap); expert_offsets[e] = j(e) * cap;
 *   rank_counts[w*R+r], rank_offsets[w*R+r], wave_offsets[W+1]: whole buckets
 *   (padding included: it is part of what each destination receives);
 *   pos[t][k]; row_token[E*cap] (-1 on padding rows); send_buf[E*cap][row]
 *   (x rows, zero bytes on padding rows). */
void oracle_dispatch_capacity(const void* x, int64_t row_bytes, const int32_t* idx,
                              int64_t T, int32_t k, int32_t E, int32_t R, int32_t W,
                              int32_t cap, int32_t* kept_counts,
                              int32_t* expert_offsets, int32_t* rank_counts,
                              int32_t* rank_offsets, int32_t* wave_offsets,
                              int32_t* pos, int32_t* row_token, void* send_buf);

/* Identity-scaled experts: out[n] = round_dtype((e(n) + 1) * in[n]) where
 * e(n) is the expert whose bucket holds row n. */
void oracle_expert_scale(const void* in, int32_t dtype, int64_t H, int32_t E,
                         const int32_t* expert_offsets,
                         const int32_t* expert_counts, void* out);

/* Combine, MoE systems survey section 1.1 eq. (1) and EP flow step 4:
 * y[t][h] = sum_i w[t][i] * out[pos[t][i]][h], all in double, unrounded. */
void oracle_combine_f64(const void* expert_out, int32_t dtype, int64_t T,
                        int64_t H, int32_t k, const double* w,
                        const int32_t* pos, int64_t nrows, double* y);

/* The same sum with the output quantised in the precision a single-precision
 * kernel decides it in: acc = 0f; acc = fmaf(w_i, out_i, acc) for i = 0..k-1
 * (pick order); y = round_to_nearest_even_dtype(acc). w is fp32 here. */
void oracle_combine_f32fma(const void* expert_out, int32_t dtype, int64_t T,
                           int64_t H, int32_t k, const float* w,
                           const int32_t* pos, int64_t nrows, void* y);

/* The whole path for identity-scaled experts, on selected tokens only: for each
 * listed token t, y[j][h] = sum_i w[t][i] * round_dtype((idx[t][i] + 1) * x[t][h])
 * (combine of the scaled copies of x[t]; survey section 1.1 eq. (1)).
 * y_f64 [n][H] is the double sum; y_q [n][H] is the same sum taken as the
 * single-precision fma chain in pick order with fp32 weights w32, rounded to
 * dtype (the kernel-precision quantisation). Either output may be NULL. */
void oracle_scaled_tokens(const void* x, int32_t dtype, int64_t H, int32_t E,
                          int32_t k, const int32_t* idx, const double* w,
                          const float* w32, const int64_t* tokens, int64_t n,
                          double* y_f64, void* y_q);

/* Completion-wave order of the tokens for a per-wave combine (irregular
 * AllToAll page, "Wave-Scheduled pipelining": each wave's dispatch -> compute
 * -> combine). Token t is complete after wave max_i wave_of(idx[t][i]) over
 * its kept picks (0 when it has none). token_wave_offsets [W+1]: first entry
 * of each wave's tokens (last = T); token_order [T]: tokens wave by wave,
 * ascending within a wave. */
void oracle_combine_order(const int32_t* idx, int64_t T, int32_t k, int32_t E,
                          int32_t R, int32_t W, int32_t* token_wave_offsets,
                          int32_t* token_order);

/* SwiGLU expert FFN of the local-layer workload, on selected send-buffer rows
 * (the pages name only an FFN; the workload fixes SwiGLU, intermediate size I,
 * bf16 weights). For row n of expert e = row_expert[n], in double:
 *   g_j = sum_h Wg[e][j][h] s[h],  u_j = sum_h Wu[e][j][h] s[h]   (j < I)
 *   h_j = round_bf16( g_j / (1 + exp(-g_j)) * u_j )   (bf16 intermediate)
 *   out[c] = sum_j Wd[e][c][j] h_j                     (c < H)
 * w_gate_up [E][2I][H] bf16 (rows 0..I-1 gate, I..2I-1 up); w_down [E][H][I].
 * out_f64 [n][H] is the double sum, out_bf16 [n][H] its bf16 rounding;
 * gu_out [n][2I] receives g_j (first I) and u_j (last I) of each row, the
 * pre-activation sums the tests' rounding-flip bound is built from (any of
 * the three may be NULL). */
void oracle_expert_swiglu_rows(const uint16_t* rows, const int32_t* row_expert,
                               int64_t n, int64_t H, int64_t I,
                               const uint16_t* w_gate_up,
                               const uint16_t* w_down, double* out_f64,
                               uint16_t* out_bf16, double* gu_out);

/* Skew statistics of S, DODOCO summary ("metrics"): per-expert max/mean and
 * Gini coefficient of per-rank loads (per-expert Gini alongside). */
typedef struct {
  double expert_max_over_mean;
  double expert_gini;
  double rank_max_over_mean;
  double rank_gini;
  int64_t total;
  int32_t expert_max;
  int32_t expert_min;
  int32_t rank_max;
  int32_t rank_min;
} oracle_stats_t;

void oracle_stats(const int32_t* expert_counts, int32_t E, int32_t R,
                  oracle_stats_t* out);

/* Fitted symmetric Dirichlet alpha of the expert counts (DODOCO summary,
 * "metrics": the third scalar summary of S, resolving near-uniform routings
 * where Gini compresses). Reading: the maximum-likelihood alpha of a
 * Dirichlet-multinomial with E equal concentrations,
 *   L(a) = lnG(E a) - lnG(N + E a) + sum_e [lnG(c_e + a) - lnG(a)],
 * whose derivative for integer counts is the finite sum
 *   L'(a) = sum_e sum_{j < c_e} 1 / (a + j) - E sum_{j < N} 1 / (E a + j).
 * The root of L' is found by bisecting its sign on ln a over [1e-8, 1e6].
 * Returns +inf when L' > 0 at 1e6 (counts as even as multinomial sampling, or
 * so close that the score's sign beyond 1e6 is below double precision in a
 * digamma evaluation), 0 when L' < 0 at 1e-8, NaN for E < 2 or N = 0. */
double oracle_dirichlet_alpha(const int32_t* counts, int32_t E);

/* Wave-scheduled exchange model (irregular AllToAll page, "optimal wave
 * count"): end-to-end time of W waves, T(W) = W a + M / b + M / (W b), with a
 * the per-wave start latency (s), b the link bandwidth (bytes/s), M the bytes
 * one link carries. */
double oracle_wave_time(double M, double a, double b, double W);

/* The minimiser of T over real W > 0: sqrt(M / (a b)) (same passage). */
double oracle_optimal_waves(double M, double a, double b);

/* The layout needs L mod W = 0: the divisor W of L with the smallest T(W)
 * (ties to the smaller W), found by trying every W = 1..L. */
int32_t oracle_plan_waves(double M, double a, double b, int32_t L);

/* 95th-percentile per-link volume under the normal approximation of the
 * multinomial (irregular AllToAll page, "long-tail latency"):
 * m_p95 = m_avg (1 + 1.645 sqrt(1 / (B p))), p = 1 / n for n destinations,
 * B tokens. The page notes the approximation fails for B p < 10. */
double oracle_link_p95(double m_avg, double B, int32_t n);

/* Gini of n non-negative integers: sum_a sum_b |v_a - v_b| / (2 n sum v). */
double oracle_gini_i64(const int64_t* v, int32_t n);

/* Round a double to the nearest bf16 (ties to even); returns the bit pattern. */
uint16_t oracle_round_bf16(double v);

#ifdef __cplusplus
}
#endif
#endif
