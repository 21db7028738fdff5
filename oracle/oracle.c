/*
 * oracle.c -- plain single-threaded CPU reference of the MoE routing path.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the CPU
 * baseline of the benchmark; never by the product path. Every function is the
 * plain definition of what it computes, written for a reader to check by eye
 * against the pages cited in oracle.h: no blocking, no fusion, no reordering.
 * Floating point is double; the only single-precision code is
 * oracle_combine_f32fma, which states the quantisation decision in the
 * precision a single-precision kernel takes it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared oracle.c -lm
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ layout */

/* Local experts per rank; expert e is on rank e / L in slot e % L
 * (experts split evenly over devices, several per card: cross-card
 * communication explainer, section 3 item 1). */
static int32_t rank_of(int32_t e, int32_t L) { return e / L; }
static int32_t slot_of(int32_t e, int32_t L) { return e % L; }
/* W waves of E / W experts each (irregular AllToAll page, "Wave-Scheduled");
 * membership by local slot so that every wave reaches every rank. */
static int32_t wave_of(int32_t e, int32_t L, int32_t W) {
  return (int32_t)(((int64_t)slot_of(e, L) * W) / L);
}

/* ---------------------------------------------------------------- rounding */

uint16_t oracle_round_bf16(double v) {
  /* bf16: 1 sign bit, 8 exponent bits (as fp32), 8 significant bits. */
  uint32_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)0x7FC0u;
  if (a == 0.0) return (uint16_t)sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  int ex;
  (void)frexp(a, &ex); /* a = m * 2^ex, m in [0.5, 1) */
  int qexp = ex - 8;   /* spacing of bf16 values around a */
  if (qexp < -133) qexp = -133; /* subnormal spacing */
  double q = ldexp(1.0, qexp);
  double r = nearbyint(a / q) * q; /* default rounding mode: ties to even */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return (uint16_t)(sign | (bits >> 16));
}

static double load_elem(const void* base, int32_t dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static double load_elem_bits_bf16(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static void store_elem(void* base, int32_t dtype, int64_t i, double v) {
  if (dtype == ORACLE_F32)
    ((float*)base)[i] = (float)v; /* C conversion: round to nearest even */
  else
    ((uint16_t*)base)[i] = oracle_round_bf16(v);
}

/* ------------------------------------------------------------------- route */

void oracle_route(const float* logits, int64_t T, int32_t E, int32_t k,
                  int32_t* idx, double* w) {
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    memset(taken, 0, (size_t)E);
    /* Selection: the i-th pick is the largest not-yet-taken logit; scanning
     * ids upward with a strict '>' keeps the lower id on ties (+0 == -0). */
    for (int32_t i = 0; i < k; ++i) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      idx[t * k + i] = best;
    }
    /* Softmax over the k kept logits (the others are -inf and contribute 0). */
    double m = (double)l[idx[t * k]];
    double s = 0.0;
    for (int32_t i = 0; i < k; ++i) s += exp((double)l[idx[t * k + i]] - m);
    for (int32_t i = 0; i < k; ++i)
      w[t * k + i] = exp((double)l[idx[t * k + i]] - m) / s;
  }
  free(taken);
}

/* ------------------------------------------------------- counts and offsets */

void oracle_counts(const int32_t* idx, int64_t T, int32_t k, int32_t E,
                   int32_t R, int32_t W, int32_t* expert_counts,
                   int32_t* rank_counts) {
  int32_t L = E / R;
  for (int32_t e = 0; e < E; ++e) expert_counts[e] = 0;
  for (int64_t p = 0; p < T * k; ++p) {
    int32_t e = idx[p];
    if (e < 0 || e >= E) continue; /* dropped pick */
    expert_counts[e] += 1;
  }
  for (int32_t j = 0; j < W * R; ++j) rank_counts[j] = 0;
  for (int32_t e = 0; e < E; ++e)
    rank_counts[wave_of(e, L, W) * R + rank_of(e, L)] += expert_counts[e];
}

void oracle_offsets(const int32_t* expert_counts, int32_t E, int32_t R,
                    int32_t W, int32_t* expert_offsets, int32_t* rank_offsets,
                    int32_t* wave_offsets) {
  int32_t L = E / R;
  int32_t running = 0;
  for (int32_t w = 0; w < W; ++w) {
    wave_offsets[w] = running;
    for (int32_t r = 0; r < R; ++r) {
      rank_offsets[w * R + r] = running;
      for (int32_t s = 0; s < L; ++s) {
        int32_t e = r * L + s;
        if (wave_of(e, L, W) != w) continue;
        expert_offsets[e] = running;
        running += expert_counts[e];
      }
    }
  }
  wave_offsets[W] = running;
}

void oracle_positions(const int32_t* idx, int64_t T, int32_t k, int32_t E,
                      const int32_t* expert_offsets, int32_t* pos,
                      int32_t* row_token) {
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int32_t e = 0; e < E; ++e) cursor[e] = expert_offsets[e];
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t i = 0; i < k; ++i) {
      int32_t e = idx[t * k + i];
      if (e < 0 || e >= E) {
        pos[t * k + i] = -1;
        continue;
      }
      int32_t p = cursor[e]++;
      pos[t * k + i] = p;
      row_token[p] = (int32_t)t;
    }
  }
  free(cursor);
}

void oracle_dispatch_copy(const void* x, int64_t row_bytes,
                          const int32_t* row_token, int64_t nrows,
                          void* send_buf) {
  for (int64_t n = 0; n < nrows; ++n)
    memcpy((char*)send_buf + n * row_bytes,
           (const char*)x + (int64_t)row_token[n] * row_bytes,
           (size_t)row_bytes);
}

/* ---------------------------------------------------- capacity dispatch */

int32_t oracle_expert_capacity(int32_t k, double f, int64_t T, int32_t E) {
  if (!(f >= 0.0) || E <= 0) return -1;
  double ec = ceil((double)k * f * (double)T / (double)E);
  if (ec > 2147483647.0) return -1;
  return (int32_t)ec;
}

void oracle_dispatch_capacity(const void* x, int64_t row_bytes, const int32_t* idx,
                              int64_t T, int32_t k, int32_t E, int32_t R, int32_t W,
                              int32_t cap, int32_t* kept_counts,
                              int32_t* expert_offsets, int32_t* rank_counts,
                              int32_t* rank_offsets, int32_t* wave_offsets,
                              int32_t* pos, int32_t* row_token, void* send_buf) {
  int32_t L = E / R;
  int64_t rows = (int64_t)E * cap;
  /* bucket starts: walk the buckets in (wave, rank, slot) order, cap rows each */
  int32_t j = 0;
  for (int32_t w = 0; w < W; ++w) {
    wave_offsets[w] = j * cap;
    for (int32_t r = 0; r < R; ++r) {
      int32_t first = j, n = 0;
      for (int32_t s = 0; s < L; ++s) {
        int32_t e = r * L + s;
        if (wave_of(e, L, W) != w) continue;
        expert_offsets[e] = j * cap;
        ++j;
        ++n;
      }
      rank_offsets[w * R + r] = first * cap;
      rank_counts[w * R + r] = n * cap;
    }
  }
  wave_offsets[W] = (int32_t)rows;
  /* padding everywhere first; kept rows overwrite it */
  for (int64_t n = 0; n < rows; ++n) row_token[n] = -1;
  memset(send_buf, 0, (size_t)(rows * row_bytes));
  for (int32_t e = 0; e < E; ++e) kept_counts[e] = 0;
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t i = 0; i < k; ++i) {
      int32_t e = idx[t * k + i];
      if (e < 0 || e >= E || kept_counts[e] >= cap) {
        pos[t * k + i] = -1;
        continue;
      }
      int32_t p = expert_offsets[e] + kept_counts[e]++;
      pos[t * k + i] = p;
      row_token[p] = (int32_t)t;
      memcpy((char*)send_buf + (int64_t)p * row_bytes, (const char*)x + t * row_bytes,
             (size_t)row_bytes);
    }
  }
}

/* ------------------------------------------------------------------ expert */

void oracle_expert_scale(const void* in, int32_t dtype, int64_t H, int32_t E,
                         const int32_t* expert_offsets,
                         const int32_t* expert_counts, void* out) {
  for (int32_t e = 0; e < E; ++e) {
    double scale = (double)(e + 1);
    for (int64_t n = expert_offsets[e];
         n < (int64_t)expert_offsets[e] + expert_counts[e]; ++n)
      for (int64_t h = 0; h < H; ++h)
        store_elem(out, dtype, n * H + h, scale * load_elem(in, dtype, n * H + h));
  }
}

void oracle_expert_swiglu_rows(const uint16_t* rows, const int32_t* row_expert,
                               int64_t n, int64_t H, int64_t I,
                               const uint16_t* w_gate_up,
                               const uint16_t* w_down, double* out_f64,
                               uint16_t* out_bf16, double* gu_out) {
  double* hmid = (double*)malloc(sizeof(double) * (size_t)I);
  for (int64_t r = 0; r < n; ++r) {
    const uint16_t* s = rows + r * H;
    const int64_t e = row_expert[r];
    const uint16_t* wg = w_gate_up + e * 2 * I * H;
    const uint16_t* wu = wg + I * H;
    const uint16_t* wd = w_down + e * H * I;
    for (int64_t j = 0; j < I; ++j) {
      double g = 0.0, u = 0.0;
      for (int64_t h = 0; h < H; ++h) {
        double sv = load_elem_bits_bf16(s[h]);
        g += load_elem_bits_bf16(wg[j * H + h]) * sv;
        u += load_elem_bits_bf16(wu[j * H + h]) * sv;
      }
      if (gu_out) {
        gu_out[r * 2 * I + j] = g;
        gu_out[r * 2 * I + I + j] = u;
      }
      double silu = g / (1.0 + exp(-g));
      hmid[j] = load_elem_bits_bf16(oracle_round_bf16(silu * u));
    }
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < I; ++j) acc += load_elem_bits_bf16(wd[c * I + j]) * hmid[j];
      if (out_f64) out_f64[r * H + c] = acc;
      if (out_bf16) out_bf16[r * H + c] = oracle_round_bf16(acc);
    }
  }
  free(hmid);
}

/* ----------------------------------------------------------------- combine */

void oracle_combine_f64(const void* expert_out, int32_t dtype, int64_t T,
                        int64_t H, int32_t k, const double* w,
                        const int32_t* pos, int64_t nrows, double* y) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h) {
      double acc = -0.0; /* additive identity: -0 + v == v for every v */
      for (int32_t i = 0; i < k; ++i) {
        int32_t p = pos[t * k + i];
        if (p < 0 || p >= nrows) continue;
        acc += w[t * k + i] * load_elem(expert_out, dtype, (int64_t)p * H + h);
      }
      y[t * H + h] = acc;
    }
}

void oracle_combine_f32fma(const void* expert_out, int32_t dtype, int64_t T,
                           int64_t H, int32_t k, const float* w,
                           const int32_t* pos, int64_t nrows, void* y) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h) {
      float acc = -0.0f;
      for (int32_t i = 0; i < k; ++i) {
        int32_t p = pos[t * k + i];
        if (p < 0 || p >= nrows) continue;
        float v = (float)load_elem(expert_out, dtype, (int64_t)p * H + h);
        acc = fmaf(w[t * k + i], v, acc);
      }
      store_elem(y, dtype, t * H + h, (double)acc);
    }
}

void oracle_scaled_tokens(const void* x, int32_t dtype, int64_t H, int32_t E,
                          int32_t k, const int32_t* idx, const double* w,
                          const float* w32, const int64_t* tokens, int64_t n,
                          double* y_f64, void* y_q) {
  for (int64_t j = 0; j < n; ++j) {
    int64_t t = tokens[j];
    for (int64_t h = 0; h < H; ++h) {
      double acc = -0.0; /* additive identity: -0 + v == v for every v */
      float acc32 = -0.0f;
      for (int32_t i = 0; i < k; ++i) {
        int32_t e = idx[t * k + i];
        if (e < 0 || e >= E) continue; /* dropped pick */
        /* the expert output element, rounded to dtype as the expert stores it */
        double prod = (double)(e + 1) * load_elem(x, dtype, t * H + h);
        double o = (dtype == ORACLE_F32) ? (double)(float)prod
                                         : load_elem_bits_bf16(oracle_round_bf16(prod));
        if (w) acc += w[t * k + i] * o;
        if (w32) acc32 = fmaf(w32[t * k + i], (float)o, acc32);
      }
      if (y_f64) y_f64[j * H + h] = acc;
      if (y_q) store_elem(y_q, dtype, j * H + h, (double)acc32);
    }
  }
}

/* ------------------------------------------------------- per-wave combine */

/* The wave after which token t's combine can run: its picks' experts sit in
 * waves wave_of(e) (irregular AllToAll page, "Wave-Scheduled pipelining": W
 * waves of E / W experts, each wave running dispatch -> compute -> combine),
 * and the token's weighted sum needs every one of them, so it is complete
 * after the last of those waves. A token without a kept pick is complete
 * before any wave: wave 0. Tokens are listed wave by wave, in token order
 * within a wave; token_wave_offsets[w] is the first entry of wave w and
 * token_wave_offsets[W] = T. */
void oracle_combine_order(const int32_t* idx, int64_t T, int32_t k, int32_t E,
                          int32_t R, int32_t W, int32_t* token_wave_offsets,
                          int32_t* token_order) {
  int32_t L = E / R;
  int32_t* done = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int64_t t = 0; t < T; ++t) {
    int32_t last = 0;
    for (int32_t i = 0; i < k; ++i) {
      int32_t e = idx[t * k + i];
      if (e < 0 || e >= E) continue; /* dropped pick */
      int32_t w = wave_of(e, L, W);
      if (w > last) last = w;
    }
    done[t] = last;
  }
  /* first entry of each wave: tokens of the waves before it */
  for (int32_t w = 0; w <= W; ++w) {
    int32_t before = 0;
    for (int64_t t = 0; t < T; ++t)
      if (done[t] < w) ++before;
    token_wave_offsets[w] = before;
  }
  for (int32_t w = 0; w < W; ++w) {
    int32_t n = token_wave_offsets[w];
    for (int64_t t = 0; t < T; ++t)
      if (done[t] == w) token_order[n++] = (int32_t)t;
  }
  free(done);
}

/* ------------------------------------------------------------------- stats */

double oracle_gini_i64(const int64_t* v, int32_t n) {
  int64_t num = 0, sum = 0;
  for (int32_t a = 0; a < n; ++a) {
    sum += v[a];
    for (int32_t b = 0; b < n; ++b) num += llabs(v[a] - v[b]);
  }
  if (sum == 0) return 0.0;
  return (double)num / (double)(2 * (int64_t)n * sum);
}

/* L'(a) for the symmetric Dirichlet-multinomial, as plain finite sums. */
static double dm_score(const int32_t* counts, int32_t E, int64_t N, double a) {
  double s = 0.0;
  for (int32_t e = 0; e < E; ++e)
    for (int32_t j = 0; j < counts[e]; ++j) s += 1.0 / (a + (double)j);
  double t = 0.0;
  for (int64_t j = 0; j < N; ++j) t += 1.0 / ((double)E * a + (double)j);
  return s - (double)E * t;
}

double oracle_dirichlet_alpha(const int32_t* counts, int32_t E) {
  int64_t N = 0;
  for (int32_t e = 0; e < E; ++e) N += counts[e];
  if (E < 2 || N == 0) return NAN;
  double lo = log(1e-8), hi = log(1e6);
  if (dm_score(counts, E, N, exp(hi)) > 0.0) return INFINITY;
  if (dm_score(counts, E, N, exp(lo)) < 0.0) return 0.0;
  for (int it = 0; it < 200 && hi - lo > 1e-15; ++it) {
    double mid = 0.5 * (lo + hi);
    if (dm_score(counts, E, N, exp(mid)) > 0.0) lo = mid;
    else hi = mid;
  }
  return exp(0.5 * (lo + hi));
}

double oracle_wave_time(double M, double a, double b, double W) {
  return W * a + M / b + M / (W * b);
}

double oracle_optimal_waves(double M, double a, double b) { return sqrt(M / (a * b)); }

int32_t oracle_plan_waves(double M, double a, double b, int32_t L) {
  int32_t best = 1;
  double tbest = oracle_wave_time(M, a, b, 1.0);
  for (int32_t W = 2; W <= L; ++W) {
    if (L % W != 0) continue;
    double t = oracle_wave_time(M, a, b, (double)W);
    if (t < tbest) {
      tbest = t;
      best = W;
    }
  }
  return best;
}

double oracle_link_p95(double m_avg, double B, int32_t n) {
  double p = 1.0 / (double)n;
  return m_avg * (1.0 + 1.645 * sqrt(1.0 / (B * p)));
}

void oracle_stats(const int32_t* expert_counts, int32_t E, int32_t R,
                  oracle_stats_t* out) {
  int32_t L = E / R;
  int64_t* ve = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  int64_t* vr = (int64_t*)calloc((size_t)R, sizeof(int64_t));
  int64_t total = 0;
  for (int32_t e = 0; e < E; ++e) {
    ve[e] = expert_counts[e];
    vr[rank_of(e, L)] += expert_counts[e];
    total += expert_counts[e];
  }
  int64_t emax = ve[0], emin = ve[0], rmax = vr[0], rmin = vr[0];
  for (int32_t e = 1; e < E; ++e) {
    if (ve[e] > emax) emax = ve[e];
    if (ve[e] < emin) emin = ve[e];
  }
  for (int32_t r = 1; r < R; ++r) {
    if (vr[r] > rmax) rmax = vr[r];
    if (vr[r] < rmin) rmin = vr[r];
  }
  out->total = total;
  out->expert_max = (int32_t)emax;
  out->expert_min = (int32_t)emin;
  out->rank_max = (int32_t)rmax;
  out->rank_min = (int32_t)rmin;
  /* max over mean, mean = total / n: ratio = n * max / total. */
  out->expert_max_over_mean =
      total ? (double)((int64_t)E * emax) / (double)total : 0.0;
  out->rank_max_over_mean =
      total ? (double)((int64_t)R * rmax) / (double)total : 0.0;
  out->expert_gini = oracle_gini_i64(ve, E);
  out->rank_gini = oracle_gini_i64(vr, R);
  free(ve);
  free(vr);
}
