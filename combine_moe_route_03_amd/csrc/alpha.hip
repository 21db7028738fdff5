// alpha.hip -- fitted symmetric Dirichlet alpha of the expert counts, the third
// scalar summary of the send-count matrix in the DODOCO summary ("metrics"):
// it separates near-uniform routings where the Gini coefficient compresses.
// Read as the maximum-likelihood alpha of a Dirichlet-multinomial with E equal
// concentrations; the score (derivative of the log-likelihood) is
//   g(a) = sum_{e: c_e > 0} [psi(c_e + a) - psi(a)] - E [psi(N + E a) - psi(E a)].
//
// One 256-thread block. Counts are staged in LDS; the start value is the
// method-of-moments alpha (the Dirichlet-multinomial variance
// N p (1-p) (N + E a) / (1 + E a), p = 1/E, solved for a); then Newton steps on
// u = ln a, each kept inside a bracket that every evaluated sign narrows
// (bisection when a step leaves it). One evaluation spreads the E experts and
// the three shared digamma terms over the threads and reduces the score and
// its derivative with DPP wave sums and one LDS exchange.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Digamma and trigamma for x > 0 in double: the recurrences
// psi(x) = psi(x+1) - 1/x and psi'(x) = psi'(x+1) + 1/x^2 carried as single
// fractions (one division each) until x >= 16, then the asymptotic series in
// 1/x with Bernoulli-number coefficients (Abramowitz & Stegun 6.3.18, 6.4.12).
__device__ inline void digamma_trigamma(double x, double& psi, double& psi1) {
  double pn = 0.0, pd = 1.0, qn = 0.0, qd = 1.0;  // sum 1/y and sum 1/y^2 as fractions
  while (x < 16.0) {
    const double y2 = x * x;
    pn = fma(pn, x, pd);
    pd *= x;
    qn = fma(qn, y2, qd);
    qd *= y2;
    x += 1.0;
  }
  const double r = 1.0 / x, r2 = r * r;
  psi = log(x) - 0.5 * r -
        r2 * (1.0 / 12 - r2 * (1.0 / 120 - r2 * (1.0 / 252 - r2 * (1.0 / 240 - r2 * (1.0 / 132))))) -
        pn / pd;
  psi1 = r + 0.5 * r2 +
         r * r2 * (1.0 / 6 - r2 * (1.0 / 30 - r2 * (1.0 / 42 - r2 * (1.0 / 30 - r2 * (5.0 / 66))))) +
         qn / qd;
}

__global__ __launch_bounds__(kThreads) void dirichlet_alpha_kernel(const int32_t* __restrict__ counts,
                                                                   int E, double* __restrict__ out) {
  __shared__ int32_t cnt[1024];
  __shared__ double part[3][kWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;

  // counts, N, experts with picks, sum of squares
  int64_t n = 0, sq = 0;
  int32_t nz = 0;
  for (int e = tid; e < E; e += kThreads) {
    const int32_t c = counts[e];
    cnt[e] = c;
    n += c;
    sq += (int64_t)c * c;
    nz += c > 0;
  }
  const auto add = [](auto x, auto y) { return x + y; };
  n = group_reduce(n, kWave, add);
  sq = group_reduce(sq, kWave, add);
  nz = group_reduce(nz, kWave, add);
  if (lane == 0) {
    part[0][wid] = (double)n;
    part[1][wid] = (double)sq;
    part[2][wid] = (double)nz;
  }
  __syncthreads();
  double N = 0.0, S2 = 0.0, NZ = 0.0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    N += part[0][q];
    S2 += part[1][q];
    NZ += part[2][q];
  }
  __syncthreads();
  if (E < 2 || N == 0.0) {
    if (tid == 0) *out = __builtin_nan("");
    return;
  }
  const double Ed = (double)E;

  // score g and dg/da at a; identical on every thread
  auto eval = [&](double a, double& g, double& gp) {
    double s0 = 0.0, s1 = 0.0;
    for (int e = tid; e < E; e += kThreads) {
      if (cnt[e] == 0) continue;
      double p, p1;
      digamma_trigamma((double)cnt[e] + a, p, p1);
      s0 += p;
      s1 += p1;
    }
    // the three shared terms, on the last three threads
    const int item = kThreads - 1 - tid;
    if (item < 3) {
      const double x = item == 0 ? a : (item == 1 ? Ed * a : N + Ed * a);
      const double c0 = item == 0 ? -NZ : (item == 1 ? Ed : -Ed);
      const double c1 = item == 0 ? -NZ : (item == 1 ? Ed * Ed : -Ed * Ed);
      double p, p1;
      digamma_trigamma(x, p, p1);
      s0 += c0 * p;
      s1 += c1 * p1;
    }
    s0 = group_reduce(s0, kWave, add);
    s1 = group_reduce(s1, kWave, add);
    if (lane == 0) {
      part[0][wid] = s0;
      part[1][wid] = s1;
    }
    __syncthreads();
    g = 0.0;
    gp = 0.0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      g += part[0][q];
      gp += part[1][q];
    }
    __syncthreads();  // part is rewritten by the next evaluation
  };

  double lo = log(1e-8), hi = log(1e6), g, gp;
  eval(exp(hi), g, gp);
  if (g > 0.0) {
    if (tid == 0) *out = __builtin_inf();
    return;
  }
  eval(exp(lo), g, gp);
  if (g < 0.0) {
    if (tid == 0) *out = 0.0;
    return;
  }
  // method-of-moments start: rho = observed variance / multinomial variance
  const double mean = N / Ed;
  const double var = S2 / Ed - mean * mean;
  const double rho = var / (N * (1.0 / Ed) * (1.0 - 1.0 / Ed));
  double u = 0.0;
  if (rho > 1.0 && N > rho) {
    const double a0 = (N - rho) / (Ed * (rho - 1.0));
    const double u0 = log(a0);
    if (u0 > lo && u0 < hi) u = u0;
  }
  for (int it = 0; it < 60; ++it) {
    const double a = exp(u);
    eval(a, g, gp);
    if (g > 0.0) lo = u;
    else hi = u;
    double un = u - g / (a * gp);  // Newton on u: dg/du = a g'(a)
    if (!(un > lo && un < hi)) un = 0.5 * (lo + hi);
    // 1e-12 in ln a: the relative precision of alpha, above the rounding
    // noise of the score near its root
    const bool done = fabs(un - u) < 1e-12 || hi - lo < 1e-12;
    u = un;
    if (done) break;
  }
  if (tid == 0) *out = exp(u);
}

}  // namespace

hipError_t launch_dirichlet_alpha(const int32_t* counts, int E, double* out, hipStream_t s) {
  return launch(dirichlet_alpha_kernel, dim3(1), dim3(kThreads), 0, s, counts, E, out);
}

}  // namespace moe
