// ffn.hip -- grouped SwiGLU expert FFN on MFMA, the dense contraction of the
// local-layer workload (expert compute on each expert's contiguous rows: MoE
// systems survey section 1.1, EP flow step 3; variable-size per-expert batched
// GEMMs driven by the expert counts, survey section 4.1).
//
//   gate/up GEMM  hbuf[n][j]  = bf16( SiLU(g) * u ),  g = s_n . Wg[e][j],
//                 u = s_n . Wu[e][j]   (fp32 accumulation, SiLU(z) = z / (1+e^-z))
//   down GEMM     out[n][c]   = bf16( hbuf_n . Wd[e][c] )
//
// Both are A[M_e x K] * B[N x K]^T with K contiguous in both operands. Tiles of
// 128 x 128 x 64 per 256-thread block (4 waves in 2 x 2, each wave 64 x 64 =
// 2 x 2 v_mfma_f32_32x32x16_bf16 tiles), LDS double-buffered with rows padded by
// 16 bytes, one barrier per K step, the next K step's global loads in flight
// during the MFMAs. A gate/up tile takes 64 gate rows and the matching 64 up rows
// of w_gate_up, so g and u of the same (row, j) land in the same lane and
// register and SiLU(g) * u is applied in the epilogue. Blocks map to (expert,
// m-tile, n-tile) with the n-tile outermost and a wave-level scan over the
// per-expert row counts; logical block ids are remapped so that consecutive
// ones run on the same XCD (workgroups are dealt to the 8 XCDs round-robin),
// which keeps the weight tile they share in that XCD's L2.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLDK = kBK + 8;  // LDS row stride in elements (144 bytes)
constexpr int kThreads = 256;
constexpr int kXCD = 8;

__device__ __forceinline__ uint16_t bf16_bits(float f) { return (uint16_t)f32_to_bf16_rne(f); }

template <bool kGateUp>
__global__ __launch_bounds__(kThreads) void ffn_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ cnts, int E, const uint16_t* __restrict__ Bw, int64_t bstride,
    int I, int K, uint16_t* __restrict__ C, int64_t ldc, int ntiles, int mt_bound) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLDK];
  __shared__ int info[4];  // expert, first row, rows in tile, n-tile

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- which tile: logical id, XCD-contiguous
  const int G = gridDim.x;  // a multiple of kXCD
  const int logical = (blockIdx.x % kXCD) * (G / kXCD) + blockIdx.x / kXCD;
  const int ntile = logical / mt_bound, mtg = logical - ntile * mt_bound;
  if (wid == 0) {
    if (lane == 0) info[0] = -1;  // no tile, unless a lane below finds one
    // Expert e owns m-tiles [base_e, base_e + ceil(cnt[e] / kBM)); lane l scans
    // experts [l*c, l*c + c).
    const int c = (E + kWave - 1) / kWave;
    const int e0 = lane * c, e1 = (e0 + c < E) ? e0 + c : E;
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += (cnts[e] + kBM - 1) / kBM;
    int incl = mine;
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int base = incl - mine;
    if (ntile < ntiles && mtg >= base && mtg < incl) {
      for (int e = e0; e < e1; ++e) {
        const int mt = (cnts[e] + kBM - 1) / kBM;
        if (mtg < base + mt) {
          const int m0 = (mtg - base) * kBM;
          const int rows = cnts[e] - m0;
          info[0] = e;
          info[1] = offs[e] + m0;
          info[2] = rows < kBM ? rows : kBM;
          info[3] = ntile;
          break;
        }
        base += mt;
      }
    }
  }
  __syncthreads();
  const int e = info[0];
  if (e < 0) return;  // uniform over the block
  const int row0 = info[1], rows = info[2];

  const uint16_t* Bexp = Bw + (int64_t)e * bstride;
  // Global -> LDS mapping: 16-byte chunk q = tid + 256*i covers tile row
  // (tid >> 3) + 32*i, columns (tid & 7)*8 .. +8 of the K step.
  const int lrow = tid >> 3, lk = (tid & 7) * 8;
  v4u ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lrow + 32 * i;
      ra[i] = (r < rows) ? *reinterpret_cast<const v4u*>(A + (int64_t)(row0 + r) * lda + k0 + lk)
                         : v4u{0u, 0u, 0u, 0u};
      const int br = kGateUp ? (r < 64 ? ntile * 64 + r : I + ntile * 64 + (r - 64))
                             : ntile * kBN + r;
      rb[i] = *reinterpret_cast<const v4u*>(Bexp + (int64_t)br * K + k0 + lk);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lrow + 32 * i;
      *reinterpret_cast<v4u*>(&As[buf][r * kLDK + lk]) = ra[i];
      *reinterpret_cast<v4u*>(&Bs[buf][r * kLDK + lk]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  const int nk = K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kc = kk * 16 + (lane >> 5) * 8;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int ar = wm * 64 + mi * 32 + (lane & 31);
        af[mi] = *reinterpret_cast<const bf16x8*>(&As[buf][ar * kLDK + kc]);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int br = kGateUp ? (ni * 64 + wn * 32 + (lane & 31)) : (wn * 64 + ni * 32 + (lane & 31));
        bfr[ni] = *reinterpret_cast<const bf16x8*>(&Bs[buf][br * kLDK + kc]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: result (row, col) of register r of a 32x32 tile is
  // row 8*(r/4) + 4*(lane/32) + r%4, col lane%32.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (tr >= rows) continue;
      uint16_t* crow = C + (int64_t)(row0 + tr) * ldc;
      if constexpr (kGateUp) {
        const float g = acc[mi][0][r], u = acc[mi][1][r];
        const float h = (g / (1.0f + expf(-g))) * u;
        crow[ntile * 64 + wn * 32 + (lane & 31)] = bf16_bits(h);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          crow[ntile * kBN + wn * 64 + ni * 32 + (lane & 31)] = bf16_bits(acc[mi][ni][r]);
      }
    }
  }
}

}  // namespace

int64_t ffn_mtile_bound(int64_t rows, int E) { return (rows + kBM - 1) / kBM + E; }

hipError_t launch_expert_swiglu(const void* send, int64_t rows, int H, int I, int E,
                                const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                                const void* w_down, void* hbuf, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int mtb = (int)ffn_mtile_bound(rows, E);
  auto grid_of = [&](int ntiles) {
    const int64_t n = (int64_t)ntiles * mtb;
    return (unsigned)((n + kXCD - 1) / kXCD * kXCD);
  };
  const uint16_t* A1 = static_cast<const uint16_t*>(send);
  uint16_t* Hb = static_cast<uint16_t*>(hbuf);
  const int nt1 = I / 64;
  hipError_t err = launch(ffn_gemm_kernel<true>, dim3(grid_of(nt1)), dim3(kThreads), 0, s, A1,
                          (int64_t)H, offs, cnts, E, static_cast<const uint16_t*>(w_gate_up),
                          (int64_t)2 * I * H, I, H, Hb, (int64_t)I, nt1, mtb);
  if (err != hipSuccess) return err;
  const int nt2 = H / kBN;
  return launch(ffn_gemm_kernel<false>, dim3(grid_of(nt2)), dim3(kThreads), 0, s,
                static_cast<const uint16_t*>(Hb), (int64_t)I, offs, cnts, E,
                static_cast<const uint16_t*>(w_down), (int64_t)H * I, I, I,
                static_cast<uint16_t*>(out), (int64_t)H, nt2, mtb);
}

}  // namespace moe
