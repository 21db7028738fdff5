// ffn.hip -- grouped SwiGLU expert FFN on MFMA, the dense contraction of the
// local-layer workload (expert compute on each expert's contiguous rows: MoE
// systems survey section 1.1, EP flow step 3; variable-size per-expert batched
// GEMMs driven by the expert counts, survey section 4.1).
//
//   gate/up GEMM  hbuf[n][j]  = bf16( SiLU(g) * u ),  g = s_n . Wg[e][j],
//                 u = s_n . Wu[e][j]   (fp32 accumulation, SiLU(z) = z / (1+e^-z))
//   down GEMM     out[n][c]   = bf16( hbuf_n . Wd[e][c] )
//
// Both are A[M_e x K] * B[N x K]^T with K contiguous in both operands, on
// v_mfma_f32_32x32x16_bf16. Two tile shapes, one kernel template:
//   large: 256 x 256 x 64 per 256-thread block, each wave 128 x 128 (4 x 4 MFMA
//          tiles, 256 fp32 accumulators per lane): 8 fragment reads per 16 MFMAs
//          and half the L2 traffic per flop of the small tile. Needs I % 128 == 0
//          and H % 256 == 0.
//   small: 128 x 128 x 64, each wave 64 x 64 (2 x 2 tiles); any I % 64 == 0 and
//          H % 128 == 0.
// LDS holds each K step's A and B tiles double-buffered; a tile row is 64 bf16
// = eight 16-byte chunks and chunk c of row r sits at chunk c ^ ((r >> 1) & 7),
// so the 16 lanes that read one fragment column in the same cycle hit distinct
// banks. One barrier per K step; the next step's global loads are in flight
// during the MFMAs. A gate/up tile takes BN/2 gate rows of w_gate_up and the
// matching BN/2 up rows, so g and u of the same (row, j) land in the same lane
// and register and SiLU(g) * u is applied in the epilogue. Blocks map to
// (expert, m-tile, n-tile) by a wave-level scan over the per-expert row
// counts. Workgroups are dealt to the 8 XCDs round-robin;
// each XCD takes one contiguous share of the m-major tile order, so it reads
// its rows once and the weights of the experts they belong to through its L2.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kXCD = 8;

__device__ __forceinline__ uint16_t bf16_bits(float f) { return (uint16_t)f32_to_bf16_rne(f); }

// Element offset of 16-byte chunk c of tile row r (XOR swizzle, no padding).
// A 64-bf16 row is 128 bytes = half of the 64 x 4-byte banks; a fragment read
// (ds_read_b128) services 16 lanes = 16 consecutive rows at once, so rows r and
// r+1 share the chunk permutation and land in opposite bank halves, while
// (r >> 1) & 7 gives the 8 row pairs 8 distinct chunk slots.
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ ((r >> 1) & 7)) << 3); }

// BM x BN block tile; each of the 2 x 2 waves computes (BM/2) x (BN/2) as
// MI x NI tiles of 32 x 32.
template <bool kGateUp, int BM, int BN>
__global__ __launch_bounds__(kThreads) void ffn_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ cnts, int E, const uint16_t* __restrict__ Bw, int64_t bstride,
    int I, int K, uint16_t* __restrict__ C, int64_t ldc, int ntiles) {
  constexpr int MI = BM / 64, NI = BN / 64;  // 32x32 tiles per wave
  constexpr int AL = BM * 8 / kThreads;      // 16-byte A chunks per thread per K step
  constexpr int BL = BN * 8 / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kBK];
  __shared__ int info[4];  // expert, first row, rows in tile, n-tile

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- which tile. Tiles are numbered m-major (all n-tiles of m-tile 0, then
  // of m-tile 1, ...) and each XCD takes one contiguous share of that order, so
  // an XCD reads its share of the rows once and the weights of the few experts
  // those rows belong to; blocks of one XCD share tiles through its L2.
  // gridDim.x is a multiple of kXCD with at least ceil(tiles / kXCD) slots per XCD.
  const int xcd = blockIdx.x % kXCD, slot = blockIdx.x / kXCD;
  int ntile = 0;
  if (wid == 0) {
    if (lane == 0) info[0] = -1;  // no tile, unless a lane below finds one
    // Expert e owns m-tiles [base_e, base_e + ceil(cnt[e] / BM)); lane l scans
    // experts [l*c, l*c + c).
    const int c = (E + kWave - 1) / kWave;
    const int e0 = lane * c, e1 = (e0 + c < E) ? e0 + c : E;
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += (cnts[e] + BM - 1) / BM;
    int incl = mine;
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, kWave - 1) * ntiles;  // tiles that exist
    const int share = (total + kXCD - 1) / kXCD;         // <= slots per XCD
    const int logical = xcd * share + slot;
    const bool live = slot < share && logical < total;
    const int mtg = live ? logical / ntiles : -1;
    ntile = live ? logical - mtg * ntiles : 0;
    int base = incl - mine;
    if (live && mtg >= base && mtg < incl) {
      for (int e = e0; e < e1; ++e) {
        const int mt = (cnts[e] + BM - 1) / BM;
        if (mtg < base + mt) {
          const int m0 = (mtg - base) * BM;
          const int rows = cnts[e] - m0;
          info[0] = e;
          info[1] = offs[e] + m0;
          info[2] = rows < BM ? rows : BM;
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
  ntile = info[3];

  const uint16_t* Bexp = Bw + (int64_t)e * bstride;
  // Global -> LDS: 16-byte chunk q = tid + 256*i is tile row (tid >> 3) + 32*i,
  // chunk (tid & 7) of the K step.
  const int lrow = tid >> 3, lc = tid & 7;
  v4u ra[AL], rb[BL];
  auto brow = [&](int r) -> int {
    if constexpr (kGateUp)
      return r < BN / 2 ? ntile * (BN / 2) + r : I + ntile * (BN / 2) + (r - BN / 2);
    else
      return ntile * BN + r;
  };
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int r = lrow + 32 * i;
      ra[i] = (r < rows)
                  ? *reinterpret_cast<const v4u*>(A + (int64_t)(row0 + r) * lda + k0 + lc * 8)
                  : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int r = lrow + 32 * i;
      rb[i] = *reinterpret_cast<const v4u*>(Bexp + (int64_t)brow(r) * K + k0 + lc * 8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i)
      *reinterpret_cast<v4u*>(&As[buf][swz(lrow + 32 * i, lc)]) = ra[i];
#pragma unroll
    for (int i = 0; i < BL; ++i)
      *reinterpret_cast<v4u*>(&Bs[buf][swz(lrow + 32 * i, lc)]) = rb[i];
  };
  // B tile row of fragment ni for this wave: gate/up tiles put the wave's gate
  // columns in ni < NI/2 and the matching up columns in ni >= NI/2.
  auto bfrag_row = [&](int ni) -> int {
    if constexpr (kGateUp)
      return ni < NI / 2 ? wn * (BN / 4) + ni * 32 : BN / 2 + wn * (BN / 4) + (ni - NI / 2) * 32;
    else
      return wn * (BN / 2) + ni * 32;
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};

  const int nk = K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kc = kk * 2 + (lane >> 5);  // 16-byte chunk this lane feeds
      bf16x8 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(
            &As[buf][swz(wm * (BM / 2) + mi * 32 + (lane & 31), kc)]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(&Bs[buf][swz(bfrag_row(ni) + (lane & 31), kc)]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: result (row, col) of register r of a 32x32 tile is
  // row 8*(r/4) + 4*(lane/32) + r%4, col lane%32.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = wm * (BM / 2) + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (tr >= rows) continue;
      uint16_t* crow = C + (int64_t)(row0 + tr) * ldc;
      if constexpr (kGateUp) {
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          const float g = acc[mi][ni][r], u = acc[mi][ni + NI / 2][r];
          const float h = (g / (1.0f + expf(-g))) * u;
          crow[ntile * (BN / 2) + wn * (BN / 4) + ni * 32 + (lane & 31)] = bf16_bits(h);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          crow[ntile * BN + wn * (BN / 2) + ni * 32 + (lane & 31)] = bf16_bits(acc[mi][ni][r]);
      }
    }
  }
}

template <int BM, int BN>
hipError_t run_ffn(const void* send, int64_t rows, int H, int I, int E, const int32_t* offs,
                   const int32_t* cnts, const void* w_gate_up, const void* w_down, void* hbuf,
                   void* out, hipStream_t s) {
  const int mtb = (int)((rows + BM - 1) / BM + E);  // each expert adds at most one partial tile
  auto grid_of = [&](int ntiles) {
    const int64_t n = (int64_t)ntiles * mtb;
    return (unsigned)((n + kXCD - 1) / kXCD * kXCD);
  };
  const int nt1 = I / (BN / 2);
  hipError_t err = launch(ffn_gemm_kernel<true, BM, BN>, dim3(grid_of(nt1)), dim3(kThreads), 0, s,
                          static_cast<const uint16_t*>(send), (int64_t)H, offs, cnts, E,
                          static_cast<const uint16_t*>(w_gate_up), (int64_t)2 * I * H, I, H,
                          static_cast<uint16_t*>(hbuf), (int64_t)I, nt1);
  if (err != hipSuccess) return err;
  const int nt2 = H / BN;
  return launch(ffn_gemm_kernel<false, BM, BN>, dim3(grid_of(nt2)), dim3(kThreads), 0, s,
                static_cast<const uint16_t*>(hbuf), (int64_t)I, offs, cnts, E,
                static_cast<const uint16_t*>(w_down), (int64_t)H * I, I, I,
                static_cast<uint16_t*>(out), (int64_t)H, nt2);
}

}  // namespace

hipError_t launch_expert_swiglu(const void* send, int64_t rows, int H, int I, int E,
                                const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                                const void* w_down, void* hbuf, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (I % 128 == 0 && H % 256 == 0)
    return run_ffn<256, 256>(send, rows, H, I, E, offs, cnts, w_gate_up, w_down, hbuf, out, s);
  return run_ffn<128, 128>(send, rows, H, I, E, offs, cnts, w_gate_up, w_down, hbuf, out, s);
}

}  // namespace moe
