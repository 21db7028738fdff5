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
//   large: 256 x 256 x 64 per 512-thread block, 8 waves as 4 x 2, each wave
//          64 x 128 (2 x 4 MFMA tiles, 128 fp32 accumulators per lane), two
//          waves per SIMD so one issues MFMAs while the other waits on LDS or
//          the barrier; no spill at 226 VGPRs (16 waves of 64 x 64, four a
//          SIMD, spilled 20 bytes a lane and measured 1.6% slower; one wave
//          of 128 x 128 per SIMD 13% slower). Needs I % 128 == 0 and
//          H % 256 == 0.
//   small: 128 x 128 x 64, 4 waves of 64 x 64 (2 x 2 tiles), two blocks per
//          compute unit; any I % 64 == 0 and H % 128 == 0.
// Global -> LDS moves go through buffer loads with the LDS bit (16 bytes a
// lane straight into LDS, no registers, hardware range check for partial
// m-tiles). LDS holds two K steps of A and B; a tile row is 64 bf16 = eight
// 16-byte chunks and chunk c of row r sits at chunk c ^ ((r >> 1) & 7), so the
// 16 lanes that read one fragment column in the same cycle hit distinct banks.
// Software pipeline: the loads of step kt+2 are issued right after the one
// barrier of step kt and land while steps kt and kt+1 compute; fragment reads
// are double-buffered in registers and interleaved one per MFMA. A gate/up
// tile takes BN/2 gate rows of w_gate_up and the matching BN/2 up rows, so g
// and u of the same (row, j) land in the same lane and register and
// SiLU(g) * u is applied in the epilogue. In an expert's partial last
// m-tile, waves with no live row skip their fragment reads and MFMAs. Blocks
// map to (expert, m-tile,
// n-tile) by a wave-level scan over the per-expert row counts. Workgroups are
// dealt to the 8 XCDs round-robin (from where the previous launch left off, so
// blocks b and b + 8 share an XCD); each XCD takes one contiguous share of the
// m-major tile order, so it reads its rows once and the weights of the experts
// they belong to through its L2. The whole FFN runs as two chains of experts
// (even and odd ids) on two streams, so that one chain's last partial round of
// tiles shares the chip with the other chain's tiles.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXCD = 8;
// m-tiles per rasterisation patch. With one chain of experts the local layer
// measured 701 us for 1 against 714 for 4; with two chains sharing each XCD's
// L2, 4 and 8 are faster than 1 (step 723-726 against 733 us, same box).
constexpr int kGroupM = 4;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a pair of bf16 (low half = a), round to nearest even: on
// gfx950 one v_cvt_pk_bf16_f32, which rounds every non-NaN float exactly as
// the bit-twiddling f32_to_bf16_rne does (checked on the device over 16M bit
// patterns: denormals, ties of both parities, overflow to infinity); a NaN
// keeps its payload instead of becoming the canonical one.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// SiLU(g) = g / (1 + e^-g), evaluated as num / (1 + e^-|g|) with num = g for
// g >= 0 and g e^-|g| below, so the denominator stays in (1, 2]: e^-|g| is
// the hardware base-2 exponential of -|g| log2(e), the product split into a
// rounded part and its error (log2(e) as a float plus its remainder, the
// error carried to first order after the exponential), and the reciprocal is
// the hardware one refined by one Newton step. For finite g (an infinite one
// gives NaN) the relative error is at most 4.6 x 2^-24 against the exact
// SiLU over 16M arguments in [-100, 100] (3.1 x 2^-24 for expf and an IEEE
// division), in ~13 instructions instead of ~25: the gate/up epilogue is
// bound by its instruction count.
__device__ __forceinline__ float silu(float g) {
  constexpr float kL1 = 1.44269504f;            // log2(e) rounded to float
  constexpr float kL2 = 1.925963033500011e-08f;  // log2(e) - kL1
  constexpr float kLn2 = 0.693147181f;
  const float a = -__builtin_fabsf(g);
  const float t = a * kL1;
  const float tl = __builtin_fmaf(a, kL1, -t) + a * kL2;  // a log2(e) - t
  const float e0 = __builtin_amdgcn_exp2f(t);
  const float e = __builtin_fmaf(e0, tl * kLn2, e0);      // e^-|g|
  const float d = 1.0f + e;
  float r = __builtin_amdgcn_rcpf(d);
  r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
  return (g >= 0.0f ? g : g * e) * r;
}

// XOR key of tile row r for a K step of BK bf16 (BK/8 16-byte chunks a row).
// The 64 four-byte banks span 256 bytes; a fragment read (ds_read_b128)
// services 16 lanes = 16 consecutive rows at one chunk index at once.
//   BK = 64: 128-byte rows, two rows per bank sweep; the key (r >> 1) & 7
//            gives the 8 row pairs distinct chunk slots.
//   BK = 32: 64-byte rows, four rows per bank sweep; the key (r >> 2) & 3
//            gives the 4 row quads distinct chunk slots.
// Either way the 16 lanes hit 64 distinct banks.
template <int BK>
__device__ __forceinline__ int swz_key(int r) {
  if constexpr (BK == 64) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// Element offset of 16-byte chunk c of tile row r in an LDS tile (no padding).
template <int BK>
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ swz_key<BK>(r)) << 3); }

typedef __attribute__((address_space(3))) void* lptr_t;

// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format,
// no swizzle, no index stride).
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediate for vmcnt <= n with the other counters left free (gfx9
// encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitVmcnt0 = wait_vmcnt(0);

// Buffer-instruction helpers (plain device functions, so that the kernel's
// lambdas stay valid in the host compilation pass).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// 16 bytes a lane from base + voff + soff into LDS at lds + 16 * lane.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)lds, 16, voff, soff, 0, 0);
}

// BM x BN block tile; each of the WM x WN waves computes (BM/WM) x (BN/WN) as
// MI x NI tiles of 32 x 32. K steps of BK, NS LDS stages.
template <bool kGateUp, int BM, int BN, int OCC, int BK, int NS, int WM, int WN>
__global__ __launch_bounds__(kWave * WM * WN, OCC) void ffn_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ cnts, int E, int sg, int sstride, int sbase,
    const uint16_t* __restrict__ Bw, int64_t bstride,
    int I, int K, uint16_t* __restrict__ C, int64_t ldc, int ntiles, int gm) {
  constexpr int NW = WM * WN;                // waves in the block
  constexpr int MI = BM / WM / 32, NI = BN / WN / 32;  // 32x32 tiles per wave
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row
  constexpr int RPI = kWave / CPR;           // tile rows per load instruction (1 KiB)
  constexpr int AI = BM / NW / RPI, BI = BN / NW / RPI;  // load instructions per wave per K step
  constexpr int kStage = (BM + BN) * BK;     // elements of one A + B stage
  static_assert(NS >= 2 && NS <= 5, "LDS stages");
  // The stages as separate arrays, so the compiler can tell the loads into one
  // stage from the fragment reads of another and need not wait for them.
  __shared__ __attribute__((aligned(1024))) uint16_t lds0[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t lds1[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t lds2[NS > 2 ? kStage : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t lds3[NS > 3 ? kStage : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t lds4[NS > 4 ? kStage : 1];
  __shared__ int info[4];  // expert, first row, rows in tile, n-tile
  const auto stage = [&](auto S) -> uint16_t* {
    constexpr int st = decltype(S)::value % NS;
    if constexpr (st == 0) return lds0;
    else if constexpr (st == 1) return lds1;
    else if constexpr (st == 2) return lds2;
    else if constexpr (st == 3) return lds3;
    else return lds4;
  };

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // Wave-uniform values are read into scalar registers (readfirstlane): then
  // the buffer descriptors and LDS addresses built from them are scalar and
  // each global->LDS load is one instruction, not a loop over lanes (local
  // layer FFN 632-637 -> 625-628 us).
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid / WN, wn = wid % WN;

  // ---- which tile. The m-tiles (every expert's rows in BM-row tiles, in
  // expert order) are split into 8 contiguous shares, one per XCD, so an XCD
  // reads its rows once and the weights of the few experts they belong to
  // through its own L2. Inside a share, tiles go in patches of GM m-tiles:
  // n-tile 0 of the patch's m-tiles, then n-tile 1, ...; the blocks resident
  // on an XCD at one time then cover a GM x (32/GM) patch, re-using each B
  // tile GM times and each A tile 32/GM times from L2.
  // gridDim.x = 8 * (max m-tiles per XCD) * ntiles.
  const int xcd = blockIdx.x % kXCD, slot = blockIdx.x / kXCD;
  int ntile = 0;
  if (wid == 0) {
    if (lane == 0) info[0] = -1;  // no tile, unless a lane below finds one
    // The launch covers E experts: the i-th is expert (i / sg) * sstride + sbase
    // + i % sg (all experts: sg = E, sbase = 0; one wave of W: sg = L/W slots
    // of each of the R ranks). Expert i owns m-tiles
    // [base_i, base_i + ceil(cnt / BM)); lane l scans experts [l*c, l*c + c).
    const auto eid = [&](int i) { return (i / sg) * sstride + sbase + i % sg; };
    const int c = (E + kWave - 1) / kWave;
    const int e0 = lane * c, e1 = (e0 + c < E) ? e0 + c : E;
    int mine = 0;
    for (int i = e0; i < e1; ++i) mine += (cnts[eid(i)] + BM - 1) / BM;
    int incl = mine;
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int MT = __shfl(incl, kWave - 1);    // m-tiles that exist
    const int mpx = (MT + kXCD - 1) / kXCD;    // m-tiles per XCD share
    const int m_lo = xcd * mpx;
    const int m_cnt = MT - m_lo < mpx ? (MT - m_lo > 0 ? MT - m_lo : 0) : mpx;
    const bool live = slot < m_cnt * ntiles;
    int mtg = -1;
    if (live) {
      const int grp = slot / (gm * ntiles), r = slot - grp * gm * ntiles;
      const int gh = (m_cnt - grp * gm < gm) ? m_cnt - grp * gm : gm;  // m-tiles in this patch
      ntile = r / gh;
      mtg = m_lo + grp * gm + (r - ntile * gh);
    }
    int base = incl - mine;
    if (live && mtg >= base && mtg < incl) {
      for (int i = e0; i < e1; ++i) {
        const int e = eid(i);
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
  const int e = __builtin_amdgcn_readfirstlane(info[0]);
  if (e < 0) return;  // uniform over the block
  const int row0 = __builtin_amdgcn_readfirstlane(info[1]);
  const int rows = __builtin_amdgcn_readfirstlane(info[2]);
  // Waves whose 32-row MFMA tiles all lie past the tile's last row (the
  // partial last m-tile of an expert) run a loop that only loads and meets the
  // barriers: no fragment reads, no MFMAs, so the SIMDs they share with live
  // waves give those the MFMA pipe (local layer FFN 674-676 -> 630-632 us;
  // zero rows computed: 11% -> 3.4% of the rows).
  const bool live = wm * (BM / WM) < rows;
  ntile = __builtin_amdgcn_readfirstlane(info[3]);

  // ---- global -> LDS without registers (global_load_lds_dwordx4): one wave
  // instruction fills 64 consecutive 16-byte LDS slots, lane l slot l, i.e.
  // RPI tile rows. Lane l therefore fetches the global chunk that the swizzle
  // puts in slot l % CPR of row l / CPR. Wave w fills A rows [w*BM/4, (w+1)*BM/4)
  // and B rows [w*BN/4, (w+1)*BN/4). A rows past the tile's last row re-read
  // that row: MFMA output rows depend on their own A row only, and those rows
  // are never stored.
  const uint16_t* Bexp = Bw + (int64_t)e * bstride;
  auto brow = [&](int r) -> int {
    if constexpr (kGateUp)
      return r < BN / 2 ? ntile * (BN / 2) + r : I + ntile * (BN / 2) + (r - BN / 2);
    else
      return ntile * BN + r;
  };
  const int lr = lane / CPR, ls = lane % CPR;
  // Buffer descriptors over this tile's A rows and this expert's weights. The
  // descriptor's range check returns zeros for A rows past the tile's last row
  // (those MFMA output rows are never stored), so no clamping is needed.
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A + (int64_t)row0 * lda, (int64_t)rows * lda * 2);
  const __amdgpu_buffer_rsrc_t brsrc =
      make_rsrc(Bexp, (int64_t)(kGateUp ? 2 * I : ntiles * BN) * K * 2);
  // Per-lane byte offsets of the K = 0 chunks; the K step goes in the scalar offset.
  uint32_t aoff[AI], boff[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int r = wid * (BM / NW) + RPI * i + lr;
    aoff[i] = (uint32_t)(((int64_t)r * lda + ((ls ^ swz_key<BK>(r)) << 3)) * 2);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = wid * (BN / NW) + RPI * i + lr;
    boff[i] = (uint32_t)(((int64_t)brow(r) * K + ((ls ^ swz_key<BK>(r)) << 3)) * 2);
  }
  auto issue = [&](uint16_t* As, int k0) __attribute__((always_inline)) {
    uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      load_lds16(arsrc, As + (wid * (BM / NW) + RPI * i) * BK, aoff[i], 2 * k0);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      load_lds16(brsrc, Bs + (wid * (BN / NW) + RPI * i) * BK, boff[i], 2 * k0);
  };

  // B tile row of fragment ni for this wave: gate/up tiles put the wave's gate
  // columns in ni < NI/2 and the matching up columns in ni >= NI/2.
  auto bfrag_row = [&](int ni) -> int {
    if constexpr (kGateUp)
      return ni < NI / 2 ? wn * (BN / 2 / WN) + ni * 32
                         : BN / 2 + wn * (BN / 2 / WN) + (ni - NI / 2) * 32;
    else
      return wn * (BN / WN) + ni * 32;
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};

  // Fragments of K sub-step kk (16 wide): lane l feeds row l % 32 with chunk
  // 2*kk + l / 32. Double-buffered in registers: the reads of sub-step kk+1
  // are in flight during the MFMAs of kk.
  bf16x8 fa[2][MI], fb[2][NI];
  auto fload = [&](int f, const uint16_t* As, int kk) __attribute__((always_inline)) {
    const uint16_t* Bs = As + BM * BK;
    const int kc = kk * 2 + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      fa[f][mi] = *reinterpret_cast<const bf16x8*>(
          &As[swz<BK>(wm * (BM / WM) + mi * 32 + (lane & 31), kc)]);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      fb[f][ni] =
          *reinterpret_cast<const bf16x8*>(&Bs[swz<BK>(bfrag_row(ni) + (lane & 31), kc)]);
  };
  auto mfmas = [&](int f) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][mi], fb[f][ni], acc[mi][ni], 0, 0, 0);
  };
  constexpr int kMF = MI * NI, kFR = MI + NI;  // MFMAs and fragment reads per sub-step

  // Software pipeline over K steps, NS LDS stages; step kt reads stage kt % NS.
  // In step kt: sub-steps 0 .. BK/16-2 run their MFMAs while reading the next
  // sub-step's fragments; then, once this wave's loads of step kt+1 have
  // landed (those of steps kt+2 .. kt+NS-1 may still be in flight), one
  // barrier, after which the loads of step kt+NS refill stage kt % NS (every
  // wave is done reading it) while the last sub-step's MFMAs run alongside the
  // first fragment reads of step kt+1. A load therefore has NS-1 steps of
  // compute to land in. Past the last step the loads repeat step nk-1 into a
  // stage nobody reads again, which keeps the loop free of branches around
  // them.
  const int nk = K / BK;
  constexpr int kLast = BK / 16 - 1;  // last sub-step of a K step
  auto step = [&](auto S, int kt) __attribute__((always_inline)) {
    const uint16_t* cur = stage(S);
    const uint16_t* nxt = stage(std::integral_constant<int, decltype(S)::value + 1>{});
    // The wave's issue priority is raised for the interleaved MFMAs and
    // fragment reads and lowered again for the wait and barrier, so a SIMD's
    // other wave (or a dead wave that only loads) yields to it (local layer
    // FFN 588.7-594.6 -> 581.2-589.5 us, three runs each, interleaved).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < kLast; ++kk) {
      fload((kk + 1) & 1, cur, kk + 1);
      mfmas(kk & 1);
      // the reads go out early, one per MFMA, so they land before sub-step kk+1
#pragma unroll
      for (int i = 0; i < kFR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
      if constexpr (kMF > kFR) __builtin_amdgcn_sched_group_barrier(0x008, kMF - kFR, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt((NS - 2) * (AI + BI)));
    __syncthreads();
    const int kn = kt + NS < nk ? kt + NS : nk - 1;
    issue(const_cast<uint16_t*>(cur), kn * BK);
    fload(0, nxt, 0);
    mfmas(kLast & 1);
#pragma unroll
    for (int i = 0; i < kFR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, (AI + BI + kFR - 1) / kFR, 0);  // global -> LDS
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    if constexpr (kMF > kFR) __builtin_amdgcn_sched_group_barrier(0x008, kMF - kFR, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  // prologue: steps 0 .. NS-1 into stages 0 .. NS-1, step 0 landed
  const auto clampk = [&](int k) { return (k < nk ? k : nk - 1) * BK; };
  issue(lds0, 0);
  issue(lds1, clampk(1));
  if constexpr (NS > 2) issue(lds2, clampk(2));
  if constexpr (NS > 3) issue(lds3, clampk(3));
  if constexpr (NS > 4) issue(lds4, clampk(4));
  __builtin_amdgcn_s_waitcnt(wait_vmcnt((NS - 1) * (AI + BI)));
  __syncthreads();
  if (live) {
    fload(0, lds0, 0);
    int kt = 0;
    for (; kt + NS <= nk; kt += NS) {
      step(I0{}, kt);
      step(I1{}, kt + 1);
      if constexpr (NS > 2) step(I2{}, kt + 2);
      if constexpr (NS > 3) step(I3{}, kt + 3);
      if constexpr (NS > 4) step(I4{}, kt + 4);
    }
    if (kt < nk) step(I0{}, kt);
    if (kt + 1 < nk) step(I1{}, kt + 1);
    if constexpr (NS > 2) if (kt + 2 < nk) step(I2{}, kt + 2);
    if constexpr (NS > 3) if (kt + 3 < nk) step(I3{}, kt + 3);
  } else {
    // the same loads and barriers, step by step (stage kt % NS refilled with
    // step kt + NS after step kt's barrier)
    auto dstep = [&](auto S, int kt) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(wait_vmcnt((NS - 2) * (AI + BI)));
      __syncthreads();
      const int kn = kt + NS < nk ? kt + NS : nk - 1;
      issue(stage(S), kn * BK);
    };
    int kt = 0;
    for (; kt + NS <= nk; kt += NS) {
      dstep(I0{}, kt);
      dstep(I1{}, kt + 1);
      if constexpr (NS > 2) dstep(I2{}, kt + 2);
      if constexpr (NS > 3) dstep(I3{}, kt + 3);
      if constexpr (NS > 4) dstep(I4{}, kt + 4);
    }
    if (kt < nk) dstep(I0{}, kt);
    if (kt + 1 < nk) dstep(I1{}, kt + 1);
    if constexpr (NS > 2) if (kt + 2 < nk) dstep(I2{}, kt + 2);
    if constexpr (NS > 3) if (kt + 3 < nk) dstep(I3{}, kt + 3);
  }
  // the trailing loads must land before the block's LDS is released
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- epilogue: result (row, col) of register r of a 32x32 tile is
  // row 8*(r/4) + 4*(lane/32) + r%4, col lane%32, so registers r and r+1 (r
  // even) are two consecutive rows of one column: one hardware conversion
  // makes both bf16 values, each stored as 2 bytes (a wave's store covers two
  // rows, 64 contiguous bytes each). The stores go through a buffer
  // descriptor over the tile's rows of C, whose range check drops the rows
  // past the tile's last one (no per-row branch); a fragment's column offset
  // is an immediate. Local layer FFN: the epilogue took 12.6 us a gate/up
  // tile and 7.8 us a down tile with per-row branches, 64-bit addresses and
  // the bit-twiddling rounding, ~900 and ~940 instructions a wave.
  const __amdgpu_buffer_rsrc_t crsrc =
      make_rsrc(C + (int64_t)row0 * ldc, (int64_t)rows * ldc * 2);
  const int ccol = kGateUp ? ntile * (BN / 2) + wn * (BN / 2 / WN) : ntile * BN + wn * (BN / WN);
  const uint32_t vbase =
      (uint32_t)(((wm * (BM / WM) + 4 * (lane >> 5)) * ldc + ccol + (lane & 31)) * 2);
  constexpr int NO = kGateUp ? NI / 2 : NI;  // output fragments of a fragment row
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const uint32_t v0 = vbase + (uint32_t)((mi * 32 + 8 * (r >> 2) + (r & 3)) * ldc * 2);
      const uint32_t v1 = v0 + (uint32_t)(ldc * 2);
#pragma unroll
      for (int ni = 0; ni < NO; ++ni) {
        float a, b;
        if constexpr (kGateUp) {
          a = silu(acc[mi][ni][r]) * acc[mi][ni + NI / 2][r];
          b = silu(acc[mi][ni][r + 1]) * acc[mi][ni + NI / 2][r + 1];
        } else {
          a = acc[mi][ni][r];
          b = acc[mi][ni][r + 1];
        }
        const uint32_t p = bf16x2_rne(a, b);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)p, crsrc, v0 + ni * 64, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(p >> 16), crsrc, v1 + ni * 64, 0, 0);
      }
    }
  }
}

// Large tiles: K step and LDS stages of the pipeline. 64 x 2 measured faster
// than 32 x 3 and 32 x 4 (local layer 806 vs 889 and 880 us): the schedule,
// not uncovered load latency, bounds this kernel.
constexpr int kLargeBK = 64;
constexpr int kLargeNS = 2;
// 4 x 2 waves, two per SIMD: local layer FFN 581.5-581.9 against 590.8-591.8
// us for 4 x 4 (16 waves) with the current epilogue, same box, interleaved
// (with the earlier, instruction-heavy epilogue 4 x 4 was the faster: 683
// against 692 us, 2 x 4 698).
constexpr int kLargeWM = 4, kLargeWN = 2;

template <int BM, int BN, int OCC, int BK, int NS, int WM, int WN>
hipError_t run_ffn(const void* send, int64_t rows, int H, int I, int E, int sg, int sstride,
                   int sbase, const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                   const void* w_down, void* hbuf, void* out, hipStream_t s) {
  const int mtb = (int)((rows + BM - 1) / BM + E);  // each expert adds at most one partial tile
  auto grid_of = [&](int ntiles) {
    return (unsigned)(kXCD * ((mtb + kXCD - 1) / kXCD) * ntiles);
  };
  const int nt1 = I / (BN / 2);
  hipError_t err = launch(ffn_gemm_kernel<true, BM, BN, OCC, BK, NS, WM, WN>, dim3(grid_of(nt1)),
                          dim3(kWave * WM * WN), 0, s,
                          static_cast<const uint16_t*>(send), (int64_t)H, offs, cnts, E, sg,
                          sstride, sbase, static_cast<const uint16_t*>(w_gate_up), (int64_t)2 * I * H, I, H,
                          static_cast<uint16_t*>(hbuf), (int64_t)I, nt1, kGroupM);
  if (err != hipSuccess) return err;
  const int nt2 = H / BN;
  return launch(ffn_gemm_kernel<false, BM, BN, OCC, BK, NS, WM, WN>, dim3(grid_of(nt2)),
                dim3(kWave * WM * WN), 0, s,
                static_cast<const uint16_t*>(hbuf), (int64_t)I, offs, cnts, E, sg, sstride,
                sbase, static_cast<const uint16_t*>(w_down), (int64_t)H * I, I, I,
                static_cast<uint16_t*>(out), (int64_t)H, nt2, kGroupM);
}

}  // namespace

hipError_t launch_expert_swiglu_subset(const void* send, int64_t rows, int H, int I, int n,
                                       int sg, int sstride, int sbase, const int32_t* offs,
                                       const int32_t* cnts, const void* w_gate_up,
                                       const void* w_down, void* hbuf, void* out, hipStream_t s) {
  if (rows == 0 || n == 0) return hipSuccess;
  if (I % 128 == 0 && H % 256 == 0)
    return run_ffn<256, 256, 1, kLargeBK, kLargeNS, kLargeWM, kLargeWN>(send, rows, H, I, n, sg, sstride, sbase, offs,
                                                    cnts, w_gate_up, w_down, hbuf, out, s);
  return run_ffn<128, 128, 2, 64, 2, 2, 2>(send, rows, H, I, n, sg, sstride, sbase, offs, cnts,
                                     w_gate_up, w_down, hbuf, out, s);
}

// The experts run as two chains, even and odd expert ids, each its gate/up
// GEMM then its down GEMM: the first on the caller's stream, the second on the
// caller's side stream, forked from the first by one caller event and joined
// back into it by another. While one chain's last, partial round of tiles
// runs, the other chain's tiles fill the idle compute units (local layer step
// 772 -> 733 us; halves by id 753, three or four chains 797 and 830 us).
// Per-element arithmetic is that of one launch. Without a side stream, one
// chain of all experts on the caller's stream.
hipError_t launch_expert_swiglu(const void* send, int64_t rows, int H, int I, int E,
                                const int32_t* offs, const int32_t* cnts, const void* w_gate_up,
                                const void* w_down, void* hbuf, void* out, hipStream_t s,
                                hipStream_t side, hipEvent_t fork, hipEvent_t join) {
  if (rows == 0 || E == 0) return hipSuccess;
  if (E < 2 || side == nullptr)
    return launch_expert_swiglu_subset(send, rows, H, I, E, E, 0, 0, offs, cnts, w_gate_up,
                                       w_down, hbuf, out, s);
  hipError_t err;
  if ((err = hipEventRecord(fork, s)) != hipSuccess) return err;
  if ((err = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return err;
  for (int c = 0; c < 2; ++c) {
    // chain c: experts 2i + c
    err = launch_expert_swiglu_subset(send, rows, H, I, (E - c + 1) / 2, 1, 2, c, offs, cnts,
                                      w_gate_up, w_down, hbuf, out, c ? side : s);
    if (err != hipSuccess) return err;
  }
  if ((err = hipEventRecord(join, side)) != hipSuccess) return err;
  return hipStreamWaitEvent(s, join, 0);
}

}  // namespace moe
