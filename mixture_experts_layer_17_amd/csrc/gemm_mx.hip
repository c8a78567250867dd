// MXFP8 grouped expert-FFN GEMMs on gfx950 MX-scaled FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, E8M0 block scales, fp32
// accumulation, bf16 outputs).
//
// Olmo-core 3 announcement, "Scaling and optimizing MoE training": MXFP8 is used
// for the expert computation where it pays, and converting into it has a cost.
// Every GEMM operand is quantised on the device (mx.hip) along that GEMM's
// contraction axis into a K-contiguous layout (activations: row blocks; forward
// weights and the token-axis operands of the weight gradients: column blocks
// stored transposed), so one "A[m][k] * B[n][k]" main loop serves all six
// products.  The token-axis operands are padded to 32 tokens per expert
// segment (block offsets from the routing metadata).
//
// The fp8 tiles (K-step of 128 bytes per row) move into LDS with the gfx950
// LDS-DMA buffer loads, 16-byte chunks XOR-swizzled by row as in the bf16
// kernels; the E8M0 scales (one 32-bit word of four blocks per tile row and
// K-step, grouped so that a tile's words for one K-step are 1 KB in a row) come
// with the data, one 1 KB LDS-DMA run per operand (half) and K-step, and are
// staged in LDS.  Where a K-step runs past the end of an expert's token range
// both operands' scales are set to 2^-127, so whatever finite codes lie there
// contribute exactly zero (products below 2^-200).
// MFMA operand layout (32x32x64 f8, checked on the hardware): lane l =
// (g = l/32, m = l%32) supplies A[m][16g .. 16g+15] in its first 16 bytes and
// A[m][32+16g .. 32+16g+15] in its last 16; its scale operand is the E8M0 scale
// of row m, block g (k in [32g, 32g+32)).  B is laid out the same way with
// n = l % 32; the accumulators are laid out as in the bf16 kernels.
#include "gemm_common.hpp"
#include "mx_common.hpp"
#include <type_traits>

namespace moe {
namespace {
using namespace gemm;

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNoSplit = 0x7FFFFFFF;

// Tile configuration: BM x BN outputs, WM x WN waves, K-step BK fp8 elements
// (128: two MFMA K-slices; 64: one), NS LDS stages per operand.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_>
struct MxCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int kA = BM * BK, kB = BN * BK;  // bytes per stage
  // scale words: per stage, two groups (the K-step's blocks may straddle two) x [A: 1 KB, B: 2 x 1 KB]
  static constexpr int kScaleStage = 2 * 3 * 1024;
  static constexpr int kScales = NS * kScaleStage;
  static_assert(BM <= 256 && BN <= 256, "one 1 KB scale run per operand (half) and group");
  static_assert(BK == 64 || BK == 128, "one or two MFMA K-slices per step");
  static constexpr int kEpi = cmax(2 * BM * (BN / 2 + 8), BM * (BN + 8));  // bf16 elements
  static constexpr int kLds = cmax((NS * kA + NS * kB + kScales) / 2, kEpi);  // bf16 elements
  static_assert(kLds * 2 <= 160 * 1024, "LDS budget");
  // LDS-DMA data loads (1 KB each) per wave per step (the scale runs come on top, one per wave at most)
  static constexpr int kDmaPerStep = (kA + kB) / 1024 / kWaves;
};
// K-step 128 on two stages.  (K-step 64 on four stages, three steps of loads
// in flight, measured 20-25% slower on every MX GEMM: each step starts with all
// waves past one barrier asking for their fragments at once, and shorter steps
// expose that LDS latency twice as often.)
using MxBig = MxCfg<256, 256, 2, 4, 128, 2>;
using MxBigP = MxBig;
using MxSmall = MxCfg<128, 128, 2, 2, 128, 2>;

// 16-byte chunk swizzle of a K-contiguous fp8 tile row (BK bytes): a fragment
// read has 16 lanes on 16 consecutive rows at one chunk; the swizzle spreads
// them over all 64 banks.
template <int BK>
__device__ __forceinline__ int mx_swz(int row) {
  return BK == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}

// K-contiguous fp8 operand with block scales: element (mn, k) at
// q[mn*ld + k_base + k]; k >= ksplit reads the second matrix at k - ksplit.
// Dual operands (template flag) take tile rows [0, W/2) from the first matrix
// and [W/2, W) from the second.  Scales are in the grouped layout: the word of
// tile row mn for block group G (blocks 4G .. 4G+3 of the row) is at
// s + G*gs + 4*mn (s already offset to the tile's first row, gs = 4 x rows of
// the scale matrix).  Rows mn >= mn_valid (of each matrix) read as zero; K
// elements past k_valid get zero-weight scales.
struct MxKc {
  const uint8_t* q0;
  const uint8_t* q1;
  const uint8_t* s0;
  const uint8_t* s1;
  int64_t ld;      // elements (bytes) per row, a multiple of 32
  int64_t k_base;  // first K element of this problem inside each row (multiple of 32)
  int k_valid;     // K elements of this problem (multiple of 32)
  int ksplit;
  int mn_valid;
  int64_t gs;      // bytes between scale groups
};

// LDS-DMA loads of a ROWS x BK-byte tile (K-step at k0).
template <class C, int ROWS, bool DUAL>
__device__ __forceinline__ void mx_dma(const MxKc& op, int k0, uint8_t* dst, int wave, int lane) {
  constexpr int CPR = C::BK / 16;  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows per 1 KB instruction
  constexpr int NI = ROWS / RPI;
  static_assert(NI % C::kWaves == 0, "tile does not split over the waves");
  const bool hi = !DUAL && k0 >= op.ksplit;
  const int64_t kk = op.k_base + (hi ? k0 - op.ksplit : k0);
  const int rl = lane / CPR, ph = lane % CPR;
#pragma unroll
  for (int u = 0; u < NI / C::kWaves; ++u) {
    const int i = wave + u * C::kWaves;
    const int trow = i * RPI + rl;
    int row = trow;
    const uint8_t* q = hi ? op.q1 : op.q0;
    if constexpr (DUAL) {
      if (i >= NI / 2) q = op.q1;
      row -= (i >= NI / 2) ? ROWS / 2 : 0;
    }
    const int rows = op.mn_valid < (DUAL ? ROWS / 2 : ROWS) ? op.mn_valid : (DUAL ? ROWS / 2 : ROWS);
    // [q + kk, q + rows*ld): ends with the last valid row
    const __amdgpu_buffer_rsrc_t r = rsrc(q + kk, static_cast<int64_t>(rows) * op.ld - kk);
    const int lc = ph ^ mx_swz<C::BK>(trow);
    dma16(r, dst + i * 1024, static_cast<int>(row * op.ld + lc * 16));
  }
}

// LDS-DMA of one scale run: the words of `rows` tile rows for block group G
// (zeros past rows_valid and for lanes past the run).
__device__ __forceinline__ void scale_dma(const uint8_t* s, int64_t gs, int64_t G, int rows_valid, uint8_t* dst,
                                          int lane) {
  const __amdgpu_buffer_rsrc_t r = rsrc(s + G * gs, static_cast<int64_t>(rows_valid) * 4);
  dma16(r, dst, lane * 16);
}

// One fp8 MFMA operand (32 bytes) from a BK-byte-row tile: row `row`, K-slice ks.
// (Read as an ext_vector type, not a struct: the compiler then knows the read
// cannot be the target of an LDS-DMA load still in flight into the other stage
// and does not wait for all of them first, which serialised each step's loads
// with its MFMAs.)
template <int BK>
__device__ __forceinline__ i32x8 mx_frag(const uint8_t* t, int row, int ks, int g) {
  const int sw = mx_swz<BK>(row);
  const lds16_t lo = *reinterpret_cast<const lds16_t*>(t + row * BK + (((ks * 4 + g) ^ sw) << 4));
  const lds16_t hi = *reinterpret_cast<const lds16_t*>(t + row * BK + (((ks * 4 + 2 + g) ^ sw) << 4));
  i32x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// B tile row of fragment j of wave column wn (dual: gate rows first, up rows at BN/2).
template <class C, bool DUAL>
__device__ __forceinline__ int b_row(int wn, int j) {
  if constexpr (DUAL) {
    constexpr int H = C::TN / 2;
    return (j >= H ? C::BN / 2 : 0) + wn * (C::WTN / 2) + (j % H) * 32;
  } else {
    return wn * C::WTN + j * 32;
  }
}

// Wait until at most `steps` K-steps of data loads (N per step) are outstanding.
template <int N, int MAXS>
__device__ __forceinline__ void mx_wait_steps(int steps) {
  static_assert(N * MAXS < 16, "vmcnt immediate");
  if constexpr (MAXS >= 2) {
    if (steps >= 2) { wait_vm<2 * N>(); return; }
  }
  if constexpr (MAXS >= 1) {
    if (steps >= 1) { wait_vm<N>(); return; }
  }
  wait_vm<0>();
}

// C = A B^T over K = [0, K), both operands K-contiguous fp8 with block scales,
// through NS LDS stages: steps 0 .. NS-2 are issued up front and, right after
// the barrier of step kt, step kt + NS - 1 (into the stage step kt - 1 used).
// Each step's scale words (the 4-block group holding its first block and,
// when its blocks run past that group, the next) come in by LDS-DMA with the
// data; a lane shifts its row's bytes out of the two words.  The wait before
// step kt leaves outstanding only as many loads as the data loads of the steps
// issued after it (loads complete in issue order; a scale run issued on top
// only makes the wait stricter).
template <class C, bool BDUAL, bool TR = false>
__device__ __forceinline__ void mx_mainloop(const MxKc& aop, const MxKc& bop, int K, uint8_t* lds, int tid,
                                            Acc<C>& acc) {
  constexpr int NS = C::NS, BK = C::BK, NSL = BK / 64;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (K + BK - 1) / BK;
  if (nk == 0) return;
  uint8_t* qa = lds;                            // A stages
  uint8_t* qb = lds + NS * C::kA;               // B stages
  uint8_t* sl = lds + NS * (C::kA + C::kB);     // [NS stages][2 groups][A 1 KB | B 2 KB]
  const int arows = aop.mn_valid < C::BM ? aop.mn_valid : C::BM;
  constexpr int BH = BDUAL ? C::BN / 2 : C::BN;
  const int brows = bop.mn_valid < BH ? bop.mn_valid : BH;
  // the wave's 32-row blocks of A that hold valid rows: fewer than TM only in the short last row tile of an
  // expert, whose empty blocks skip their fragment reads and MFMAs
  const int wrows = arows - wm * C::WTM;
  const int tmv = __builtin_amdgcn_readfirstlane(wrows <= 0 ? 0 : (wrows >= C::WTM ? C::TM : (wrows + 31) / 32));
  // first block of step kt inside its matrix (K-steps of a split operand restart at the split)
  auto first_block = [&](int kt) -> int64_t {
    const int k0 = kt * BK;
    const bool hi = !BDUAL && k0 >= aop.ksplit;
    return aop.k_base / 32 + (hi ? k0 - aop.ksplit : k0) / 32;
  };
  auto issue = [&](int kt) {
    const int k0 = kt * BK;
    const int st = kt % NS;
    mx_dma<C, C::BM, false>(aop, k0, qa + st * C::kA, wave, lane);
    mx_dma<C, C::BN, BDUAL>(bop, k0, qb + st * C::kB, wave, lane);
    // scale runs, dealt round-robin over the waves: run = group (0, 1) x {A, B half 0, B half 1}
    const bool hi = !BDUAL && k0 >= aop.ksplit;
    const int64_t b0 = first_block(kt);
    const int64_t G = b0 >> 2;
    const bool two = (b0 & 3) + BK / 32 > 4;  // the step's blocks run into the next group
#pragma unroll
    for (int run = 0; run < 6; ++run) {
      const int grp = run / 3, part = run % 3;
      if (run % C::kWaves != wave || (grp == 1 && !two) || (part == 2 && !BDUAL)) continue;
      uint8_t* dst = sl + st * C::kScaleStage + grp * 3072 + part * 1024;
      if (part == 0)
        scale_dma(hi ? aop.s1 : aop.s0, aop.gs, G + grp, arows, dst, lane);
      else
        scale_dma((part == 2 || (!BDUAL && hi)) ? bop.s1 : bop.s0, bop.gs, G + grp, brows, dst, lane);
    }
  };
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < nk) issue(s0);
  // the K loop for TMV valid row blocks of the wave (TM: a full tile; 2 covers any short last tile of up to 64
  // rows; 0: wave rows past the valid ones, which only load and synchronise)
  auto kloop = [&](auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    for (int kt = 0; kt < nk; ++kt) {
      const int ahead = nk - 1 - kt < NS - 2 ? nk - 1 - kt : NS - 2;
      mx_wait_steps<C::kDmaPerStep, NS - 2>(ahead);
      __syncthreads();
      if (kt + NS - 1 < nk) issue(kt + NS - 1);
      const int st = kt % NS;
      const uint8_t* as = qa + st * C::kA;
      const uint8_t* bs = qb + st * C::kB;
      const uint8_t* ss = sl + st * C::kScaleStage;
      // the step's blocks from byte o of the staged group word on; those past the problem's K range get
      // zero-weight scales
      const int o = static_cast<int>(first_block(kt) & 3);
      const int nb = (aop.k_valid - kt * BK) / 32;
      const uint32_t m = nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - nb))));
      auto word = [&](int part, int row) -> uint32_t {
        const uint32_t w0 = reinterpret_cast<const uint32_t*>(ss + part * 1024)[row];
        if (o == 0) return w0;
        const uint32_t w1 = reinterpret_cast<const uint32_t*>(ss + 3072 + part * 1024)[row];
        return (w0 >> (8 * o)) | (w1 << (32 - 8 * o));
      };
      // lane (g, m) needs block 2 ks + g of its row for K-slice ks: the word shifted down by g bytes puts it at
      // byte 2 ks, which the MFMA's scale operand selects (op_sel)
      uint32_t ca[C::TM], cb[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) ca[i] = (word(0, wm * C::WTM + i * 32 + (lane & 31)) & m) >> (8 * g);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int r = b_row<C, BDUAL>(wn, j) + (lane & 31);
        cb[j] = ((BDUAL && r >= C::BN / 2 ? word(2, r - C::BN / 2) : word(1, r)) & m) >> (8 * g);
      }
#pragma unroll
      for (int ks = 0; ks < NSL; ++ks) {
        i32x8 a[TMV > 0 ? TMV : 1], b[C::TN];
#pragma unroll
        for (int i = 0; i < TMV; ++i) a[i] = mx_frag<BK>(as, wm * C::WTM + i * 32 + (lane & 31), ks, g);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) b[j] = mx_frag<BK>(bs, b_row<C, BDUAL>(wn, j) + (lane & 31), ks, g);
#pragma unroll
        for (int i = 0; i < TMV; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j) {
            const int sa = static_cast<int>(ca[i]), sb = static_cast<int>(cb[j]);
            // TR: the tile transposed (B in the first operand slot), so a lane holds four consecutive output
            // columns of one row (the register-direct and wave-staged epilogues)
            if (ks == 0)
              acc[i][j] = TR ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, sb, 0, sa)
                             : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, sa, 0, sb);
            else
              acc[i][j] = TR ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 2, sb, 2, sa)
                             : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 2, sa, 2, sb);
          }
      }
    }
  };
  if (tmv > 2 || C::TM <= 2) {
    if (tmv > 0) kloop(std::integral_constant<int, C::TM>{});
    else kloop(std::integral_constant<int, 0>{});
  } else if (tmv > 0) {
    kloop(std::integral_constant<int, (C::TM < 2 ? C::TM : 2)>{});
  } else {
    kloop(std::integral_constant<int, 0>{});
  }
  __syncthreads();  // the epilogue reuses the LDS
}

// Quantised operands of one FFN call (device pointers into the scratch area).
struct MxArgs {
  FfnArgs f;
  const int32_t* blk;  // MX block offsets per expert (token axis), E+1
  int64_t ldt;         // padded token length of the transposed token-axis operands
  const uint8_t *xq, *xs, *aq, *as, *dyq, *dys, *dhgq, *dhgs, *dhuq, *dhus;          // row-blocked [R, K]
  const uint8_t *wgq, *wgs, *wuq, *wus, *wdq, *wds;                                   // weights, K-contiguous
  const uint8_t *xtq, *xts, *dytq, *dyts, *atq, *ats, *dhgtq, *dhgts, *dhutq, *dhuts;  // [cols, ldt]
  uint8_t *oaq, *oas;  // G1 on 256 x 256 tiles: A's rows layout (G2's operand), written by its epilogue
};

// Workgroup barrier that waits for the wave's LDS accesses only: __syncthreads()
// (whose release fence also covers LDS-DMA loads, which write LDS under the
// vector memory counter) would make every wave wait for all its outstanding
// vector memory operations, the next tile's loads and the epilogue's stores
// included.  Used where the loads a step needs have been waited for explicitly
// (wait_vm); the memory clobber keeps the compiler from moving accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// G1's register-direct epilogue (as epi_regs_swiglu_fwd: Hg, Hu and A = silu(Hg) * Hu
// as bf16) that also encodes A into its MX rows layout for G2 (codes [R][f],
// grouped scales), so no separate pass reads A back.  Each wave's 32-column
// slice of the tile is one 32-element block of every row: a lane holds 16 of
// its values (to_chunks), lane l ^ 32 the other 16.  The block is encoded from
// A rounded to bf16, the values the quantiser would read, with its arithmetic,
// so the bytes equal its output.  The tile's 128 columns (n0 a multiple of 128)
// are whole 128-byte code lines and whole scale words (one block group), so
// codes and scale bytes are gathered in the idle LDS and leave as whole lines
// and one 1 KB run of words: stored from registers, the 16-byte pieces of 32
// rows per instruction cost G1 about 4% (measured).
template <class C>
__device__ __forceinline__ void epi_regs_swiglu_fwd_mx(const Acc<C>& acc, const FfnArgs& p, int64_t row0, int rows,
                                                       int n0, int lane, int wm, int wn, int wave, uint8_t* aq,
                                                       uint8_t* as, uint8_t* stage) {
  static_assert(C::BN / 2 == 128, "a tile's 128 columns of A: whole 128-byte code lines, one scale group");
  static_assert(C::BM * 128 + C::BM * 4 <= C::kLds * 2, "codes and scale words staged in the tile's LDS");
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  uint8_t* sq = stage;                  // [BM][128] codes, 16-byte chunks XOR-swizzled by row
  uint8_t* sw = stage + C::BM * 128;    // [BM] scale words
  constexpr int H = C::TN / 2;
  static_assert(C::WTN / 2 == 32 * H, "one 32-column block per fragment column");
  const int rl = lane & 31, h = lane >> 5, hc = 8 * h;
  const int64_t f = p.f, R = p.R;
  uint16_t* hg = static_cast<uint16_t*>(p.o_hg) + row0 * f + n0;
  uint16_t* hu = static_cast<uint16_t*>(p.o_hu) + row0 * f + n0;
  uint16_t* ac = static_cast<uint16_t*>(p.o_act) + row0 * f + n0;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * C::WTM + i * 32 + rl;
    const bool rv = row < rows;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      float g[2][8], u[2][8];
      to_chunks(acc[i][j], g);
      to_chunks(acc[i][j + H], u);
      uint4 ab[2];
      float v[2][8];
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float a[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) a[t] = silu_f(g[c][t]) * u[c][t];
        ab[c] = pack8(a);
        Elem<uint16_t>::unpack(ab[c], v[c]);
#pragma unroll
        for (int t = 0; t < 8; ++t) amax = fmaxf(amax, fabsf(v[c][t]));
      }
      {  // with lane l ^ 32 (the row's other 16 values): a VALU lane swap, no LDS round trip
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const int e = mx_block_exponent(amax);
      const float inv = mx_inv_scale(e);
      const int col = wn * (C::WTN / 2) + j * 32;  // the block's first column in the tile
      // codes of the lane's two runs of eight (columns 16c + 8h ..)
      uint2 cw[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        cw[c] = make_uint2(e4m3_pack4(v[c][0] * inv, v[c][1] * inv, v[c][2] * inv, v[c][3] * inv),
                           e4m3_pack4(v[c][4] * inv, v[c][5] * inv, v[c][6] * inv, v[c][7] * inv));
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x2 w2 = {cw[c].x, cw[c].y};
        *reinterpret_cast<u32x2*>(sq + row * 128 + ((((col >> 4) + c) ^ (row & 7)) << 4) + hc) = w2;
      }
      if (h == 0) sw[row * 4 + col / 32] = static_cast<uint8_t>(e + 127);  // byte (block within the group)
      if (rv) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int64_t o = row * f + col + 16 * c + hc;
          store16<false>(hg + o, pack8(g[c]));
          store16<false>(hu + o, pack8(u[c]));
          store16<false>(ac + o, ab[c]);
        }
      }
    }
  }
  lds_barrier();  // the staged codes and scale bytes of all waves (the bf16 stores stay in flight)
  // wave w: rows 32w .. 32w + 31, eight lanes (one 128-byte line) per row
#pragma unroll
  for (int t = 0; t < C::BM / 8 / C::kWaves; ++t) {
    const int rr = (wave * (C::BM / 8 / C::kWaves) + t) * 8 + (lane >> 3), k = lane & 7;
    if (rr < rows) {
      const uint4 v = lds_get16(sq + rr * 128 + ((k ^ (rr & 7)) << 4));
      *reinterpret_cast<uint4*>(aq + (row0 + rr) * f + n0 + 16 * k) = v;
    }
  }
  // the words of the tile's rows for block group n0 / 128: rows row0 .. row0 + rows - 1, contiguous
  // (4-byte aligned only: the run starts at any row), 256 bytes per store instruction
  if (wave == C::kWaves - 1) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(as + ((n0 / 128) * R + row0) * 4);
#pragma unroll
    for (int t = 0; t < C::BM / 64; ++t) {
      const int r = t * 64 + lane;
      if (r < rows) dst[r] = reinterpret_cast<const uint32_t*>(sw)[r];
    }
  }
}

template <class C, int KIND>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(2))) void ffn_mx_kernel(MxArgs m) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLds];
  uint8_t* lds8 = reinterpret_cast<uint8_t*>(lds);
  const FfnArgs& p = m.f;
  const int tid = threadIdx.x;
  // 256 x 256 tiles on 8 waves of 128 x 64: computed transposed; G1 and G2 store from registers, the others
  // through 8 KB of LDS per wave (whole-line stores); smaller tiles stage the whole tile in LDS
  constexpr bool TR = C::BM == 256 && C::BN == 256 && C::kWaves == 8 && C::WTN == 64;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  uint16_t* wbuf = lds + wave * 4096;  // this wave's 8 KB of the (then idle) LDS
  const int d = p.d, f = p.f;
  const int64_t wsz = static_cast<int64_t>(d) * f;
  Acc<C> acc;

  if constexpr (KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5) {
    const int gx = KIND == kG1 ? (f + C::BN / 2 - 1) / (C::BN / 2)
                               : KIND == kG3 ? (f + C::BN - 1) / C::BN : (d + C::BN - 1) / C::BN;
    const int64_t lid = xcd_tile(blockIdx.x, static_cast<int64_t>(p.tiles[p.max_tiles].x) * gx);
    if (lid < 0) return;
    int nt;
    const int4 t = p.tiles[expert_tile(lid, gx, p.tiles, p.max_tiles, nt)];
    if (t.x < 0) return;
    const int e = __builtin_amdgcn_readfirstlane(t.x), rows = __builtin_amdgcn_readfirstlane(t.z);
    const int64_t row0 = __builtin_amdgcn_readfirstlane(t.y);
    if constexpr (KIND == kG1) {
      const int n0 = nt * (C::BN / 2);
      const int64_t R = p.R;
      const MxKc a{m.xq + row0 * d, nullptr, m.xs + row0 * 4, nullptr, d, 0, d, kNoSplit, rows, R * 4};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * d;  // transposed Wg, Wu: [E][f][d]
      const int64_t so = e * wsz / 32 + static_cast<int64_t>(n0) * 4;  // scales grouped per expert over f rows
      const MxKc b{m.wgq + wo, m.wuq + wo, m.wgs + so, m.wus + so, d, 0, d, kNoSplit, f - n0,
                   static_cast<int64_t>(f) * 4};
      mx_mainloop<C, true, TR>(a, b, d, lds8, tid, acc);
      if constexpr (TR) epi_regs_swiglu_fwd_mx<C>(acc, p, row0, rows, n0, lane, wm, wn, wave, m.oaq, m.oas, lds8);
      else epi_swiglu_fwd<C>(acc, lds, p, row0, rows, n0, tid);
    } else if constexpr (KIND == kG2) {
      const int n0 = nt * C::BN;  // over d
      const MxKc a{m.aq + row0 * f, nullptr, m.as + row0 * 4, nullptr, f, 0, f, kNoSplit, rows, p.R * 4};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * f;  // transposed Wd: [E][d][f]
      const int64_t so = e * wsz / 32 + static_cast<int64_t>(n0) * 4;  // scales grouped per expert over d rows
      const MxKc b{m.wdq + wo, nullptr, m.wds + so, nullptr, f, 0, f, kNoSplit, d - n0, static_cast<int64_t>(d) * 4};
      mx_mainloop<C, false, TR>(a, b, f, lds8, tid, acc);
      // Y is read by the combine right after: ordinary (cached) stores
      if constexpr (TR) epi_regs_store<C>(acc, static_cast<uint16_t*>(p.o_y) + row0 * d + n0, d, rows, d - n0, lane, wm, wn);
      else epi_store<C, false>(acc, lds, static_cast<uint16_t*>(p.o_y) + row0 * d + n0, d, rows, d - n0, tid);
    } else if constexpr (KIND == kG3) {
      const int n0 = nt * C::BN;  // over f
      const MxKc a{m.dyq + row0 * d, nullptr, m.dys + row0 * 4, nullptr, d, 0, d, kNoSplit, rows, p.R * 4};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * d;  // natural Wd: [E][f][d]
      const int64_t so = (static_cast<int64_t>(e) * f + n0) * 4;  // scales grouped over all E*f rows
      const MxKc b{m.wdq + wo, nullptr, m.wds + so, nullptr, d, 0, d, kNoSplit, f - n0,
                   static_cast<int64_t>(p.E) * f * 4};
      mx_mainloop<C, false>(a, b, d, lds8, tid, acc);
      epi_swiglu_bwd<C>(acc, lds, p, row0, rows, n0, tid);
    } else {  // kG5
      const int n0 = nt * C::BN;  // over d
      const MxKc a{m.dhgq + row0 * f, m.dhuq + row0 * f, m.dhgs + row0 * 4, m.dhus + row0 * 4,
                   f, 0, 2 * f, f, rows, p.R * 4};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * f;  // natural Wg, Wu: [E][d][f]
      const int64_t so = (static_cast<int64_t>(e) * d + n0) * 4;  // scales grouped over all E*d rows
      const MxKc b{m.wgq + wo, m.wuq + wo, m.wgs + so, m.wus + so, f, 0, 2 * f, f, d - n0,
                   static_cast<int64_t>(p.E) * d * 4};
      mx_mainloop<C, false, TR>(a, b, 2 * f, lds8, tid, acc);
      // dX rows are read by the dispatch backward right after: ordinary stores
      if constexpr (TR)
        epi_staged_store<C, false>(acc, wbuf, static_cast<uint16_t*>(p.o_dx) + row0 * d + n0, d, rows, d - n0, lane, wm,
                                   wn);
      else epi_store<C>(acc, lds, static_cast<uint16_t*>(p.o_dx) + row0 * d + n0, d, rows, d - n0, tid);
    }
  } else {  // weight gradients: K = 32-padded token blocks of expert e
    const int gm = KIND == kG4 ? (f + C::BM - 1) / C::BM : (d + C::BM - 1) / C::BM;
    const int gn = KIND == kG4 ? (d + C::BN - 1) / C::BN : 2 * ((f + C::BN - 1) / C::BN);
    int e, local;
    if (!wgrad_tile_sorted(blockIdx.x, p.E, gm * gn, p.wsched, e, local)) return;
    e = __builtin_amdgcn_readfirstlane(e);
    const int mt = local / gn, ntile = local % gn;
    const int b0 = __builtin_amdgcn_readfirstlane(ld_uniform(m.blk + e));
    const int64_t kb = static_cast<int64_t>(b0) * 32;
    const int K = (__builtin_amdgcn_readfirstlane(ld_uniform(m.blk + e + 1)) - b0) * 32;
    const int m0 = mt * C::BM;
    uint16_t* Cp;
    int n0, ldc, mvalid, nvalid;
    MxKc a, b;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      n0 = ntile * C::BN;
      a = MxKc{m.atq + static_cast<int64_t>(m0) * m.ldt, nullptr, m.ats + static_cast<int64_t>(m0) * 4, nullptr,
               m.ldt, kb, K, kNoSplit, f - m0, static_cast<int64_t>(f) * 4};
      b = MxKc{m.dytq + static_cast<int64_t>(n0) * m.ldt, nullptr, m.dyts + static_cast<int64_t>(n0) * 4, nullptr,
               m.ldt, kb, K, kNoSplit, d - n0, static_cast<int64_t>(d) * 4};
      Cp = static_cast<uint16_t*>(p.o_dwd) + e * wsz;
      ldc = d;
      mvalid = f;
      nvalid = d;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + C::BN - 1) / C::BN;
      const int which = ntile / per;
      n0 = (ntile % per) * C::BN;
      a = MxKc{m.xtq + static_cast<int64_t>(m0) * m.ldt, nullptr, m.xts + static_cast<int64_t>(m0) * 4, nullptr,
               m.ldt, kb, K, kNoSplit, d - m0, static_cast<int64_t>(d) * 4};
      const uint8_t* bq = which ? m.dhutq : m.dhgtq;
      const uint8_t* bs = which ? m.dhuts : m.dhgts;
      b = MxKc{bq + static_cast<int64_t>(n0) * m.ldt, nullptr, bs + static_cast<int64_t>(n0) * 4, nullptr, m.ldt, kb,
               K, kNoSplit, f - n0, static_cast<int64_t>(f) * 4};
      Cp = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz;
      ldc = f;
      mvalid = d;
      nvalid = f;
    }
    mx_mainloop<C, false, TR>(a, b, K, lds8, tid, acc);
    if constexpr (TR)
      epi_staged_store<C, true>(acc, wbuf, Cp + static_cast<int64_t>(m0) * ldc + n0, ldc, mvalid - m0, nvalid - n0,
                                lane, wm, wn);
    else epi_store<C>(acc, lds, Cp + static_cast<int64_t>(m0) * ldc + n0, ldc, mvalid - m0, nvalid - n0, tid);
  }
}

// ---------------------------------------------------------------------------
// Persistent 256 x 256 MX kernel for the SwiGLU backward (G3) and the down
// projection (G2).  Workgroups loop over tiles (ids b, b + G, ... in the
// XCD-contiguous order), and the K-steps of consecutive tiles form one stream
// through the two LDS stages: each step's loads are issued right after the
// barrier of the step before.  Tiles are computed transposed (mfma(B, A)) so
// the epilogues run from registers.  G2's last step issues the next tile's
// first step, so those loads are in flight during its epilogue, which stores
// the same number of 16-byte lines in every wave (buffer stores into a range
// that ends with the tile's last valid row: the hardware drops the lanes past
// it instead of the wave branching around them; tiles are whole in N, d a
// multiple of 256); the next tile then waits for its own first loads alone,
// which went out before these stores (loads and stores retire in issue order),
// while the stores drain.  G3 stages its Hg, Hu loads through both LDS stages
// (the next tile then starts after its epilogue).  Measured on the MXFP8
// E = 128 workload: G3 621 us against 789 one workgroup per tile, G2 560
// against 574; G1 and G5 (24-32 K-steps a tile against G2's 12) the same way
// as G2 983 against 964 and 1002 against 994, so they keep one workgroup per
// tile.  So do the weight gradients: a new workgroup's loads do not wait for
// the previous tile's 128 KB of dW stores, which a persistent workgroup's
// single vmcnt counter would (measured 21% slower persistent).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, int off, const uint4& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
}

// G2's epilogue: TM x TN x 2 stores per wave.
template <class C>
__device__ __forceinline__ void epi_regs_store_all(const Acc<C>& acc, uint16_t* dst, int64_t ld, int rows_valid,
                                                   int lane, int wm, int wn) {
  const __amdgpu_buffer_rsrc_t r = rsrc(dst, static_cast<int64_t>(rows_valid) * ld * 2);
  const int rl = lane & 31, hc = 8 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * C::WTM + i * 32 + rl;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      float v[2][8];
      to_chunks(acc[i][j], v);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        bstore16(r, static_cast<int>((row * ld + wn * C::WTN + j * 32 + 16 * c + hc) * 2), pack8(v[c]));
    }
  }
}

struct MxTile {
  MxKc a, b;
  int K;            // contraction length (0: zero outputs)
  int rows, cols;   // valid output rows / columns from the tile origin
  int64_t row0;     // rows-by-expert GEMMs: first row of the tile
  int n0;           // first output column (over f for G1 and G3)
  uint16_t* out;    // plain-store GEMMs: output tile origin
  int64_t ldo;      // and its row stride
};

// Tile of hardware-order id `id` over the live table entries times the N
// tiles (rows-by-expert GEMMs).  False past the last tile.
template <class C, int KIND>
__device__ __forceinline__ bool mx_tile(const MxArgs& m, int64_t id, int64_t live, MxTile& t) {
  const FfnArgs& p = m.f;
  const int d = p.d, f = p.f;
  const int64_t wsz = static_cast<int64_t>(d) * f;
  static_assert(KIND == kG2 || KIND == kG3, "the persistent GEMMs");
  {
    const int gx = KIND == kG3 ? (f + C::BN - 1) / C::BN : (d + C::BN - 1) / C::BN;
    const int64_t lid = xcd_tile(id, live * gx);
    if (lid < 0) return false;
    int nt;
    const int4 tt = ld_uniform(p.tiles + expert_tile(lid, gx, p.tiles, p.max_tiles, nt));
    const int e = __builtin_amdgcn_readfirstlane(tt.x);
    const int rows = e < 0 ? 0 : __builtin_amdgcn_readfirstlane(tt.z);
    const int64_t row0 = e < 0 ? 0 : __builtin_amdgcn_readfirstlane(tt.y);
    const int64_t ee = e < 0 ? 0 : e;
    const int64_t R = p.R;
    t.row0 = row0;
    t.rows = rows;
    if constexpr (KIND == kG2) {
      t.n0 = nt * C::BN;  // over d
      t.a = MxKc{m.aq + row0 * f, nullptr, m.as + row0 * 4, nullptr, f, 0, f, kNoSplit, rows, R * 4};
      const int64_t wo = ee * wsz + static_cast<int64_t>(t.n0) * f;      // transposed Wd: [E][d][f]
      const int64_t so = ee * wsz / 32 + static_cast<int64_t>(t.n0) * 4;  // scales grouped per expert over d rows
      t.b = MxKc{m.wdq + wo, nullptr, m.wds + so, nullptr, f, 0, f, kNoSplit, d - t.n0, static_cast<int64_t>(d) * 4};
      t.K = f;
      t.cols = d - t.n0;
      t.out = static_cast<uint16_t*>(p.o_y) + row0 * d + t.n0;
      t.ldo = d;
    } else {  // kG3
      t.n0 = nt * C::BN;  // over f
      t.a = MxKc{m.dyq + row0 * d, nullptr, m.dys + row0 * 4, nullptr, d, 0, d, kNoSplit, rows, R * 4};
      const int64_t wo = ee * wsz + static_cast<int64_t>(t.n0) * d;    // natural Wd: [E][f][d]
      const int64_t so = (ee * f + t.n0) * 4;                           // scales grouped over all E*f rows
      t.b = MxKc{m.wdq + wo, nullptr, m.wds + so, nullptr, d, 0, d, kNoSplit, f - t.n0,
                 static_cast<int64_t>(p.E) * f * 4};
      t.K = d;
      t.cols = f - t.n0;
    }
    if (rows == 0) t.K = 0;
  }
  return true;
}

// Whether hardware-order id `id` names a tile (as mx_tile, without building it).
template <class C, int KIND>
__device__ __forceinline__ bool mx_tile_valid(const FfnArgs& p, int64_t id, int64_t live) {
  const int gx = KIND == kG3 ? (p.f + C::BN - 1) / C::BN : (p.d + C::BN - 1) / C::BN;
  return xcd_tile(id, live * gx) >= 0;
}

template <class C, int KIND>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::kWaves / 4)))
void ffn_mx_persistent(MxArgs m) {
  static_assert(C::BM == 256 && C::BN == 256 && C::kWaves == 8 && C::TM == 4 && C::WTN == 64,
                "256 x 256 tiles on 8 waves of 128 x 64");
  constexpr bool kStaged = KIND == kG3;
  constexpr int kEpiOps = C::TM * C::TN * 2;  // stores of one wave's G2 epilogue (epi_regs_store_all)
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLds];
  uint8_t* l8 = reinterpret_cast<uint8_t*>(lds);
  const FfnArgs& p = m.f;
  const int tid = threadIdx.x, lane = tid & 63, g32 = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t live = __builtin_amdgcn_readfirstlane(ld_uniform(p.tiles + p.max_tiles).x);
  const int64_t step = gridDim.x;
  int64_t id = blockIdx.x;
  MxTile cur;
  if (!mx_tile<C, KIND>(m, id, live, cur)) return;

  uint8_t* const qa = l8;                          // A stages
  uint8_t* const qb = l8 + 2 * C::kA;              // B stages
  uint8_t* const sl = l8 + 2 * C::kA + 2 * C::kB;  // scale stages: [2 groups][A 1 KB | B 2 KB]
  // this wave's 8 KB of stage `slot` (bf16 elements) for G3's staged epilogue
  auto stage_buf = [&](int slot) -> uint16_t* {
    return reinterpret_cast<uint16_t*>(wave < 4 ? qa + slot * C::kA + wave * 8192
                                                : qb + slot * C::kB + (wave - 4) * 8192);
  };
  // step kt of tile t into stage `slot`: the A and B tiles and the scale runs (one per wave:
  // group (0, 1) x {A, B}; group 1 only for K-steps that straddle two groups)
  auto issue = [&](const MxTile& t, int kt, int slot) {
    const int k0 = kt * C::BK;
    mx_dma<C, C::BM, false>(t.a, k0, qa + slot * C::kA, wave, lane);
    mx_dma<C, C::BN, false>(t.b, k0, qb + slot * C::kB, wave, lane);
    const int o = static_cast<int>((t.a.k_base / 32) & 3);
    const int grp = wave / 3, part = wave % 3;
    if (wave < 6 && !(grp == 1 && o == 0) && part != 2) {
      const int arows = t.a.mn_valid < C::BM ? t.a.mn_valid : C::BM;
      const int brows = t.b.mn_valid < C::BN ? t.b.mn_valid : C::BN;
      const bool hi = k0 >= t.a.ksplit;
      const int kk = hi ? k0 - t.a.ksplit : k0;
      const int64_t G = (t.a.k_base / 32 + kk / 32) >> 2;
      uint8_t* dst = sl + slot * C::kScaleStage + grp * 3072 + part * 1024;
      if (part == 0)
        scale_dma(hi ? t.a.s1 : t.a.s0, t.a.gs, G + grp, arows, dst, lane);
      else
        scale_dma(hi ? t.b.s1 : t.b.s0, t.b.gs, G + grp, brows, dst, lane);
    }
  };

  int g = 0;         // stage position of the current tile's step 0
  bool pre = false;  // the current tile's step 0 already issued
  for (;;) {
    const int64_t nid = id + step;
    const bool more = mx_tile_valid<C, KIND>(p, nid, live);
    const int nk = (cur.K + C::BK - 1) / C::BK;
    if (!pre && nk > 0) issue(cur, 0, g & 1);
    const int o = static_cast<int>((cur.a.k_base / 32) & 3);
    Acc<C> acc;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      // step 0 of a tile whose loads went out during the previous tile: only the previous epilogue's stores may
      // still be in flight after them
      if (!kStaged && kt == 0 && pre) wait_vm<kEpiOps>();
      else wait_vm<0>();
      lds_barrier();
      const int slot = (g + kt) & 1;
      // the next step's loads into the other stage: this tile's, or at its last step the next tile's first
      if (kt + 1 < nk) {
        issue(cur, kt + 1, slot ^ 1);
      } else if (kStaged) {
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 0, stage_buf(slot ^ 1), wm, wn, lane);
      } else if (more) {
        MxTile t2;
        mx_tile<C, KIND>(m, nid, live, t2);
        if (t2.K > 0) issue(t2, 0, slot ^ 1);
      }
      const uint8_t* as = qa + slot * C::kA;
      const uint8_t* bs = qb + slot * C::kB;
      const uint8_t* ss = sl + slot * C::kScaleStage;
      // bytes of this step's four blocks that lie inside the tile's K range
      const int nb = (cur.a.k_valid - kt * C::BK) / 32;
      const uint32_t msk = nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - nb))));
      auto word = [&](int part, int row) -> uint32_t {
        const uint32_t w0 = reinterpret_cast<const uint32_t*>(ss + part * 1024)[row];
        if (o == 0) return w0;
        const uint32_t w1 = reinterpret_cast<const uint32_t*>(ss + 3072 + part * 1024)[row];
        return (w0 >> (8 * o)) | (w1 << (32 - 8 * o));
      };
      // lane (g, m): block 2 ks + g of its row at byte 2 ks of the word shifted down by g bytes (op_sel)
      uint32_t ca[C::TM], cb[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) ca[i] = (word(0, wm * C::WTM + i * 32 + (lane & 31)) & msk) >> (8 * g32);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        cb[j] = (word(1, b_row<C, false>(wn, j) + (lane & 31)) & msk) >> (8 * g32);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        i32x8 a[C::TM], b[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) a[i] = mx_frag<C::BK>(as, wm * C::WTM + i * 32 + (lane & 31), ks, g32);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) b[j] = mx_frag<C::BK>(bs, b_row<C, false>(wn, j) + (lane & 31), ks, g32);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
            acc[i][j] = ks == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                      b[j], a[i], acc[i][j], 0, 0, 0, static_cast<int>(cb[j]), 0, static_cast<int>(ca[i]))
                                : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                      b[j], a[i], acc[i][j], 0, 0, 2, static_cast<int>(cb[j]), 2, static_cast<int>(ca[i]));
      }
    }
    pre = nk > 0 && !kStaged && more;
    g += nk;
    if constexpr (kStaged) {
      // blocks 0, 1 in the two stage buffers, then 2, 3; block 0 was issued at the last K-step
      if (nk > 0) {
        uint16_t* b0 = stage_buf(g & 1);
        uint16_t* b1 = stage_buf((g + 1) & 1);
        __syncthreads();  // the last step's stage is free
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 1, b1, wm, wn, lane);
        wait_vm<0>();
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 0, b0, wm, wn, lane);
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 1, b1, wm, wn, lane);
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 2, b0, wm, wn, lane);
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 3, b1, wm, wn, lane);
        wait_vm<0>();
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 2, b0, wm, wn, lane);
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 3, b1, wm, wn, lane);
        __syncthreads();  // the LDS holds stages again
      }
    } else {  // G2: Y is read by the combine right after: ordinary stores
      epi_regs_store_all<C>(acc, cur.out, cur.ldo, cur.rows, lane, wm, wn);
    }
    if (!more) break;
    mx_tile<C, KIND>(m, nid, live, cur);
    id = nid;
  }
}

template <int KIND>
void launch_mx_persistent(const char* name, const MxArgs& a, int64_t tiles, hipStream_t s) {
  using C = MxBigP;
  static const int occ = occupancy(reinterpret_cast<const void*>(&ffn_mx_persistent<C, KIND>), C::kThreads);
  MOE_LAUNCH(name, (ffn_mx_persistent<C, KIND>), dim3(persistent_grid(occ, tiles)), dim3(C::kThreads), 0, s, a);
}

template <class C>
int launch_mx_cfg(int kind, const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t nd = cdiv(a.f.d, C::BN), nf = cdiv(a.f.f, C::BN);
  const dim3 blk(C::kThreads);
  switch (kind) {
    case kG1:
      MOE_LAUNCH("G1_mx", (ffn_mx_kernel<C, kG1>), dim3(xcd_grid(cdiv(a.f.f, C::BN / 2) * max_tiles)), blk, 0, s, a);
      break;
    case kG2: MOE_LAUNCH("G2_mx", (ffn_mx_kernel<C, kG2>), dim3(xcd_grid(nd * max_tiles)), blk, 0, s, a); break;
    case kG3: MOE_LAUNCH("G3_mx", (ffn_mx_kernel<C, kG3>), dim3(xcd_grid(nf * max_tiles)), blk, 0, s, a); break;
    case kG5: MOE_LAUNCH("G5_mx", (ffn_mx_kernel<C, kG5>), dim3(xcd_grid(nd * max_tiles)), blk, 0, s, a); break;
    case kG4:
      MOE_LAUNCH("G4_mx", (ffn_mx_kernel<C, kG4>),
                 dim3(static_cast<unsigned>(wgrad_sorted_grid(a.f.E, static_cast<int>(cdiv(a.f.f, C::BM) * nd)))), blk,
                 0, s, a);
      break;
    case kG6:
      MOE_LAUNCH("G6_mx", (ffn_mx_kernel<C, kG6>),
                 dim3(static_cast<unsigned>(wgrad_sorted_grid(a.f.E, static_cast<int>(cdiv(a.f.d, C::BM) * 2 * nf)))),
                 blk, 0, s, a);
      break;
    default: return MOE_EINVAL;
  }
  return launch_status();
}

bool mx_big_rows(int64_t R, int E) { return R >= static_cast<int64_t>(E) * 512; }
bool mx_big_wgrad(const FfnArgs& a) { return a.d % 256 == 0 && a.f % 256 == 0; }

// 256 x 256 tiles: the SwiGLU-backward GEMM (G3) and the down projection (G2)
// on the persistent kernel, the others one workgroup per tile.  G3 persistent:
// 621 us against 789 with one workgroup per tile (MXFP8 E = 128 workload).
int launch_mx_kind(int kind, const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  using C = MxBig;
  const bool wgrad = kind == kG4 || kind == kG6;
  const bool big = wgrad ? mx_big_wgrad(a.f) : a.f.bm == C::BM;
  if (!big) return launch_mx_cfg<MxSmall>(kind, a, max_tiles, s);
  if (kind == kG3) {
    launch_mx_persistent<kG3>("G3_mx", a, cdiv(a.f.f, C::BN) * max_tiles, s);
    return launch_status();
  }
  // G2 (12 K-steps a tile at f = 1536) persistent, its next tile's first loads in flight during the epilogue
  // (needs whole tiles in N: its epilogue stores every column of a row).  Measured on the MXFP8 E = 128 workload:
  // G2 574 -> 560 us; G1 and G5 (24-32 K-steps a tile) persistent the same way: 964 -> 983 and 994 -> 1002.
  if (kind == kG2 && a.f.d % C::BN == 0) {
    launch_mx_persistent<kG2>("G2_mx", a, cdiv(a.f.d, C::BN) * max_tiles, s);
    return launch_status();
  }
  return launch_mx_cfg<C>(kind, a, max_tiles, s);
}

// Scratch carving: a bump allocator over the caller's workspace.
struct Carve {
  char* p;
  size_t used = 0;
  uint8_t* take(size_t n) {
    uint8_t* r = p ? reinterpret_cast<uint8_t*>(p + used) : nullptr;
    used += align_up(n, 256);
    return r;
  }
};

struct QPair {
  uint8_t* q;
  uint8_t* s;
};

QPair take_q(Carve& c, int64_t elems) {
  QPair r;
  r.q = c.take(static_cast<size_t>(elems));
  r.s = c.take(static_cast<size_t>(elems / 32));
  return r;
}

int64_t token_pad(int64_t R, int E) { return mx_token_rows(R, E); }

// Lay out (or size, when base is null) the forward and backward scratch areas.
struct FwdBufs {
  QPair x, wg, wu, wd, a;
};
struct BwdBufs {
  QPair dy, wd, wg, wu, dhg, dhu, xt, dyt, at, dhgt, dhut;
};

FwdBufs carve_fwd(Carve& c, int64_t R, int E, int d, int f) {
  const int64_t w = static_cast<int64_t>(E) * d * f;
  FwdBufs b;
  b.x = take_q(c, R * d);
  b.wg = take_q(c, w);
  b.wu = take_q(c, w);
  b.wd = take_q(c, w);
  b.a = take_q(c, R * f);
  return b;
}

BwdBufs carve_bwd(Carve& c, int64_t R, int E, int d, int f) {
  const int64_t w = static_cast<int64_t>(E) * d * f;
  const int64_t rp = token_pad(R, E);
  BwdBufs b;
  b.dy = take_q(c, R * d);
  b.wd = take_q(c, w);
  b.wg = take_q(c, w);
  b.wu = take_q(c, w);
  b.dhg = take_q(c, R * f);
  b.dhu = take_q(c, R * f);
  b.xt = take_q(c, static_cast<int64_t>(d) * rp);
  b.dyt = take_q(c, static_cast<int64_t>(d) * rp);
  b.at = take_q(c, static_cast<int64_t>(f) * rp);
  b.dhgt = take_q(c, static_cast<int64_t>(f) * rp);
  b.dhut = take_q(c, static_cast<int64_t>(f) * rp);
  return b;
}

// Pre-quantised weights: every weight in the forward orientation (blocks along
// the forward GEMM's K, stored K-contiguous: Wg, Wu as [E][f][d], Wd as
// [E][d][f]) and the backward one (natural layouts, blocks along the last axis).
struct WCache {
  QPair wg_f, wu_f, wd_f, wg_b, wu_b, wd_b;
};

WCache carve_wcache(Carve& c, int E, int d, int f) {
  const int64_t w = static_cast<int64_t>(E) * d * f;
  WCache r;
  r.wg_f = take_q(c, w);
  r.wu_f = take_q(c, w);
  r.wd_f = take_q(c, w);
  r.wg_b = take_q(c, w);
  r.wu_b = take_q(c, w);
  r.wd_b = take_q(c, w);
  return r;
}

}  // namespace

int ffn_mx_bm(int64_t R, int E) { return mx_big_rows(R, E) ? MxBig::BM : MxSmall::BM; }

size_t mx_wcache_bytes(int E, int d, int f) {
  Carve c{nullptr};
  carve_wcache(c, E, d, f);
  return c.used;
}

void mx_wcache_build(const void* wg, const void* wu, const void* wd, int E, int d, int f, char* cache,
                     hipStream_t s) {
  Carve c{cache};
  const WCache w = carve_wcache(c, E, d, f);
  const int bf = MOE_BF16;
  // Wg, Wu [E][d][f]: along d -> [E][f][d] (forward), along f -> [E][d][f] (backward)
  launch_mx_both(wg, bf, E, d, f, w.wg_f.q, w.wg_f.s, w.wg_b.q, w.wg_b.s, s);
  launch_mx_both(wu, bf, E, d, f, w.wu_f.q, w.wu_f.s, w.wu_b.q, w.wu_b.s, s);
  // Wd [E][f][d]: along f -> [E][d][f] (forward), along d -> [E][f][d] (backward)
  launch_mx_both(wd, bf, E, f, d, w.wd_f.q, w.wd_f.s, w.wd_b.q, w.wd_b.s, s);
}

size_t mx_ffn_scratch_bytes(int64_t R, int E, int d, int f, int is_bwd) {
  Carve c{nullptr};
  if (is_bwd)
    carve_bwd(c, R, E, d, f);
  else
    carve_fwd(c, R, E, d, f);
  return c.used;
}

int mx_ffn_fwd(const FfnArgs& a, int64_t max_tiles, const char* wcache, const uint8_t* x_mx, char* scratch,
               hipStream_t s) {
  Carve c{scratch};
  const FwdBufs b = carve_fwd(c, a.R, a.E, a.d, a.f);
  const int bf = MOE_BF16;
  MxArgs m{};
  m.f = a;
  // X along d (rows); Wg, Wu [E][d][f] along d -> [E][f][d]; Wd [E][f][d] along f -> [E][d][f]
  if (!x_mx) launch_mx_rows(a.x, bf, a.R, a.d, b.x.q, b.x.s, s, true);
  if (wcache) {
    Carve cc{const_cast<char*>(wcache)};
    const WCache w = carve_wcache(cc, a.E, a.d, a.f);
    m.wgq = w.wg_f.q; m.wgs = w.wg_f.s; m.wuq = w.wu_f.q; m.wus = w.wu_f.s; m.wdq = w.wd_f.q; m.wds = w.wd_f.s;
  } else {
    launch_mx_cols(a.wg, bf, a.E, a.d, a.f, nullptr, 0, a.d, b.wg.q, b.wg.s, s, true, nullptr);
    launch_mx_cols(a.wu, bf, a.E, a.d, a.f, nullptr, 0, a.d, b.wu.q, b.wu.s, s, true, nullptr);
    launch_mx_cols(a.wd, bf, a.E, a.f, a.d, nullptr, 0, a.f, b.wd.q, b.wd.s, s, true, nullptr);
    m.wgq = b.wg.q; m.wgs = b.wg.s; m.wuq = b.wu.q; m.wus = b.wu.s; m.wdq = b.wd.q; m.wds = b.wd.s;
  }
  m.xq = x_mx ? x_mx : b.x.q;
  m.xs = x_mx ? x_mx + align_up(static_cast<size_t>(a.R) * a.d, 256) : b.x.s;
  // A along f for G2: encoded by G1's epilogue on 256 x 256 tiles, else by the quantiser from the stored A
  m.oaq = b.a.q; m.oas = b.a.s;
  int st = launch_mx_kind(kG1, m, max_tiles, s);
  if (st != MOE_OK) return st;
  if (ffn_mx_bm(a.R, a.E) != MxBig::BM) launch_mx_rows(a.o_act, bf, a.R, a.f, b.a.q, b.a.s, s, true);
  m.aq = b.a.q; m.as = b.a.s;
  return launch_mx_kind(kG2, m, max_tiles, s);
}

int mx_ffn_bwd(const FfnArgs& a, int64_t max_tiles, const int32_t* mx_blk_offsets, const char* wcache,
               const uint8_t* dy_mx, const uint8_t* x_mxt, const uint8_t* dy_mxt, char* scratch, hipStream_t s) {
  Carve c{scratch};
  const BwdBufs b = carve_bwd(c, a.R, a.E, a.d, a.f);
  const int bf = MOE_BF16;
  const int64_t rp = token_pad(a.R, a.E);
  MxArgs m{};
  m.f = a;
  m.blk = mx_blk_offsets;
  m.ldt = rp;
  int st = MOE_OK;
  if (a.R > 0) {
    // weights in the backward orientation: natural layouts, blocks along the last axis
    if (wcache) {
      Carve cc{const_cast<char*>(wcache)};
      const WCache w = carve_wcache(cc, a.E, a.d, a.f);
      m.wdq = w.wd_b.q; m.wds = w.wd_b.s; m.wgq = w.wg_b.q; m.wgs = w.wg_b.s; m.wuq = w.wu_b.q; m.wus = w.wu_b.s;
    } else {
      launch_mx_rows(a.wd, bf, static_cast<int64_t>(a.E) * a.f, a.d, b.wd.q, b.wd.s, s, true);
      m.wdq = b.wd.q; m.wds = b.wd.s;
    }
    // G3: dA = dY Wd^T: dY along d, Wd natural [E][f][d] along d
    if (!dy_mx) launch_mx_rows(a.dy, bf, a.R, a.d, b.dy.q, b.dy.s, s, true);
    m.dyq = dy_mx ? dy_mx : b.dy.q;
    m.dys = dy_mx ? dy_mx + align_up(static_cast<size_t>(a.R) * a.d, 256) : b.dy.s;
    st = launch_mx_kind(kG3, m, max_tiles, s);
    if (st != MOE_OK) return st;
    // G5: dX = dHg Wg^T + dHu Wu^T: dH along f, Wg/Wu natural [E][d][f] along f; from the same read dH along
    // the tokens of each expert segment for the weight gradient G6
    const uint16_t* dhg = static_cast<const uint16_t*>(a.dhg);
    const uint16_t* dhu = static_cast<const uint16_t*>(a.dhu);
    launch_mx_gather(dhg, a.R, a.f, 1, nullptr, nullptr, a.offsets, mx_blk_offsets, a.E, nullptr, b.dhg.q, b.dhg.s,
                     b.dhgt.q, b.dhgt.s, s);
    launch_mx_gather(dhu, a.R, a.f, 1, nullptr, nullptr, a.offsets, mx_blk_offsets, a.E, nullptr, b.dhu.q, b.dhu.s,
                     b.dhut.q, b.dhut.s, s);
    if (!wcache) {
      launch_mx_rows(a.wg, bf, static_cast<int64_t>(a.E) * a.d, a.f, b.wg.q, b.wg.s, s, true);
      launch_mx_rows(a.wu, bf, static_cast<int64_t>(a.E) * a.d, a.f, b.wu.q, b.wu.s, s, true);
      m.wgq = b.wg.q; m.wgs = b.wg.s; m.wuq = b.wu.q; m.wus = b.wu.s;
    }
    m.dhgq = b.dhg.q; m.dhgs = b.dhg.s; m.dhuq = b.dhu.q; m.dhus = b.dhu.s;
    st = launch_mx_kind(kG5, m, max_tiles, s);
    if (st != MOE_OK) return st;
    // weight gradients: every operand along tokens, per expert segment, transposed
    launch_mx_cols(a.act, bf, 1, a.R, a.f, a.offsets, a.E, rp, b.at.q, b.at.s, s, true, mx_blk_offsets);
    if (!dy_mxt) launch_mx_cols(a.dy, bf, 1, a.R, a.d, a.offsets, a.E, rp, b.dyt.q, b.dyt.s, s, true, mx_blk_offsets);
    if (!x_mxt) launch_mx_cols(a.x, bf, 1, a.R, a.d, a.offsets, a.E, rp, b.xt.q, b.xt.s, s, true, mx_blk_offsets);
  }
  const size_t tcodes = align_up(static_cast<size_t>(a.d) * rp, 256);  // token-axis codes of a d-wide operand
  m.atq = b.at.q; m.ats = b.at.s;
  m.dytq = dy_mxt ? dy_mxt : b.dyt.q;
  m.dyts = dy_mxt ? dy_mxt + tcodes : b.dyt.s;
  m.xtq = x_mxt ? x_mxt : b.xt.q;
  m.xts = x_mxt ? x_mxt + tcodes : b.xt.s;
  m.dhgtq = b.dhgt.q; m.dhgts = b.dhgt.s; m.dhutq = b.dhut.q; m.dhuts = b.dhut.s;
  st = launch_mx_kind(kG4, m, max_tiles, s);
  if (st == MOE_OK) st = launch_mx_kind(kG6, m, max_tiles, s);
  return st;
}

}  // namespace moe
