// BF16 grouped expert-FFN GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Operand tiles move from global memory straight into LDS with the gfx950
// 16-byte LDS-DMA buffer loads (buffer_load_dwordx4 ... lds): no register
// staging, and an LDS ring per operand keeps K-steps in flight while one is
// consumed, with one barrier per K-step.  Buffer range checks supply the zeros
// of ragged row tiles and of the token-axis tail of the weight gradients, so
// the loads carry no predicates.
//
// Every operand keeps its memory layout in LDS, with 16-byte chunks XOR-
// swizzled by row so that the fragment reads are free of bank conflicts:
// K-contiguous operands (activation rows, the weights of the dgrad GEMMs) are
// read as 16-byte fragments; operands contiguous along M or N (the weights of
// the forward GEMMs, both operands of the weight-gradient GEMMs, whose K is the
// token axis) are read with the transposing LDS read ds_read_b64_tr_b16, two
// per fragment.
//
// Tile shapes: 256 x 256 outputs per workgroup (8 waves of 128 x 64) for long
// expert segments and the weight gradients, on a persistent grid with the
// epilogue straight from registers (or through the ring slot the last K-step
// released) while the next tile's first loads are in flight; otherwise 128-row
// tiles, 128 x 256 (8 waves of 64 x 64, K step 32) for the forward GEMMs and
// 128 x 128 (4 waves of 64 x 64) for the backward ones, two workgroups per CU
// so that one's LDS-staged epilogue overlaps the other's main loop.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies A[m = l % 32][k = 8(l/32) .. +7]
// and B[k = 8(l/32) .. +7][n = l % 32]; accumulator register r of lane l holds
// C[8(r/4) + 4(l/32) + r%4][l % 32].
#include <type_traits>

#include "gemm_common.hpp"


namespace moe {
namespace {
using namespace gemm;

constexpr int kNoSplit = 0x7FFFFFFF;

// Tile configuration: BM x BN outputs, WM x WN waves, K-step BK, LDS ring of
// NA stages for the A tile and NB stages for the B tile (equal, or 3 and 2).
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NA_, int NB_, int SPREAD_, bool REGEPI_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NA = NA_, NB = NB_;
  // equal rings: 0 issues a K-step's loads right after the barrier; 1 spreads
  // them over the step's first two 16-deep MFMA slices (A, then B); 2 over all four
  static constexpr int kSpread = SPREAD_;
  // epilogue: straight from registers (tiles computed transposed, the next
  // tile's first steps in flight meanwhile), or staged through LDS as bf16 for
  // 16-byte streaming stores of whole rows (the two-workgroup-per-CU tiles,
  // where the other workgroup's main loop overlaps it)
  static constexpr bool kRegEpi = REGEPI_;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int kA = BM * BK, kB = BN * BK;  // elements per stage
  static constexpr int kBOff = NA * kA;              // the B ring follows the A ring
  // resident waves per SIMD the register allocation must allow: two
  // workgroups per compute unit for the 128-row tiles, one for 256 x 256
  static constexpr int kWavesPerSimd = (BM == 128 ? 2 : 1) * kWaves / 4;
  // LDS-staged epilogue tiles: G1 two BM x (BN/2 + 8), the others BM x (BN + 8)
  static constexpr int kEpi = REGEPI_ ? 0 : cmax(2 * BM * (BN / 2 + 8), BM * (BN + 8));
  static constexpr int kLds = cmax(NA * kA + NB * kB, kEpi);  // elements (bf16)
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(NA >= 2 && NB >= 2 && (NA == NB ? NA <= 5 : NA + NB == 5), "LDS ring depths: equal, or 3 and 2");
  static_assert(kLds * 2 <= 160 * 1024, "LDS budget");
  static_assert(SPREAD_ == 0 || (NA == NB && BK / 16 >= 2 * SPREAD_), "spread loads need equal rings and the slices");
};
// 256 x 256, 8 waves of 128 x 64, K step 64, two stages per operand, each
// step's loads issued over the first two MFMA slices
using Big = Cfg<256, 256, 2, 4, 64, 2, 2, 1, true>;
// 128 x 128, 4 waves of 64 x 64, K step 64, three A stages (two workgroups per CU)
using Small = Cfg<128, 128, 2, 2, 64, 3, 2, 0, false>;
// 128 x 256, 8 waves of 64 x 64, K step 32: two workgroups per CU (short segments, forward GEMMs)
using Mid = Cfg<128, 256, 2, 4, 32, 3, 2, 0, false>;

// K-contiguous operand: element (mn, k) at m0[mn*ld + k] for k < ksplit, else
// m1[mn*ld + k - ksplit]; rows mn >= mn_valid read as zero.
struct KcOp {
  const uint16_t* m0;
  const uint16_t* m1;
  int64_t ld;
  int ksplit;
  int mn_valid;
};

// M/N-contiguous operand: element (mn, k) at m0[k*ld + c0 + mn]; k >= k_valid
// reads as zero.  Dual: tile columns [0, W/2) come from m0 and [W/2, W) from
// m1, both at column c0 + (mn mod W/2).
struct McOp {
  const uint16_t* m0;
  const uint16_t* m1;
  int64_t ld;
  int c0;
  int k_valid;
};

// 16-byte chunk swizzles.  K-contiguous tile rows hold BK elements; a fragment
// read has 16 lanes on 16 consecutive rows at one chunk.  M/N-contiguous tile
// rows (one k each) hold RS elements; a transposing read has 32 lanes on 4
// consecutive k-rows x 4 consecutive chunks.
template <int BK>
__device__ __forceinline__ int kc_swz(int row) {
  return BK == 64 ? (row >> 1) & 7 : (row >> 2) & 3;
}
template <int RS>
__device__ __forceinline__ int mc_swz(int k) {
  static_assert(RS >= 64, "M/N-contiguous tile rows of at least 64 elements");
  return RS >= 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

// Issue the LDS-DMA loads of a ROWS x BK K-contiguous tile (K-step at k0).
// Loads u in [U0, U1) of this wave's share (U1 < 0: all).
template <class C, int ROWS, int U0 = 0, int U1 = -1>
__device__ __forceinline__ void dma_kc(const KcOp& op, int k0, uint16_t* dst, int wave, int lane) {
  constexpr int CPR = C::BK / 8;          // chunks per row
  constexpr int RPI = 64 / CPR;           // rows per instruction (1 KB)
  constexpr int NI = ROWS / RPI;
  static_assert(NI % C::kWaves == 0, "K-contiguous tile does not split over the waves");
  const bool hi = k0 >= op.ksplit;
  const uint16_t* m = hi ? op.m1 : op.m0;
  const int kk = hi ? k0 - op.ksplit : k0;
  const int rows = op.mn_valid < ROWS ? op.mn_valid : ROWS;
  const __amdgpu_buffer_rsrc_t r = rsrc(m, static_cast<int64_t>(rows) * op.ld * 2);
  const int rl = lane / CPR, ph = lane % CPR;
  constexpr int UE = U1 < 0 ? NI / C::kWaves : U1;
#pragma unroll
  for (int u = U0; u < UE; ++u) {
    const int i = wave + u * C::kWaves;
    const int row = i * RPI + rl;
    const int lc = ph ^ kc_swz<C::BK>(row);
    dma16(r, dst + i * 512, static_cast<int>((row * op.ld + kk + lc * 8) * 2));
  }
}

// Issue the LDS-DMA loads of a BK x ROWS M/N-contiguous tile, as NSUB
// sub-tiles of BK x ROWS/NSUB (dual: one per matrix).
template <class C, int ROWS, int NSUB, int U0 = 0, int U1 = -1>
__device__ __forceinline__ void dma_mc(const McOp& op, int k0, uint16_t* dst, int wave, int lane) {
  constexpr int RS = ROWS / NSUB;
  constexpr int CPR = RS / 8;             // chunks per k-row
  constexpr int KPI = 64 / CPR;           // k-rows per instruction (1 KB)
  constexpr int NIS = C::BK / KPI;        // instructions per sub-tile
  constexpr int NI = NIS * NSUB;
  static_assert(KPI >= 1 && C::BK % KPI == 0 && NI % C::kWaves == 0, "M/N-contiguous tile split");
  int kv = op.k_valid - k0;
  kv = kv < 0 ? 0 : (kv > C::BK ? C::BK : kv);
  const int kl = lane / CPR, ph = lane % CPR;
  constexpr int UE = U1 < 0 ? NI / C::kWaves : U1;
#pragma unroll
  for (int u = U0; u < UE; ++u) {
    const int i = wave + u * C::kWaves;
    const int sub = i / NIS, ii = i % NIS;
    const uint16_t* m = (NSUB == 2 && sub == 1 ? op.m1 : op.m0) + k0 * op.ld;
    const __amdgpu_buffer_rsrc_t r = rsrc(m, static_cast<int64_t>(kv) * op.ld * 2);
    const int kr = ii * KPI + kl;
    const int lc = ph ^ mc_swz<RS>(kr);
    dma16(r, dst + sub * (C::BK * RS) + ii * 512, static_cast<int>((kr * op.ld + op.c0 + lc * 8) * 2));
  }
}

// MFMA fragment from a K-contiguous tile: rows base .. base+31, k-slice ks.
template <class C>
__device__ __forceinline__ bf16x8 frag_kc(const uint16_t* t, int base, int ks, int lane) {
  const int row = base + (lane & 31);
  const int ph = (ks * 2 + (lane >> 5)) ^ kc_swz<C::BK>(row);
  return *reinterpret_cast<const bf16x8*>(t + row * C::BK + ph * 8);
}

// MFMA fragment from an M/N-contiguous (sub-)tile of RS columns: columns
// col .. col+31, k-slice ks.  Two transposing reads: within each 16-lane
// group G, lane i gets slot s from element i%4 of the address of lane 4s + i/4;
// lane L points at k-row 16 ks + 8(G/2) + 4 half + L/4, columns col + 16(G%2) + 4(L%4).
template <class C, int RS>
__device__ __forceinline__ bf16x8 frag_mc(const uint16_t* t, int col, int ks, int lane) {
  const int G = lane >> 4, L = lane & 15;
  const int k = ks * 16 + 8 * (G >> 1) + (L >> 2);
  const int c = col + 16 * (G & 1) + 4 * (L & 3);
  const int ph = (c >> 3) ^ mc_swz<RS>(k);  // same swizzle for k + 4
  const uint16_t* p = t + k * RS + ph * 8 + (c & 7);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * RS));
  bf16x8 r;
  short tmp[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  __builtin_memcpy(&r, tmp, 16);
  return r;
}

template <bool KC>
struct OpFor;
template <>
struct OpFor<true> {
  using T = KcOp;
};
template <>
struct OpFor<false> {
  using T = McOp;
};

template <class C, bool AKC, bool BKC, bool BDUAL>
__device__ __forceinline__ bf16x8 frag_b(const uint16_t* Bs, int wn, int j, int ks, int lane) {
  if constexpr (BKC) {
    return frag_kc<C>(Bs, wn * C::WTN + j * 32, ks, lane);
  } else if constexpr (BDUAL) {
    // gate fragments j < TN/2, up fragments j >= TN/2, each matrix a BN/2-wide sub-tile
    constexpr int H = C::TN / 2;
    const int sub = j >= H ? 1 : 0;
    return frag_mc<C, C::BN / 2>(Bs + sub * (C::BK * C::BN / 2), wn * (C::WTN / 2) + (j - sub * H) * 32, ks, lane);
  } else {
    return frag_mc<C, C::BN>(Bs, wn * C::WTN + j * 32, ks, lane);
  }
}

template <class C, bool AKC, bool BKC, bool BDUAL>
__device__ __forceinline__ void load_frags(const uint16_t* As, const uint16_t* Bs, int wm, int wn, int ks, int lane,
                                           bf16x8* a, bf16x8* b) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    a[i] = AKC ? frag_kc<C>(As, wm * C::WTM + i * 32, ks, lane) : frag_mc<C, C::BM>(As, wm * C::WTM + i * 32, ks, lane);
#pragma unroll
  for (int j = 0; j < C::TN; ++j) b[j] = frag_b<C, AKC, BKC, BDUAL>(Bs, wn, j, ks, lane);
}

// One K-step.  With register-direct epilogues each 32 x 32 tile is computed
// transposed (B fragment in the MFMA's first operand slot), which leaves four
// consecutive output columns of one row in each lane.
template <class C, bool AKC, bool BKC, bool BDUAL, class Hook>
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, int wm,
                                          int wn, int lane, Acc<C>& acc, Hook&& hook) {
#pragma unroll
  for (int ks = 0; ks < C::BK / 16; ++ks) {
    hook(ks);
    bf16x8 a[C::TM], b[C::TN];
    load_frags<C, AKC, BKC, BDUAL>(As, Bs, wm, wn, ks, lane, a, b);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = C::kRegEpi ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// One output tile: its operands, K, and where its outputs go.  All fields are
// workgroup-uniform.
struct Tile {
  KcOp ka, kb;      // K-contiguous operands (the kinds that use them)
  McOp ma, mb;      // M/N-contiguous operands
  int K;            // contraction length (0: no loads, zero outputs)
  int rows, cols;   // valid output rows / columns from the tile origin
  int64_t row0;     // rows-by-expert GEMMs: first row of the tile
  int n0;           // first output column (over f for G1 and G3)
  uint16_t* out;    // plain-store GEMMs: output tile origin
  int64_t ldo;      // and its row stride
};

// Tile of hardware id h (rows-by-expert GEMMs: XCD-contiguous ranges over the
// `live` table entries times the N tiles; weight gradients: wgrad_tile_sorted).
// False once h is past the last tile; for a fixed h mod 8 that holds for every
// larger h too, so a workgroup stepping h by the grid size stops there.
template <class C, int KIND>
__device__ __forceinline__ bool make_tile(const FfnArgs& p, int64_t h, int64_t live, Tile& t) {
  const int d = p.d, f = p.f;
  const int64_t wsz = static_cast<int64_t>(d) * f;
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* Wg = static_cast<const uint16_t*>(p.wg);
  const uint16_t* Wu = static_cast<const uint16_t*>(p.wu);
  const uint16_t* Wd = static_cast<const uint16_t*>(p.wd);
  if constexpr (KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5) {
    // logical tile = (row tile, N tile) in the expert column-major order (expert_tile)
    const int gx = KIND == kG1 ? (f + C::BN / 2 - 1) / (C::BN / 2)
                               : KIND == kG3 ? (f + C::BN - 1) / C::BN : (d + C::BN - 1) / C::BN;
    const int64_t lid = xcd_tile(h, live * gx);
    if (lid < 0) return false;
    int nt;
    const int4 tt = p.tiles[expert_tile(lid, gx, p.tiles, p.max_tiles, nt)];
    // tile-table values are workgroup-uniform: keep them (and the buffer
    // descriptors built from them) in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(tt.x);
    const int rows = e < 0 ? 0 : __builtin_amdgcn_readfirstlane(tt.z);
    const int64_t row0 = e < 0 ? 0 : __builtin_amdgcn_readfirstlane(tt.y);
    const int64_t eo = e < 0 ? 0 : static_cast<int64_t>(e) * wsz;
    t.row0 = row0;
    t.rows = rows;
    if constexpr (KIND == kG1) {
      t.n0 = nt * (C::BN / 2);
      t.ka = KcOp{X + row0 * d, nullptr, d, kNoSplit, rows};
      t.mb = McOp{Wg + eo, Wu + eo, f, t.n0, d};
      t.K = d;
      t.cols = f - t.n0;
    } else if constexpr (KIND == kG2) {
      t.n0 = nt * C::BN;
      t.ka = KcOp{static_cast<const uint16_t*>(p.act) + row0 * f, nullptr, f, kNoSplit, rows};
      t.mb = McOp{Wd + eo, nullptr, d, t.n0, f};
      t.K = f;
      t.cols = d - t.n0;
      t.out = static_cast<uint16_t*>(p.o_y) + row0 * d + t.n0;
      t.ldo = d;
    } else if constexpr (KIND == kG3) {
      t.n0 = nt * C::BN;  // over f
      t.ka = KcOp{static_cast<const uint16_t*>(p.dy) + row0 * d, nullptr, d, kNoSplit, rows};
      t.kb = KcOp{Wd + eo + static_cast<int64_t>(t.n0) * d, nullptr, d, kNoSplit, f - t.n0};
      t.K = d;
      t.cols = f - t.n0;
    } else {  // kG5
      t.n0 = nt * C::BN;  // over d
      t.ka = KcOp{static_cast<const uint16_t*>(p.dhg) + row0 * f, static_cast<const uint16_t*>(p.dhu) + row0 * f, f,
                  f, rows};
      t.kb = KcOp{Wg + eo + static_cast<int64_t>(t.n0) * f, Wu + eo + static_cast<int64_t>(t.n0) * f, f, f, d - t.n0};
      t.K = 2 * f;
      t.cols = d - t.n0;
      t.out = static_cast<uint16_t*>(p.o_dx) + row0 * d + t.n0;
      t.ldo = d;
    }
    if (rows == 0) t.K = 0;
  } else {  // weight gradients: K = rows of expert e
    // logical tile = (expert, M tile, N tile), blocks of tiles sharing operand
    // slices kept on one XCD, an expert's blocks spread over all XCDs
    const int gm = KIND == kG4 ? (f + C::BM - 1) / C::BM : (d + C::BM - 1) / C::BM;
    const int gn = KIND == kG4 ? (d + C::BN - 1) / C::BN : 2 * ((f + C::BN - 1) / C::BN);
    int e, local;
    if (!wgrad_tile_sorted(h, p.E, gm * gn, p.wsched, e, local)) return false;
    const int mt = local / gn, ntile = local % gn;
    e = __builtin_amdgcn_readfirstlane(e);
    const int64_t seg0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
    const int K = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]) - static_cast<int>(seg0);
    const int m0 = __builtin_amdgcn_readfirstlane(mt * C::BM);
    t.K = K;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      t.n0 = __builtin_amdgcn_readfirstlane(ntile * C::BN);
      t.ma = McOp{static_cast<const uint16_t*>(p.act) + seg0 * f, nullptr, f, m0, K};
      t.mb = McOp{static_cast<const uint16_t*>(p.dy) + seg0 * d, nullptr, d, t.n0, K};
      t.out = static_cast<uint16_t*>(p.o_dwd) + e * wsz + static_cast<int64_t>(m0) * d + t.n0;
      t.ldo = d;
      t.rows = f - m0;
      t.cols = d - t.n0;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + C::BN - 1) / C::BN;
      const int which = __builtin_amdgcn_readfirstlane(ntile / per);
      t.n0 = __builtin_amdgcn_readfirstlane((ntile % per) * C::BN);
      t.ma = McOp{X + seg0 * d, nullptr, d, m0, K};
      t.mb = McOp{static_cast<const uint16_t*>(which ? p.dhu : p.dhg) + seg0 * f, nullptr, f, t.n0, K};
      t.out = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz + static_cast<int64_t>(m0) * f + t.n0;
      t.ldo = f;
      t.rows = d - m0;
      t.cols = f - t.n0;
    }
  }
  return true;
}

// Persistent grid (workgroups loop over tiles) or one workgroup per tile; see
// launch_kind.
template <class C, int KIND>
constexpr bool persistent() {
  return C::kRegEpi && KIND != kG4 && KIND != kG6;
}

// Wait until at most `steps` K-steps of loads (n loads each) are outstanding.
template <int N, int MAXS>
__device__ __forceinline__ void wait_steps(int steps) {
  static_assert(N * MAXS < 16, "vmcnt immediate");
  if constexpr (MAXS >= 3) {
    if (steps >= 3) { wait_vm<3 * N>(); return; }
  }
  if constexpr (MAXS >= 2) {
    if (steps == 2) { wait_vm<2 * N>(); return; }
  }
  if constexpr (MAXS >= 1) {
    if (steps == 1) { wait_vm<N>(); return; }
  }
  wait_vm<0>();
}

// Grouped GEMM over tiles: workgroup b takes hardware tile ids b, b + G,
// b + 2G, ... (G = grid size, a multiple of 8, so every id of one workgroup
// maps to the same XCD); with one workgroup per tile the loop runs once.  The
// K-steps of consecutive tiles form one stream through the LDS rings (ring
// position g counts steps across tiles).
//
// Register-direct epilogues (256 x 256 tiles, persistent grid): at the last
// K-step of a tile, right after the barrier that frees their slots, the first
// steps of the next tile are issued, so their loads are in flight during the
// epilogue.  That epilogue uses at most the other ring slot, which the last
// step has just released: G3 stages its Hg, Hu loads there (g3_stage; the next
// tile's loads then wait for the epilogue), G4, G5, G6 stage their rows for
// streaming stores, G1 and G2 store straight from registers.  LDS-staged
// epilogues (128-row tiles) take the whole LDS between two barriers.
//
// Rings of equal depth N: right after the barrier of step kt, step kt + N - 1
// of both operands is issued (at kt = 0 first the leading steps not issued
// yet), so step kt + 1 waits with the loads of steps kt + 2 .. kt + N - 2 still
// outstanding.  Rings of depths 3 and 2: a tile's first loads are step 0 of
// both operands and step 1 of the 3-deep one; after the barrier of step kt the
// 2-deep operand's step kt + 1 and then the 3-deep operand's step kt + 2 are
// issued, so step kt + 1 waits with only the 3-deep operand's step kt + 2
// outstanding.  Step 0 of a tile that follows an epilogue of the same
// workgroup waits for everything outstanding (that epilogue's stores included).
template <class C, int KIND>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::kWavesPerSimd)))
void ffn_bf16_kernel(FfnArgs p) {
  constexpr bool MG = KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5;
  constexpr bool AKC = MG, BKC = KIND == kG3 || KIND == kG5, BDUAL = KIND == kG1;
  constexpr bool kEven = C::NA == C::NB;
  constexpr int N = C::NA;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t live = MG ? __builtin_amdgcn_readfirstlane(p.tiles[p.max_tiles].x) : 0;
  const int64_t G = gridDim.x;
  int64_t h = blockIdx.x;
  Tile cur, nxt;
  if (!make_tile<C, KIND>(p, h, live, cur)) return;

  constexpr int kLA = (C::BM * C::BK * 2 / 1024) / C::kWaves;  // LDS-DMA instructions per wave per step
  constexpr int kLB = (C::BN * C::BK * 2 / 1024) / C::kWaves;
  constexpr int kAhead = C::NA == 3 ? kLA : (C::NB == 3 ? kLB : 0);
  auto issue_a = [&](const Tile& t, int kt, int pos) {
    uint16_t* st = lds + (pos % C::NA) * C::kA;
    if constexpr (AKC) dma_kc<C, C::BM>(t.ka, kt * C::BK, st, wave, lane);
    else dma_mc<C, C::BM, 1>(t.ma, kt * C::BK, st, wave, lane);
  };
  auto issue_b = [&](const Tile& t, int kt, int pos) {
    uint16_t* st = lds + C::kBOff + (pos % C::NB) * C::kB;
    if constexpr (BKC) dma_kc<C, C::BN>(t.kb, kt * C::BK, st, wave, lane);
    else dma_mc<C, C::BN, BDUAL ? 2 : 1>(t.mb, kt * C::BK, st, wave, lane);
  };
  // parts [U0, U1) of one step's loads
  auto part_a = [&](const Tile& t, int kt, int pos, auto u0, auto u1) {
    uint16_t* st = lds + (pos % C::NA) * C::kA;
    constexpr int U0 = decltype(u0)::value, U1 = decltype(u1)::value;
    if constexpr (AKC) dma_kc<C, C::BM, U0, U1>(t.ka, kt * C::BK, st, wave, lane);
    else dma_mc<C, C::BM, 1, U0, U1>(t.ma, kt * C::BK, st, wave, lane);
  };
  auto part_b = [&](const Tile& t, int kt, int pos, auto u0, auto u1) {
    uint16_t* st = lds + C::kBOff + (pos % C::NB) * C::kB;
    constexpr int U0 = decltype(u0)::value, U1 = decltype(u1)::value;
    if constexpr (BKC) dma_kc<C, C::BN, U0, U1>(t.kb, kt * C::BK, st, wave, lane);
    else dma_mc<C, C::BN, BDUAL ? 2 : 1, U0, U1>(t.mb, kt * C::BK, st, wave, lane);
  };
  using I0 = std::integral_constant<int, 0>;
  using IHA = std::integral_constant<int, kLA / 2>;
  using IA = std::integral_constant<int, kLA>;
  using IHB = std::integral_constant<int, kLB / 2>;
  using IB = std::integral_constant<int, kLB>;
  // steps issued ahead of a tile: N - 1 with even rings, else 1
  constexpr int kPre = kEven ? N - 1 : 1;
  // G3 on 2-deep equal rings: Hg, Hu staged through the rings' LDS (g3_stage);
  // stage_buf(s) is this wave's 8 KB in ring slot s
  constexpr bool kStaged = C::kRegEpi && KIND == kG3 && kEven && N == 2 && C::kWaves == 8 && C::TM == 4;
  // G4, G5, G6 on the same tiles: streaming stores of whole rows through the
  // idle ring slot (epi_staged_store); G2's Y keeps cached register-direct stores
  constexpr bool kStagedStore = C::kRegEpi && (KIND == kG4 || KIND == kG5 || KIND == kG6) && kEven && N == 2 &&
                                C::kWaves == 8 && C::TM == 4;
  auto stage_buf = [&](int slot) -> uint16_t* {
    return wave < 4 ? lds + slot * C::kA + wave * 4096 : lds + C::kBOff + slot * C::kB + (wave - 4) * 4096;
  };

  int g = 0;    // ring position of the current tile's step 0
  int pre = 0;  // leading steps of the current tile already issued
  for (;;) {
    const bool more = persistent<C, KIND>() && make_tile<C, KIND>(p, h + G, live, nxt);
    const int nk = (cur.K + C::BK - 1) / C::BK;
    if (pre == 0 && nk > 0) {
      issue_a(cur, 0, g);
      issue_b(cur, 0, g);
      pre = 1;
      if constexpr (!kEven) {  // and the 3-deep operand's step 1
        if (1 < nk) {
          if constexpr (C::NA == 3) issue_a(cur, 1, g + 1);
          else issue_b(cur, 1, g + 1);
          pre = 2;
        }
      }
    }
    Acc<C> acc;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      if constexpr (kEven) {
        if (kt == 0) wait_vm<0>();
        else {
          const int ahead = nk - 1 - kt < N - 2 ? nk - 1 - kt : N - 2;
          wait_steps<kLA + kLB, N - 2>(ahead);
        }
      } else {
        // step 0 of a workgroup's first tile leaves the 3-deep operand's step 1
        // outstanding; after an epilogue, whose stores are outstanding too, it
        // waits for everything
        if (kt + 1 >= nk || (kt == 0 && h != blockIdx.x)) wait_vm<0>();
        else wait_vm<kAhead>();
      }
      __syncthreads();
      if constexpr (kEven) {
        if (kt == 0)
          for (int s = pre; s <= N - 2 && s < nk; ++s) {
            issue_a(cur, s, g + s);
            issue_b(cur, s, g + s);
          }
        if (C::kSpread == 0 && kt + N - 1 < nk) {
          issue_a(cur, kt + N - 1, g + kt + N - 1);
          issue_b(cur, kt + N - 1, g + kt + N - 1);
        }
      } else if constexpr (C::NA == 3) {
        if (kt + 1 < nk) issue_b(cur, kt + 1, g + kt + 1);
        if (kt == 0 && 1 < nk && pre < 2) issue_a(cur, 1, g + 1);
        if (kt + 2 < nk) issue_a(cur, kt + 2, g + kt + 2);
      } else {  // NB == 3
        if (kt + 1 < nk) issue_a(cur, kt + 1, g + kt + 1);
        if (kt == 0 && 1 < nk && pre < 2) issue_b(cur, 1, g + 1);
        if (kt + 2 < nk) issue_b(cur, kt + 2, g + kt + 2);
      }
      if (kStaged && kt + 1 == nk) g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 0, stage_buf((g + nk) % 2), wm, wn, lane);
      if (C::kRegEpi && !kStaged && kt + 1 == nk && more) {
        const int nk2 = (nxt.K + C::BK - 1) / C::BK;
        for (int s = 0; s < kPre && s < nk2; ++s) {
          issue_a(nxt, s, g + nk + s);
          issue_b(nxt, s, g + nk + s);
        }
      }
      const bool spread = kEven && C::kSpread != 0 && kt + N - 1 < nk;
      const int ks_ = kt + N - 1, ps_ = g + kt + N - 1;
      mma_stage<C, AKC, BKC, BDUAL>(lds + ((g + kt) % C::NA) * C::kA, lds + C::kBOff + ((g + kt) % C::NB) * C::kB,
                                    wm, wn, lane, acc, [&](int ks) {
                                      if constexpr (C::kSpread == 1) {
                                        if (spread && ks == 0) part_a(cur, ks_, ps_, I0{}, IA{});
                                        if (spread && ks == 1) part_b(cur, ks_, ps_, I0{}, IB{});
                                      } else if constexpr (C::kSpread == 2) {
                                        if (spread && ks == 0) part_a(cur, ks_, ps_, I0{}, IHA{});
                                        if (spread && ks == 1) part_a(cur, ks_, ps_, IHA{}, IA{});
                                        if (spread && ks == 2) part_b(cur, ks_, ps_, I0{}, IHB{});
                                        if (spread && ks == 3) part_b(cur, ks_, ps_, IHB{}, IB{});
                                      }
                                    });
    }
    if (C::kRegEpi && !kStaged && nk > 0 && more) {
      const int nk2 = (nxt.K + C::BK - 1) / C::BK;
      pre = nk2 < kPre ? nk2 : kPre;
    } else {
      pre = 0;
    }
    g += nk;
    if constexpr (kStaged) {
      // blocks 0, 1 in the two buffers, then 2, 3; block 0 was issued at the last K-step
      if (nk > 0) {
        uint16_t* b0 = stage_buf(g % 2);
        uint16_t* b1 = stage_buf((g + 1) % 2);
        __syncthreads();  // the last step's slot is free
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 1, b1, wm, wn, lane);
        wait_vm<0>();
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 0, b0, wm, wn, lane);
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 1, b1, wm, wn, lane);
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 2, b0, wm, wn, lane);
        g3_stage<C>(p, cur.row0, cur.rows, cur.n0, 3, b1, wm, wn, lane);
        wait_vm<0>();
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 2, b0, wm, wn, lane);
        g3_block<C>(acc, p, cur.row0, cur.rows, cur.n0, cur.cols, 3, b1, wm, wn, lane);
        __syncthreads();  // the LDS is the ring again
      }
    } else if constexpr (!C::kRegEpi) {
      __syncthreads();  // the epilogue reuses the LDS
      if constexpr (KIND == kG1) epi_swiglu_fwd<C>(acc, lds, p, cur.row0, cur.rows, cur.n0, tid);
      else if constexpr (KIND == kG3) epi_swiglu_bwd<C>(acc, lds, p, cur.row0, cur.rows, cur.n0, tid);
      else if constexpr (KIND == kG2)  // Y is read by the combine right after: ordinary (cached) stores
        epi_store<C, false>(acc, lds, cur.out, cur.ldo, cur.rows, cur.cols, tid);
      else epi_store<C>(acc, lds, cur.out, cur.ldo, cur.rows, cur.cols, tid);
      __syncthreads();  // the LDS is the ring again
    } else if constexpr (kStagedStore) {
      if (nk > 0) __syncthreads();  // the last step's slot is free
      epi_staged_store<C, KIND != kG5>(acc, stage_buf((g + 1) % 2), cur.out, cur.ldo, cur.rows, cur.cols, lane, wm, wn);
    } else if constexpr (KIND == kG1) epi_regs_swiglu_fwd<C>(acc, p, cur.row0, cur.rows, cur.n0, lane, wm, wn);
    else if constexpr (KIND == kG3) epi_regs_swiglu_bwd<C>(acc, p, cur.row0, cur.rows, cur.n0, lane, wm, wn);
    else epi_regs_store<C>(acc, cur.out, cur.ldo, cur.rows, cur.cols, lane, wm, wn);
    if (!more) break;
    cur = nxt;
    h += G;
  }
}

// Launch kind KIND over at most `tiles` tiles (a host-known bound).  The
// rows-by-expert GEMMs with register-direct epilogues run on a persistent grid
// (as many workgroups as can be resident at once, each looping over tiles of
// equal cost with the next tile's loads in flight during an epilogue).  The
// others get one workgroup per tile, so that the hardware hands out tiles as
// compute units free up: weight-gradient tiles cost as much as their expert's
// row count, which routing can make very uneven.
template <class C, int KIND>
void launch_kind(const char* name, const FfnArgs& a, int64_t tiles, hipStream_t s) {
  unsigned grid = xcd_grid(tiles);
  if constexpr (persistent<C, KIND>()) {
    static const int occ = occupancy(reinterpret_cast<const void*>(&ffn_bf16_kernel<C, KIND>), C::kThreads);
    grid = persistent_grid(occ, tiles);
  }
  MOE_LAUNCH(name, (ffn_bf16_kernel<C, KIND>), dim3(grid), dim3(C::kThreads), 0, s, a);
}

template <class C>
int launch_cfg(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t nd = cdiv(a.d, C::BN), nf = cdiv(a.f, C::BN);
  switch (kind) {
    case kG1: launch_kind<C, kG1>("G1_bf16", a, cdiv(a.f, C::BN / 2) * max_tiles, s); break;
    case kG2: launch_kind<C, kG2>("G2_bf16", a, nd * max_tiles, s); break;
    case kG3: launch_kind<C, kG3>("G3_bf16", a, nf * max_tiles, s); break;
    case kG5: launch_kind<C, kG5>("G5_bf16", a, nd * max_tiles, s); break;
    case kG4: launch_kind<C, kG4>("G4_bf16", a, wgrad_sorted_grid(a.E, static_cast<int>(cdiv(a.f, C::BM) * nd)), s); break;
    case kG6:
      launch_kind<C, kG6>("G6_bf16", a, wgrad_sorted_grid(a.E, static_cast<int>(cdiv(a.d, C::BM) * 2 * nf)), s);
      break;
    default: return MOE_EINVAL;
  }
  return launch_status();
}

// Row-tile height of the rows-by-expert GEMMs: 256 when the average expert
// segment holds at least two such tiles, else 128 (Small and Mid share it).
// (At 512 rows per expert the 256 x 256 tiles measured 6-7% faster per step:
// each expert's weights are re-read once per row tile.)
bool big_rows(int64_t R, int E) { return R >= static_cast<int64_t>(E) * 512; }
// Weight-gradient tiles: 256 x 256 when d and f fill them.
// (128 x 128 tiles for short token segments measured slower: the 256 x 256
// tile's reuse outweighs its unoverlapped epilogue.)
bool big_wgrad(const FfnArgs& a) { return a.d % 256 == 0 && a.f % 256 == 0; }

}  // namespace

int ffn_bf16_bm(int64_t R, int E) { return big_rows(R, E) ? Big::BM : Small::BM; }

int launch_ffn_bf16(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s) {
  const bool wgrad = kind == kG4 || kind == kG6;
  const bool big = wgrad ? big_wgrad(a) : a.bm == Big::BM;
  if (big) return launch_cfg<Big>(kind, a, max_tiles, s);
  // short segments: 128-row tiles; the forward GEMMs do better 256 wide at two workgroups per CU
  if (kind == kG1) launch_kind<Mid, kG1>("G1_bf16", a, cdiv(a.f, Mid::BN / 2) * max_tiles, s);
  else if (kind == kG2) launch_kind<Mid, kG2>("G2_bf16", a, cdiv(a.d, Mid::BN) * max_tiles, s);
  else return launch_cfg<Small>(kind, a, max_tiles, s);
  return launch_status();
}

}  // namespace moe
