// BF16 grouped expert-FFN GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Operand tiles move from global memory straight into LDS with the gfx950
// 16-byte LDS-DMA buffer loads (buffer_load_dwordx4 ... lds): no register
// staging, and a 2- or 3-deep LDS ring per operand keeps K-steps in flight while one is
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
// per fragment.  Tile shapes: 256 x 256 outputs per workgroup (8 waves of
// 128 x 64) for long expert segments (except the SwiGLU-backward GEMM) and the
// weight gradients; otherwise 128-row tiles: 128 x 256 (8 waves of 64 x 64, K
// step 32, two workgroups per CU) for the forward GEMMs and 128 x 128 (4 waves
// of 64 x 64, two workgroups per CU, so that one's epilogue overlaps the
// other's main loop) for the backward ones.  Epilogues go through LDS so that
// global stores (and the Hg/Hu loads of the SwiGLU backward) are 16-byte vectors.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies A[m = l % 32][k = 8(l/32) .. +7]
// and B[k = 8(l/32) .. +7][n = l % 32]; accumulator register r of lane l holds
// C[8(r/4) + 4(l/32) + r%4][l % 32].
#include "gemm_common.hpp"


namespace moe {
namespace {
using namespace gemm;

constexpr int kNoSplit = 0x7FFFFFFF;

// Tile configuration: BM x BN outputs, WM x WN waves, K-step BK, LDS ring of
// NA stages for the A tile and NB stages for the B tile (2 or 3, not both 3).
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NA_, int NB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NA = NA_, NB = NB_;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int kA = BM * BK, kB = BN * BK;  // elements per stage
  static constexpr int kBOff = NA * kA;              // the B ring follows the A ring
  // epilogue tiles: G1 two BM x (BN/2 + 8), the others BM x (BN + 8) (G3 may halve)
  static constexpr int kEpi = cmax(2 * BM * (BN / 2 + 8), BM * (BN + 8));
  static constexpr int kLds = cmax(NA * kA + NB * kB, kEpi);  // elements (bf16)
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(NA >= 2 && NA <= 3 && NB >= 2 && NB <= 3 && NA + NB <= 5, "LDS ring depth");
  static_assert(kLds * 2 <= 160 * 1024, "LDS budget");
};
// 256 x 256, 8 waves of 128 x 64, K step 64, two stages per operand
using Big = Cfg<256, 256, 2, 4, 64, 2, 2>;
// 128 x 128, 4 waves of 64 x 64, K step 64, three A stages (two workgroups per CU)
using Small = Cfg<128, 128, 2, 2, 64, 3, 2>;
// 128 x 256, 8 waves of 64 x 64, K step 32: two workgroups per CU (short segments, forward GEMMs)
using Mid = Cfg<128, 256, 2, 4, 32, 3, 2>;

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
template <class C, int ROWS>
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
#pragma unroll
  for (int u = 0; u < NI / C::kWaves; ++u) {
    const int i = wave + u * C::kWaves;
    const int row = i * RPI + rl;
    const int lc = ph ^ kc_swz<C::BK>(row);
    dma16(r, dst + i * 512, static_cast<int>((row * op.ld + kk + lc * 8) * 2));
  }
}

// Issue the LDS-DMA loads of a BK x ROWS M/N-contiguous tile, as NSUB
// sub-tiles of BK x ROWS/NSUB (dual: one per matrix).
template <class C, int ROWS, int NSUB>
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
#pragma unroll
  for (int u = 0; u < NI / C::kWaves; ++u) {
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

template <class C, bool AKC, bool BKC, bool BDUAL>
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, int wm,
                                          int wn, int lane, Acc<C>& acc) {
#pragma unroll
  for (int ks = 0; ks < C::BK / 16; ++ks) {
    bf16x8 a[C::TM], b[C::TN];
    load_frags<C, AKC, BKC, BDUAL>(As, Bs, wm, wn, ks, lane, a, b);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// C = A B over K = [0, K).  K-step kt of A lives in A slot kt % NA and of B in
// B slot kt % NB.  Right after the barrier that retires step kt - 1, step
// kt + N - 1 of each operand is issued, the 2-deep operand first; so when step
// kt + 1 is waited for, only the loads of the 3-deep operand's step kt + 2 (if
// any) were issued after the last load it needs.
template <class C, bool AKC, bool BKC, bool BDUAL>
__device__ __forceinline__ void mainloop(const typename OpFor<AKC>::T& aop, const typename OpFor<BKC>::T& bop, int K,
                                         uint16_t* lds, int tid, Acc<C>& acc) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (K + C::BK - 1) / C::BK;
  if (nk == 0) return;
  // LDS-DMA instructions per wave per K-step
  constexpr int kLA = (C::BM * C::BK * 2 / 1024) / C::kWaves;
  constexpr int kLB = (C::BN * C::BK * 2 / 1024) / C::kWaves;
  constexpr int kAhead = C::NA == 3 ? kLA : (C::NB == 3 ? kLB : 0);
  auto issue_a = [&](int kt) {
    uint16_t* st = lds + (kt % C::NA) * C::kA;
    if constexpr (AKC) dma_kc<C, C::BM>(aop, kt * C::BK, st, wave, lane);
    else dma_mc<C, C::BM, 1>(aop, kt * C::BK, st, wave, lane);
  };
  auto issue_b = [&](int kt) {
    uint16_t* st = lds + C::kBOff + (kt % C::NB) * C::kB;
    if constexpr (BKC) dma_kc<C, C::BN>(bop, kt * C::BK, st, wave, lane);
    else dma_mc<C, C::BN, BDUAL ? 2 : 1>(bop, kt * C::BK, st, wave, lane);
  };
  auto issue = [&](int ka, int kb) {  // 2-deep operand first
    if constexpr (C::NA == 3) {
      if (kb < nk) issue_b(kb);
      if (ka < nk) issue_a(ka);
    } else {
      if (ka < nk) issue_a(ka);
      if (kb < nk) issue_b(kb);
    }
  };
  issue(0, 0);
  if (C::NA == 3) issue(1, nk);
  if (C::NB == 3) issue(nk, 1);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vm<kAhead>();
    else wait_vm<0>();
    __syncthreads();
    issue(kt + C::NA - 1, kt + C::NB - 1);
    const uint16_t* as = lds + (kt % C::NA) * C::kA;
    const uint16_t* bs = lds + C::kBOff + (kt % C::NB) * C::kB;
    mma_stage<C, AKC, BKC, BDUAL>(as, bs, wm, wn, lane, acc);
  }
  __syncthreads();  // the epilogue reuses the LDS
}

template <class C, int KIND>
__global__ __launch_bounds__(C::kThreads) void ffn_bf16_kernel(FfnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int d = p.d, f = p.f;
  Acc<C> acc;

  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* Wg = static_cast<const uint16_t*>(p.wg);
  const uint16_t* Wu = static_cast<const uint16_t*>(p.wu);
  const uint16_t* Wd = static_cast<const uint16_t*>(p.wd);
  const int64_t wsz = static_cast<int64_t>(d) * f;

  if constexpr (KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5) {
    // logical tile = (row tile, N tile), N tile fastest, XCD-contiguous ranges
    const int gx = KIND == kG1 ? (f + C::BN / 2 - 1) / (C::BN / 2)
                               : KIND == kG3 ? (f + C::BN - 1) / C::BN : (d + C::BN - 1) / C::BN;
    const int64_t lid = xcd_tile(blockIdx.x, static_cast<int64_t>(p.tiles[p.max_tiles].x) * gx);
    if (lid < 0) return;
    const int4 t = p.tiles[lid / gx];
    if (t.x < 0) return;
    // tile-table values are workgroup-uniform: keep them (and the buffer
    // descriptors built from them) in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(t.x), rows = __builtin_amdgcn_readfirstlane(t.z);
    const int64_t row0 = __builtin_amdgcn_readfirstlane(t.y);
    const int nt = static_cast<int>(lid % gx);
    if constexpr (KIND == kG1) {
      const int n0 = nt * (C::BN / 2);
      const KcOp a{X + row0 * d, nullptr, d, kNoSplit, rows};
      const McOp b{Wg + e * wsz, Wu + e * wsz, f, n0, d};
      mainloop<C, true, false, true>(a, b, d, lds, tid, acc);
      epi_swiglu_fwd<C>(acc, lds, p, row0, rows, n0, tid);
    } else if constexpr (KIND == kG2) {
      const int n0 = nt * C::BN;
      const KcOp a{static_cast<const uint16_t*>(p.act) + row0 * f, nullptr, f, kNoSplit, rows};
      const McOp b{Wd + e * wsz, nullptr, d, n0, f};
      mainloop<C, true, false, false>(a, b, f, lds, tid, acc);
      // Y is read by the combine right after: ordinary (cached) stores
      epi_store<C, false>(acc, lds, static_cast<uint16_t*>(p.o_y) + row0 * d + n0, d, rows, d - n0, tid);
    } else if constexpr (KIND == kG3) {
      const int n0 = nt * C::BN;  // over f
      const KcOp a{static_cast<const uint16_t*>(p.dy) + row0 * d, nullptr, d, kNoSplit, rows};
      const KcOp b{Wd + e * wsz + static_cast<int64_t>(n0) * d, nullptr, d, kNoSplit, f - n0};
      mainloop<C, true, true, false>(a, b, d, lds, tid, acc);
      epi_swiglu_bwd<C>(acc, lds, p, row0, rows, n0, tid);
    } else {  // kG5
      const int n0 = nt * C::BN;  // over d
      const KcOp a{static_cast<const uint16_t*>(p.dhg) + row0 * f, static_cast<const uint16_t*>(p.dhu) + row0 * f, f,
                   f, rows};
      const KcOp b{Wg + e * wsz + static_cast<int64_t>(n0) * f, Wu + e * wsz + static_cast<int64_t>(n0) * f, f, f,
                   d - n0};
      mainloop<C, true, true, false>(a, b, 2 * f, lds, tid, acc);
      epi_store<C>(acc, lds, static_cast<uint16_t*>(p.o_dx) + row0 * d + n0, d, rows, d - n0, tid);
    }
  } else {  // weight gradients: K = rows of expert e
    // logical tile = (expert, M tile, N tile), blocks of tiles sharing operand
    // slices kept on one XCD, an expert's blocks spread over all XCDs
    const int gm = KIND == kG4 ? (f + C::BM - 1) / C::BM : (d + C::BM - 1) / C::BM;
    const int gn = KIND == kG4 ? (d + C::BN - 1) / C::BN : 2 * ((f + C::BN - 1) / C::BN);
    int e, mt, ntile;
    if (!wgrad_tile(blockIdx.x, p.E, gm, gn, e, mt, ntile)) return;
    const int64_t seg0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
    const int K = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]) - static_cast<int>(seg0);
    const int m0 = mt * C::BM;
    uint16_t* Cp;
    int n0, ldc, mvalid, nvalid;
    McOp a, b;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      n0 = ntile * C::BN;
      a = McOp{static_cast<const uint16_t*>(p.act) + seg0 * f, nullptr, f, m0, K};
      b = McOp{static_cast<const uint16_t*>(p.dy) + seg0 * d, nullptr, d, n0, K};
      Cp = static_cast<uint16_t*>(p.o_dwd) + e * wsz;
      ldc = d;
      mvalid = f;
      nvalid = d;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + C::BN - 1) / C::BN;
      const int which = ntile / per;
      n0 = (ntile % per) * C::BN;
      a = McOp{X + seg0 * d, nullptr, d, m0, K};
      b = McOp{static_cast<const uint16_t*>(which ? p.dhu : p.dhg) + seg0 * f, nullptr, f, n0, K};
      Cp = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz;
      ldc = f;
      mvalid = d;
      nvalid = f;
    }
    mainloop<C, false, false, false>(a, b, K, lds, tid, acc);
    epi_store<C>(acc, lds, Cp + static_cast<int64_t>(m0) * ldc + n0, ldc, mvalid - m0, nvalid - n0, tid);
  }
}

template <class C>
int launch_cfg(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t nd = cdiv(a.d, C::BN), nf = cdiv(a.f, C::BN);
  const dim3 blk(C::kThreads);
  switch (kind) {
    case kG1:
      MOE_LAUNCH("G1_bf16", (ffn_bf16_kernel<C, kG1>), dim3(xcd_grid(cdiv(a.f, C::BN / 2) * max_tiles)), blk, 0, s,
                 a);
      break;
    case kG2: MOE_LAUNCH("G2_bf16", (ffn_bf16_kernel<C, kG2>), dim3(xcd_grid(nd * max_tiles)), blk, 0, s, a); break;
    case kG3: MOE_LAUNCH("G3_bf16", (ffn_bf16_kernel<C, kG3>), dim3(xcd_grid(nf * max_tiles)), blk, 0, s, a); break;
    case kG5: MOE_LAUNCH("G5_bf16", (ffn_bf16_kernel<C, kG5>), dim3(xcd_grid(nd * max_tiles)), blk, 0, s, a); break;
    case kG4:
      MOE_LAUNCH("G4_bf16", (ffn_bf16_kernel<C, kG4>), dim3(static_cast<unsigned>(a.E * cdiv(a.f, C::BM) * nd)), blk,
                 0, s, a);
      break;
    case kG6:
      MOE_LAUNCH("G6_bf16", (ffn_bf16_kernel<C, kG6>), dim3(static_cast<unsigned>(a.E * cdiv(a.d, C::BM) * 2 * nf)),
                 blk, 0, s, a);
      break;
    default: return MOE_EINVAL;
  }
  return launch_status();
}

// Row-tile height of the rows-by-expert GEMMs: 256 when the average expert
// segment holds at least four such tiles, else 128 (Small and Mid share it).
bool big_rows(int64_t R, int E) { return R >= static_cast<int64_t>(E) * 1024; }
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
  if (kind == kG1 || kind == kG2) return launch_cfg<Mid>(kind, a, max_tiles, s);
  return launch_cfg<Small>(kind, a, max_tiles, s);
}

}  // namespace moe
