// BF16 grouped expert-FFN GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Two tile shapes share one kernel template: 256 x 256 outputs per workgroup
// for large expert segments and the weight gradients, and 128 x 128 with 4
// waves (each 64 x 64) for short segments (about 512 rows per expert), where a
// 256-row tile would mostly compute padding.  The K loop steps by 64 through
// two LDS stages with one or two register stages of global-load prefetch, one
// barrier per step.  Every global load is a 16-byte vector and every operand keeps its
// memory layout in LDS: K-contiguous operands (activation rows, the weights of
// the dgrad GEMMs) are read as 16-byte fragments; operands contiguous along M
// or N (the weights of the forward GEMMs, both operands of the weight-gradient
// GEMMs, whose K is the token axis) are read with the gfx950 transposing LDS
// read ds_read_b64_tr_b16, two per fragment.  Epilogues go through LDS so that
// global stores (and the Hg/Hu loads of the SwiGLU backward) are 16-byte
// vectors along rows.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies A[m = l % 32][k = 8(l/32) .. +7]
// and B[k = 8(l/32) .. +7][n = l % 32]; accumulator register r of lane l holds
// C[8(r/4) + 4(l/32) + r%4][l % 32].
#include "ffn_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNoSplit = 0x7FFFFFFF;
constexpr int kBK = 64;
constexpr int kLdK = kBK + 8;  // K-contiguous LDS rows: 144 B, 16-byte reads of 16 rows cover all banks

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Tile configuration: BM x BN outputs, WM x WN waves, DIST register stages of
// global-load prefetch (1: tile kt+1 in flight, 2: tiles kt+1 and kt+2).
template <int BM_, int BN_, int WM_, int WN_, int DIST_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, DIST = DIST_;
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  // M/N-contiguous LDS rows: rows + 32 elements.  A transposing read resolves
  // banks over 32 lanes (four k-rows x 64 bytes); a row stride of 16 banks
  // modulo 64 spreads them over all 64 banks.
  static constexpr int ldm(int rows) { return rows + 32; }
  static constexpr int tile(int rows) { return cmax(kBK * ldm(rows), rows * kLdK); }
  static constexpr int kA = tile(BM), kB = tile(BN);
  static constexpr int kStage = kA + kB;
  static constexpr int kLds = 2 * kStage;  // elements (bf16)
};
#ifndef MOE_BIG_TILE
#define MOE_BIG_TILE 1
#endif
#if MOE_BIG_TILE == 1
using Big = Cfg<256, 256, 2, 4, 1>;  // 8 waves of 128 x 64, one register stage
#else
using Big = Cfg<256, 256, 2, 2, 2>;  // 4 waves of 128 x 128, two register stages
#endif
using Small = Cfg<128, 128, 2, 2, 2>;

// K-contiguous operand: element (mn, k) at p[mn*ld + k]; for k >= ksplit the
// element comes from the second matrix at column k - ksplit.
struct KcOp {
  const uint16_t* p0;
  const uint16_t* p1;
  int64_t ld;
  int ksplit;
  int mn_valid;
  __device__ const uint16_t* at(int mn, int k) const {
    return k < ksplit ? p0 + mn * ld + k : p1 + mn * ld + (k - ksplit);
  }
};

// M/N-contiguous operand: element (mn, k) at p[k*ld + col].  With dual_w > 0 the
// tile's N index alternates between two matrices in groups of dual_w/2 columns
// (dual_w = one wave's N width), so every wave holds matching gate and up columns.
struct McOp {
  const uint16_t* p0;
  const uint16_t* p1;
  int64_t ld;
  int mn_valid;  // valid columns (of each matrix when dual)
  int k_valid;
  int dual_w;
  __device__ void col_of(int mn, const uint16_t*& p, int& col) const {
    if (dual_w > 0) {
      const int h = dual_w / 2, w = mn / dual_w, r = mn % dual_w;
      p = r >= h ? p1 : p0;
      col = w * h + r % h;
    } else {
      p = p0;
      col = mn;
    }
  }
};

// One operand's tile loader: 16-byte global loads into registers, 16-byte LDS
// stores.  The M/N-contiguous form resolves each chunk's column pointer once
// (the chunk keeps its M/N position for the whole K loop).
template <class C, int ROWS, bool KC>
struct Loader {
  static constexpr int kChunks = ROWS * kBK / 8 / C::kThreads;
  static_assert(kChunks >= 1 && ROWS * kBK / 8 % C::kThreads == 0, "tile does not split evenly");
  static constexpr int kLd = C::ldm(ROWS);
  uint4 v[kChunks];

  struct Bases {
    const uint16_t* p[kChunks];
  };
  __device__ static void setup(const McOp& op, int tid, Bases& b) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int mn = ((tid + i * C::kThreads) % (ROWS / 8)) * 8;
      const uint16_t* p;
      int col;
      op.col_of(mn, p, col);
      b.p[i] = col < op.mn_valid ? p + col : nullptr;
    }
  }
  __device__ static void setup(const KcOp&, int, Bases&) {}

  __device__ void load(const KcOp& op, const Bases&, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * C::kThreads;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      v[i] = row < op.mn_valid ? *reinterpret_cast<const uint4*>(op.at(row, k0 + kc)) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void load(const McOp& op, const Bases& b, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int k = k0 + (tid + i * C::kThreads) / (ROWS / 8);
      v[i] = (b.p[i] != nullptr && k < op.k_valid) ? *reinterpret_cast<const uint4*>(b.p[i] + k * op.ld)
                                                   : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * C::kThreads;
      if constexpr (KC) {
        const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        *reinterpret_cast<uint4*>(lds + row * kLdK + kc) = v[i];
      } else {
        const int kr = c / (ROWS / 8), mn = (c % (ROWS / 8)) * 8;
        *reinterpret_cast<uint4*>(lds + kr * kLd + mn) = v[i];
      }
    }
  }
};

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

// MFMA fragment (8 consecutive k for one m or n) of the 32-row block starting at
// `base` (M or N index) and k offset `k0` inside a stage.
template <bool KC, int LDM>
__device__ __forceinline__ bf16x8 frag(const uint16_t* lds, int base, int k0, int lane) {
  if constexpr (KC) {
    return *reinterpret_cast<const bf16x8*>(lds + (base + (lane & 31)) * kLdK + k0 + (lane >> 5) * 8);
  } else {
    // Two transposing reads.  Within each 16-lane group G, lane i gets slot s
    // from element i%4 of the address given by lane 4s + i/4; lane L points at
    // row k = k0 + 8*(G/2) + 4*half + L/4, columns base + 16*(G%2) + 4*(L%4).
    const int G = lane >> 4, L = lane & 15;
    const uint16_t* p = lds + (k0 + 8 * (G >> 1) + (L >> 2)) * LDM + base + 16 * (G & 1) + 4 * (L & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * LDM));
    bf16x8 r;
    short tmp[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    __builtin_memcpy(&r, tmp, 16);
    return r;
  }
}

template <class C>
using Acc = f32x16[C::TM][C::TN];

template <class C, bool AKC, bool BKC>
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, int wm,
                                          int wn, int lane, Acc<C>& acc) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    bf16x8 a[C::TM], b[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) a[i] = frag<AKC, C::ldm(C::BM)>(As, wm * C::WTM + i * 32, ks * 16, lane);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) b[j] = frag<BKC, C::ldm(C::BN)>(Bs, wn * C::WTN + j * 32, ks * 16, lane);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// C = A B over K = [0, K).  Tile kt+2 is fetched into registers while tile kt
// is consumed from LDS and tile kt+1 waits in the other register set, so every
// global load has two compute steps to arrive.
template <class C, bool AKC, bool BKC>
__device__ __forceinline__ void mainloop(const typename OpFor<AKC>::T& aop, const typename OpFor<BKC>::T& bop, int K,
                                         uint16_t* lds, int tid, Acc<C>& acc) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (K + kBK - 1) / kBK;
  if (nk == 0) return;
  using LA = Loader<C, C::BM, AKC>;
  using LB = Loader<C, C::BN, BKC>;
  typename LA::Bases ba;
  typename LB::Bases bb;
  LA::setup(aop, tid, ba);
  LB::setup(bop, tid, bb);
  if constexpr (C::DIST == 1) {
    // one register stage: tile kt+1 is fetched while tile kt is consumed
    LA la;
    LB lb;
    la.load(aop, ba, 0, tid);
    lb.load(bop, bb, 0, tid);
    la.store(lds, tid);
    lb.store(lds + C::kA, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint16_t* cur = lds + (kt & 1) * C::kStage;
      uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStage;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(aop, ba, (kt + 1) * kBK, tid);
        lb.load(bop, bb, (kt + 1) * kBK, tid);
      }
      mma_stage<C, AKC, BKC>(cur, cur + C::kA, wm, wn, lane, acc);
      if (more) {
        la.store(nxt, tid);
        lb.store(nxt + C::kA, tid);
      }
      __syncthreads();
    }
    return;
  }
  LA la0, la1;
  LB lb0, lb1;
  la0.load(aop, ba, 0, tid);
  lb0.load(bop, bb, 0, tid);
  if (nk > 1) {
    la1.load(aop, ba, kBK, tid);
    lb1.load(bop, bb, kBK, tid);
  }
  la0.store(lds, tid);
  lb0.store(lds + C::kA, tid);
  __syncthreads();
  auto step = [&](int kt, LA& la_next, LB& lb_next, LA& la_free, LB& lb_free) {
    uint16_t* cur = lds + (kt & 1) * C::kStage;
    uint16_t* nxt = lds + ((kt + 1) & 1) * C::kStage;
    if (kt + 2 < nk) {
      la_free.load(aop, ba, (kt + 2) * kBK, tid);
      lb_free.load(bop, bb, (kt + 2) * kBK, tid);
    }
    mma_stage<C, AKC, BKC>(cur, cur + C::kA, wm, wn, lane, acc);
    if (kt + 1 < nk) {
      la_next.store(nxt, tid);
      lb_next.store(nxt + C::kA, tid);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, la1, lb1, la0, lb0);
    if (kt + 1 < nk) step(kt + 1, la0, lb0, la1, lb1);
  }
}

// ---------------------------------------------------------------------------
// Epilogue through LDS: accumulators -> bf16 tile in LDS -> 16-byte stores.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * C::WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * C::WTN + j * 32 + (lane & 31);
}

// Copy a rows x cols bf16 tile from LDS (row stride ldc) to global memory with
// 16-byte stores; only rows < rows_valid and columns < cols_valid are written.
template <class C>
__device__ __forceinline__ void flush_tile(const uint16_t* ct, int ldc, int rows, int cols, uint16_t* dst,
                                           int64_t ld, int rows_valid, int cols_valid, int tid) {
  const int cpr = cols / 8;
  for (int c = tid; c < rows * cpr; c += C::kThreads) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    if (r < rows_valid && cc < cols_valid)
      *reinterpret_cast<uint4*>(dst + r * ld + cc) = *reinterpret_cast<const uint4*>(ct + r * ldc + cc);
  }
}

template <class C>
__device__ __forceinline__ void load_tile(uint16_t* ct, int ldc, int rows, int cols, const uint16_t* src, int64_t ld,
                                          int rows_valid, int cols_valid, int tid) {
  const int cpr = cols / 8;
  for (int c = tid; c < rows * cpr; c += C::kThreads) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    const uint4 v = (r < rows_valid && cc < cols_valid) ? *reinterpret_cast<const uint4*>(src + r * ld + cc)
                                                        : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(ct + r * ldc + cc) = v;
  }
}

// Store the plain accumulator tile (bf16) to dst[r*ld + c].
template <class C>
__device__ __forceinline__ void store_acc(const Acc<C>& acc, uint16_t* lds, uint16_t* dst, int64_t ld,
                                          int rows_valid, int cols_valid, int tid) {
  constexpr int ldc = C::BN + 8;
  static_assert(C::BM * ldc <= C::kLds, "output tile exceeds LDS");
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        lds[acc_row<C>(wm, i, r, lane) * ldc + acc_col<C>(wn, j, lane)] =
            static_cast<uint16_t>(f32_to_bf16(acc[i][j][r]));
  __syncthreads();
  flush_tile<C>(lds, ldc, C::BM, C::BN, dst, ld, rows_valid, cols_valid, tid);
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
    const int e = t.x, rows = t.z;
    const int64_t row0 = t.y;
    const int nt = static_cast<int>(lid % gx);
    if constexpr (KIND == kG1) {
      const int n0 = nt * (C::BN / 2);
      const KcOp a{X + row0 * d, nullptr, d, kNoSplit, rows};
      const McOp b{Wg + e * wsz + n0, Wu + e * wsz + n0, f, f - n0, d, C::WTN};
      mainloop<C, true, false>(a, b, d, lds, tid, acc);
      // Hg and Hu tiles (BM x BN/2 each), then A in the Hg buffer
      constexpr int ldh = C::BN / 2 + 8;
      static_assert(2 * C::BM * ldh <= C::kLds, "G1 epilogue tiles exceed LDS");
      uint16_t* tg = lds;
      uint16_t* tu = lds + C::BM * ldh;
      const int64_t o0 = row0 * f + n0;
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN / 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = acc_row<C>(wm, i, r, lane) * ldh + wn * (C::WTN / 2) + j * 32 + (lane & 31);
            tg[o] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][r]));
            tu[o] = static_cast<uint16_t>(f32_to_bf16(acc[i][j + C::TN / 2][r]));
          }
      __syncthreads();
      flush_tile<C>(tg, ldh, C::BM, C::BN / 2, static_cast<uint16_t*>(p.o_hg) + o0, f, rows, f - n0, tid);
      flush_tile<C>(tu, ldh, C::BM, C::BN / 2, static_cast<uint16_t*>(p.o_hu) + o0, f, rows, f - n0, tid);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN / 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = acc_row<C>(wm, i, r, lane) * ldh + wn * (C::WTN / 2) + j * 32 + (lane & 31);
            const float g = acc[i][j][r], u = acc[i][j + C::TN / 2][r];
            tg[o] = static_cast<uint16_t>(f32_to_bf16(silu_f(g) * u));
          }
      __syncthreads();
      flush_tile<C>(tg, ldh, C::BM, C::BN / 2, static_cast<uint16_t*>(p.o_act) + o0, f, rows, f - n0, tid);
    } else if constexpr (KIND == kG2) {
      const int n0 = nt * C::BN;
      const KcOp a{static_cast<const uint16_t*>(p.act) + row0 * f, nullptr, f, kNoSplit, rows};
      const McOp b{Wd + e * wsz + n0, nullptr, d, d - n0, f, 0};
      mainloop<C, true, false>(a, b, f, lds, tid, acc);
      store_acc<C>(acc, lds, static_cast<uint16_t*>(p.o_y) + row0 * d + n0, d, rows, d - n0, tid);
    } else if constexpr (KIND == kG3) {
      const int n0 = nt * C::BN;  // over f
      const KcOp a{static_cast<const uint16_t*>(p.dy) + row0 * d, nullptr, d, kNoSplit, rows};
      const KcOp b{Wd + e * wsz + static_cast<int64_t>(n0) * d, nullptr, d, kNoSplit, f - n0};
      mainloop<C, true, true>(a, b, d, lds, tid, acc);
      // SwiGLU backward: stage Hg, Hu with 16-byte loads, compute dHg, dHu in
      // place, 16-byte stores.  When both full tiles do not fit in LDS the tile
      // is processed in two row halves, each by the waves owning those rows.
      constexpr int ldc = C::BN + 8;
      constexpr int halves = (2 * C::BM * ldc <= C::kLds) ? 1 : 2;
      constexpr int hr = C::BM / halves;
      static_assert(2 * hr * ldc <= C::kLds, "G3 epilogue tiles exceed LDS");
      static_assert(halves == 1 || C::WM == 2, "the half split assumes two wave rows");
      uint16_t* tg = lds;
      uint16_t* tu = lds + hr * ldc;
      for (int h = 0; h < halves; ++h) {
        const int64_t o0 = (row0 + h * hr) * f + n0;
        const int rv = rows - h * hr;
        load_tile<C>(tg, ldc, hr, C::BN, static_cast<const uint16_t*>(p.hg) + o0, f, rv, f - n0, tid);
        load_tile<C>(tu, ldc, hr, C::BN, static_cast<const uint16_t*>(p.hu) + o0, f, rv, f - n0, tid);
        __syncthreads();
        if (halves == 1 || wm == h) {
#pragma unroll
          for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int o = (acc_row<C>(wm, i, r, lane) - h * hr) * ldc + acc_col<C>(wn, j, lane);
                const float g = bf16_to_f32(tg[o]), u = bf16_to_f32(tu[o]);
                const float da = acc[i][j][r];
                const float sg = sigmoid_f(g);
                tu[o] = static_cast<uint16_t>(f32_to_bf16(da * g * sg));
                tg[o] = static_cast<uint16_t>(f32_to_bf16(da * u * sg * (1.0f + g * (1.0f - sg))));
              }
        }
        __syncthreads();
        flush_tile<C>(tg, ldc, hr, C::BN, static_cast<uint16_t*>(p.o_dhg) + o0, f, rv, f - n0, tid);
        flush_tile<C>(tu, ldc, hr, C::BN, static_cast<uint16_t*>(p.o_dhu) + o0, f, rv, f - n0, tid);
        __syncthreads();
      }
    } else {  // kG5
      const int n0 = nt * C::BN;  // over d
      const KcOp a{static_cast<const uint16_t*>(p.dhg) + row0 * f, static_cast<const uint16_t*>(p.dhu) + row0 * f, f,
                   f, rows};
      const KcOp b{Wg + e * wsz + static_cast<int64_t>(n0) * f, Wu + e * wsz + static_cast<int64_t>(n0) * f, f, f,
                   d - n0};
      mainloop<C, true, true>(a, b, 2 * f, lds, tid, acc);
      store_acc<C>(acc, lds, static_cast<uint16_t*>(p.o_dx) + row0 * d + n0, d, rows, d - n0, tid);
    }
  } else {  // weight gradients: K = rows of expert e
    // logical tile = (expert, M tile, N tile), N fastest, in hardware order so
    // that a heavily loaded expert spreads over every XCD
    const int gm = KIND == kG4 ? (f + C::BM - 1) / C::BM : (d + C::BM - 1) / C::BM;
    const int gn = KIND == kG4 ? (d + C::BN - 1) / C::BN : 2 * ((f + C::BN - 1) / C::BN);
    const int64_t lid = blockIdx.x;
    if (lid >= static_cast<int64_t>(p.E) * gm * gn) return;
    const int e = static_cast<int>(lid / (gm * gn));
    const int mt = static_cast<int>((lid / gn) % gm), ntile = static_cast<int>(lid % gn);
    const int64_t seg0 = p.offsets[e];
    const int K = p.offsets[e + 1] - static_cast<int>(seg0);
    const int m0 = mt * C::BM;
    uint16_t* Cp;
    int n0, ldc, mvalid, nvalid;
    McOp a, b;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      n0 = ntile * C::BN;
      a = McOp{static_cast<const uint16_t*>(p.act) + seg0 * f + m0, nullptr, f, f - m0, K, 0};
      b = McOp{static_cast<const uint16_t*>(p.dy) + seg0 * d + n0, nullptr, d, d - n0, K, 0};
      Cp = static_cast<uint16_t*>(p.o_dwd) + e * wsz;
      ldc = d;
      mvalid = f;
      nvalid = d;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + C::BN - 1) / C::BN;
      const int which = ntile / per;
      n0 = (ntile % per) * C::BN;
      a = McOp{X + seg0 * d + m0, nullptr, d, d - m0, K, 0};
      b = McOp{static_cast<const uint16_t*>(which ? p.dhu : p.dhg) + seg0 * f + n0, nullptr, f, f - n0, K, 0};
      Cp = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz;
      ldc = f;
      mvalid = d;
      nvalid = f;
    }
    mainloop<C, false, false>(a, b, K, lds, tid, acc);
    store_acc<C>(acc, lds, Cp + static_cast<int64_t>(m0) * ldc + n0, ldc, mvalid - m0, nvalid - n0, tid);
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
// segment holds at least four such tiles, else 128.
bool big_rows(int64_t R, int E) { return R >= static_cast<int64_t>(E) * 1024; }
// Weight-gradient tiles: 256 x 256 when d and f fill them.
bool big_wgrad(const FfnArgs& a) { return a.d % 256 == 0 && a.f % 256 == 0; }

}  // namespace

int ffn_bf16_bm(int64_t R, int E) { return big_rows(R, E) ? Big::BM : Small::BM; }

int launch_ffn_bf16(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s) {
  const bool wgrad = kind == kG4 || kind == kG6;
  const bool big = wgrad ? big_wgrad(a) : big_rows(a.R, a.E);
  return big ? launch_cfg<Big>(kind, a, max_tiles, s) : launch_cfg<Small>(kind, a, max_tiles, s);
}

}  // namespace moe
