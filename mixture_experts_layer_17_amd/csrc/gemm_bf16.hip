// BF16 grouped expert-FFN GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// One workgroup computes a 128 x 128 output tile with 4 waves (2 x 2), each wave
// a 64 x 64 sub-tile as 2 x 2 MFMA 32x32 blocks with fp32 accumulators.  The K
// loop steps by 64 with two register stages and two LDS stages: tile kt+2 is
// being fetched while tile kt is consumed, one barrier per step.  Every global
// load is a 16-byte vector and every operand keeps its memory layout in LDS:
// K-contiguous operands (activation rows, the weights of the dgrad GEMMs) are
// read as 16-byte fragments; operands contiguous along M or N (the weights of
// the forward GEMMs, both operands of the weight-gradient GEMMs, whose K is the
// token axis) are read with the gfx950 transposing LDS read ds_read_b64_tr_b16,
// two per fragment.  Epilogues go through LDS so that global stores (and the
// Hg/Hu loads of the SwiGLU backward) are 16-byte vectors along rows.
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

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kWM = 2, kWN = 2;
constexpr int kThreads = 64 * kWM * kWN;
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;
constexpr int kNoSplit = 0x7FFFFFFF;
// LDS tiles.  K-contiguous operand: [rows][kBK + 8] (row stride 144 B: the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks).
// MN-contiguous operand: [kBK][rows + 32] (row stride 320 B = 80 banks: a
// transposing read resolves banks over 32 lanes, i.e. four k-rows x 64 bytes,
// which this stride spreads over all 64 banks).
constexpr int kLdK = kBK + 8;
constexpr int kLdM = 128 + 32;
constexpr int kTileElems = (kBK * kLdM > 128 * kLdK) ? kBK * kLdM : 128 * kLdK;  // one operand, one stage
constexpr int kStageElems = 2 * kTileElems;                                        // A + B
constexpr int kLdsElems = 2 * kStageElems;                                         // two stages

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

// MN-contiguous operand: element (mn, k) at p[k*ld + col].  With `dual`, the
// tile's N index alternates between two matrices in groups of kWTN/2 columns so
// that each wave's N range holds matching gate and up columns.
struct McOp {
  const uint16_t* p0;
  const uint16_t* p1;
  int64_t ld;
  int mn_valid;  // valid columns (of each matrix when dual)
  int k_valid;
  bool dual;
  __device__ void col_of(int mn, const uint16_t*& p, int& col) const {
    if (dual) {
      const int w = mn / kWTN, r = mn % kWTN;
      p = (r >= kWTN / 2) ? p1 : p0;
      col = w * (kWTN / 2) + r % (kWTN / 2);
    } else {
      p = p0;
      col = mn;
    }
  }
};

// 16-byte global loads of one 128 x kBK (K-contiguous) or kBK x 128
// (MN-contiguous) tile into registers, then 16-byte LDS stores.  Each thread's
// chunks keep the same M/N position for the whole K loop, so their base
// pointers are resolved once (setup) and a step only adds the K offset.
template <bool KC>
struct Loader {
  static constexpr int kChunks = 128 * kBK / 8 / kThreads;  // 4
  uint4 v[kChunks];
  __device__ void load(const KcOp& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      v[i] = row < op.mn_valid ? *reinterpret_cast<const uint4*>(op.at(row, k0 + kc)) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void load(const McOp& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int kr = (tid + i * kThreads) / 16;
      const int k = k0 + kr;
      v[i] = (base[i] != nullptr && k < op.k_valid) ? *reinterpret_cast<const uint4*>(base[i] + k * op.ld)
                                                    : make_uint4(0, 0, 0, 0);
    }
  }
  // MN-contiguous operands: per-chunk column pointer (null when out of range).
  const uint16_t* base[kChunks];
  __device__ void setup(const McOp& op, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int mn = ((tid + i * kThreads) % 16) * 8;
      const uint16_t* p;
      int col;
      op.col_of(mn, p, col);
      base[i] = col < op.mn_valid ? p + col : nullptr;
    }
  }
  __device__ void setup(const KcOp&, int) {}
  __device__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      if constexpr (KC) {
        const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        *reinterpret_cast<uint4*>(lds + row * kLdK + kc) = v[i];
      } else {
        const int kr = c / 16, mn = (c % 16) * 8;
        *reinterpret_cast<uint4*>(lds + kr * kLdM + mn) = v[i];
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

// MFMA fragment (8 consecutive k for one m or n) of a 32-row block starting at
// `base` (M or N index) and k offset `k0` inside the stage.
template <bool KC>
__device__ __forceinline__ bf16x8 frag(const uint16_t* lds, int base, int k0, int lane) {
  if constexpr (KC) {
    return *reinterpret_cast<const bf16x8*>(lds + (base + (lane & 31)) * kLdK + k0 + (lane >> 5) * 8);
  } else {
    // Two transposing reads.  Within each 16-lane group G, lane i gets slot s
    // from element i%4 of the address given by lane 4s + i/4; lane L points at
    // row k = k0 + 8*(G/2) + 4*half + L/4, columns base + 16*(G%2) + 4*(L%4).
    const int G = lane >> 4, L = lane & 15;
    const uint16_t* p = lds + (k0 + 8 * (G >> 1) + (L >> 2)) * kLdM + base + 16 * (G & 1) + 4 * (L & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * kLdM));
    bf16x8 r;
    const short* lo_s = reinterpret_cast<const short*>(&lo);
    const short* hi_s = reinterpret_cast<const short*>(&hi);
    short tmp[8] = {lo_s[0], lo_s[1], lo_s[2], lo_s[3], hi_s[0], hi_s[1], hi_s[2], hi_s[3]};
    __builtin_memcpy(&r, tmp, 16);
    return r;
  }
}

template <bool AKC, bool BKC>
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, int wm,
                                          int wn, int lane, f32x16 (&acc)[kTM][kTN]) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    bf16x8 a[kTM], b[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) a[i] = frag<AKC>(As, wm * kWTM + i * 32, ks * 16, lane);
#pragma unroll
    for (int j = 0; j < kTN; ++j) b[j] = frag<BKC>(Bs, wn * kWTN + j * 32, ks * 16, lane);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// C = A B over K = [0, K).  Tile kt+2 is fetched into registers while tile kt
// is consumed from LDS and tile kt+1 waits in the other register set, so every
// global load has two compute steps to arrive.
template <bool AKC, bool BKC>
__device__ __forceinline__ void mainloop(const typename OpFor<AKC>::T& aop, const typename OpFor<BKC>::T& bop, int K,
                                         uint16_t* lds, int tid, f32x16 (&acc)[kTM][kTN]) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (K + kBK - 1) / kBK;
  if (nk == 0) return;
  Loader<AKC> la0, la1;
  Loader<BKC> lb0, lb1;
  la0.setup(aop, tid);
  la1.setup(aop, tid);
  lb0.setup(bop, tid);
  lb1.setup(bop, tid);
  la0.load(aop, 0, tid);
  lb0.load(bop, 0, tid);
  if (nk > 1) {
    la1.load(aop, kBK, tid);
    lb1.load(bop, kBK, tid);
  }
  la0.store(lds, tid);
  lb0.store(lds + kTileElems, tid);
  __syncthreads();
  auto step = [&](int kt, Loader<AKC>& la_next, Loader<BKC>& lb_next, Loader<AKC>& la_free,
                  Loader<BKC>& lb_free) {
    uint16_t* cur = lds + (kt & 1) * kStageElems;
    uint16_t* nxt = lds + ((kt + 1) & 1) * kStageElems;
    if (kt + 2 < nk) {
      la_free.load(aop, (kt + 2) * kBK, tid);
      lb_free.load(bop, (kt + 2) * kBK, tid);
    }
    mma_stage<AKC, BKC>(cur, cur + kTileElems, wm, wn, lane, acc);
    if (kt + 1 < nk) {
      la_next.store(nxt, tid);
      lb_next.store(nxt + kTileElems, tid);
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
constexpr int kLdC = 128 + 8;  // bf16 elements per LDS output row (272 bytes)
static_assert(kBM * kLdC <= kLdsElems, "output tile exceeds LDS");

// Row/column (inside the 128 x 128 tile) of accumulator register r of block (i, j).
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * kWTN + j * 32 + (lane & 31); }

// Copy a rows x cols bf16 tile from LDS (row stride kLdC) to global memory with
// 16-byte stores; only rows < rows_valid and columns < cols_valid are written.
__device__ __forceinline__ void flush_tile(const uint16_t* ct, int ldc, int rows, int cols, uint16_t* dst,
                                           int64_t ld, int rows_valid, int cols_valid, int tid) {
  const int cpr = cols / 8;
  for (int c = tid; c < rows * cpr; c += kThreads) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    if (r < rows_valid && cc < cols_valid)
      *reinterpret_cast<uint4*>(dst + r * ld + cc) = *reinterpret_cast<const uint4*>(ct + r * ldc + cc);
  }
}

__device__ __forceinline__ void load_tile(uint16_t* ct, int rows, int cols, const uint16_t* src, int64_t ld,
                                          int rows_valid, int cols_valid, int tid) {
  const int cpr = cols / 8;
  for (int c = tid; c < rows * cpr; c += kThreads) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    const uint4 v = (r < rows_valid && cc < cols_valid) ? *reinterpret_cast<const uint4*>(src + r * ld + cc)
                                                        : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(ct + r * kLdC + cc) = v;
  }
}

// Store the plain accumulator tile (bf16) to dst[r*ld + c].
__device__ __forceinline__ void store_acc(const f32x16 (&acc)[kTM][kTN], uint16_t* lds, uint16_t* dst, int64_t ld,
                                          int rows_valid, int cols_valid, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        lds[acc_row(wm, i, r, lane) * kLdC + acc_col(wn, j, lane)] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][r]));
  __syncthreads();
  flush_tile(lds, kLdC, kBM, kBN, dst, ld, rows_valid, cols_valid, tid);
}

template <int KIND>
__global__ __launch_bounds__(kThreads, 2) void ffn_bf16_kernel(FfnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int d = p.d, f = p.f;
  f32x16 acc[kTM][kTN];

  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* Wg = static_cast<const uint16_t*>(p.wg);
  const uint16_t* Wu = static_cast<const uint16_t*>(p.wu);
  const uint16_t* Wd = static_cast<const uint16_t*>(p.wd);
  const int64_t wsz = static_cast<int64_t>(d) * f;

  if constexpr (KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5) {
    const int4 t = p.tiles[blockIdx.y];
    if (t.x < 0) return;
    const int e = t.x, rows = t.z;
    const int64_t row0 = t.y;
    if constexpr (KIND == kG1) {
      const int n0 = blockIdx.x * (kBN / 2);
      const KcOp a{X + row0 * d, nullptr, d, kNoSplit, rows};
      const McOp b{Wg + e * wsz + n0, Wu + e * wsz + n0, f, f - n0, d, true};
      mainloop<true, false>(a, b, d, lds, tid, acc);
      // three 128 x 64 bf16 tiles: Hg, Hu, A (row stride kLdH)
      constexpr int kLdH = kBN / 2 + 8;
      static_assert(3 * kBM * kLdH <= kLdsElems, "G1 epilogue tiles exceed LDS");
      uint16_t* tg = lds;
      uint16_t* tu = lds + kBM * kLdH;
      uint16_t* ta = lds + 2 * kBM * kLdH;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN / 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = acc_row(wm, i, r, lane) * kLdH + wn * (kWTN / 2) + j * 32 + (lane & 31);
            const float g = acc[i][j][r], u = acc[i][j + kTN / 2][r];
            tg[o] = static_cast<uint16_t>(f32_to_bf16(g));
            tu[o] = static_cast<uint16_t>(f32_to_bf16(u));
            ta[o] = static_cast<uint16_t>(f32_to_bf16(silu_f(g) * u));
          }
      __syncthreads();
      const int64_t o0 = row0 * f + n0;
      flush_tile(tg, kLdH, kBM, kBN / 2, static_cast<uint16_t*>(p.o_hg) + o0, f, rows, f - n0, tid);
      flush_tile(tu, kLdH, kBM, kBN / 2, static_cast<uint16_t*>(p.o_hu) + o0, f, rows, f - n0, tid);
      flush_tile(ta, kLdH, kBM, kBN / 2, static_cast<uint16_t*>(p.o_act) + o0, f, rows, f - n0, tid);
    } else if constexpr (KIND == kG2) {
      const int n0 = blockIdx.x * kBN;
      const KcOp a{static_cast<const uint16_t*>(p.act) + row0 * f, nullptr, f, kNoSplit, rows};
      const McOp b{Wd + e * wsz + n0, nullptr, d, d - n0, f, false};
      mainloop<true, false>(a, b, f, lds, tid, acc);
      store_acc(acc, lds, static_cast<uint16_t*>(p.o_y) + row0 * d + n0, d, rows, d - n0, tid);
    } else if constexpr (KIND == kG3) {
      const int n0 = blockIdx.x * kBN;  // over f
      const KcOp a{static_cast<const uint16_t*>(p.dy) + row0 * d, nullptr, d, kNoSplit, rows};
      const KcOp b{Wd + e * wsz + static_cast<int64_t>(n0) * d, nullptr, d, kNoSplit, f - n0};
      mainloop<true, true>(a, b, d, lds, tid, acc);
      // stage Hg, Hu tiles with 16-byte loads, compute dHg, dHu in place, store
      static_assert(2 * kBM * kLdC <= kLdsElems, "G3 epilogue tiles exceed LDS");
      uint16_t* tg = lds;
      uint16_t* tu = lds + kBM * kLdC;
      const int64_t o0 = row0 * f + n0;
      load_tile(tg, kBM, kBN, static_cast<const uint16_t*>(p.hg) + o0, f, rows, f - n0, tid);
      load_tile(tu, kBM, kBN, static_cast<const uint16_t*>(p.hu) + o0, f, rows, f - n0, tid);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = acc_row(wm, i, r, lane) * kLdC + acc_col(wn, j, lane);
            const float g = bf16_to_f32(tg[o]), u = bf16_to_f32(tu[o]);
            const float da = acc[i][j][r];
            const float sg = sigmoid_f(g);
            tu[o] = static_cast<uint16_t>(f32_to_bf16(da * g * sg));
            tg[o] = static_cast<uint16_t>(f32_to_bf16(da * u * sg * (1.0f + g * (1.0f - sg))));
          }
      __syncthreads();
      flush_tile(tg, kLdC, kBM, kBN, static_cast<uint16_t*>(p.o_dhg) + o0, f, rows, f - n0, tid);
      flush_tile(tu, kLdC, kBM, kBN, static_cast<uint16_t*>(p.o_dhu) + o0, f, rows, f - n0, tid);
    } else {  // kG5
      const int n0 = blockIdx.x * kBN;  // over d
      const KcOp a{static_cast<const uint16_t*>(p.dhg) + row0 * f, static_cast<const uint16_t*>(p.dhu) + row0 * f, f,
                   f, rows};
      const KcOp b{Wg + e * wsz + static_cast<int64_t>(n0) * f, Wu + e * wsz + static_cast<int64_t>(n0) * f, f, f,
                   d - n0};
      mainloop<true, true>(a, b, 2 * f, lds, tid, acc);
      store_acc(acc, lds, static_cast<uint16_t*>(p.o_dx) + row0 * d + n0, d, rows, d - n0, tid);
    }
  } else {  // weight gradients: K = rows of expert e
    const int e = blockIdx.z;
    const int64_t seg0 = p.offsets[e];
    const int K = p.offsets[e + 1] - static_cast<int>(seg0);
    const int m0 = blockIdx.y * kBM;
    uint16_t* C;
    int n0, ldc, mvalid, nvalid;
    McOp a, b;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      n0 = blockIdx.x * kBN;
      a = McOp{static_cast<const uint16_t*>(p.act) + seg0 * f + m0, nullptr, f, f - m0, K, false};
      b = McOp{static_cast<const uint16_t*>(p.dy) + seg0 * d + n0, nullptr, d, d - n0, K, false};
      C = static_cast<uint16_t*>(p.o_dwd) + e * wsz;
      ldc = d;
      mvalid = f;
      nvalid = d;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + kBN - 1) / kBN;
      const int which = blockIdx.x / per;
      n0 = (blockIdx.x % per) * kBN;
      a = McOp{X + seg0 * d + m0, nullptr, d, d - m0, K, false};
      b = McOp{static_cast<const uint16_t*>(which ? p.dhu : p.dhg) + seg0 * f + n0, nullptr, f, f - n0, K, false};
      C = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz;
      ldc = f;
      mvalid = d;
      nvalid = f;
    }
    mainloop<false, false>(a, b, K, lds, tid, acc);
    store_acc(acc, lds, C + static_cast<int64_t>(m0) * ldc + n0, ldc, mvalid - m0, nvalid - n0, tid);
  }
}

}  // namespace

int ffn_bf16_bm() { return kBM; }

int launch_ffn_bf16(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s) {
  const unsigned mt = static_cast<unsigned>(max_tiles);
  const unsigned nd = static_cast<unsigned>(cdiv(a.d, kBN));
  const unsigned nf = static_cast<unsigned>(cdiv(a.f, kBN));
  switch (kind) {
    case kG1:
      MOE_LAUNCH("G1_bf16", ffn_bf16_kernel<kG1>, dim3(static_cast<unsigned>(cdiv(a.f, kBN / 2)), mt), dim3(kThreads), 0,
                         s, a);
      break;
    case kG2: MOE_LAUNCH("G2_bf16", ffn_bf16_kernel<kG2>, dim3(nd, mt), dim3(kThreads), 0, s, a); break;
    case kG3: MOE_LAUNCH("G3_bf16", ffn_bf16_kernel<kG3>, dim3(nf, mt), dim3(kThreads), 0, s, a); break;
    case kG5: MOE_LAUNCH("G5_bf16", ffn_bf16_kernel<kG5>, dim3(nd, mt), dim3(kThreads), 0, s, a); break;
    case kG4:
      MOE_LAUNCH("G4_bf16", ffn_bf16_kernel<kG4>, dim3(nd, static_cast<unsigned>(cdiv(a.f, kBM)), a.E), dim3(kThreads),
                         0, s, a);
      break;
    case kG6:
      MOE_LAUNCH("G6_bf16", ffn_bf16_kernel<kG6>, dim3(2 * nf, static_cast<unsigned>(cdiv(a.d, kBM)), a.E),
                         dim3(kThreads), 0, s, a);
      break;
    default: return MOE_EINVAL;
  }
  return launch_status();
}

}  // namespace moe
