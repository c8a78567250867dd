// BF16 grouped expert-FFN GEMMs on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// One workgroup computes a 128 x 128 output tile with 4 waves (2 x 2), each wave
// a 64 x 64 sub-tile as 2 x 2 MFMA 32x32 blocks with fp32 accumulators.  The K
// loop steps by 64: the next A and B tiles are fetched from HBM into registers
// while the current ones are consumed from LDS (two LDS buffers, one barrier per
// step).  In LDS both operands are stored K-contiguous (row = M or N index, 64
// K values + 8 bf16 of padding, so the 16-byte fragment reads of 8 consecutive
// rows hit distinct banks).  Operands that are K-contiguous in memory (token
// rows of activations, the transposed weights of the dgrad GEMMs) are copied
// with 16-byte loads; operands that are contiguous along M or N (the weights of
// the forward GEMMs, and both operands of the weight-gradient GEMMs, whose K is
// the token axis) are read as 8 k-rows x 4 columns per thread and transposed in
// registers before the 16-byte LDS stores.
//
// MFMA operand layout (32x32x16 bf16): lane l supplies A[m = l % 32][k = 8(l/32) .. +7]
// and B[k = 8(l/32) .. +7][n = l % 32]; accumulator register r of lane l holds
// C[8(r/4) + 4(l/32) + r%4][l % 32].
#include "ffn_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kWM = 2, kWN = 2;
constexpr int kThreads = 64 * kWM * kWN;
constexpr int kLd = kBK + 8;  // LDS row stride in bf16 elements (144 bytes)
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;
constexpr int kNoSplit = 0x7FFFFFFF;

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

template <int ROWS>
struct KcLoader {
  static constexpr int kChunks = ROWS * kBK / 8 / kThreads;
  uint4 v[kChunks];
  __device__ void load(const KcOp& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      v[i] = row < op.mn_valid ? *reinterpret_cast<const uint4*>(op.at(row, k0 + kc)) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      *reinterpret_cast<uint4*>(lds + row * kLd + kc) = v[i];
    }
  }
};

template <int ROWS>
struct McLoader {
  static constexpr int kBlocks = (kBK / 8) * (ROWS / 4) / kThreads;
  static_assert(kBlocks >= 1, "tile too small for the transposing loader");
  uint2 v[kBlocks][8];
  __device__ void load(const McOp& op, int k0, int tid) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      const int blk = tid + b * kThreads;
      const int mn = (blk % (ROWS / 4)) * 4, kb = blk / (ROWS / 4);
      const uint16_t* p;
      int col;
      op.col_of(mn, p, col);
      const bool mn_ok = col < op.mn_valid;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int k = k0 + kb * 8 + r;
        v[b][r] = (mn_ok && k < op.k_valid) ? *reinterpret_cast<const uint2*>(p + k * op.ld + col)
                                            : make_uint2(0, 0);
      }
    }
  }
  __device__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      const int blk = tid + b * kThreads;
      const int mn = (blk % (ROWS / 4)) * 4, kb = blk / (ROWS / 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = (m < 2 ? v[b][2 * j].x : v[b][2 * j].y);
          const uint32_t hi = (m < 2 ? v[b][2 * j + 1].x : v[b][2 * j + 1].y);
          w[j] = (m & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        *reinterpret_cast<uint4*>(lds + (mn + m) * kLd + kb * 8) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
};

template <bool KC>
struct LoaderFor;
template <>
struct LoaderFor<true> {
  using A = KcLoader<kBM>;
  using B = KcLoader<kBN>;
  using Op = KcOp;
};
template <>
struct LoaderFor<false> {
  using A = McLoader<kBM>;
  using B = McLoader<kBN>;
  using Op = McOp;
};

__device__ __forceinline__ void mma_step(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs, int wm,
                                         int wn, int lane, f32x16 (&acc)[kTM][kTN]) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    bf16x8 a[kTM], b[kTN];
    const int kof = ks * 16 + (lane >> 5) * 8;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(As + (wm * kWTM + i * 32 + (lane & 31)) * kLd + kof);
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * kWTN + j * 32 + (lane & 31)) * kLd + kof);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// C = A B over K = [0, K) with A: BM x K and B: K x BN described by the ops.
template <bool AKC, bool BKC>
__device__ __forceinline__ void mainloop(const typename LoaderFor<AKC>::Op& aop,
                                         const typename LoaderFor<BKC>::Op& bop, int K, uint16_t* lds, int tid,
                                         f32x16 (&acc)[kTM][kTN]) {
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
  constexpr int kBuf = (kBM + kBN) * kLd;
  typename LoaderFor<AKC>::A la;
  typename LoaderFor<BKC>::B lb;
  la.load(aop, 0, tid);
  lb.load(bop, 0, tid);
  la.store(lds, tid);
  lb.store(lds + kBM * kLd, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint16_t* cur = lds + (kt & 1) * kBuf;
    uint16_t* nxt = lds + ((kt + 1) & 1) * kBuf;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(aop, (kt + 1) * kBK, tid);
      lb.load(bop, (kt + 1) * kBK, tid);
    }
    mma_step(cur, cur + kBM * kLd, wm, wn, lane, acc);
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + kBM * kLd, tid);
    }
    __syncthreads();
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void ffn_bf16_kernel(FfnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (kBM + kBN) * kLd];
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
      uint16_t* Hg = static_cast<uint16_t*>(p.o_hg);
      uint16_t* Hu = static_cast<uint16_t*>(p.o_hu);
      uint16_t* A = static_cast<uint16_t*>(p.o_act);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN / 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = n0 + wn * (kWTN / 2) + j * 32 + (lane & 31);
            if (rl < rows && col < f) {
              const float g = acc[i][j][r], u = acc[i][j + kTN / 2][r];
              const int64_t o = (row0 + rl) * f + col;
              Hg[o] = static_cast<uint16_t>(f32_to_bf16(g));
              Hu[o] = static_cast<uint16_t>(f32_to_bf16(u));
              A[o] = static_cast<uint16_t>(f32_to_bf16(silu_f(g) * u));
            }
          }
    } else if constexpr (KIND == kG2) {
      const int n0 = blockIdx.x * kBN;
      const KcOp a{static_cast<const uint16_t*>(p.act) + row0 * f, nullptr, f, kNoSplit, rows};
      const McOp b{Wd + e * wsz + n0, nullptr, d, d - n0, f, false};
      mainloop<true, false>(a, b, f, lds, tid, acc);
      uint16_t* Y = static_cast<uint16_t*>(p.o_y);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
            if (rl < rows && col < d) Y[(row0 + rl) * d + col] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][r]));
          }
    } else if constexpr (KIND == kG3) {
      const int n0 = blockIdx.x * kBN;  // over f
      const KcOp a{static_cast<const uint16_t*>(p.dy) + row0 * d, nullptr, d, kNoSplit, rows};
      const KcOp b{Wd + e * wsz + static_cast<int64_t>(n0) * d, nullptr, d, kNoSplit, f - n0};
      mainloop<true, true>(a, b, d, lds, tid, acc);
      const uint16_t* Hg = static_cast<const uint16_t*>(p.hg);
      const uint16_t* Hu = static_cast<const uint16_t*>(p.hu);
      uint16_t* dHg = static_cast<uint16_t*>(p.o_dhg);
      uint16_t* dHu = static_cast<uint16_t*>(p.o_dhu);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
            if (rl < rows && col < f) {
              const int64_t o = (row0 + rl) * f + col;
              const float g = bf16_to_f32(Hg[o]), u = bf16_to_f32(Hu[o]);
              const float da = acc[i][j][r];
              const float s = sigmoid_f(g);
              dHu[o] = static_cast<uint16_t>(f32_to_bf16(da * g * s));
              dHg[o] = static_cast<uint16_t>(f32_to_bf16(da * u * s * (1.0f + g * (1.0f - s))));
            }
          }
    } else {  // kG5
      const int n0 = blockIdx.x * kBN;  // over d
      const KcOp a{static_cast<const uint16_t*>(p.dhg) + row0 * f, static_cast<const uint16_t*>(p.dhu) + row0 * f, f,
                   f, rows};
      const KcOp b{Wg + e * wsz + static_cast<int64_t>(n0) * f, Wu + e * wsz + static_cast<int64_t>(n0) * f, f, f,
                   d - n0};
      mainloop<true, true>(a, b, 2 * f, lds, tid, acc);
      uint16_t* DX = static_cast<uint16_t*>(p.o_dx);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
            if (rl < rows && col < d) DX[(row0 + rl) * d + col] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][r]));
          }
    }
  } else {  // weight gradients: K = rows of expert e
    const int e = blockIdx.z;
    const int64_t seg0 = p.offsets[e];
    const int K = p.offsets[e + 1] - static_cast<int>(seg0);
    const int m0 = blockIdx.y * kBM;
    const uint16_t* Bsrc;
    uint16_t* C;
    int n0, ldc, mvalid, nvalid;
    McOp a, b;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      n0 = blockIdx.x * kBN;
      a = McOp{static_cast<const uint16_t*>(p.act) + seg0 * f + m0, nullptr, f, f - m0, K, false};
      Bsrc = static_cast<const uint16_t*>(p.dy) + seg0 * d + n0;
      b = McOp{Bsrc, nullptr, d, d - n0, K, false};
      C = static_cast<uint16_t*>(p.o_dwd) + e * wsz;
      ldc = d;
      mvalid = f;
      nvalid = d;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + kBN - 1) / kBN;
      const int which = blockIdx.x / per;
      n0 = (blockIdx.x % per) * kBN;
      a = McOp{X + seg0 * d + m0, nullptr, d, d - m0, K, false};
      Bsrc = static_cast<const uint16_t*>(which ? p.dhu : p.dhg) + seg0 * f + n0;
      b = McOp{Bsrc, nullptr, f, f - n0, K, false};
      C = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz;
      ldc = f;
      mvalid = d;
      nvalid = f;
    }
    mainloop<false, false>(a, b, K, lds, tid, acc);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = m0 + wm * kWTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
          if (rl < mvalid && col < nvalid)
            C[static_cast<int64_t>(rl) * ldc + col] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][r]));
        }
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
