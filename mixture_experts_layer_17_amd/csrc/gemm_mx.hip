// MXFP8 grouped expert-FFN GEMMs on gfx950 MX-scaled FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, E8M0 block scales, fp32
// accumulation, bf16 outputs).
//
// Olmo-core 3 announcement, "Scaling and optimizing MoE training": MXFP8 is used
// for the expert computation where it pays, and converting into it has a cost.
// Every GEMM operand is quantised on the device (mx.hip) along that GEMM's
// contraction axis into a K-contiguous layout (activations: row blocks; forward
// weights and the token-axis operands of the weight gradients: column blocks
// stored transposed), so a single "A[m][k] * B[n][k]" kernel serves all six
// products.  The token-axis operands are padded to 32 tokens per expert
// segment (block offsets from the routing metadata); their K range is masked at
// segment ends.
//
// Tile: 128 x 128 outputs per workgroup, 4 waves of 64 x 64, K step 128 bytes
// (two MFMA K-steps of 64).  LDS rows are 128 bytes + 16 of padding; each row's
// four E8M0 scales of the K step sit in a 32-bit LDS word.  MFMA operand layout
// (32x32x64 f8, checked on the hardware): lane l = (g = l/32, m = l%32) supplies
// A[m][16g .. 16g+15] in its first 16 bytes and A[m][32+16g .. 32+16g+15] in
// its last 16; its scale operand is the E8M0 scale of row m, block g (k in
// [32g, 32g+32)).  B is laid out the same way with n = l % 32.
#include "mx_common.hpp"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 128;  // kBK in fp8 elements (bytes)
constexpr int kWM = 2, kWN = 2;
constexpr int kThreads = 64 * kWM * kWN;
constexpr int kLd = kBK + 16;  // LDS row stride in bytes
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;
constexpr int kNoSplit = 0x7FFFFFFF;

// K-contiguous fp8 operand with block scales: element (mn, k) at q[mn*ld + k],
// scale of (mn, k) at s[mn*(ld/32) + k/32].  k >= ksplit reads the second
// matrix at k - ksplit.  `dual` maps the tile's N index onto two matrices in
// groups of kWTN/2 rows (gate and up columns side by side in every wave).
struct MxOp {
  const uint8_t* q0;
  const uint8_t* q1;
  const uint8_t* s0;
  const uint8_t* s1;
  int64_t ld;      // elements per row (a multiple of 32)
  int64_t k_base;  // first K element of this problem inside each row
  int k_valid;     // K elements of this problem
  int ksplit;
  int mn_valid;
  bool dual;
  __device__ void row_of(int mn, int k, const uint8_t*& q, const uint8_t*& s, int& row, int& kk) const {
    const bool second = dual ? ((mn % kWTN) >= kWTN / 2) : (k >= ksplit);
    row = dual ? (mn / kWTN) * (kWTN / 2) + mn % (kWTN / 2) : mn;
    kk = (!dual && k >= ksplit) ? k - ksplit : k;
    q = second ? q1 : q0;
    s = second ? s1 : s0;
  }
};

struct MxLoader {
  static constexpr int kChunks = 128 * kBK / 16 / kThreads;  // 16-byte chunks per thread (4)
  uint4 v[kChunks];
  uint32_t sc;  // four scale bytes of one row (threads < 128)
  __device__ void load(const MxOp& op, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int mn = c / (kBK / 16), kc = (c % (kBK / 16)) * 16;
      const uint8_t *q, *s;
      int row, kk;
      op.row_of(mn, k0 + kc, q, s, row, kk);
      const bool ok = row < op.mn_valid && k0 + kc < op.k_valid;
      v[i] = ok ? *reinterpret_cast<const uint4*>(q + row * op.ld + op.k_base + kk) : make_uint4(0, 0, 0, 0);
    }
    sc = 0;
    if (tid < 128) {
      const uint8_t *q, *s;
      int row, kk;
      op.row_of(tid, k0, q, s, row, kk);
      if (row < op.mn_valid) {
        const uint8_t* sp = s + row * (op.ld / 32) + (op.k_base + kk) / 32;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k0 + 32 * j < op.k_valid) sc |= static_cast<uint32_t>(sp[j]) << (8 * j);
      }
    }
  }
  __device__ void store(uint8_t* lds, uint32_t* lds_s, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int mn = c / (kBK / 16), kc = (c % (kBK / 16)) * 16;
      *reinterpret_cast<uint4*>(lds + mn * kLd + kc) = v[i];
    }
    if (tid < 128) lds_s[tid] = sc;
  }
};

struct Smem {
  uint8_t a[2][kBM * kLd];
  uint8_t b[2][kBN * kLd];
  uint32_t sa[2][kBM];
  uint32_t sb[2][kBN];
};

__device__ __forceinline__ i32x8 frag(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 32);
  i32x8 v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

__device__ __forceinline__ void mx_step(const Smem& sm, int buf, int wm, int wn, int lane, f32x16 (&acc)[kTM][kTN]) {
#pragma unroll
  for (int ks = 0; ks < kBK / 64; ++ks) {
    i32x8 a[kTM], b[kTN];
    int sa[kTM], sb[kTN];
    // lane l = (g = l/32, row l%32): bytes k = 16g..16g+15 and 32+16g..32+16g+15
    // of this 64-wide K step; its scale operand is the row's block g.
    const int kof = ks * 64 + (lane >> 5) * 16;
    const int sh = 8 * (ks * 2 + (lane >> 5));
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int r = wm * kWTM + i * 32 + (lane & 31);
      a[i] = frag(sm.a[buf] + r * kLd + kof);
      sa[i] = static_cast<int>((sm.sa[buf][r] >> sh) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int r = wn * kWTN + j * 32 + (lane & 31);
      b[j] = frag(sm.b[buf] + r * kLd + kof);
      sb[j] = static_cast<int>((sm.sb[buf][r] >> sh) & 0xFFu);
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
  }
}

__device__ __forceinline__ void mx_mainloop(const MxOp& aop, const MxOp& bop, int K, Smem& sm, int tid,
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
  MxLoader la, lb;
  la.load(aop, 0, tid);
  lb.load(bop, 0, tid);
  la.store(sm.a[0], sm.sa[0], tid);
  lb.store(sm.b[0], sm.sb[0], tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(aop, (kt + 1) * kBK, tid);
      lb.load(bop, (kt + 1) * kBK, tid);
    }
    mx_step(sm, cur, wm, wn, lane, acc);
    if (more) {
      la.store(sm.a[cur ^ 1], sm.sa[cur ^ 1], tid);
      lb.store(sm.b[cur ^ 1], sm.sb[cur ^ 1], tid);
    }
    __syncthreads();
  }
}

// Quantised operands of one FFN call (device pointers into the scratch area).
struct MxArgs {
  FfnArgs f;
  const int32_t* blk;  // MX block offsets per expert (token axis), E+1
  int64_t ldt;         // padded token length of the transposed token-axis operands
  const uint8_t *xq, *xs, *aq, *as, *dyq, *dys, *dhgq, *dhgs, *dhuq, *dhus;          // row-blocked [R, K]
  const uint8_t *wgq, *wgs, *wuq, *wus, *wdq, *wds;                                   // weights, K-contiguous
  const uint8_t *xtq, *xts, *dytq, *dyts, *atq, *ats, *dhgtq, *dhgts, *dhutq, *dhuts;  // [cols, ldt]
};

template <int KIND>
__global__ __launch_bounds__(kThreads) void ffn_mx_kernel(MxArgs m) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const FfnArgs& p = m.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int d = p.d, f = p.f;
  const int64_t wsz = static_cast<int64_t>(d) * f;
  f32x16 acc[kTM][kTN];

  if constexpr (KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5) {
    const int4 t = p.tiles[blockIdx.y];
    if (t.x < 0) return;
    const int e = t.x, rows = t.z;
    const int64_t row0 = t.y;
    if constexpr (KIND == kG1) {
      const int n0 = blockIdx.x * (kBN / 2);
      const MxOp a{m.xq + row0 * d, nullptr, m.xs + row0 * (d / 32), nullptr, d, 0, d, kNoSplit, rows, false};
      const MxOp b{m.wgq + e * wsz + static_cast<int64_t>(n0) * d, m.wuq + e * wsz + static_cast<int64_t>(n0) * d,
                   m.wgs + (e * wsz + static_cast<int64_t>(n0) * d) / 32,
                   m.wus + (e * wsz + static_cast<int64_t>(n0) * d) / 32, d, 0, d, kNoSplit, f - n0, true};
      mx_mainloop(a, b, d, sm, tid, acc);
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
      const int n0 = blockIdx.x * kBN;  // over d
      const MxOp a{m.aq + row0 * f, nullptr, m.as + row0 * (f / 32), nullptr, f, 0, f, kNoSplit, rows, false};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * f;  // transposed Wd: [E][d][f]
      const MxOp b{m.wdq + wo, nullptr, m.wds + wo / 32, nullptr, f, 0, f, kNoSplit, d - n0, false};
      mx_mainloop(a, b, f, sm, tid, acc);
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
      const MxOp a{m.dyq + row0 * d, nullptr, m.dys + row0 * (d / 32), nullptr, d, 0, d, kNoSplit, rows, false};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * d;  // natural Wd: [E][f][d]
      const MxOp b{m.wdq + wo, nullptr, m.wds + wo / 32, nullptr, d, 0, d, kNoSplit, f - n0, false};
      mx_mainloop(a, b, d, sm, tid, acc);
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
      const MxOp a{m.dhgq + row0 * f, m.dhuq + row0 * f, m.dhgs + row0 * (f / 32), m.dhus + row0 * (f / 32),
                   f, 0, 2 * f, f, rows, false};
      const int64_t wo = e * wsz + static_cast<int64_t>(n0) * f;  // natural Wg, Wu: [E][d][f]
      const MxOp b{m.wgq + wo, m.wuq + wo, m.wgs + wo / 32, m.wus + wo / 32, f, 0, 2 * f, f, d - n0, false};
      mx_mainloop(a, b, 2 * f, sm, tid, acc);
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
  } else {  // weight gradients: K = 32-padded token blocks of expert e
    const int e = blockIdx.z;
    const int64_t kb = static_cast<int64_t>(m.blk[e]) * 32;
    const int K = (m.blk[e + 1] - m.blk[e]) * 32;
    const int m0 = blockIdx.y * kBM;
    uint16_t* C;
    int n0, ldc, mvalid, nvalid;
    MxOp a, b;
    if constexpr (KIND == kG4) {  // dWd_e [f, d] = A_e^T dY_e
      n0 = blockIdx.x * kBN;
      a = MxOp{m.atq + static_cast<int64_t>(m0) * m.ldt, nullptr, m.ats + static_cast<int64_t>(m0) * (m.ldt / 32),
               nullptr, m.ldt, kb, K, kNoSplit, f - m0, false};
      b = MxOp{m.dytq + static_cast<int64_t>(n0) * m.ldt, nullptr, m.dyts + static_cast<int64_t>(n0) * (m.ldt / 32),
               nullptr, m.ldt, kb, K, kNoSplit, d - n0, false};
      C = static_cast<uint16_t*>(p.o_dwd) + e * wsz;
      ldc = d;
      mvalid = f;
      nvalid = d;
    } else {  // kG6: dWg_e, dWu_e [d, f] = X_e^T dH_e
      const int per = (f + kBN - 1) / kBN;
      const int which = blockIdx.x / per;
      n0 = (blockIdx.x % per) * kBN;
      a = MxOp{m.xtq + static_cast<int64_t>(m0) * m.ldt, nullptr, m.xts + static_cast<int64_t>(m0) * (m.ldt / 32),
               nullptr, m.ldt, kb, K, kNoSplit, d - m0, false};
      const uint8_t* bq = which ? m.dhutq : m.dhgtq;
      const uint8_t* bs = which ? m.dhuts : m.dhgts;
      b = MxOp{bq + static_cast<int64_t>(n0) * m.ldt, nullptr, bs + static_cast<int64_t>(n0) * (m.ldt / 32), nullptr,
               m.ldt, kb, K, kNoSplit, f - n0, false};
      C = static_cast<uint16_t*>(which ? p.o_dwu : p.o_dwg) + e * wsz;
      ldc = f;
      mvalid = d;
      nvalid = f;
    }
    mx_mainloop(a, b, K, sm, tid, acc);
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

int launch_mx_kind(int kind, const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  const unsigned mt = static_cast<unsigned>(max_tiles);
  const unsigned nd = static_cast<unsigned>(cdiv(a.f.d, kBN));
  const unsigned nf = static_cast<unsigned>(cdiv(a.f.f, kBN));
  const dim3 blk(kThreads);
  switch (kind) {
    case kG1:
      MOE_LAUNCH("G1_mx", ffn_mx_kernel<kG1>, dim3(static_cast<unsigned>(cdiv(a.f.f, kBN / 2)), mt), blk, 0, s, a);
      break;
    case kG2: MOE_LAUNCH("G2_mx", ffn_mx_kernel<kG2>, dim3(nd, mt), blk, 0, s, a); break;
    case kG3: MOE_LAUNCH("G3_mx", ffn_mx_kernel<kG3>, dim3(nf, mt), blk, 0, s, a); break;
    case kG5: MOE_LAUNCH("G5_mx", ffn_mx_kernel<kG5>, dim3(nd, mt), blk, 0, s, a); break;
    case kG4:
      MOE_LAUNCH("G4_mx", ffn_mx_kernel<kG4>, dim3(nd, static_cast<unsigned>(cdiv(a.f.f, kBM)), a.f.E), blk, 0, s,
                 a);
      break;
    case kG6:
      MOE_LAUNCH("G6_mx", ffn_mx_kernel<kG6>, dim3(2 * nf, static_cast<unsigned>(cdiv(a.f.d, kBM)), a.f.E), blk, 0,
                 s, a);
      break;
    default: return MOE_EINVAL;
  }
  return launch_status();
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

int64_t token_pad(int64_t R, int E) { return 32 * (cdiv(R, 32) + E); }

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

}  // namespace

size_t mx_ffn_scratch_bytes(int64_t R, int E, int d, int f, int is_bwd) {
  Carve c{nullptr};
  if (is_bwd)
    carve_bwd(c, R, E, d, f);
  else
    carve_fwd(c, R, E, d, f);
  return c.used;
}

int mx_ffn_fwd(const FfnArgs& a, int64_t max_tiles, char* scratch, hipStream_t s) {
  Carve c{scratch};
  const FwdBufs b = carve_fwd(c, a.R, a.E, a.d, a.f);
  const int bf = MOE_BF16;
  // X along d (rows); Wg, Wu [E][d][f] along d -> [E][f][d]; Wd [E][f][d] along f -> [E][d][f]
  launch_mx_rows(a.x, bf, a.R, a.d, b.x.q, b.x.s, s);
  launch_mx_cols(a.wg, bf, a.E, a.d, a.f, nullptr, 0, a.d, b.wg.q, b.wg.s, s);
  launch_mx_cols(a.wu, bf, a.E, a.d, a.f, nullptr, 0, a.d, b.wu.q, b.wu.s, s);
  launch_mx_cols(a.wd, bf, a.E, a.f, a.d, nullptr, 0, a.f, b.wd.q, b.wd.s, s);
  MxArgs m{};
  m.f = a;
  m.xq = b.x.q; m.xs = b.x.s;
  m.wgq = b.wg.q; m.wgs = b.wg.s; m.wuq = b.wu.q; m.wus = b.wu.s;
  int st = launch_mx_kind(kG1, m, max_tiles, s);
  if (st != MOE_OK) return st;
  launch_mx_rows(a.o_act, bf, a.R, a.f, b.a.q, b.a.s, s);
  m.aq = b.a.q; m.as = b.a.s;
  m.wdq = b.wd.q; m.wds = b.wd.s;
  return launch_mx_kind(kG2, m, max_tiles, s);
}

int mx_ffn_bwd(const FfnArgs& a, int64_t max_tiles, const int32_t* mx_blk_offsets, char* scratch, hipStream_t s) {
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
    // G3: dA = dY Wd^T: dY along d, Wd natural [E][f][d] along d
    launch_mx_rows(a.dy, bf, a.R, a.d, b.dy.q, b.dy.s, s);
    launch_mx_rows(a.wd, bf, static_cast<int64_t>(a.E) * a.f, a.d, b.wd.q, b.wd.s, s);
    m.dyq = b.dy.q; m.dys = b.dy.s; m.wdq = b.wd.q; m.wds = b.wd.s;
    st = launch_mx_kind(kG3, m, max_tiles, s);
    if (st != MOE_OK) return st;
    // G5: dX = dHg Wg^T + dHu Wu^T: dH along f, Wg/Wu natural [E][d][f] along f
    launch_mx_rows(a.dhg, bf, a.R, a.f, b.dhg.q, b.dhg.s, s);
    launch_mx_rows(a.dhu, bf, a.R, a.f, b.dhu.q, b.dhu.s, s);
    launch_mx_rows(a.wg, bf, static_cast<int64_t>(a.E) * a.d, a.f, b.wg.q, b.wg.s, s);
    launch_mx_rows(a.wu, bf, static_cast<int64_t>(a.E) * a.d, a.f, b.wu.q, b.wu.s, s);
    m.dhgq = b.dhg.q; m.dhgs = b.dhg.s; m.dhuq = b.dhu.q; m.dhus = b.dhu.s;
    m.wgq = b.wg.q; m.wgs = b.wg.s; m.wuq = b.wu.q; m.wus = b.wu.s;
    st = launch_mx_kind(kG5, m, max_tiles, s);
    if (st != MOE_OK) return st;
    // weight gradients: every operand along tokens, per expert segment, transposed
    launch_mx_cols(a.act, bf, 1, a.R, a.f, a.offsets, a.E, rp, b.at.q, b.at.s, s);
    launch_mx_cols(a.dy, bf, 1, a.R, a.d, a.offsets, a.E, rp, b.dyt.q, b.dyt.s, s);
    launch_mx_cols(a.x, bf, 1, a.R, a.d, a.offsets, a.E, rp, b.xt.q, b.xt.s, s);
    launch_mx_cols(a.dhg, bf, 1, a.R, a.f, a.offsets, a.E, rp, b.dhgt.q, b.dhgt.s, s);
    launch_mx_cols(a.dhu, bf, 1, a.R, a.f, a.offsets, a.E, rp, b.dhut.q, b.dhut.s, s);
  }
  m.atq = b.at.q; m.ats = b.at.s; m.dytq = b.dyt.q; m.dyts = b.dyt.s;
  m.xtq = b.xt.q; m.xts = b.xt.s;
  m.dhgtq = b.dhgt.q; m.dhgts = b.dhgt.s; m.dhutq = b.dhut.q; m.dhuts = b.dhut.s;
  st = launch_mx_kind(kG4, m, max_tiles, s);
  if (st == MOE_OK) st = launch_mx_kind(kG6, m, max_tiles, s);
  return st;
}

}  // namespace moe
