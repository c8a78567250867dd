// FP32 grouped expert-FFN GEMMs (fp32 storage and math, fp32 FMA on the vector
// ALUs).  Used for fp32 layers, whose sizes are small (the tiny fp32 workload
// has d = 64, f = 128); one thread computes one output element (G1: one gate/up
// pair) with a straight K loop in index order.  Rows-by-expert GEMMs walk the
// same device tile table as the BF16 kernels, with 16-row tiles.
#include "ffn_common.hpp"

namespace moe {
namespace {

constexpr int kBM = 16, kBN = 16;

template <int KIND>
__global__ __launch_bounds__(kBM * kBN) void ffn_f32_kernel(FfnArgs p) {
  const int d = p.d, f = p.f;
  const int64_t wsz = static_cast<int64_t>(d) * f;
  const float* X = static_cast<const float*>(p.x);
  const float* Wg = static_cast<const float*>(p.wg);
  const float* Wu = static_cast<const float*>(p.wu);
  const float* Wd = static_cast<const float*>(p.wd);
  const int ty = threadIdx.x / kBN, tx = threadIdx.x % kBN;

  if constexpr (KIND == kG1 || KIND == kG2 || KIND == kG3 || KIND == kG5) {
    const int4 t = p.tiles[blockIdx.y];
    if (t.x < 0 || ty >= t.z) return;
    const int e = t.x;
    const int64_t row = static_cast<int64_t>(t.y) + ty;
    const int col = blockIdx.x * kBN + tx;
    if constexpr (KIND == kG1) {
      if (col >= f) return;
      float g = 0.f, u = 0.f;
      for (int k = 0; k < d; ++k) {
        const float xv = X[row * d + k];
        g += xv * Wg[e * wsz + static_cast<int64_t>(k) * f + col];
        u += xv * Wu[e * wsz + static_cast<int64_t>(k) * f + col];
      }
      static_cast<float*>(p.o_hg)[row * f + col] = g;
      static_cast<float*>(p.o_hu)[row * f + col] = u;
      static_cast<float*>(p.o_act)[row * f + col] = silu_f(g) * u;
    } else if constexpr (KIND == kG2) {
      if (col >= d) return;
      const float* A = static_cast<const float*>(p.act);
      float acc = 0.f;
      for (int k = 0; k < f; ++k) acc += A[row * f + k] * Wd[e * wsz + static_cast<int64_t>(k) * d + col];
      static_cast<float*>(p.o_y)[row * d + col] = acc;
    } else if constexpr (KIND == kG3) {
      if (col >= f) return;
      const float* DY = static_cast<const float*>(p.dy);
      float da = 0.f;
      for (int k = 0; k < d; ++k) da += DY[row * d + k] * Wd[e * wsz + static_cast<int64_t>(col) * d + k];
      const float g = static_cast<const float*>(p.hg)[row * f + col];
      const float u = static_cast<const float*>(p.hu)[row * f + col];
      const float s = sigmoid_f(g);
      static_cast<float*>(p.o_dhu)[row * f + col] = da * g * s;
      static_cast<float*>(p.o_dhg)[row * f + col] = da * u * s * (1.0f + g * (1.0f - s));
    } else {
      if (col >= d) return;
      const float* DHG = static_cast<const float*>(p.dhg);
      const float* DHU = static_cast<const float*>(p.dhu);
      float acc = 0.f;
      for (int k = 0; k < f; ++k)
        acc += DHG[row * f + k] * Wg[e * wsz + static_cast<int64_t>(col) * f + k] +
               DHU[row * f + k] * Wu[e * wsz + static_cast<int64_t>(col) * f + k];
      static_cast<float*>(p.o_dx)[row * d + col] = acc;
    }
  } else {
    const int e = blockIdx.z;
    const int64_t seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
    const int m = blockIdx.y * kBM + ty;
    const int n = blockIdx.x * kBN + tx;
    if constexpr (KIND == kG4) {  // dWd_e [f, d]
      if (m >= f || n >= d) return;
      const float* A = static_cast<const float*>(p.act);
      const float* DY = static_cast<const float*>(p.dy);
      float acc = 0.f;
      for (int64_t r = seg0; r < seg1; ++r) acc += A[r * f + m] * DY[r * d + n];
      static_cast<float*>(p.o_dwd)[e * wsz + static_cast<int64_t>(m) * d + n] = acc;
    } else {  // kG6: dWg_e, dWu_e [d, f]
      if (m >= d || n >= f) return;
      const float* DHG = static_cast<const float*>(p.dhg);
      const float* DHU = static_cast<const float*>(p.dhu);
      float ag = 0.f, au = 0.f;
      for (int64_t r = seg0; r < seg1; ++r) {
        const float xv = X[r * d + m];
        ag += xv * DHG[r * f + n];
        au += xv * DHU[r * f + n];
      }
      static_cast<float*>(p.o_dwg)[e * wsz + static_cast<int64_t>(m) * f + n] = ag;
      static_cast<float*>(p.o_dwu)[e * wsz + static_cast<int64_t>(m) * f + n] = au;
    }
  }
}

}  // namespace

int ffn_f32_bm() { return kBM; }

int launch_ffn_f32(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s) {
  const unsigned mt = static_cast<unsigned>(max_tiles);
  const unsigned nd = static_cast<unsigned>(cdiv(a.d, kBN));
  const unsigned nf = static_cast<unsigned>(cdiv(a.f, kBN));
  const dim3 blk(kBM * kBN);
  switch (kind) {
    case kG1: MOE_LAUNCH("G1_f32", ffn_f32_kernel<kG1>, dim3(nf, mt), blk, 0, s, a); break;
    case kG2: MOE_LAUNCH("G2_f32", ffn_f32_kernel<kG2>, dim3(nd, mt), blk, 0, s, a); break;
    case kG3: MOE_LAUNCH("G3_f32", ffn_f32_kernel<kG3>, dim3(nf, mt), blk, 0, s, a); break;
    case kG5: MOE_LAUNCH("G5_f32", ffn_f32_kernel<kG5>, dim3(nd, mt), blk, 0, s, a); break;
    case kG4:
      MOE_LAUNCH("G4_f32", ffn_f32_kernel<kG4>, dim3(nd, static_cast<unsigned>(cdiv(a.f, kBM)), a.E), blk, 0, s, a);
      break;
    case kG6:
      MOE_LAUNCH("G6_f32", ffn_f32_kernel<kG6>, dim3(nf, static_cast<unsigned>(cdiv(a.d, kBM)), a.E), blk, 0, s, a);
      break;
    default: return MOE_EINVAL;
  }
  return launch_status();
}

}  // namespace moe
