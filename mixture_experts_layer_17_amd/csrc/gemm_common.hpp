// Shared pieces of the grouped expert-FFN GEMMs (internal): the gfx950 LDS-DMA
// load helpers and the LDS-staged epilogues.  A tile configuration C provides
// BM x BN outputs per workgroup over WM x WN waves of WTM x WTN (TM x TN MFMA
// tiles of 32 x 32 each), kThreads, and kLds (bf16 elements of LDS).
//
// Accumulator layout of the 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16 and
// v_mfma_scale_f32_32x32x64_f8f6f4 alike): register r of lane l holds
// C[8(r/4) + 4(l/32) + r%4][l % 32].
#pragma once

#include "ffn_common.hpp"

namespace moe {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// 16-byte LDS accesses go through an ext_vector type rather than a struct such
// as uint4: only then does the compiler's alias information tell an LDS read
// or write apart from the LDS-DMA loads still in flight into another ring slot,
// instead of waiting for all of them before it (a full vmcnt wait).
typedef int lds16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_get16(const void* p) {
  const lds16_t v = *reinterpret_cast<const lds16_t*>(p);
  return make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                    static_cast<uint32_t>(v[3]));
}
__device__ __forceinline__ void lds_put16(void* p, const uint4& u) {
  const lds16_t v = {static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z), static_cast<int>(u.w)};
  *reinterpret_cast<lds16_t*>(p) = v;
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format: range-checked, out of range reads 0

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <class C>
using Acc = f32x16[C::TM][C::TN];

// Buffer descriptor over [base, base + bytes).  Every caller passes
// workgroup-uniform values; readfirstlane keeps the descriptor in scalar
// registers (a descriptor in vector registers would need a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int n = __builtin_amdgcn_readfirstlane(bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : static_cast<int>(bytes)));
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  void* pb = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pb, 0, n, kRsrcWord3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_dst), 16, voff, 0, 0, 0);
}

// Wait until at most N vector memory operations of this wave are outstanding
// (N < 64: the counter's low four bits sit in bits 3:0 of the immediate, its
// high two in bits 15:14; expcnt and lgkmcnt left alone).  On this
// architecture loads and stores share the counter and retire in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
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
// NT: streaming (non-temporal) stores, for outputs the next kernel does not read.
template <class C, bool NT = true>
__device__ __forceinline__ void flush_tile(const uint16_t* ct, int ldc, int rows, int cols, uint16_t* dst,
                                           int64_t ld, int rows_valid, int cols_valid, int tid) {
  const int cpr = cols / 8;
  for (int c = tid; c < rows * cpr; c += C::kThreads) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    if (r < rows_valid && cc < cols_valid) {
      const uint4 v = *reinterpret_cast<const uint4*>(ct + r * ldc + cc);
      if constexpr (NT) store16_nt(dst + r * ld + cc, v);
      else *reinterpret_cast<uint4*>(dst + r * ld + cc) = v;
    }
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
template <class C, bool NT = true>
__device__ __forceinline__ void epi_store(const Acc<C>& acc, uint16_t* lds, uint16_t* dst, int64_t ld,
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
  flush_tile<C, NT>(lds, ldc, C::BM, C::BN, dst, ld, rows_valid, cols_valid, tid);
}

// G1 epilogue: Hg and Hu tiles (BM x BN/2 each: the gate columns are
// accumulator tiles j < TN/2, the up columns j >= TN/2), then A = silu(Hg) * Hu
// (SwiGLU) in the Hg buffer; all three stored as bf16.
template <class C>
__device__ __forceinline__ void epi_swiglu_fwd(const Acc<C>& acc, uint16_t* lds, const FfnArgs& p, int64_t row0,
                                               int rows, int n0, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int f = p.f;
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
}

// G3 epilogue: SwiGLU backward from dA (the accumulators) and the stored Hg, Hu:
// dHu = dA * silu(Hg), dHg = dA * Hu * silu'(Hg), stored as bf16.
template <class C>
__device__ __forceinline__ void epi_swiglu_bwd(const Acc<C>& acc, uint16_t* lds, const FfnArgs& p, int64_t row0,
                                               int rows, int n0, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int f = p.f;
  // Stage Hg, Hu with 16-byte loads, compute dHg, dHu in
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
}

// ---------------------------------------------------------------------------
// Register-direct epilogues.  The kernels using them compute every 32 x 32
// tile transposed, as mfma(B fragment, A fragment): then register r of lane l
// holds C[l % 32][8(r/4) + 4(l/32) + r%4], four consecutive columns of one
// row.  to_chunks exchanges halves between lanes l and l + 32
// (v_permlane32_swap) so that each lane holds two runs of eight: chunk c of
// lane l is row l % 32, columns 16c + 8(l/32) .. +7, stored as one 16-byte
// vector.  No LDS and no barrier: the next tile's loads can be in flight.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void to_chunks(const f32x16& a, float (&o)[2][8]) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[8 * c + s]),
                                                      __float_as_uint(a[8 * c + 4 + s]), false, false);
      o[c][s] = __uint_as_float(r[0]);
      o[c][4 + s] = __uint_as_float(r[1]);
    }
}

__device__ __forceinline__ uint4 pack8(const float* v) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

template <bool NT>
__device__ __forceinline__ void store16(uint16_t* p, const uint4& v) {
  if constexpr (NT) store16_nt(p, v);
  else *reinterpret_cast<uint4*>(p) = v;
}

// Plain bf16 output tile at dst (row stride ld): rows < rows_valid, columns < cols_valid.
// Ordinary (cached) stores: each instruction writes 32 bytes of 32 rows, and the
// L2 merges them into whole lines (streaming stores of such pieces measured slower).
template <class C, bool NT = false>
__device__ __forceinline__ void epi_regs_store(const Acc<C>& acc, uint16_t* dst, int64_t ld, int rows_valid,
                                               int cols_valid, int lane, int wm, int wn) {
  const int rl = lane & 31, hc = 8 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * C::WTM + i * 32 + rl;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      float v[2][8];
      to_chunks(acc[i][j], v);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = wn * C::WTN + j * 32 + 16 * c + hc;
        if (row < rows_valid && col < cols_valid) store16<NT>(dst + row * ld + col, pack8(v[c]));
      }
    }
  }
}

// G1: gate tiles j < TN/2 and up tiles j >= TN/2 cover the same f columns;
// stores Hg, Hu and A = silu(Hg) * Hu (SwiGLU, from the fp32 accumulators).
template <class C>
__device__ __forceinline__ void epi_regs_swiglu_fwd(const Acc<C>& acc, const FfnArgs& p, int64_t row0, int rows,
                                                    int n0, int lane, int wm, int wn) {
  constexpr int H = C::TN / 2;
  const int rl = lane & 31, hc = 8 * (lane >> 5);
  const int64_t f = p.f;
  uint16_t* hg = static_cast<uint16_t*>(p.o_hg) + row0 * f + n0;
  uint16_t* hu = static_cast<uint16_t*>(p.o_hu) + row0 * f + n0;
  uint16_t* ac = static_cast<uint16_t*>(p.o_act) + row0 * f + n0;
  const int cols = p.f - n0;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * C::WTM + i * 32 + rl;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      float g[2][8], u[2][8];
      to_chunks(acc[i][j], g);
      to_chunks(acc[i][j + H], u);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = wn * (C::WTN / 2) + j * 32 + 16 * c + hc;
        if (row < rows && col < cols) {
          float a[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) a[t] = silu_f(g[c][t]) * u[c][t];
          const int64_t o = row * f + col;
          store16<false>(hg + o, pack8(g[c]));
          store16<false>(hu + o, pack8(u[c]));
          store16<false>(ac + o, pack8(a));
        }
      }
    }
  }
}

// G3: SwiGLU backward from dA (the accumulators) and the stored Hg, Hu:
// dHu = dA * silu(Hg), dHg = dA * Hu * silu'(Hg), stored as bf16.  The Hg, Hu
// chunks of row block i + 1 are loaded while block i is computed, and all loads
// of a block precede its stores (which could alias them as far as the compiler
// knows), so the load latencies overlap.
template <class C>
__device__ __forceinline__ void epi_regs_swiglu_bwd(const Acc<C>& acc, const FfnArgs& p, int64_t row0, int rows,
                                                    int n0, int lane, int wm, int wn) {
  const int rl = lane & 31, hc = 8 * (lane >> 5);
  const int64_t f = p.f;
  const uint16_t* hg = static_cast<const uint16_t*>(p.hg) + row0 * f + n0;
  const uint16_t* hu = static_cast<const uint16_t*>(p.hu) + row0 * f + n0;
  uint16_t* dg = static_cast<uint16_t*>(p.o_dhg) + row0 * f + n0;
  uint16_t* du = static_cast<uint16_t*>(p.o_dhu) + row0 * f + n0;
  const int cols = p.f - n0;
  auto load = [&](int i, uint4 (&lg)[C::TN][2], uint4 (&lu)[C::TN][2]) {
    const int row = wm * C::WTM + i * 32 + rl;
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = wn * C::WTN + j * 32 + 16 * c + hc;
        const bool ok = row < rows && col < cols;
        const int64_t o = row * f + col;
        lg[j][c] = ok ? *reinterpret_cast<const uint4*>(hg + o) : make_uint4(0, 0, 0, 0);
        lu[j][c] = ok ? *reinterpret_cast<const uint4*>(hu + o) : make_uint4(0, 0, 0, 0);
      }
  };
  uint4 lg[2][C::TN][2], lu[2][C::TN][2];
  load(0, lg[0], lu[0]);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = wm * C::WTM + i * 32 + rl;
    if (i + 1 < C::TM) load(i + 1, lg[(i + 1) & 1], lu[(i + 1) & 1]);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      float da[2][8];
      to_chunks(acc[i][j], da);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = wn * C::WTN + j * 32 + 16 * c + hc;
        if (row < rows && col < cols) {
          const int64_t o = row * f + col;
          float g[8], u[8], og[8], ou[8];
          Elem<uint16_t>::unpack(lg[i & 1][j][c], g);
          Elem<uint16_t>::unpack(lu[i & 1][j][c], u);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float sg = sigmoid_f(g[t]);
            ou[t] = da[c][t] * g[t] * sg;
            og[t] = da[c][t] * u[t] * sg * (1.0f + g[t] * (1.0f - sg));
          }
          store16<false>(dg + o, pack8(og));
          store16<false>(du + o, pack8(ou));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wave-private epilogues of the 256 x 256 tiles (8 waves of 128 x 64, tiles
// computed transposed) through LDS the main loop no longer uses: each wave
// owns 8 KB of a ring slot (stage buffer `buf`, bf16 elements).
// ---------------------------------------------------------------------------

// SwiGLU-backward epilogue of the 256 x 256 tiles (G3) with Hg, Hu staged
// through LDS.  Each wave owns 16 KB of the (then idle) LDS rings: two buffers
// of one 32-row block of its 128 x 64 sub-tile, Hg then Hu (4 KB each), filled
// with coalesced LDS-DMA loads (eight whole 128-byte rows per instruction).
// Within a buffer, 128-byte row r keeps global 16-byte chunk q at physical
// chunk q ^ ((r >> 1) & 7), so that reading 32 rows at one chunk (the
// accumulator layout) is free of bank conflicts.
template <class C>
__device__ __forceinline__ void g3_stage(const FfnArgs& p, int64_t row0, int rows, int n0, int i, uint16_t* buf,
                                         int wm, int wn, int lane) {
  static_assert(C::WTN == 64, "one 128-byte row per wave and block");
  const int64_t f = p.f;
  const int64_t colbase = n0 + wn * C::WTN;
  const int64_t bytes = (static_cast<int64_t>(rows) * f - colbase) * 2;
  const int64_t o = row0 * f + colbase;
  const __amdgpu_buffer_rsrc_t rg = rsrc(static_cast<const uint16_t*>(p.hg) + o, bytes);
  const __amdgpu_buffer_rsrc_t ru = rsrc(static_cast<const uint16_t*>(p.hu) + o, bytes);
  const int rbase = wm * C::WTM + i * 32;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = u * 8 + (lane >> 3);
    const int q = (lane & 7) ^ ((r >> 1) & 7);
    const int voff = static_cast<int>(((rbase + r) * f + q * 8) * 2);
    dma16(rg, buf + u * 512, voff);
    dma16(ru, buf + 2048 + u * 512, voff);
  }
}

template <class C>
__device__ __forceinline__ void g3_block(const Acc<C>& acc, const FfnArgs& p, int64_t row0, int rows, int n0,
                                         int cols, int i, const uint16_t* buf, int wm, int wn, int lane) {
  const int rl = lane & 31, h = lane >> 5;
  const int64_t f = p.f;
  uint16_t* dg = static_cast<uint16_t*>(p.o_dhg) + row0 * f + n0;
  uint16_t* du = static_cast<uint16_t*>(p.o_dhu) + row0 * f + n0;
  const int row = wm * C::WTM + i * 32 + rl;
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    float da[2][8];
    to_chunks(acc[i][j], da);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = 4 * j + 2 * c + h;  // 16-byte chunk of the wave's 64 columns
      const int ph = q ^ ((rl >> 1) & 7);
      const uint4 vg = lds_get16(buf + rl * 64 + ph * 8);
      const uint4 vu = lds_get16(buf + 2048 + rl * 64 + ph * 8);
      const int col = wn * C::WTN + q * 8;
      if (row < rows && col < cols) {
        float g[8], u[8], og[8], ou[8];
        Elem<uint16_t>::unpack(vg, g);
        Elem<uint16_t>::unpack(vu, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = sigmoid_f(g[e]);
          ou[e] = da[c][e] * g[e] * sg;
          og[e] = da[c][e] * u[e] * sg * (1.0f + g[e] * (1.0f - sg));
        }
        const int64_t o = row * f + col;
        store16<false>(dg + o, pack8(og));
        store16<false>(du + o, pack8(ou));
      }
    }
  }
}

// Plain output of the 256 x 256 tiles through LDS, as whole lines.  Each wave
// writes two 32-row blocks of its 128 x 64 sub-tile as bf16 into its 8 KB of
// the idle ring slot (row r keeps 16-byte chunk q at q ^ ((r >> 1) & 7):
// conflict-free both ways), reads them back eight whole 128-byte rows per
// instruction and stores those; twice.  Only this wave touches its buffer.
// NT: the non-temporal hint, for outputs no kernel reads soon (the weight
// gradients); G5's dX rows, read by the dispatch backward right after, keep
// ordinary stores.
template <class C, bool NT = true>
__device__ __forceinline__ void epi_staged_store(const Acc<C>& acc, uint16_t* buf, uint16_t* dst, int64_t ld,
                                                 int rows_valid, int cols_valid, int lane, int wm, int wn) {
  static_assert(C::WTN == 64 && C::TM % 2 == 0, "two 32 x 64 blocks per pass");
  const int rl = lane & 31, h = lane >> 5;
#pragma unroll
  for (int pass = 0; pass < C::TM / 2; ++pass) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        float v[2][8];
        to_chunks(acc[2 * pass + b][j], v);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int q = 4 * j + 2 * c + h;
          lds_put16(buf + b * 2048 + rl * 64 + (q ^ ((rl >> 1) & 7)) * 8, pack8(v[c]));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = u * 8 + (lane >> 3), p = lane & 7;
        const int q = p ^ ((r >> 1) & 7);
        const uint4 v = lds_get16(buf + b * 2048 + r * 64 + p * 8);
        const int row = wm * C::WTM + (2 * pass + b) * 32 + r, col = wn * C::WTN + q * 8;
        if (row < rows_valid && col < cols_valid) {
          if (NT) store16_nt(dst + row * ld + col, v);
          else *reinterpret_cast<uint4*>(dst + row * ld + col) = v;
        }
      }
  }
}

}  // namespace gemm
}  // namespace moe
