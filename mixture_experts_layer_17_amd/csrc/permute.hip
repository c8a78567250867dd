// Row-wise dispatch into the expert-major buffer and the weighted combine, with
// their backward passes.
//
// Olmo-core 3 announcement, "Scaling and optimizing MoE training": routed data
// is written directly into the experts' input buffers, keeping the reordering
// work minimal; the gains of MXFP8 came mostly from the expert FFN and from
// moving data between experts, so these kernels are pure HBM streams.
//
// All four kernels are token-major: each token row is read (or written) exactly
// once, by one wave (the combine and the dispatch backward: one wave per part of
// 64 x 4 vectors of the row), and the k expert-buffer rows it touches are whole
// 16-byte-vector rows.  Every access is a 16-byte vector, 1 KiB per wave
// instruction.  The k row indices of a token are wave-uniform scalar loads.
// Sums run in fp32 in slot order j = 0..k-1.
#include "mx_common.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;       // tokens per workgroup
constexpr int kDispatchWaves = 8;  // tokens per workgroup of the plain dispatch (measured 4-5% faster than 4)
constexpr int kMaxChunks = 16;  // 16-byte vectors per lane held in registers (d <= 8192 bf16)

template <typename T>
__global__ __launch_bounds__(64 * kDispatchWaves) void dispatch_kernel(const T* __restrict__ x, int64_t Tn, int d,
                                                                      int k, const int32_t* __restrict__ perm_dst,
                                                                      T* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kDispatchWaves + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nvec = d / Elem<T>::kVec;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  int rows[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) rows[j] = j < k ? perm_dst[t * k + j] : 0;
  for (int c0 = 0; c0 < nvec; c0 += 64 * kMaxChunks) {
    uint4 v[kMaxChunks];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = c0 + i * 64 + lane;
      if (c < nvec) v[i] = src[c];
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      uint4* dst = reinterpret_cast<uint4*>(x_perm + static_cast<int64_t>(rows[j]) * d);
#pragma unroll
      for (int i = 0; i < kMaxChunks; ++i) {
        const int c = c0 + i * 64 + lane;
        if (c < nvec) store16_nt(dst + c, v[i]);
      }
    }
  }
}

// Up to KP slots per token (k <= KP); every lane loads kBatch 16-byte vectors of
// each of the k rows before it uses any, so a wave keeps k * kBatch KiB in flight.
constexpr int kBatch = 4;

template <typename T, int KP>
__global__ __launch_bounds__(64 * kWaves) void gather_sum_kernel(const T* __restrict__ src_rows, int64_t Tn, int d,
                                                                int k, const int32_t* __restrict__ perm_dst,
                                                                const float* __restrict__ gates,
                                                                T* __restrict__ out) {
  // out[t] = sum_j w_j * src_rows[perm_dst[t*k+j]], w_j = gates[t,j] or 1 (gates == nullptr).  A token's row
  // is split into parts of 64 x kBatch vectors, one wave each, so that every wave issues all of its loads at
  // once (with one wave per token, d = 4096 took two rounds of loads per wave: 4.8 against 5.8 TB/s at d = 2048)
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nvec = d / V;
  const int parts = (nvec + 64 * kBatch - 1) / (64 * kBatch);
  const int64_t wv = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t t = wv / parts;
  if (t >= Tn) return;
  const int cbeg = static_cast<int>(wv - t * parts) * 64 * kBatch;
  const uint4* rows[KP];
  float w[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    rows[j] = reinterpret_cast<const uint4*>(src_rows + static_cast<int64_t>(j < k ? perm_dst[t * k + j] : 0) * d);
    w[j] = j < k ? (gates ? gates[t * k + j] : 1.0f) : 0.f;
  }
  uint4* dst = reinterpret_cast<uint4*>(out + t * d);
  {
    const int c0 = cbeg;
    uint4 v[KP][kBatch];
#pragma unroll
    for (int j = 0; j < KP; ++j)
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int c = c0 + b * 64 + lane;
        if (j < k && c < nvec) v[j][b] = rows[j][c];
      }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * 64 + lane;
      if (c >= nvec) break;
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        if (j < k) {
          float f[V];
          Elem<T>::unpack(v[j][b], f);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += w[j] * f[i];
        }
      }
      // streaming stores: the layer output and dX are not read again in the step, and cached stores of them
      // evict the expert rows that the combine backward reads next (144 -> 126 us for it at E = 128, d = 4096)
      store16_nt(dst + c, Elem<T>::pack(acc));
    }
  }
}

// With WRITE_DY false only dgates is computed (dY goes to its MX layouts
// through mx_gather_kernel instead).
template <typename T, int KP, bool WRITE_DY = true>
__global__ __launch_bounds__(64 * kWaves) void combine_bwd_kernel(const T* __restrict__ dout,
                                                                 const T* __restrict__ y_perm, int64_t Tn, int d,
                                                                 int k, const int32_t* __restrict__ perm_dst,
                                                                 const float* __restrict__ gates,
                                                                 T* __restrict__ dy_perm, float* __restrict__ dgates) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nvec = d / V;
  int64_t rows[KP];
  float g[KP], dot[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    rows[j] = static_cast<int64_t>(j < k ? perm_dst[t * k + j] : 0) * d;
    g[j] = j < k ? gates[t * k + j] : 0.f;
    dot[j] = 0.f;
  }
  const uint4* src = reinterpret_cast<const uint4*>(dout + t * d);
  for (int c0 = 0; c0 < nvec; c0 += 64 * kBatch) {
    uint4 ov[kBatch], yv[KP][kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * 64 + lane;
      if (c < nvec) ov[b] = src[c];
    }
#pragma unroll
    for (int j = 0; j < KP; ++j)
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int c = c0 + b * 64 + lane;
        if (j < k && c < nvec) yv[j][b] = reinterpret_cast<const uint4*>(y_perm + rows[j])[c];
      }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * 64 + lane;
      if (c >= nvec) break;
      float o[V];
      Elem<T>::unpack(ov[b], o);
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        if (j < k) {
          float y[V], sv[V];
          Elem<T>::unpack(yv[j][b], y);
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < V; ++i) { p += o[i] * y[i]; sv[i] = g[j] * o[i]; }
          dot[j] += p;
          if constexpr (WRITE_DY) reinterpret_cast<uint4*>(dy_perm + rows[j])[c] = Elem<T>::pack(sv);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    if (j < k) {
      const float s = wave_sum(dot[j]);
      if (lane == 0) dgates[t * k + j] = s;
    }
  }
}

// MX rows layout of one expert-buffer row segment, computed where the row is
// written (Olmo-core 3 announcement, "Scaling and optimizing MoE training":
// MXFP8 gains come from the expert FFN and from moving data between experts).
// Lane l holds 16-byte vector c (8 bf16 values, c = 64 i + l) of the row: four
// lanes form a 32-element block (amax over two lane exchanges), sixteen a group
// of four blocks whose E8M0 bytes make one 32-bit word (two more exchanges).
// Returns the 8 E4M3 codes; *word is the group's scale word (valid in every lane).
__device__ __forceinline__ uint2 mx_encode8(const float* v, uint32_t* word, int c) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = mx_block_exponent(amax);
  const float inv = mx_inv_scale(e);
  uint32_t sw = static_cast<uint32_t>(e + 127) << (8 * ((c >> 2) & 3));
  sw |= __shfl_xor(sw, 4, 64);
  sw |= __shfl_xor(sw, 8, 64);
  *word = sw;
  return make_uint2(e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                    e4m3_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv));
}

// Dispatch that also writes the MX rows layout of every expert row: codes
// q[row * d + col], scale word of (row, group G) at sw[G * R + row].  bf16,
// d % 128 == 0 (a group never straddles lanes of different waves).
__global__ __launch_bounds__(64 * kWaves) void dispatch_mx_kernel(const uint16_t* __restrict__ x, int64_t Tn, int d,
                                                                 int k, const int32_t* __restrict__ perm_dst,
                                                                 uint16_t* __restrict__ x_perm,
                                                                 uint8_t* __restrict__ q, uint32_t* __restrict__ sw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int64_t R = Tn * k;
  const int nvec = d / 8;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  int rows[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) rows[j] = j < k ? perm_dst[t * k + j] : 0;
  for (int c0 = 0; c0 < nvec; c0 += 64 * kMaxChunks) {
    uint4 v[kMaxChunks];
    uint2 cq[kMaxChunks];
    uint32_t cw[kMaxChunks];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = c0 + i * 64 + lane;
      if (c0 + i * 64 < nvec) {  // wave-uniform: whole groups of 16 lanes are valid together
        v[i] = c < nvec ? src[c] : make_uint4(0, 0, 0, 0);
        float f[8];
        Elem<uint16_t>::unpack(v[i], f);
        cq[i] = mx_encode8(f, &cw[i], c);
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const int64_t row = rows[j];
      uint4* dst = reinterpret_cast<uint4*>(x_perm + row * d);
      uint2* dq = reinterpret_cast<uint2*>(q + row * d);
#pragma unroll
      for (int i = 0; i < kMaxChunks; ++i) {
        const int c = c0 + i * 64 + lane;
        if (c < nvec) {
          store16_nt(dst + c, v[i]);
          dq[c] = cq[i];
          if ((c & 15) == 0) sw[static_cast<int64_t>(c >> 4) * R + row] = cw[i];
        }
      }
    }
  }
}

// combine_bwd that also writes the MX rows layout of dy_perm (codes and scale
// words as in dispatch_mx_kernel), encoded from the stored bf16 values.
// bf16, d % 128 == 0.
template <int KP>
__global__ __launch_bounds__(64 * kWaves) void combine_bwd_mx_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y_perm, int64_t Tn, int d, int k,
    const int32_t* __restrict__ perm_dst, const float* __restrict__ gates, uint16_t* __restrict__ dy_perm,
    float* __restrict__ dgates, uint8_t* __restrict__ q, uint32_t* __restrict__ sw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int64_t R = Tn * k;
  const int nvec = d / 8;
  int64_t rows[KP];
  float g[KP], dot[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    rows[j] = j < k ? perm_dst[t * k + j] : 0;
    g[j] = j < k ? gates[t * k + j] : 0.f;
    dot[j] = 0.f;
  }
  const uint4* src = reinterpret_cast<const uint4*>(dout + t * d);
  // wave-uniform trip counts; groups of 16 lanes are valid together (d % 128 == 0)
  for (int c0 = 0; c0 < nvec; c0 += 64 * kBatch) {
    uint4 ov[kBatch], yv[KP][kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * 64 + lane;
      ov[b] = c < nvec ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < KP; ++j)
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int c = c0 + b * 64 + lane;
        if (j < k) yv[j][b] = c < nvec ? reinterpret_cast<const uint4*>(y_perm + rows[j] * d)[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (c0 + b * 64 >= nvec) break;  // wave-uniform
      const int c = c0 + b * 64 + lane;
      const bool ok = c < nvec;
      float o[8];
      Elem<uint16_t>::unpack(ov[b], o);
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        if (j < k) {
          float y[8], sv[8];
          Elem<uint16_t>::unpack(yv[j][b], y);
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) { p += o[i] * y[i]; sv[i] = g[j] * o[i]; }
          dot[j] += p;
          const uint4 packed = Elem<uint16_t>::pack(sv);
          float r[8];
          Elem<uint16_t>::unpack(packed, r);  // quantise the stored (bf16) values
          uint32_t word;
          const uint2 cq = mx_encode8(r, &word, c);
          if (ok) {
            const int64_t row = rows[j];
            reinterpret_cast<uint4*>(dy_perm + row * d)[c] = packed;
            reinterpret_cast<uint2*>(q + row * d)[c] = cq;
            if ((c & 15) == 0) sw[static_cast<int64_t>(c >> 4) * R + row] = word;
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    if (j < k) {
      const float s = wave_sum(dot[j]);
      if (lane == 0) dgates[t * k + j] = s;
    }
  }
}

bool dims_ok(int dtype, int64_t T, int d, int k) {
  return (dtype == MOE_F32 || dtype == MOE_BF16) && T >= 0 && d > 0 && d % 8 == 0 && k >= 1 && k <= kMaxK &&
         T * k < (1ll << 31) && static_cast<int64_t>(d) * (T * k) < (1ll << 62);
}

inline dim3 grid_for(int64_t T) { return dim3(static_cast<unsigned>(cdiv(T, kWaves))); }
// waves per token row of gather_sum_kernel
template <typename T>
int gather_parts(int d) { return static_cast<int>(cdiv(d / Elem<T>::kVec, 64 * kBatch)); }

// k <= 4 (the workloads' top-4) takes the 4-slot kernels, whose register
// footprint allows twice the resident waves of the 8-slot ones.
template <typename T>
int launch_gather_sum(const char* name, const T* src, int64_t Tn, int d, int k, const int32_t* perm_dst,
                      const float* gates, T* out, hipStream_t s) {
  if (k <= 4)
    MOE_LAUNCH(name, (gather_sum_kernel<T, 4>), grid_for(Tn * gather_parts<T>(d)), dim3(64 * kWaves), 0, s, src, Tn, d,
               k, perm_dst, gates, out);
  else
    MOE_LAUNCH(name, (gather_sum_kernel<T, kMaxK>), grid_for(Tn * gather_parts<T>(d)), dim3(64 * kWaves), 0, s, src,
               Tn, d, k, perm_dst, gates, out);
  return launch_status();
}

template <typename T, bool WRITE_DY = true>
int launch_combine_bwd(const T* dout, const T* y_perm, int64_t Tn, int d, int k, const int32_t* perm_dst,
                       const float* gates, T* dy_perm, float* dgates, hipStream_t s) {
  if (k <= 4)
    MOE_LAUNCH("combine_bwd", (combine_bwd_kernel<T, 4, WRITE_DY>), grid_for(Tn), dim3(64 * kWaves), 0, s, dout,
               y_perm, Tn, d, k, perm_dst, gates, dy_perm, dgates);
  else
    MOE_LAUNCH("combine_bwd", (combine_bwd_kernel<T, kMaxK, WRITE_DY>), grid_for(Tn), dim3(64 * kWaves), 0, s, dout,
               y_perm, Tn, d, k, perm_dst, gates, dy_perm, dgates);
  return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_dispatch(const void* x, int dtype, int64_t T, int32_t d, int32_t k, const int32_t* perm_dst,
                            void* x_perm, void* stream) {
  if (!dims_ok(dtype, T, d, k)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !perm_dst || !x_perm || !aligned16(x) || !aligned16(x_perm)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(cdiv(T, kDispatchWaves)));
  if (dtype == MOE_F32)
    MOE_LAUNCH("dispatch", dispatch_kernel<float>, grid, dim3(64 * kDispatchWaves), 0, s, static_cast<const float*>(x),
               T, d, k, perm_dst, static_cast<float*>(x_perm));
  else
    MOE_LAUNCH("dispatch", dispatch_kernel<uint16_t>, grid, dim3(64 * kDispatchWaves), 0, s,
               static_cast<const uint16_t*>(x), T, d, k, perm_dst, static_cast<uint16_t*>(x_perm));
  return launch_status();
}

extern "C" size_t moe_mx_act_bytes(int64_t rows, int32_t cols) {
  if (rows < 0 || cols <= 0 || cols % 128) return 0;
  return align_up(static_cast<size_t>(rows) * cols, 256) + static_cast<size_t>(rows) * (cols / 32);
}

extern "C" int moe_dispatch_mx(const void* x, int64_t T, int32_t d, int32_t k, const int32_t* perm_dst,
                               void* x_perm, void* x_mx, void* stream) {
  if (!dims_ok(MOE_BF16, T, d, k)) return MOE_EINVAL;
  if (d % 128) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !perm_dst || !x_perm || !x_mx || !aligned16(x) || !aligned16(x_perm) || !aligned16(x_mx))
    return MOE_EINVAL;
  const int64_t R = T * k;
  uint8_t* q = static_cast<uint8_t*>(x_mx);
  uint32_t* sw = reinterpret_cast<uint32_t*>(q + align_up(static_cast<size_t>(R) * d, 256));
  MOE_LAUNCH("dispatch", dispatch_mx_kernel, grid_for(T), dim3(64 * kWaves), 0, static_cast<hipStream_t>(stream),
             static_cast<const uint16_t*>(x), T, d, k, perm_dst, static_cast<uint16_t*>(x_perm), q, sw);
  return launch_status();
}

extern "C" int moe_combine_bwd_mx(const void* dout, const void* y_perm, const float* gates, const int32_t* perm_dst,
                                  int64_t T, int32_t d, int32_t k, void* dy_perm, float* dgates, void* dy_mx,
                                  void* stream) {
  if (!dims_ok(MOE_BF16, T, d, k)) return MOE_EINVAL;
  if (d % 128) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dout || !y_perm || !gates || !perm_dst || !dy_perm || !dgates || !dy_mx || !aligned16(dout) ||
      !aligned16(y_perm) || !aligned16(dy_perm) || !aligned16(dy_mx))
    return MOE_EINVAL;
  const int64_t R = T * k;
  uint8_t* q = static_cast<uint8_t*>(dy_mx);
  uint32_t* sw = reinterpret_cast<uint32_t*>(q + align_up(static_cast<size_t>(R) * d, 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* dout16 = static_cast<const uint16_t*>(dout);
  const uint16_t* y16 = static_cast<const uint16_t*>(y_perm);
  uint16_t* dy16 = static_cast<uint16_t*>(dy_perm);
  if (k <= 4)
    MOE_LAUNCH("combine_bwd", combine_bwd_mx_kernel<4>, grid_for(T), dim3(64 * kWaves), 0, s, dout16, y16, T, d, k,
               perm_dst, gates, dy16, dgates, q, sw);
  else
    MOE_LAUNCH("combine_bwd", combine_bwd_mx_kernel<kMaxK>, grid_for(T), dim3(64 * kWaves), 0, s, dout16, y16, T, d,
               k, perm_dst, gates, dy16, dgates, q, sw);
  return launch_status();
}

extern "C" int64_t moe_mx_tok_rows(int64_t R, int32_t E) {
  if (R < 0 || E < 1 || E > kMaxE) return 0;
  return mx_token_rows(R, E);
}

extern "C" size_t moe_mx_tok_bytes(int64_t R, int32_t E, int32_t cols) {
  if (R < 0 || E < 1 || E > kMaxE || cols <= 0 || cols % 128) return 0;
  const int64_t rp = mx_token_rows(R, E);
  return align_up(static_cast<size_t>(rp) * cols, 256) + static_cast<size_t>(rp / 32) * cols;
}

namespace {
// Shared checks of the two token-axis calls; R = T k.
int tok_args_ok(int64_t T, int32_t d, int32_t k, int32_t E, const int32_t* perm_src, const int32_t* offsets,
                const int32_t* mx_blk_offsets, const void* rows_out, const void* mx, const void* mxt) {
  if (!dims_ok(MOE_BF16, T, d, k) || E < 1 || E > kMaxE) return MOE_EINVAL;
  if (d % 128) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!perm_src || !offsets || !mx_blk_offsets || !mx || !mxt || !aligned16(mx) || !aligned16(mxt) ||
      (rows_out && !aligned16(rows_out)))
    return MOE_EINVAL;
  return MOE_OK;
}
}  // namespace

extern "C" int moe_dispatch_mx_tok(const void* x, int64_t T, int32_t d, int32_t k, int32_t E, const int32_t* perm_src,
                                   const int32_t* offsets, const int32_t* mx_blk_offsets, void* x_perm, void* x_mx,
                                   void* x_mxt, void* stream) {
  const int st = tok_args_ok(T, d, k, E, perm_src, offsets, mx_blk_offsets, x_perm, x_mx, x_mxt);
  if (st != MOE_OK || T == 0) return st;
  if (!x || !aligned16(x)) return MOE_EINVAL;
  const int64_t R = T * k;
  uint8_t* q = static_cast<uint8_t*>(x_mx);
  uint8_t* qt = static_cast<uint8_t*>(x_mxt);
  launch_mx_gather(static_cast<const uint16_t*>(x), R, d, k, perm_src, nullptr, offsets, mx_blk_offsets, E,
                   static_cast<uint16_t*>(x_perm), q, q + align_up(static_cast<size_t>(R) * d, 256), qt,
                   qt + align_up(static_cast<size_t>(mx_token_rows(R, E)) * d, 256), static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" int moe_combine_bwd_mx_tok(const void* dout, const void* y_perm, const float* gates,
                                      const int32_t* perm_dst, const int32_t* perm_src, const int32_t* offsets,
                                      const int32_t* mx_blk_offsets, int64_t T, int32_t d, int32_t k, int32_t E,
                                      void* dy_perm, float* dgates, void* dy_mx, void* dy_mxt, void* stream) {
  const int st = tok_args_ok(T, d, k, E, perm_src, offsets, mx_blk_offsets, dy_perm, dy_mx, dy_mxt);
  if (st != MOE_OK || T == 0) return st;
  if (!dout || !y_perm || !gates || !perm_dst || !dgates || !aligned16(dout) || !aligned16(y_perm)) return MOE_EINVAL;
  const int64_t R = T * k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* dout16 = static_cast<const uint16_t*>(dout);
  // dgates (token-major: each token's k dot products), then dY = gate x dout into both MX layouts
  const int r = launch_combine_bwd<uint16_t, false>(dout16, static_cast<const uint16_t*>(y_perm), T, d, k, perm_dst,
                                                    gates, nullptr, dgates, s);
  if (r != MOE_OK) return r;
  uint8_t* q = static_cast<uint8_t*>(dy_mx);
  uint8_t* qt = static_cast<uint8_t*>(dy_mxt);
  launch_mx_gather(dout16, R, d, k, perm_src, gates, offsets, mx_blk_offsets, E, static_cast<uint16_t*>(dy_perm), q,
                   q + align_up(static_cast<size_t>(R) * d, 256), qt,
                   qt + align_up(static_cast<size_t>(mx_token_rows(R, E)) * d, 256), s);
  return launch_status();
}

extern "C" int moe_dispatch_bwd(const void* dx_perm, int dtype, int64_t T, int32_t d, int32_t k,
                                const int32_t* perm_dst, void* dx, void* stream) {
  if (!dims_ok(dtype, T, d, k)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!dx_perm || !perm_dst || !dx || !aligned16(dx_perm) || !aligned16(dx)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MOE_F32)
    return launch_gather_sum("dispatch_bwd", static_cast<const float*>(dx_perm), T, d, k, perm_dst, nullptr,
                             static_cast<float*>(dx), s);
  return launch_gather_sum("dispatch_bwd", static_cast<const uint16_t*>(dx_perm), T, d, k, perm_dst, nullptr,
                           static_cast<uint16_t*>(dx), s);
}

extern "C" int moe_combine(const void* y_perm, int dtype, const float* gates, const int32_t* perm_dst, int64_t T,
                           int32_t d, int32_t k, void* out, void* stream) {
  if (!dims_ok(dtype, T, d, k)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!y_perm || !gates || !perm_dst || !out || !aligned16(y_perm) || !aligned16(out)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MOE_F32)
    return launch_gather_sum("combine", static_cast<const float*>(y_perm), T, d, k, perm_dst, gates,
                             static_cast<float*>(out), s);
  return launch_gather_sum("combine", static_cast<const uint16_t*>(y_perm), T, d, k, perm_dst, gates,
                           static_cast<uint16_t*>(out), s);
}

extern "C" int moe_combine_bwd(const void* dout, const void* y_perm, int dtype, const float* gates,
                               const int32_t* perm_dst, int64_t T, int32_t d, int32_t k, void* dy_perm,
                               float* dgates, void* stream) {
  if (!dims_ok(dtype, T, d, k)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!dout || !y_perm || !gates || !perm_dst || !dy_perm || !dgates || !aligned16(dout) || !aligned16(y_perm) ||
      !aligned16(dy_perm))
    return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MOE_F32)
    return launch_combine_bwd(static_cast<const float*>(dout), static_cast<const float*>(y_perm), T, d, k, perm_dst,
                              gates, static_cast<float*>(dy_perm), dgates, s);
  return launch_combine_bwd(static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y_perm), T, d, k,
                            perm_dst, gates, static_cast<uint16_t*>(dy_perm), dgates, s);
}
