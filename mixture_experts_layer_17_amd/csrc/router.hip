// Router logits l = x W_r and their backward (the linear router; the pages give
// no router formula).  Small next to the expert GEMMs: the router is a [d, E]
// matrix with E <= 256, so these are plain fp32-FMA kernels.
//
// For E <= 16 (the linear-router workloads) W_r is staged in LDS and one wave
// owns one token: 16-byte activation loads, per-lane expert sums reduced across
// the wave (forward) or per-feature dot products over the experts (dx).  Wider
// routers use plain one-thread-per-output kernels.  dW_r = x^T dl is reduced in
// two deterministic passes: fixed 64-token chunks write fp32 partials to the
// workspace, then one thread per (feature, expert) sums them in chunk order.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kChunk = 32;        // tokens per dW_r partial
constexpr int kTokPerBlk = 32;    // tokens per workgroup in the wave-per-token kernels
constexpr size_t kMaxLdsW = 64 * 1024;

// Row i of W_r [d, E] widened to fp32 from LDS (EP >= E experts, zero padded),
// read as 16-byte vectors (EP * sizeof(T) is a multiple of 16).
template <typename T, int EP>
__device__ __forceinline__ void w_row(const T* __restrict__ wl, int i, float* o) {
  constexpr int V = Elem<T>::kVec;
  static_assert(EP % V == 0, "W_r rows must be whole 16-byte vectors");
  const uint4* r = reinterpret_cast<const uint4*>(wl + static_cast<int64_t>(i) * EP);
#pragma unroll
  for (int q = 0; q < EP / V; ++q) Elem<T>::unpack(r[q], o + q * V);
}

template <typename T, int EP>
__device__ __forceinline__ void stage_w(const T* __restrict__ w, int d, int E, T* wl) {
  for (int i = threadIdx.x; i < d * EP; i += blockDim.x) {
    const int r = i / EP, e = i - r * EP;
    if constexpr (sizeof(T) == 4)
      wl[i] = e < E ? w[static_cast<int64_t>(r) * E + e] : 0.f;
    else
      wl[i] = e < E ? w[static_cast<int64_t>(r) * E + e] : static_cast<T>(0);
  }
  __syncthreads();
}

// logits: one wave per token, 16-byte activation loads, per-lane expert sums
// reduced across the wave.  W_r is staged in LDS once per workgroup.
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_fwd_fast_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                             int64_t Tn, int d, int E, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* wl = reinterpret_cast<T*>(smem_raw);
  stage_w<T, EP>(w, d, E, wl);
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = d / V;
  for (int tl = wave; tl < kTokPerBlk; tl += 4) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlk + tl;
    if (t >= Tn) break;
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * d);
    for (int c = lane; c < nvec; c += 64) {
      float xv[V];
      Elem<T>::unpack(xr[c], xv);
#pragma unroll
      for (int q = 0; q < V; ++q) {
        float wr[EP];
        w_row<T, EP>(wl, c * V + q, wr);
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[e] += xv[q] * wr[e];
      }
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = wave_sum(acc[e]);
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (lane == e && e < E) logits[t * E + e] = acc[e];
  }
}

// dx (+)= dl W_r^T: one wave per token, 16-byte output vectors.
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_bwd_dx_fast_kernel(const float* __restrict__ dl,
                                                                const T* __restrict__ w, int64_t Tn, int d, int E,
                                                                T* __restrict__ dx, int accumulate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* wl = reinterpret_cast<T*>(smem_raw);
  stage_w<T, EP>(w, d, E, wl);
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = d / V;
  for (int tl = wave; tl < kTokPerBlk; tl += 4) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlk + tl;
    if (t >= Tn) break;
    float g[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) g[e] = e < E ? dl[t * E + e] : 0.f;
    uint4* out = reinterpret_cast<uint4*>(dx + t * d);
    for (int c = lane; c < nvec; c += 64) {
      float o[V];
      if (accumulate) {
        Elem<T>::unpack(out[c], o);
      } else {
#pragma unroll
        for (int q = 0; q < V; ++q) o[q] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < V; ++q) {
        float wr[EP];
        w_row<T, EP>(wl, c * V + q, wr);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EP; ++e) s += g[e] * wr[e];
        o[q] += s;
      }
      out[c] = Elem<T>::pack(o);
    }
  }
}

// dW_r partials over fixed 64-token chunks: thread = 8 consecutive features x
// all experts; the chunk's dl rows are staged in LDS.
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_bwd_dw_fast_kernel(const T* __restrict__ x,
                                                                const float* __restrict__ dl, int64_t Tn, int d,
                                                                int E, float* __restrict__ part) {
  __shared__ float dls[kChunk * EP];
  const int64_t c = blockIdx.x;
  const int64_t t0 = c * kChunk;
  const int nt = static_cast<int>(Tn - t0 < kChunk ? Tn - t0 : kChunk);
  for (int i = threadIdx.x; i < kChunk * EP; i += blockDim.x) {
    const int r = i / EP, e = i - r * EP;
    dls[i] = (r < nt && e < E) ? dl[(t0 + r) * E + e] : 0.f;
  }
  __syncthreads();
  const int i0 = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (i0 >= d) return;
  float acc[8][EP];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[q][e] = 0.f;
  for (int r = 0; r < nt; ++r) {
    float xv[8];
    if constexpr (sizeof(T) == 2) {
      Elem<T>::unpack(*reinterpret_cast<const uint4*>(x + (t0 + r) * d + i0), xv);
    } else {
      Elem<T>::unpack(reinterpret_cast<const uint4*>(x + (t0 + r) * d + i0)[0], xv);
      Elem<T>::unpack(reinterpret_cast<const uint4*>(x + (t0 + r) * d + i0)[1], xv + 4);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[q][e] += xv[q] * dls[r * EP + e];
  }
  const int64_t n = static_cast<int64_t>(d) * E;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (e < E) part[c * n + static_cast<int64_t>(i0 + q) * E + e] = acc[q][e];
}

template <typename T>
__global__ __launch_bounds__(256) void router_fwd_kernel(const T* __restrict__ x, const T* __restrict__ w, int64_t Tn,
                                                        int d, int E, float* __restrict__ logits) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= Tn * E) return;
  const int64_t t = i / E;
  const int e = static_cast<int>(i - t * E);
  const T* xr = x + t * d;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc += Elem<T>::load1(xr, c) * Elem<T>::load1(w, static_cast<int64_t>(c) * E + e);
  logits[i] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void router_bwd_dx_kernel(const float* __restrict__ dl, const T* __restrict__ w,
                                                           int64_t Tn, int d, int E, T* __restrict__ dx,
                                                           int accumulate) {
  const int nch = d / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= Tn * nch) return;
  const int64_t t = i / nch;
  const int c0 = static_cast<int>(i - t * nch) * 8;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  const float* dlr = dl + t * E;
  for (int e = 0; e < E; ++e) {
    const float g = dlr[e];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += g * Elem<T>::load1(w, static_cast<int64_t>(c0 + q) * E + e);
  }
  T* out = dx + t * d + c0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float prev = accumulate ? Elem<T>::load1(out, q) : 0.f;
    Elem<T>::store1(out, q, prev + acc[q]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void router_bwd_dw_partial_kernel(const T* __restrict__ x,
                                                                   const float* __restrict__ dl, int64_t Tn, int d,
                                                                   int E, float* __restrict__ part) {
  // part[c][i][e] = sum over tokens t of chunk c of x[t][i] * dl[t][e]
  const int64_t n = static_cast<int64_t>(d) * E;
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t c = blockIdx.y;
  if (gi >= n) return;
  const int i = static_cast<int>(gi / E);
  const int e = static_cast<int>(gi - static_cast<int64_t>(i) * E);
  const int64_t t0 = c * kChunk;
  const int64_t t1 = t0 + kChunk < Tn ? t0 + kChunk : Tn;
  float acc = 0.f;
  for (int64_t t = t0; t < t1; ++t) acc += Elem<T>::load1(x, t * d + i) * dl[t * E + e];
  part[c * n + gi] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void router_bwd_dw_reduce_kernel(const float* __restrict__ part, int nchunk,
                                                                  int64_t n, T* __restrict__ dw) {
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gi >= n) return;
  // fixed chunk order; eight loads in flight per step
  float acc = 0.f;
  int c = 0;
  for (; c + 8 <= nchunk; c += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = part[(c + q) * n + gi];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += v[q];
  }
  for (; c < nchunk; ++c) acc += part[c * n + gi];
  Elem<T>::store1(dw, gi, acc);
}

bool router_ok(int dtype, int64_t T, int d, int E) {
  return (dtype == MOE_F32 || dtype == MOE_BF16) && T >= 0 && d > 0 && d % 8 == 0 && E >= 1 && E <= kMaxE &&
         T < (1ll << 31);
}

template <typename T, int EP>
bool fast_ok(int d, int E) {
  return E <= EP && static_cast<size_t>(d) * EP * sizeof(T) <= kMaxLdsW;
}

template <typename T>
int router_fwd_impl(const void* x, const void* w_r, int64_t Tn, int d, int E, float* logits, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(cdiv(Tn, kTokPerBlk)));
  if (fast_ok<T, 8>(d, E)) {
    MOE_LAUNCH("router_logits", (router_fwd_fast_kernel<T, 8>), g, dim3(256), static_cast<size_t>(d) * 8 * sizeof(T),
               s, static_cast<const T*>(x), static_cast<const T*>(w_r), Tn, d, E, logits);
  } else if (fast_ok<T, 16>(d, E)) {
    MOE_LAUNCH("router_logits", (router_fwd_fast_kernel<T, 16>), g, dim3(256),
               static_cast<size_t>(d) * 16 * sizeof(T), s, static_cast<const T*>(x), static_cast<const T*>(w_r), Tn,
               d, E, logits);
  } else {
    const int64_t n = Tn * E;
    MOE_LAUNCH("router_logits", router_fwd_kernel<T>, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s,
               static_cast<const T*>(x), static_cast<const T*>(w_r), Tn, d, E, logits);
  }
  return launch_status();
}

template <typename T>
int router_bwd_impl(const void* x, const void* w_r, const float* dlogits, int64_t Tn, int d, int E, void* dx,
                    int accumulate_dx, void* dw_r, float* part, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(cdiv(Tn, kTokPerBlk)));
  const int64_t n = static_cast<int64_t>(d) * E;
  const int nchunk = static_cast<int>(cdiv(Tn, kChunk));
  const dim3 gdw(static_cast<unsigned>(nchunk), static_cast<unsigned>(cdiv(d / 8, 256)));
  if (fast_ok<T, 8>(d, E)) {
    MOE_LAUNCH("router_bwd_dx", (router_bwd_dx_fast_kernel<T, 8>), g, dim3(256),
               static_cast<size_t>(d) * 8 * sizeof(T), s, dlogits, static_cast<const T*>(w_r), Tn, d, E,
               static_cast<T*>(dx), accumulate_dx);
    MOE_LAUNCH("router_bwd_dw_partial", (router_bwd_dw_fast_kernel<T, 8>), gdw, dim3(256), 0, s,
               static_cast<const T*>(x), dlogits, Tn, d, E, part);
  } else if (fast_ok<T, 16>(d, E)) {
    MOE_LAUNCH("router_bwd_dx", (router_bwd_dx_fast_kernel<T, 16>), g, dim3(256),
               static_cast<size_t>(d) * 16 * sizeof(T), s, dlogits, static_cast<const T*>(w_r), Tn, d, E,
               static_cast<T*>(dx), accumulate_dx);
    MOE_LAUNCH("router_bwd_dw_partial", (router_bwd_dw_fast_kernel<T, 16>), gdw, dim3(256), 0, s,
               static_cast<const T*>(x), dlogits, Tn, d, E, part);
  } else {
    const int64_t nch = Tn * (d / 8);
    MOE_LAUNCH("router_bwd_dx", router_bwd_dx_kernel<T>, dim3(static_cast<unsigned>(cdiv(nch, 256))), dim3(256), 0,
               s, dlogits, static_cast<const T*>(w_r), Tn, d, E, static_cast<T*>(dx), accumulate_dx);
    MOE_LAUNCH("router_bwd_dw_partial", router_bwd_dw_partial_kernel<T>,
               dim3(static_cast<unsigned>(cdiv(n, 256)), nchunk), dim3(256), 0, s, static_cast<const T*>(x), dlogits,
               Tn, d, E, part);
  }
  MOE_LAUNCH("router_bwd_dw_reduce", router_bwd_dw_reduce_kernel<T>, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s,
                     part, nchunk, n, static_cast<T*>(dw_r));
  return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_router_logits(const void* x, const void* w_r, int dtype, int64_t T, int32_t d, int32_t E,
                                 float* logits, void* stream) {
  if (!router_ok(dtype, T, d, E)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !w_r || !logits) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MOE_F32) return router_fwd_impl<float>(x, w_r, T, d, E, logits, s);
  return router_fwd_impl<uint16_t>(x, w_r, T, d, E, logits, s);
}

extern "C" size_t moe_router_logits_bwd_workspace(int64_t T, int32_t d, int32_t E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  return static_cast<size_t>(cdiv(T, kChunk) > 0 ? cdiv(T, kChunk) : 1) * d * E * sizeof(float);
}

extern "C" int moe_router_logits_bwd(const void* x, const void* w_r, int dtype, const float* dlogits, int64_t T,
                                     int32_t d, int32_t E, void* dx, int accumulate_dx, void* dw_r, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!router_ok(dtype, T, d, E)) return MOE_EINVAL;
  if (!x || !w_r || !dlogits || !dx || !dw_r || !ws) return MOE_EINVAL;
  if (ws_bytes < moe_router_logits_bwd_workspace(T, d, E)) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    // Overwrite semantics: dW_r of an empty batch is zero.
    const size_t bytes = static_cast<size_t>(d) * E * (dtype == MOE_F32 ? 4 : 2);
    launch_zero(dw_r, bytes, s);
    return launch_status();
  }
  if (dtype == MOE_F32)
    return router_bwd_impl<float>(x, w_r, dlogits, T, d, E, dx, accumulate_dx, dw_r, static_cast<float*>(ws), s);
  return router_bwd_impl<uint16_t>(x, w_r, dlogits, T, d, E, dx, accumulate_dx, dw_r, static_cast<float*>(ws), s);
}
