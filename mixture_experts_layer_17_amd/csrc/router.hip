// Router logits l = x W_r and their backward (the linear router; the pages give
// no router formula).  Small next to the expert GEMMs: the router is a [d, E]
// matrix with E <= 256, so these are plain fp32-FMA kernels.
//
// Forward: one thread per (token, expert), fp32 accumulation in index order.
// Backward: dx (+)= dl W_r^T one thread per (token, 8 features); dW_r = x^T dl in
// two deterministic passes: fixed 256-token chunks write fp32 partials to the
// workspace, then one thread per (feature, expert) sums the partials in chunk
// order.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kChunk = 256;

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
  float acc = 0.f;
  for (int c = 0; c < nchunk; ++c) acc += part[c * n + gi];
  Elem<T>::store1(dw, gi, acc);
}

bool router_ok(int dtype, int64_t T, int d, int E) {
  return (dtype == MOE_F32 || dtype == MOE_BF16) && T >= 0 && d > 0 && d % 8 == 0 && E >= 1 && E <= kMaxE &&
         T < (1ll << 31);
}

template <typename T>
int router_bwd_impl(const void* x, const void* w_r, const float* dlogits, int64_t Tn, int d, int E, void* dx,
                    int accumulate_dx, void* dw_r, float* part, hipStream_t s) {
  const int64_t nch = Tn * (d / 8);
  MOE_LAUNCH("router_bwd_dx", router_bwd_dx_kernel<T>, dim3(static_cast<unsigned>(cdiv(nch, 256))), dim3(256), 0, s, dlogits,
                     static_cast<const T*>(w_r), Tn, d, E, static_cast<T*>(dx), accumulate_dx);
  const int64_t n = static_cast<int64_t>(d) * E;
  const int nchunk = static_cast<int>(cdiv(Tn, kChunk));
  MOE_LAUNCH("router_bwd_dw_partial", router_bwd_dw_partial_kernel<T>, dim3(static_cast<unsigned>(cdiv(n, 256)), nchunk), dim3(256),
                     0, s, static_cast<const T*>(x), dlogits, Tn, d, E, part);
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
  const int64_t n = T * E;
  if (dtype == MOE_F32)
    MOE_LAUNCH("router_logits", router_fwd_kernel<float>, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w_r), T, d, E, logits);
  else
    MOE_LAUNCH("router_logits", router_fwd_kernel<uint16_t>, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_r), T, d, E, logits);
  return launch_status();
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
