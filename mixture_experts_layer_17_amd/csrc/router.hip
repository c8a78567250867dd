// Router logits l = x W_r and their backward (the linear router; the pages give
// no router formula).  Small next to the expert GEMMs: the router is a [d, E]
// matrix with E <= 256, so these are plain fp32-FMA kernels bound by reading x.
//
// For E <= 16 (the linear-router workloads) W_r is staged in LDS and one wave
// owns a token (two at a time, so that more loads are in flight): 16-byte
// activation loads, per-lane expert sums reduced across the wave (forward) or
// per-feature dot products over the experts (dx).  Wider routers use plain
// one-thread-per-output kernels.  dW_r = x^T dl is reduced in two
// deterministic passes: fixed token chunks write fp32 partials to the
// workspace, then the partials are summed in chunk order.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kChunk = 32;        // tokens per dW_r partial (generic path)
constexpr int kDwTok = 64;        // tokens per dW_r partial (E <= 16 path)
constexpr int kDwFeat = 512;      // features per workgroup of the E <= 16 dW_r path (64 lanes x 8)
constexpr int kTokPerBlk = 8;     // tokens per workgroup in the wave-per-token kernels (2 per wave; more
                                  // per workgroup measured slower: fewer workgroups to hide the loads)
constexpr int kTokPar = 2;        // tokens a wave works on at once
constexpr int kXBatch = 4;        // 16-byte activation vectors per lane and token loaded before any is used
constexpr int kDwBatch = 4;       // tokens per wave whose activation loads are in flight together (dW_r)
constexpr size_t kMaxLdsW = 64 * 1024;

// W_r [d, E] in LDS, widened per read.  Feature i = V*c + q (c: 16-byte vector
// of x, q: position in it) is stored at row q*nvec + c, so the lanes of a wave
// (consecutive c) read consecutive rows; rows hold EP >= E experts, zero padded.
template <typename T, int EP>
__device__ __forceinline__ void w_row(const T* __restrict__ wl, int nvec, int c, int q, float* o) {
  constexpr int V = Elem<T>::kVec;
  static_assert(EP % V == 0, "W_r rows must be whole 16-byte vectors");
  const uint4* r = reinterpret_cast<const uint4*>(wl + (static_cast<int64_t>(q) * nvec + c) * EP);
#pragma unroll
  for (int u = 0; u < EP / V; ++u) Elem<T>::unpack(r[u], o + u * V);
}

template <typename T, int EP>
__device__ __forceinline__ void stage_w(const T* __restrict__ w, int d, int E, T* wl) {
  constexpr int V = Elem<T>::kVec;
  const int nvec = d / V;
  if (E == EP) {
    // rows of W_r are whole 16-byte vectors: one vector load per (row, part)
    constexpr int P = EP / V;  // vectors per row
    constexpr int NB = 8;      // vectors per thread whose loads are in flight together
    const uint4* src = reinterpret_cast<const uint4*>(w);
    const int n = d * P;
    for (int i0 = threadIdx.x; i0 < n; i0 += NB * blockDim.x) {
      uint4 v[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = i0 + b * blockDim.x;
        v[b] = i < n ? src[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = i0 + b * blockDim.x;
        if (i >= n) break;
        const int r = i / P, u = i - r * P;
        const int c = r / V, q = r - c * V;
        reinterpret_cast<uint4*>(wl + (static_cast<int64_t>(q) * nvec + c) * EP)[u] = v[b];
      }
    }
    __syncthreads();
    return;
  }
  for (int i = threadIdx.x; i < d * EP; i += blockDim.x) {
    const int r = i / EP, e = i - r * EP;
    const int c = r / V, q = r - c * V;
    const int64_t o = (static_cast<int64_t>(q) * nvec + c) * EP + e;
    if constexpr (sizeof(T) == 4)
      wl[o] = e < E ? w[static_cast<int64_t>(r) * E + e] : 0.f;
    else
      wl[o] = e < E ? w[static_cast<int64_t>(r) * E + e] : static_cast<T>(0);
  }
  __syncthreads();
}

// logits: a wave takes kTokPar tokens at a time, 16-byte activation loads,
// per-lane expert sums reduced across the wave.  W_r is staged once per workgroup.
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_fwd_fast_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                             int64_t Tn, int d, int E, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* wl = reinterpret_cast<T*>(smem_raw);
  stage_w<T, EP>(w, d, E, wl);
  constexpr int V = Elem<T>::kVec;
  constexpr int kPerWave = kTokPerBlk / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = d / V;
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * kTokPerBlk + wave * kPerWave;
  for (int tt = 0; tt < kPerWave; tt += kTokPar) {
    float acc[kTokPar][EP];
#pragma unroll
    for (int p = 0; p < kTokPar; ++p)
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[p][e] = 0.f;
    for (int c0 = lane; c0 < nvec; c0 += 64 * kXBatch) {
      uint4 raw[kXBatch][kTokPar];  // every load of the batch in flight before the first is used
#pragma unroll
      for (int b = 0; b < kXBatch; ++b)
#pragma unroll
        for (int p = 0; p < kTokPar; ++p) {
          const int64_t t = tw + tt + p;
          const int c = c0 + b * 64;
          raw[b][p] = (t < Tn && c < nvec) ? reinterpret_cast<const uint4*>(x + t * d)[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int b = 0; b < kXBatch; ++b) {
        const int c = c0 + b * 64;
        if (c >= nvec) break;
        float xv[kTokPar][V];
#pragma unroll
        for (int p = 0; p < kTokPar; ++p) Elem<T>::unpack(raw[b][p], xv[p]);
#pragma unroll
        for (int q = 0; q < V; ++q) {
          float wr[EP];
          w_row<T, EP>(wl, nvec, c, q, wr);
#pragma unroll
          for (int p = 0; p < kTokPar; ++p)
#pragma unroll
            for (int e = 0; e < EP; ++e) acc[p][e] += xv[p][q] * wr[e];
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kTokPar; ++p) {
      const int64_t t = tw + tt + p;
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[p][e] = wave_sum(acc[p][e]);
      if (t < Tn) {
#pragma unroll
        for (int e = 0; e < EP; ++e)
          if (lane == e && e < E) logits[t * E + e] = acc[p][e];
      }
    }
  }
}

// bf16 logits on the packed dot product v_dot2_f32_bf16 (two bf16 products and
// an fp32 accumulate per instruction; the products of bf16 values are exact in
// fp32).  W_r is staged as pairs of consecutive features: the 32-bit word for
// expert e and feature pair (8c + 2pp, 8c + 2pp + 1) holds both bf16 values, so
// an activation word (two consecutive features) meets its weights without any
// unpacking.  Words for experts 4h .. 4h+3 form one 16-byte vector at
// ((h * 4 + pp) * nvec + c): the lanes of a wave (consecutive c) read
// consecutive vectors.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int EP>
__device__ __forceinline__ void stage_w_pairs(const uint16_t* __restrict__ w, int d, int E, uint4* wl) {
  static_assert(EP % 4 == 0, "whole 16-byte vectors of expert words");
  const int nvec = d / 8;
  const int npair = d / 2;
  if (E == EP) {
    // rows i, i + 1 of W_r are EP bf16 each (whole 16-byte vectors)
    constexpr int P = EP / 8;  // 16-byte vectors per row
    for (int m = threadIdx.x; m < npair; m += blockDim.x) {
      const int c = m >> 2, pp = m & 3;
      const uint4* r0 = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(2 * m) * EP);
      const uint4* r1 = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(2 * m + 1) * EP);
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const uint4 a = r0[u], b = r1[u];
        // experts 8u .. 8u+3 from words x, y; 8u+4 .. 8u+7 from z, w
        const uint4 lo = make_uint4((a.x & 0xFFFFu) | (b.x << 16), (a.x >> 16) | (b.x & 0xFFFF0000u),
                                    (a.y & 0xFFFFu) | (b.y << 16), (a.y >> 16) | (b.y & 0xFFFF0000u));
        const uint4 hi = make_uint4((a.z & 0xFFFFu) | (b.z << 16), (a.z >> 16) | (b.z & 0xFFFF0000u),
                                    (a.w & 0xFFFFu) | (b.w << 16), (a.w >> 16) | (b.w & 0xFFFF0000u));
        wl[((2 * u) * 4 + pp) * nvec + c] = lo;
        wl[((2 * u + 1) * 4 + pp) * nvec + c] = hi;
      }
    }
  } else {
    uint32_t* ww = reinterpret_cast<uint32_t*>(wl);
    for (int i = threadIdx.x; i < npair * EP; i += blockDim.x) {
      const int m = i / EP, e = i - m * EP;
      const int c = m >> 2, pp = m & 3, h = e >> 2, j = e & 3;
      uint32_t word = 0;
      if (e < E)
        word = static_cast<uint32_t>(w[static_cast<int64_t>(2 * m) * E + e]) |
               (static_cast<uint32_t>(w[static_cast<int64_t>(2 * m + 1) * E + e]) << 16);
      ww[((h * 4 + pp) * nvec + c) * 4 + j] = word;
    }
  }
  __syncthreads();
}

template <int EP>
__global__ __launch_bounds__(256) void router_fwd_dot2_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ w, int64_t Tn, int d,
                                                             int E, float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  uint4* wl = reinterpret_cast<uint4*>(smem_raw);
  stage_w_pairs<EP>(w, d, E, wl);
  constexpr int kPerWave = kTokPerBlk / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = d / 8;
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * kTokPerBlk + wave * kPerWave;
  for (int tt = 0; tt < kPerWave; tt += kTokPar) {
    float acc[kTokPar][EP];
#pragma unroll
    for (int p = 0; p < kTokPar; ++p)
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[p][e] = 0.f;
    for (int c0 = lane; c0 < nvec; c0 += 64 * kXBatch) {
      uint4 raw[kXBatch][kTokPar];  // every load of the batch in flight before the first is used
#pragma unroll
      for (int b = 0; b < kXBatch; ++b)
#pragma unroll
        for (int p = 0; p < kTokPar; ++p) {
          const int64_t t = tw + tt + p;
          const int c = c0 + b * 64;
          raw[b][p] = (t < Tn && c < nvec) ? reinterpret_cast<const uint4*>(x + t * d)[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int b = 0; b < kXBatch; ++b) {
        const int c = c0 + b * 64;
        if (c >= nvec) break;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
          for (int h = 0; h < EP / 4; ++h) {
            const uint4 wq = wl[(h * 4 + pp) * nvec + c];
#pragma unroll
            for (int p = 0; p < kTokPar; ++p) {
              const uint32_t xw = pp == 0 ? raw[b][p].x : pp == 1 ? raw[b][p].y : pp == 2 ? raw[b][p].z : raw[b][p].w;
              acc[p][4 * h + 0] = dot2_bf16(xw, wq.x, acc[p][4 * h + 0]);
              acc[p][4 * h + 1] = dot2_bf16(xw, wq.y, acc[p][4 * h + 1]);
              acc[p][4 * h + 2] = dot2_bf16(xw, wq.z, acc[p][4 * h + 2]);
              acc[p][4 * h + 3] = dot2_bf16(xw, wq.w, acc[p][4 * h + 3]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kTokPar; ++p) {
      const int64_t t = tw + tt + p;
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[p][e] = wave_sum(acc[p][e]);
      if (t < Tn) {
#pragma unroll
        for (int e = 0; e < EP; ++e)
          if (lane == e && e < E) logits[t * E + e] = acc[p][e];
      }
    }
  }
}

// dx (+)= dl W_r^T: a wave takes kTokPar tokens at a time, 16-byte output vectors.
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_bwd_dx_fast_kernel(const float* __restrict__ dl,
                                                                const T* __restrict__ w, int64_t Tn, int d, int E,
                                                                T* __restrict__ dx, int accumulate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* wl = reinterpret_cast<T*>(smem_raw);
  constexpr int V = Elem<T>::kVec;
  constexpr int kPerWave = kTokPerBlk / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = d / V;
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * kTokPerBlk + wave * kPerWave;
  uint4 raw[kXBatch][kTokPar];  // a batch's dx loads in flight before the first is used
  auto load_batch = [&](int tt, int c0) {
#pragma unroll
    for (int b = 0; b < kXBatch; ++b)
#pragma unroll
      for (int p = 0; p < kTokPar; ++p) {
        const int64_t t = tw + tt + p;
        const int c = c0 + b * 64;
        raw[b][p] = (accumulate && t < Tn && c < nvec) ? reinterpret_cast<const uint4*>(dx + t * d)[c]
                                                      : make_uint4(0, 0, 0, 0);
      }
  };
  load_batch(0, lane);  // the first batch is in flight while W_r is staged
  stage_w<T, EP>(w, d, E, wl);
  for (int tt = 0; tt < kPerWave; tt += kTokPar) {
    float g[kTokPar][EP];
#pragma unroll
    for (int p = 0; p < kTokPar; ++p) {
      const int64_t t = tw + tt + p;
#pragma unroll
      for (int e = 0; e < EP; ++e) g[p][e] = (t < Tn && e < E) ? dl[t * E + e] : 0.f;
    }
    for (int c0 = lane; c0 < nvec; c0 += 64 * kXBatch) {
      if (tt != 0 || c0 != lane) load_batch(tt, c0);
#pragma unroll
      for (int b = 0; b < kXBatch; ++b) {
        const int c = c0 + b * 64;
        if (c >= nvec) break;
        float o[kTokPar][V];
#pragma unroll
        for (int p = 0; p < kTokPar; ++p) Elem<T>::unpack(raw[b][p], o[p]);
#pragma unroll
        for (int q = 0; q < V; ++q) {
          float wr[EP];
          w_row<T, EP>(wl, nvec, c, q, wr);
#pragma unroll
          for (int p = 0; p < kTokPar; ++p) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EP; ++e) s += g[p][e] * wr[e];
            o[p][q] += s;
          }
        }
#pragma unroll
        for (int p = 0; p < kTokPar; ++p) {
          const int64_t t = tw + tt + p;
          if (t < Tn) reinterpret_cast<uint4*>(dx + t * d)[c] = Elem<T>::pack(o[p]);
        }
      }
    }
  }
}

// dW_r partials, E <= 16: workgroup = (64-token chunk, 512 features); wave w
// takes tokens w, w+4, ... of the chunk, lane = 8 consecutive features x EP
// experts.  The four waves' sums are added in wave order through LDS and
// written as part[chunk][feature group][q][lane][EP] (feature = group*512 +
// 8*lane + q), so every store of a wave is one contiguous run.
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_bwd_dw_fast_kernel(const T* __restrict__ x,
                                                                const float* __restrict__ dl, int64_t Tn, int d,
                                                                int E, float* __restrict__ part) {
  __shared__ float dls[kDwTok * EP];
  __shared__ float red[4][64][EP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int fg = blockIdx.y, ng = gridDim.y;
  const int64_t t0 = c * kDwTok;
  const int nt = static_cast<int>(Tn - t0 < kDwTok ? Tn - t0 : kDwTok);
  for (int i = tid; i < kDwTok * EP; i += blockDim.x) {
    const int r = i / EP, e = i - r * EP;
    dls[i] = (r < nt && e < E) ? dl[(t0 + r) * E + e] : 0.f;
  }
  __syncthreads();
  const int i0 = fg * kDwFeat + lane * 8;
  float acc[8][EP];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[q][e] = 0.f;
  if (i0 < d) {
    // tokens wave, wave + 4, ...: kDwBatch tokens' loads in flight before the first is used
    constexpr int NV = sizeof(T) == 2 ? 1 : 2;  // 16-byte vectors per 8 features
    for (int r0 = wave; r0 < nt; r0 += 4 * kDwBatch) {
      uint4 raw[kDwBatch][NV];
#pragma unroll
      for (int b = 0; b < kDwBatch; ++b) {
        const int r = r0 + 4 * b;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          raw[b][v] = r < nt ? reinterpret_cast<const uint4*>(x + (t0 + r) * d + i0)[v] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < kDwBatch; ++b) {
        const int r = r0 + 4 * b;
        if (r >= nt) break;
        float xv[8];
#pragma unroll
        for (int v = 0; v < NV; ++v) Elem<T>::unpack(raw[b][v], xv + v * (8 / NV));
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int e = 0; e < EP; ++e) acc[q][e] += xv[q] * dls[r * EP + e];
      }
    }
  }
  float* out = part + (c * ng + fg) * static_cast<int64_t>(kDwFeat * EP);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
#pragma unroll
    for (int e = 0; e < EP; ++e) red[wave][lane][e] = acc[q][e];
    __syncthreads();
    for (int o = tid; o < 64 * EP; o += blockDim.x) {
      const int l = o / EP, e = o - l * EP;
      out[q * 64 * EP + o] = ((red[0][l][e] + red[1][l][e]) + red[2][l][e]) + red[3][l][e];
    }
    __syncthreads();
  }
}

// Sum of the E <= 16 partials over the chunks.  A workgroup takes 64 outputs j
// (the partial layout's order); wave s sums the chunks c = s (mod 4) in
// increasing order, kReduceBatch loads in flight per lane, and the four wave
// sums are added in wave order: a fixed order, so identical inputs give
// identical bits.
constexpr int kReduceBatch = 16;

template <typename T, int EP>
__global__ __launch_bounds__(256) void router_bwd_dw_fast_reduce_kernel(const float* __restrict__ part, int nchunk,
                                                                       int ng, int d, int E, T* __restrict__ dw) {
  __shared__ float red[4][64];
  const int64_t per = static_cast<int64_t>(ng) * kDwFeat * EP;
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  float acc = 0.f;
  if (j < per) {
    for (int c0 = s; c0 < nchunk; c0 += 4 * kReduceBatch) {
      float v[kReduceBatch];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u) {
        const int c = c0 + 4 * u;
        v[u] = c < nchunk ? part[c * per + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (c0 + 4 * u < nchunk) acc += v[u];
    }
  }
  red[s][lane] = acc;
  __syncthreads();
  if (s != 0 || j >= per) return;
  const int e = static_cast<int>(j % EP);
  const int l = static_cast<int>((j / EP) % 64);
  const int q = static_cast<int>((j / (EP * 64)) % 8);
  const int fg = static_cast<int>(j / (EP * kDwFeat));
  const int i = fg * kDwFeat + l * 8 + q;
  if (e >= E || i >= d) return;
  Elem<T>::store1(dw, static_cast<int64_t>(i) * E + e, ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
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
  if constexpr (sizeof(T) == 2) {  // bf16: packed dot products on bf16 pairs
    if (fast_ok<T, 8>(d, E) || fast_ok<T, 16>(d, E)) {
      if (E <= 8)
        MOE_LAUNCH("router_logits", router_fwd_dot2_kernel<8>, g, dim3(256), static_cast<size_t>(d) * 8 * 2, s,
                   static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_r), Tn, d, E, logits);
      else
        MOE_LAUNCH("router_logits", router_fwd_dot2_kernel<16>, g, dim3(256), static_cast<size_t>(d) * 16 * 2, s,
                   static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_r), Tn, d, E, logits);
      return launch_status();
    }
  }
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

template <typename T, int EP>
void router_bwd_fast(const void* x, const void* w_r, const float* dlogits, int64_t Tn, int d, int E, void* dx,
                     int accumulate_dx, void* dw_r, float* part, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(cdiv(Tn, kTokPerBlk)));
  MOE_LAUNCH("router_bwd_dx", (router_bwd_dx_fast_kernel<T, EP>), g, dim3(256),
             static_cast<size_t>(d) * EP * sizeof(T), s, dlogits, static_cast<const T*>(w_r), Tn, d, E,
             static_cast<T*>(dx), accumulate_dx);
  const int nchunk = static_cast<int>(cdiv(Tn, kDwTok));
  const int ng = static_cast<int>(cdiv(d, kDwFeat));
  MOE_LAUNCH("router_bwd_dw_partial", (router_bwd_dw_fast_kernel<T, EP>),
             dim3(static_cast<unsigned>(nchunk), static_cast<unsigned>(ng)), dim3(256), 0, s,
             static_cast<const T*>(x), dlogits, Tn, d, E, part);
  const int64_t per = static_cast<int64_t>(ng) * kDwFeat * EP;
  MOE_LAUNCH("router_bwd_dw_reduce", (router_bwd_dw_fast_reduce_kernel<T, EP>),
             dim3(static_cast<unsigned>(cdiv(per, 64))), dim3(256), 0, s, part, nchunk, ng, d, E,
             static_cast<T*>(dw_r));
}

template <typename T>
int router_bwd_impl(const void* x, const void* w_r, const float* dlogits, int64_t Tn, int d, int E, void* dx,
                    int accumulate_dx, void* dw_r, float* part, hipStream_t s) {
  if (fast_ok<T, 8>(d, E)) {
    router_bwd_fast<T, 8>(x, w_r, dlogits, Tn, d, E, dx, accumulate_dx, dw_r, part, s);
    return launch_status();
  }
  if (fast_ok<T, 16>(d, E)) {
    router_bwd_fast<T, 16>(x, w_r, dlogits, Tn, d, E, dx, accumulate_dx, dw_r, part, s);
    return launch_status();
  }
  const int64_t n = static_cast<int64_t>(d) * E;
  const int nchunk = static_cast<int>(cdiv(Tn, kChunk));
  const int64_t nch = Tn * (d / 8);
  MOE_LAUNCH("router_bwd_dx", router_bwd_dx_kernel<T>, dim3(static_cast<unsigned>(cdiv(nch, 256))), dim3(256), 0, s,
             dlogits, static_cast<const T*>(w_r), Tn, d, E, static_cast<T*>(dx), accumulate_dx);
  MOE_LAUNCH("router_bwd_dw_partial", router_bwd_dw_partial_kernel<T>,
             dim3(static_cast<unsigned>(cdiv(n, 256)), nchunk), dim3(256), 0, s, static_cast<const T*>(x), dlogits,
             Tn, d, E, part);
  MOE_LAUNCH("router_bwd_dw_reduce", router_bwd_dw_reduce_kernel<T>, dim3(static_cast<unsigned>(cdiv(n, 256))),
             dim3(256), 0, s, part, nchunk, n, static_cast<T*>(dw_r));
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
  // generic path: [ceil(T/32)][d][E]; E <= 16 path: [ceil(T/64)][ceil(d/512)*512][EP]
  const size_t generic = static_cast<size_t>(cdiv(T, kChunk) > 0 ? cdiv(T, kChunk) : 1) * d * E;
  const int ep = E <= 8 ? 8 : 16;
  const size_t fast = static_cast<size_t>(cdiv(T, kDwTok) > 0 ? cdiv(T, kDwTok) : 1) * cdiv(d, kDwFeat) * kDwFeat * ep;
  return (generic > fast ? generic : fast) * sizeof(float);
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
