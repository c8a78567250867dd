// Top-k routing and device-built routing metadata.
//
// Olmo-core 3 announcement, "Scaling and optimizing MoE training": routing
// metadata stays on the GPU so the host can keep enqueuing work without
// waiting for it; routed rows go straight into the experts' input buffers.
// Introduction: a fixed number of experts (four of 8 or 128) per token.
//
// Three launches, no host synchronisation and no atomics that decide an order:
//  1. route_select: one workgroup per 64 tokens.  The 64 x E logit tile is
//     staged through LDS with coalesced loads; one to four lanes per token each
//     keep a sorted top-k list of a part of its row (logit descending, index
//     ascending) and merge them over lane shuffles; the token's first lane writes
//     indices and renormalised gates, then ORs the token's bit into a per-expert
//     64-bit mask.  The rank of a token inside its block for expert e is the
//     popcount of the mask bits below its own (token order), and the block's
//     count for e is the popcount of the whole mask.
//  2. route_scan: one workgroup turns the [blocks x E] count matrix into
//     counts, offsets, MX block offsets and per-(block, expert) base rows.
//  3. route_scatter: row = base[block][e] + rank; writes perm_dst and perm_src.
#include <mutex>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kTokPerBlk = 64;   // tokens per routing block (one wave)
constexpr int kStageMaxE = 128;  // widest logit row staged through LDS
constexpr int kStageBatch = 8;   // 16-byte logit loads per lane in flight while staging
constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 8;    // block counts per thread loaded before any is used

// Order of the selection: a ranks above b when it is larger, or when a is a
// number and b is NaN (NaN ranks below every number, -inf included); equal
// values (-0.0 and +0.0 among them) and two NaNs do not rank above each other,
// so the lower expert index keeps the earlier slot.
__device__ __forceinline__ bool ranks_above(float a, float b) { return a > b || (b != b && a == a); }

// The selection's total order: a before b when a ranks above b, or neither
// ranks above the other and a has the lower expert index.
__device__ __forceinline__ bool before(float av, int ai, float bv, int bi) {
  return ranks_above(av, bv) || (!ranks_above(bv, av) && ai < bi);
}

// P lanes per token (1, 2 or 4, and at least K experts each): lane p of a token
// scans the experts [p E / P, (p + 1) E / P) in index order with the insertion
// rule below, and the P sorted lists then meet over lane shuffles, each lane
// inserting its partner's entries into its own list under the total order.
// The top K of a row under that (strict) order is unique, so the result does
// not depend on P.  A workgroup still takes 64 tokens (one mask bit each).
template <int K>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ logits, int64_t T,
                                                           int E, int P, int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ gates,
                                                           int32_t* __restrict__ rank,
                                                           int32_t* __restrict__ blk_counts) {
  extern __shared__ float smem[];
  // For E <= kStageMaxE the [64, E] logit tile is staged through LDS with
  // coalesced loads (odd row stride: lane-private rows hit distinct banks);
  // wider rows are read by each lane straight from global memory.
  const bool stage = E <= kStageMaxE;
  const int ld = E + 1;
  float* tile = smem;
  unsigned long long* mask =
      reinterpret_cast<unsigned long long*>(smem + (stage ? kTokPerBlk * ld : 0));
  const int tid = threadIdx.x, nthr = blockDim.x;  // 64 P threads
  const int tok = tid / P, part = tid - tok * P;   // the block's token (0 .. 63) and the part of its row
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlk;
  const int ntok = static_cast<int>(T - t0 < kTokPerBlk ? T - t0 : kTokPerBlk);

  const float* src = logits + t0 * E;
  if (stage) {
    // 16-byte loads, kStageBatch per thread issued before any is written to LDS
    // (src is 16-byte aligned when logits is: t0 * E * 4 is a multiple of 256)
    const int nel = ntok * E;
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
    const int nv = vec ? nel / 4 : 0;
    const float4* s4 = reinterpret_cast<const float4*>(src);
    for (int v0 = 0; v0 < nv; v0 += nthr * kStageBatch) {
      float4 buf[kStageBatch];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const int v = v0 + u * nthr + tid;
        if (v < nv) buf[u] = s4[v];
      }
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const int v = v0 + u * nthr + tid;
        if (v < nv) {
          int r = (4 * v) / E, c = 4 * v - r * E;
          const float f[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            tile[r * ld + c] = f[q];
            if (++c == E) { c = 0; ++r; }
          }
        }
      }
    }
    for (int i = 4 * nv + tid; i < nel; i += nthr) {
      const int r = i / E;
      tile[r * ld + (i - r * E)] = src[i];
    }
  }
  for (int e = tid; e < E; e += nthr) mask[e] = 0ull;
  __syncthreads();

  const bool live = tok < ntok;
  float val[K];
  int idx[K];
#pragma unroll
  for (int i = 0; i < K; ++i) { val[i] = 0.f; idx[i] = i; }

  if (live) {
    const float* row = stage ? tile + tok * ld : src + static_cast<int64_t>(tok) * E;
    const int e0 = part * E / P, e1 = (part + 1) * E / P;
    for (int e = e0; e < e1; ++e) {
      const float v = row[e];
      // Candidate e has a larger index than every entry held, so it goes in
      // front of an entry only when it ranks strictly above it.  The first K
      // experts of the part fill the list unconditionally; entries are never
      // duplicated, so the result is K distinct valid experts for any input.
      const int q = e - e0;
      const bool take = (q < K) || ranks_above(v, val[K - 1]);
      if (take) {
        const int pos = q < K ? q : K - 1;
#pragma unroll
        for (int i = 0; i < K; ++i)
          if (i == pos) { val[i] = v; idx[i] = e; }
#pragma unroll
        for (int i = K - 1; i >= 1; --i) {
          if (i <= pos && ranks_above(val[i], val[i - 1])) {
            const float tv = val[i]; val[i] = val[i - 1]; val[i - 1] = tv;
            const int ti = idx[i]; idx[i] = idx[i - 1]; idx[i - 1] = ti;
          }
        }
      }
    }
  }
  // the parts' lists meet (lanes tok P .. tok P + P - 1 share a wave); every lane of a token ends with its top K
  for (int m = 1; m < P; m <<= 1) {
    float pv[K];
    int pi[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      pv[i] = __shfl_xor(val[i], m, 64);
      pi[i] = __shfl_xor(idx[i], m, 64);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (before(pv[j], pi[j], val[K - 1], idx[K - 1])) {
        val[K - 1] = pv[j];
        idx[K - 1] = pi[j];
#pragma unroll
        for (int i = K - 1; i >= 1; --i) {
          if (before(val[i], idx[i], val[i - 1], idx[i - 1])) {
            const float tv = val[i]; val[i] = val[i - 1]; val[i - 1] = tv;
            const int ti = idx[i]; idx[i] = idx[i - 1]; idx[i - 1] = ti;
          }
        }
      }
    }
  }
  if (live && part == 0) {
    // Renormalised gates: softmax over the K chosen logits.
    float z[K];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < K; ++i) { z[i] = __expf(val[i] - val[0]); s += z[i]; }
    const float inv = 1.0f / s;
    const int64_t t = t0 + tok;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      topk_idx[t * K + i] = idx[i];
      gates[t * K + i] = z[i] * inv;
      atomicOr(&mask[idx[i]], 1ull << tok);
    }
  }
  __syncthreads();
  if (live && part == 0) {
    const unsigned long long below = (1ull << tok) - 1ull;
    const int64_t t = t0 + tok;
#pragma unroll
    for (int i = 0; i < K; ++i) rank[t * K + i] = __popcll(mask[idx[i]] & below);
  }
  int32_t* cnt = blk_counts + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = tid; e < E; e += nthr) cnt[e] = __popcll(mask[e]);
}

// One workgroup.  blk_base has the layout of blk_counts and is written in place.
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(int32_t* __restrict__ blk, int nblk, int E,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ mx_blk_offsets) {
  __shared__ int32_t part[kScanThreads];
  __shared__ int32_t tot[kMaxE + 1];
  __shared__ int32_t mxb[kMaxE + 1];
  __shared__ int32_t sc[2][kMaxE], scb[2][kMaxE];
  const int tid = threadIdx.x;
  const int parts = kScanThreads / E;  // >= 4 for E <= 256
  const int e = tid % E;
  const int p = tid / E;
  const bool active = p < parts;
  const int per = (nblk + parts - 1) / parts;
  const int b0 = active ? min(nblk, p * per) : 0;
  const int b1 = active ? min(nblk, b0 + per) : 0;
  int s = 0;
  if (active)
    for (int b = b0; b < b1; b += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) c[u] = b + u < b1 ? blk[static_cast<int64_t>(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) s += c[u];
    }
  part[tid] = s;
  __syncthreads();
  // per-expert totals, then exclusive scans over the E (<= 256) experts:
  // Hillis-Steele in LDS (integer sums, so the order of additions is immaterial)
  int own = 0, ownb = 0;
  if (tid < E) {
    for (int q = 0; q < parts; ++q) own += part[q * E + tid];
    ownb = (own + 31) / 32;
    sc[0][tid] = own;
    scb[0][tid] = ownb;
  }
  __syncthreads();
  int cur = 0;
  for (int o = 1; o < E; o <<= 1) {
    if (tid < E) {
      sc[cur ^ 1][tid] = sc[cur][tid] + (tid >= o ? sc[cur][tid - o] : 0);
      scb[cur ^ 1][tid] = scb[cur][tid] + (tid >= o ? scb[cur][tid - o] : 0);
    }
    __syncthreads();
    cur ^= 1;
  }
  if (tid < E) {
    tot[tid] = sc[cur][tid] - own;
    mxb[tid] = scb[cur][tid] - ownb;
    if (tid == E - 1) {
      tot[E] = sc[cur][tid];
      mxb[E] = scb[cur][tid];
    }
  }
  __syncthreads();
  if (tid <= E) {
    offsets[tid] = tot[tid];
    if (mx_blk_offsets) mx_blk_offsets[tid] = mxb[tid];
    if (tid < E) counts[tid] = tot[tid + 1] - tot[tid];
  }
  // Base of each part = expert offset + counts of earlier parts.
  if (active) {
    int base = tot[e];
    for (int q = 0; q < p; ++q) base += part[q * E + e];
    for (int b = b0; b < b1; b += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) c[u] = b + u < b1 ? blk[static_cast<int64_t>(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        if (b + u < b1) {
          blk[static_cast<int64_t>(b + u) * E + e] = base;
          base += c[u];
        }
    }
  }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                            const int32_t* __restrict__ rank,
                                                            const int32_t* __restrict__ blk_base,
                                                            int64_t R, int k, int E,
                                                            int32_t* __restrict__ perm_src,
                                                            int32_t* __restrict__ perm_dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= R) return;
  const int64_t t = i / k;
  const int64_t b = t / kTokPerBlk;
  const int e = topk_idx[i];
  const int row = blk_base[b * E + e] + rank[i];
  perm_dst[i] = row;
  perm_src[row] = static_cast<int32_t>(i);
}

// dlogits[t, e] = g_j (dg_j - sum_i g_i dg_i) if e = S_j, else 0.  A thread
// takes V consecutive experts of one token (V = 4: one 16-byte store) and
// reads the token's K gates, gate gradients and indices once.
template <int K, int V>
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* __restrict__ gates,
                                                        const float* __restrict__ dgates,
                                                        const int32_t* __restrict__ topk_idx, int64_t T,
                                                        int E, float* __restrict__ dlogits) {
  const int ev = E / V;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= T * ev) return;
  const int64_t t = i / ev;
  const int e0 = static_cast<int>(i - t * ev) * V;
  float g[K], dg[K];
  int id[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    g[j] = gates[t * K + j];
    dg[j] = dgates[t * K + j];
    id[j] = topk_idx[t * K + j];
  }
  float inner = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) inner += g[j] * dg[j];
  float out[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    // an unselected expert gets exactly zero
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (id[j] == e0 + v) mine = g[j] * (dg[j] - inner);
    out[v] = mine;
  }
  if constexpr (V == 4)
    *reinterpret_cast<float4*>(dlogits + t * E + e0) = make_float4(out[0], out[1], out[2], out[3]);
  else
    dlogits[t * E + e0] = out[0];
}

size_t route_ws_bytes(int64_t T, int E, int k) {
  const int64_t nblk = cdiv(T, kTokPerBlk);
  return align_up(static_cast<size_t>(T * k) * 4, 256) + align_up(static_cast<size_t>(nblk * E) * 4, 256);
}

template <int K>
void launch_select(const float* logits, int64_t T, int E, int32_t* idx, float* gates, int32_t* rank,
                   int32_t* blk, hipStream_t s) {
  const int64_t nblk = cdiv(T, kTokPerBlk);
  const size_t tile = E <= kStageMaxE ? static_cast<size_t>(kTokPerBlk) * (E + 1) * sizeof(float) : 0;
  const size_t lds = tile + static_cast<size_t>(E) * 8;
  const int P = E >= 4 * K ? 4 : (E >= 2 * K ? 2 : 1);  // lanes per token, at least K experts each
  MOE_LAUNCH("route_select", route_select_kernel<K>, dim3(static_cast<unsigned>(nblk)), dim3(64 * P), lds, s, logits,
                     T, E, P, idx, gates, rank, blk);
}

template <int K>
void launch_bwd(const float* g, const float* dg, const int32_t* idx, int64_t T, int E, float* dl,
                hipStream_t s) {
  if (E % 4 == 0 && (reinterpret_cast<uintptr_t>(dl) & 15u) == 0) {
    const int64_t n = T * (E / 4);
    MOE_LAUNCH("route_topk_bwd", (route_bwd_kernel<K, 4>), dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s,
               g, dg, idx, T, E, dl);
  } else {
    const int64_t n = T * E;
    MOE_LAUNCH("route_topk_bwd", (route_bwd_kernel<K, 1>), dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s,
               g, dg, idx, T, E, dl);
  }
}

bool route_args_ok(int64_t T, int E, int k) {
  return T >= 0 && E >= 1 && E <= kMaxE && k >= 1 && k <= kMaxK && k <= E && T * k < (1ll << 31);
}

// Load statistics of one routing from its per-expert row counts: max, min,
// number of empty experts, total rows (one workgroup, E <= 256).
__global__ __launch_bounds__(256) void route_stats_kernel(const int32_t* __restrict__ counts, int E,
                                                          int32_t* __restrict__ stats) {
  __shared__ int32_t mx[256], mn[256], em[256], sm[256];
  const int t = threadIdx.x;
  const int32_t c = t < E ? counts[t] : 0;
  mx[t] = t < E ? c : INT32_MIN;
  mn[t] = t < E ? c : INT32_MAX;
  em[t] = (t < E && c == 0) ? 1 : 0;
  sm[t] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) {
      mx[t] = mx[t] > mx[t + o] ? mx[t] : mx[t + o];
      mn[t] = mn[t] < mn[t + o] ? mn[t] : mn[t + o];
      em[t] += em[t + o];
      sm[t] += sm[t + o];
    }
    __syncthreads();
  }
  if (t == 0) {
    stats[0] = mx[0];
    stats[1] = mn[0];
    stats[2] = em[0];
    stats[3] = sm[0];
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_route_stats(const int32_t* counts, int32_t E, int32_t* stats, void* stream) {
  if (E < 1 || E > kMaxE || !counts || !stats) return MOE_EINVAL;
  MOE_LAUNCH("route_stats", route_stats_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), counts, E,
             stats);
  return launch_status();
}

extern "C" size_t moe_route_topk_workspace(int64_t T, int32_t E, int32_t k) {
  if (!route_args_ok(T, E, k)) return 0;
  return route_ws_bytes(T, E, k);
}

namespace moe {
namespace {

// Validation shared by moe_route_topk and moe_route_topk_noalloc (everything but the workspace).
int route_check(const float* logits, int64_t T, int E, int k, const int32_t* topk_idx, const float* gates,
                const int32_t* counts, const int32_t* offsets, const int32_t* perm_src, const int32_t* perm_dst) {
  if (!route_args_ok(T, E, k)) return (E > kMaxE || k > kMaxK) ? MOE_EUNSUPPORTED : MOE_EINVAL;
  if (!counts || !offsets) return MOE_EINVAL;
  if (T > 0 && (!logits || !topk_idx || !gates || !perm_src || !perm_dst)) return MOE_EINVAL;
  return MOE_OK;
}

// The three routing launches over a scratch area of route_ws_bytes(T, E, k)
// bytes at ws (every byte of it is written before it is read).
int route_launch(const float* logits, int64_t T, int E, int k, int32_t* topk_idx, float* gates, int32_t* counts,
                 int32_t* offsets, int32_t* perm_src, int32_t* perm_dst, int32_t* mx_blk_offsets, void* ws,
                 hipStream_t s) {
  const int64_t nblk = cdiv(T, kTokPerBlk);
  int32_t* rank = static_cast<int32_t*>(ws);
  int32_t* blk = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(static_cast<size_t>(T * k) * 4, 256));
  if (T > 0) {
    switch (k) {
      case 1: launch_select<1>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      case 2: launch_select<2>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      case 3: launch_select<3>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      case 4: launch_select<4>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      case 5: launch_select<5>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      case 6: launch_select<6>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      case 7: launch_select<7>(logits, T, E, topk_idx, gates, rank, blk, s); break;
      default: launch_select<8>(logits, T, E, topk_idx, gates, rank, blk, s); break;
    }
  }
  MOE_LAUNCH("route_scan", route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk, static_cast<int>(nblk), E,
                     counts, offsets, mx_blk_offsets);
  if (T > 0) {
    const int64_t R = T * k;
    MOE_LAUNCH("route_scatter", route_scatter_kernel, dim3(static_cast<unsigned>(cdiv(R, 256))), dim3(256), 0, s,
                       topk_idx, rank, blk, R, k, E, perm_src, perm_dst);
  }
  return launch_status();
}

// ---------------------------------------------------------------------------
// Routing without allocation (moe_route_topk_noalloc): the same launches with
// their scratch in a static device array of kNoAllocBytes per GPU, which each
// GPU the library runs on holds until the process ends.  Limits: T*k and
// ceil(T/64)*E at most 2^20 each, so route_ws_bytes <= 4 MiB + 4 MiB.
// ---------------------------------------------------------------------------
constexpr int64_t kNoAllocRows = int64_t{1} << 20;
constexpr int64_t kNoAllocBlkCounts = int64_t{1} << 20;
constexpr size_t kNoAllocBytes = static_cast<size_t>(kNoAllocRows + kNoAllocBlkCounts) * 4;

static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

// Device address of `scratch` on the current device, looked up once per device
// with hipGetSymbolAddress (in host code the array's name is only a stand-in).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                              float* gates, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                              int32_t* perm_dst, int32_t* mx_blk_offsets, void* ws, size_t ws_bytes,
                              void* stream) {
  const int st = route_check(logits, T, E, k, topk_idx, gates, counts, offsets, perm_src, perm_dst);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_EINVAL;
  if (ws_bytes < route_ws_bytes(T, E, k)) return MOE_EWORKSPACE;
  return route_launch(logits, T, E, k, topk_idx, gates, counts, offsets, perm_src, perm_dst, mx_blk_offsets, ws,
                      static_cast<hipStream_t>(stream));
}

extern "C" int moe_route_topk_noalloc(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                                      float* gates, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                                      int32_t* perm_dst, int32_t* mx_blk_offsets, void* stream) {
  const int st = route_check(logits, T, E, k, topk_idx, gates, counts, offsets, perm_src, perm_dst);
  if (st != MOE_OK) return st;
  if (T * k > kNoAllocRows || cdiv(T, kTokPerBlk) * E > kNoAllocBlkCounts) return MOE_EWORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return MOE_EHIP;
  return route_launch(logits, T, E, k, topk_idx, gates, counts, offsets, perm_src, perm_dst, mx_blk_offsets, ws,
                      static_cast<hipStream_t>(stream));
}

extern "C" int moe_route_topk_bwd(const float* gates, const float* dgates, const int32_t* topk_idx,
                                  int64_t T, int32_t E, int32_t k, float* dlogits, void* stream) {
  if (!route_args_ok(T, E, k)) return (E > kMaxE || k > kMaxK) ? MOE_EUNSUPPORTED : MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!gates || !dgates || !topk_idx || !dlogits) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (k) {
    case 1: launch_bwd<1>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    case 2: launch_bwd<2>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    case 3: launch_bwd<3>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    case 4: launch_bwd<4>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    case 5: launch_bwd<5>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    case 6: launch_bwd<6>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    case 7: launch_bwd<7>(gates, dgates, topk_idx, T, E, dlogits, s); break;
    default: launch_bwd<8>(gates, dgates, topk_idx, T, E, dlogits, s); break;
  }
  return launch_status();
}
