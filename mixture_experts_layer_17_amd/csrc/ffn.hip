// Host entry points of the grouped SwiGLU expert FFN, the device tile table,
// and the library's version / status helpers.
//
// Olmo-core 3 announcement, "Scaling and optimizing MoE training": the expert
// products run as one grouped computation, and the routing metadata stays on
// the GPU.  The host therefore sizes every launch from host-known bounds
// (R, E, d, f) only; a one-workgroup kernel turns the device offsets into a
// table of BM-row tiles, and each GEMM workgroup reads its tile from it.
#include "ffn_common.hpp"
#include "mx_common.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void tile_map_kernel(const int32_t* __restrict__ offsets, int E, int BM,
                                                       int64_t R, int64_t max_tiles, int4* __restrict__ tiles,
                                                       int32_t* __restrict__ sched) {
  // tile counts per expert, their inclusive prefix sum (Hillis-Steele over
  // kMaxE = 256 entries), then one thread per table slot
  __shared__ int64_t cum[kMaxE];
  __shared__ int32_t off_s[kMaxE], n_s[kMaxE];
  static_assert(kMaxE == 256, "one thread per expert");
  const int tid = threadIdx.x;
  int64_t cnt = 0;
  if (tid < E) {
    const int32_t o = offsets[tid];
    int32_t n = offsets[tid + 1] - o;
    if (n < 0) n = 0;
    off_s[tid] = o;
    n_s[tid] = n;
    cnt = (n + BM - 1) / BM;
  }
  cum[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    const int64_t v = tid >= o ? cum[tid - o] : 0;
    __syncthreads();
    cum[tid] += v;
    __syncthreads();
  }
  const int64_t total = cum[E - 1];
  const int64_t used = total < max_tiles ? total : max_tiles;
  for (int64_t slot = tid; slot < max_tiles; slot += blockDim.x) {
    int4 t = make_int4(-1, 0, 0, 0);
    if (slot < used) {
      // expert e: first with cum[e] > slot
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid] > slot) hi = mid; else lo = mid + 1;
      }
      const int e = lo;
      const int64_t i = slot - (cum[e] - (n_s[e] + BM - 1) / BM);
      const int64_t r0 = off_s[e] + i * BM;
      int64_t rows = n_s[e] - i * BM < BM ? n_s[e] - i * BM : BM;
      if (r0 + rows > R) rows = R - r0 > 0 ? R - r0 : 0;  // memory safety against bad offsets
      t = make_int4(rows > 0 ? e : -1, static_cast<int>(r0), static_cast<int>(rows), e);
    }
    tiles[slot] = t;
  }
  if (tid == 0) tiles[max_tiles] = make_int4(static_cast<int>(used), 0, 0, 0);
  // each expert's run of entries, cut at the live count
  if (tid < E) {
    const int64_t first = cum[tid] - cnt;
    int64_t n = used - first < cnt ? used - first : cnt;
    if (n < 0) n = 0;
    tiles[max_tiles + 1 + tid] = make_int4(static_cast<int>(first), static_cast<int>(n), 0, 0);
  }
  if (sched) {
    // the backward's weight-gradient order (wgrad_tile_sorted): experts by cost ceil(n_e / 64) + 3 (K-steps plus
    // an allowance for the epilogue), largest first, ties by lower index
    __shared__ int32_t cost[kMaxE];
    if (tid < E) cost[tid] = (n_s[tid] + 63) / 64 + 3;
    __syncthreads();
    if (tid < E) {
      const int32_t c = cost[tid];
      int rank = 0;
      for (int e = 0; e < E; ++e) rank += (cost[e] > c || (cost[e] == c && e < tid)) ? 1 : 0;
      sched[rank] = tid;
    }
  }
}


struct FfnShape {
  int64_t R;
  int E, d, f, prec;
};

bool shape_ok(const FfnShape& s) {
  if (s.R < 0 || s.R >= (1ll << 31) || s.E < 1 || s.E > kMaxE || s.d <= 0 || s.f <= 0) return false;
  if (s.prec != MOE_F32 && s.prec != MOE_BF16 && s.prec != MOE_MXFP8) return false;
  return true;
}

bool shape_supported(const FfnShape& s) {
  const int q = s.prec == MOE_MXFP8 ? 128 : 64;
  return s.d % q == 0 && s.f % q == 0;
}

int tile_bm(int prec, int64_t R, int E) {
  return prec == MOE_F32 ? ffn_f32_bm() : prec == MOE_MXFP8 ? ffn_mx_bm(R, E) : ffn_bf16_bm(R, E);
}

size_t elem_bytes(int prec) { return prec == MOE_F32 ? 4 : 2; }

// Workspace layout: [tile table][experts sorted by weight-gradient cost][dHg][dHu] (backward only)[MX scratch]
// (MXFP8 only).
size_t tiles_bytes(const FfnShape& s) {
  return align_up(static_cast<size_t>(max_m_tiles(s.R, s.E, tile_bm(s.prec, s.R, s.E)) + 1 + kMaxE) * sizeof(int4),
                  256);
}

size_t ffn_ws_bytes(const FfnShape& s, int is_bwd) {
  size_t b = tiles_bytes(s);
  if (is_bwd) b += wgrad_sched_bytes() + 2 * align_up(static_cast<size_t>(s.R) * s.f * elem_bytes(s.prec), 256);
  if (s.prec == MOE_MXFP8) b += mx_ffn_scratch_bytes(s.R, s.E, s.d, s.f, is_bwd);
  return b;
}

}  // namespace

int occupancy(const void* kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) n = 1;
  return n < 1 ? 1 : n;
}

unsigned persistent_grid(int occ, int64_t work) {
  constexpr int kMaxDev = 64;
  static int cus[kMaxDev] = {};  // compute units per device, looked up once
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int n = dev < kMaxDev ? __atomic_load_n(&cus[dev], __ATOMIC_RELAXED) : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = kNumXcd;
    if (dev < kMaxDev) __atomic_store_n(&cus[dev], n, __ATOMIC_RELAXED);
  }
  int64_t g = static_cast<int64_t>(n) * occ / kNumXcd * kNumXcd;
  if (g < kNumXcd) g = kNumXcd;
  const int64_t w = static_cast<int64_t>(xcd_grid(work < 1 ? 1 : work));
  return static_cast<unsigned>(g < w ? g : w);
}


void launch_tile_map(const int32_t* offsets, int E, int BM, int64_t R, int64_t max_tiles, int4* tiles,
                     hipStream_t s, int32_t* sched) {
  MOE_LAUNCH("tile_map", tile_map_kernel, dim3(1), dim3(256), 0, s, offsets, E, BM, R, max_tiles, tiles, sched);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_abi_version(void) { return 4; }

extern "C" const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or type";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

extern "C" size_t moe_grouped_ffn_workspace(int64_t R, int32_t E, int32_t d, int32_t f, int prec, int is_bwd) {
  const FfnShape s{R, E, d, f, prec};
  if (!shape_ok(s)) return 0;
  return ffn_ws_bytes(s, is_bwd);
}

extern "C" size_t moe_mx_weight_cache_bytes(int32_t E, int32_t d, int32_t f) {
  if (E < 1 || E > kMaxE || d <= 0 || f <= 0) return 0;
  return mx_wcache_bytes(E, d, f);
}

extern "C" int moe_mx_weight_cache_build(const void* w_gate, const void* w_up, const void* w_down, int32_t E,
                                         int32_t d, int32_t f, void* cache, size_t cache_bytes, void* stream) {
  if (E < 1 || E > kMaxE || d <= 0 || f <= 0) return MOE_EINVAL;
  if (d % 128 || f % 128) return MOE_EUNSUPPORTED;
  if (!w_gate || !w_up || !w_down || !cache) return MOE_EINVAL;
  for (const void* p : {w_gate, w_up, w_down, (const void*)cache})
    if (!aligned16(p)) return MOE_EINVAL;
  if (cache_bytes < mx_wcache_bytes(E, d, f)) return MOE_EWORKSPACE;
  mx_wcache_build(w_gate, w_up, w_down, E, d, f, static_cast<char*>(cache), static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" int moe_grouped_ffn_fwd(int64_t R, int32_t E, int32_t d, int32_t f, int prec, const int32_t* offsets,
                                   const void* x_perm, const void* w_gate, const void* w_up, const void* w_down,
                                   const void* mx_wcache, const void* x_mx, void* h_gate, void* h_up, void* a_act,
                                   void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  const FfnShape sh{R, E, d, f, prec};
  if (!shape_ok(sh)) return MOE_EINVAL;
  if (!shape_supported(sh)) return MOE_EUNSUPPORTED;
  if (!offsets || !w_gate || !w_up || !w_down || !ws) return MOE_EINVAL;
  if (R > 0 && ((!x_perm && !(x_mx && prec == MOE_MXFP8)) || !h_gate || !h_up || !a_act || !y_perm))
    return MOE_EINVAL;
  for (const void* p : {x_perm, w_gate, w_up, w_down, mx_wcache, x_mx, (const void*)h_gate, (const void*)h_up,
                        (const void*)a_act, (const void*)y_perm, (const void*)ws})
    if (p && !aligned16(p)) return MOE_EINVAL;
  if (x_mx && prec != MOE_MXFP8) return MOE_EINVAL;
  if (ws_bytes < ffn_ws_bytes(sh, 0)) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (R == 0) return MOE_OK;
  const int bm = tile_bm(prec, R, E);
  const int64_t mt = max_m_tiles(R, E, bm);
  int4* tiles = static_cast<int4*>(ws);
  launch_tile_map(offsets, E, bm, R, mt, tiles, s, nullptr);
  FfnArgs a{};
  a.offsets = offsets;
  a.tiles = tiles;
  a.max_tiles = mt;
  a.bm = bm;
  a.E = E; a.d = d; a.f = f; a.R = R;
  a.x = x_perm; a.wg = w_gate; a.wu = w_up; a.wd = w_down;
  a.o_hg = h_gate; a.o_hu = h_up; a.o_act = a_act; a.act = a_act; a.o_y = y_perm;
  if (prec == MOE_MXFP8) {
    char* mxs = static_cast<char*>(ws) + tiles_bytes(sh);
    return mx_ffn_fwd(a, mt, static_cast<const char*>(mx_wcache), static_cast<const uint8_t*>(x_mx), mxs, s);
  }
  auto launch = prec == MOE_F32 ? launch_ffn_f32 : launch_ffn_bf16;
  int st = launch(kG1, a, mt, s);
  if (st == MOE_OK) st = launch(kG2, a, mt, s);
  return st;
}

extern "C" int moe_grouped_ffn_bwd(int64_t R, int32_t E, int32_t d, int32_t f, int prec, const int32_t* offsets,
                                   const int32_t* mx_blk_offsets, const void* dy_perm, const void* x_perm,
                                   const void* h_gate, const void* h_up, const void* a_act, const void* w_gate,
                                   const void* w_up, const void* w_down, const void* mx_wcache, const void* dy_mx,
                                   const void* x_mxt, const void* dy_mxt, void* dx_perm, void* dw_gate,
                                   void* dw_up, void* dw_down, void* ws, size_t ws_bytes, void* stream) {
  const FfnShape sh{R, E, d, f, prec};
  if (!shape_ok(sh)) return MOE_EINVAL;
  if (!shape_supported(sh)) return MOE_EUNSUPPORTED;
  if (!offsets || !w_gate || !w_up || !w_down || !dw_gate || !dw_up || !dw_down || !ws) return MOE_EINVAL;
  if ((dy_mx || x_mxt || dy_mxt) && prec != MOE_MXFP8) return MOE_EINVAL;
  // x_perm is read only for its token-axis MX layout, dy_perm only for its two MX layouts (MOE_MXFP8)
  const bool need_x = prec != MOE_MXFP8 || !x_mxt;
  const bool need_dy = prec != MOE_MXFP8 || !dy_mx || !dy_mxt;
  if (R > 0 && ((need_dy && !dy_perm) || (need_x && !x_perm) || !h_gate || !h_up || !a_act || !dx_perm))
    return MOE_EINVAL;
  if (prec == MOE_MXFP8 && !mx_blk_offsets) return MOE_EINVAL;
  for (const void* p : {dy_perm, x_perm, h_gate, h_up, a_act, w_gate, w_up, w_down, mx_wcache, dy_mx, x_mxt, dy_mxt,
                        (const void*)dx_perm, (const void*)dw_gate, (const void*)dw_up, (const void*)dw_down,
                        (const void*)ws})
    if (p && !aligned16(p)) return MOE_EINVAL;
  if (ws_bytes < ffn_ws_bytes(sh, 1)) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bm = tile_bm(prec, R, E);
  const int64_t mt = max_m_tiles(R, E, bm);
  char* wsb = static_cast<char*>(ws);
  int4* tiles = reinterpret_cast<int4*>(wsb);
  const size_t hbytes = align_up(static_cast<size_t>(R) * f * elem_bytes(prec), 256);
  const size_t tb = tiles_bytes(sh) + wgrad_sched_bytes();
  void* dhg = wsb + tb;
  void* dhu = wsb + tb + hbytes;
  // the tile table and, in the same launch, the weight gradients' expert order
  int32_t* wsched = reinterpret_cast<int32_t*>(wsb + tiles_bytes(sh));
  launch_tile_map(offsets, E, bm, R, mt, tiles, s, wsched);
  FfnArgs a{};
  a.offsets = offsets;
  a.tiles = tiles;
  a.max_tiles = mt;
  a.bm = bm;
  a.E = E; a.d = d; a.f = f; a.R = R;
  a.x = x_perm; a.wg = w_gate; a.wu = w_up; a.wd = w_down;
  a.hg = h_gate; a.hu = h_up; a.act = a_act; a.dy = dy_perm;
  a.o_dhg = dhg; a.o_dhu = dhu; a.dhg = dhg; a.dhu = dhu;
  a.o_dx = dx_perm; a.o_dwg = dw_gate; a.o_dwu = dw_up; a.o_dwd = dw_down;
  a.wsched = wsched;
  if (prec == MOE_MXFP8) {
    char* mxs = wsb + tb + 2 * hbytes;
    return mx_ffn_bwd(a, mt, mx_blk_offsets, static_cast<const char*>(mx_wcache), static_cast<const uint8_t*>(dy_mx),
                      static_cast<const uint8_t*>(x_mxt), static_cast<const uint8_t*>(dy_mxt), mxs, s);
  }
  auto launch = prec == MOE_F32 ? launch_ffn_f32 : launch_ffn_bf16;
  int st = MOE_OK;
  // G5 last: its dX rows (ordinary stores) are then still in the caches when
  // the dispatch backward reads them right after (3-4% faster than G5 before G6)
  if (R > 0) st = launch(kG3, a, mt, s);
  if (st == MOE_OK) st = launch(kG4, a, mt, s);
  if (st == MOE_OK) st = launch(kG6, a, mt, s);
  if (R > 0 && st == MOE_OK) st = launch(kG5, a, mt, s);
  return st;
}
