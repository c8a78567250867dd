// Shared definitions of the grouped expert-FFN GEMMs (internal).
//
// The six products of one SwiGLU expert FFN, forward and backward, run as
// grouped GEMMs over the expert-major buffer (Olmo-core 3 announcement,
// "Scaling and optimizing MoE training": the many small expert products become
// one grouped computation):
//   G1  [Hg | Hu] = X Wg_e | X Wu_e, epilogue A = silu(Hg) * Hu   rows by expert
//   G2  Y = A Wd_e                                                rows by expert
//   G3  dA = dY Wd_e^T, epilogue dHg, dHu (SwiGLU backward)        rows by expert
//   G4  dWd_e = A_e^T dY_e                                        K = rows of e
//   G5  dX = dHg Wg_e^T + dHu Wu_e^T                              rows by expert
//   G6  dWg_e = X_e^T dHg_e, dWu_e = X_e^T dHu_e                  K = rows of e
// "Rows by expert" GEMMs walk a device-built tile table (one entry per
// BM-row tile of each expert segment), so the grid size is a host-known bound
// and the host never reads the routing counts.
#pragma once

#include "common.hpp"

namespace moe {

enum FfnKind { kG1 = 1, kG2 = 2, kG3 = 3, kG4 = 4, kG5 = 5, kG6 = 6 };

struct FfnArgs {
  const int32_t* offsets;  // [E+1] expert segment offsets (device)
  const int4* tiles;       // M-tile table: {expert (< 0: no rows), row0, rows, expert}, expert < 0 past
                           // the end; entry [max_tiles] = {number of live tiles, 0, 0, 0}; entry
                           // [max_tiles + 1 + e] = {first entry of expert e, its number of entries, 0, 0}
  int64_t max_tiles;
  int bm;                  // row-tile height the tile table was built for
  const int32_t* wsched;   // backward: the experts sorted by weight-gradient cost (wgrad_tile_sorted)
  int E, d, f;
  int64_t R;
  // inputs
  const void *x, *wg, *wu, *wd, *hg, *hu, *act, *dy, *dhg, *dhu;
  // outputs
  void *o_hg, *o_hu, *o_act, *o_y, *o_dhg, *o_dhu, *o_dx, *o_dwg, *o_dwu, *o_dwd;
};

// Upper bound of BM-row tiles over all expert segments: sum ceil(n_e / BM).
inline int64_t max_m_tiles(int64_t R, int E, int BM) { return cdiv(R, BM) + E; }

// XCD-aware tile order.  The hardware deals consecutive workgroup ids round-robin
// over the 8 XCDs (each with its own L2); giving XCD x the contiguous logical
// range [x*per, (x+1)*per) keeps the tiles that share operands (the N-tiles of
// one row block, the row blocks of one expert) on one L2.  Returns -1 for
// workgroups with no tile.  Launch grids are rounded up to a multiple of 8.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int64_t xcd_tile(int64_t hw_id, int64_t total) {
  const int64_t per = (total + kNumXcd - 1) / kNumXcd;
  if (hw_id >= per * kNumXcd) return -1;
  const int64_t lid = (hw_id % kNumXcd) * per + hw_id / kNumXcd;
  return lid < total ? lid : -1;
}
inline unsigned xcd_grid(int64_t total) {
  return static_cast<unsigned>(cdiv(total, kNumXcd) * kNumXcd);
}

// Rows-by-expert tile order over the live entries of the tile table times gx
// column tiles: each expert's run of entries [T, T + n) is taken in groups of
// row tiles, and inside a group the column tile is the major index, so the row
// tiles that read the same weight columns take consecutive logical ids (hence,
// through xcd_tile, CUs of one XCD at about the same time) and fetch those
// columns into its L2 once, while an expert with many row tiles still works on
// few of them at a time (its X rows stay in L2 too).  Groups are pairs; an odd
// run ends with a triple (n = 1: a single), so a short last row tile (an
// expert's rows just past a multiple of the tile height) shares its weight
// columns with the two before it instead of fetching them again alone.
// Returns the table entry and the column tile of logical id lid (< live * gx).
__device__ __forceinline__ int64_t expert_tile(int64_t lid, int gx, const int4* tiles, int64_t max_tiles, int& nt) {
  const int e = __builtin_amdgcn_readfirstlane(ld_uniform(tiles + lid / gx).w);
  const int4 run = ld_uniform(tiles + max_tiles + 1 + e);
  const int64_t first = __builtin_amdgcn_readfirstlane(run.x);
  const int n = __builtin_amdgcn_readfirstlane(run.y);
  const int64_t l = lid - first * gx;
  int64_t grp = l / (2 * gx);
  int m = 2;  // row tiles in this group
  if (n == 1) {
    m = 1;
  } else if ((n & 1) && grp >= (n - 3) / 2) {
    grp = (n - 3) / 2;  // the closing triple: entries n - 3 .. n - 1
    m = 3;
  }
  const int64_t l2 = l - grp * 2 * gx;
  nt = static_cast<int>(l2 / m);
  return first + 2 * grp + l2 % m;
}

// Weight-gradient tile order for one workgroup per tile (G4, G6), from the
// experts sorted by cost (sched[0, E), as launch_tile_map writes it).  The
// hardware deals workgroup ids round-robin over the 8 XCDs; id h runs on XCD
// x = h % 8 as that XCD's q-th workgroup (q = h / 8).  The sorted experts go in
// rounds of 8: in round 0 (the 8 costliest) each expert's tiles spread over all
// 8 XCDs, so a heavily routed expert still fills the chip; in every later round
// XCD x takes expert 8r + x whole, so one L2 serves all of that expert's operand
// slices.  Each XCD holds ntile slots per round, heaviest rounds first, and the
// grid is 8 * ntile * ceil(E / 8).  False for slots past the last expert.
__device__ __forceinline__ bool wgrad_tile_sorted(int64_t h, int E, int ntile, const int32_t* sched, int& e,
                                                  int& local) {
  const int x = static_cast<int>(h % kNumXcd);
  const int64_t q = h / kNumXcd;
  const int r = static_cast<int>(q / ntile);
  int j;
  if (r == 0) {
    const int64_t t = q * kNumXcd + x;  // the round's 8 * ntile tiles, dealt over the XCDs
    j = static_cast<int>(t / ntile);
    local = static_cast<int>(t % ntile);
  } else {
    j = r * kNumXcd + x;
    local = static_cast<int>(q - static_cast<int64_t>(r) * ntile);
  }
  if (j >= E) return false;
  e = ld_uniform(sched + __builtin_amdgcn_readfirstlane(j));
  return true;
}
inline int64_t wgrad_sorted_grid(int E, int ntile) {
  return static_cast<int64_t>(kNumXcd) * ntile * ((E + kNumXcd - 1) / kNumXcd);
}

// The experts sorted by weight-gradient cost, largest first (ties: lower
// index), written on the device from the routing offsets (by the tile-table
// launch) so the host never waits: sched[0, E) int32.  An expert's cost is
// ceil(n_e / 64) + 3 (its K-steps plus an allowance for the epilogue).
inline size_t wgrad_sched_bytes() { return align_up(static_cast<size_t>(kMaxE) * 4, 256); }

// Persistent launches (ffn.hip).  occupancy: resident workgroups per compute
// unit of `kernel` at `threads` per workgroup (at least 1).  persistent_grid:
// compute units x occ of the current device, rounded down to a multiple of the
// XCD count, and at most xcd_grid(work).
int occupancy(const void* kernel, int threads);
unsigned persistent_grid(int occ, int64_t work);

// Launch the tile-table builder (defined in ffn.hip); with sched (not NULL) the
// same launch also writes the weight gradients' expert order.
void launch_tile_map(const int32_t* offsets, int E, int BM, int64_t R, int64_t max_tiles, int4* tiles,
                     hipStream_t s, int32_t* sched);

// GEMM launchers (defined in gemm_bf16.hip / gemm_f32.hip).
int launch_ffn_bf16(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s);
int launch_ffn_f32(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s);
int ffn_bf16_bm(int64_t R, int E);  // row-tile height for this workload
int ffn_f32_bm();

}  // namespace moe
