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
  const int4* tiles;       // M-tile table: {expert, row0, rows, 0}; expert < 0 past the end;
                           // entry [max_tiles] = {number of live tiles, 0, 0, 0}
  int64_t max_tiles;
  int bm;                  // row-tile height the tile table was built for
  const int4* tiles128;    // MXFP8 backward with bm = 256: a 128-row table for the SwiGLU-backward GEMM, else null
  int64_t max_tiles128;
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

// Weight-gradient tile order.  Expert e has a gm x gn grid of output tiles;
// tiles in a block of GM x GN read the same GM operand slices along M and GN
// along N.  Workgroups are handed to the XCDs round-robin by hardware id, so
// the S = GM*GN tiles of one block get ids h, h+8, ..., h+8(S-1) (one XCD, one
// L2), while the 8 blocks of a run of 8*S ids sit on 8 different XCDs (a heavily
// loaded expert still spreads over the whole chip).  Returns false for ids
// past the last tile; the grid is E*gm*gn.
__device__ __forceinline__ bool wgrad_tile(int64_t h, int E, int gm, int gn, int& e, int& mt, int& nt) {
  const int GM = gm % 2 == 0 ? 2 : 1;
  const int GN = gn % 4 == 0 ? 4 : gn % 2 == 0 ? 2 : 1;
  const int S = GM * GN;
  const int64_t per_e = static_cast<int64_t>(gm / GM) * (gn / GN);
  const int64_t ng = per_e * E;  // blocks
  const int64_t run = h / (kNumXcd * S), q = h % (kNumXcd * S);
  int64_t g;
  int w;
  if ((run + 1) * kNumXcd <= ng) {
    g = run * kNumXcd + q % kNumXcd;
    w = static_cast<int>(q / kNumXcd);
  } else {  // last, partial run: blocks in hardware order
    g = run * kNumXcd + q / S;
    w = static_cast<int>(q % S);
    if (g >= ng) return false;
  }
  e = static_cast<int>(g / per_e);
  const int rem = static_cast<int>(g % per_e), bn = gn / GN;
  mt = (rem / bn) * GM + w / GN;
  nt = (rem % bn) * GN + w % GN;
  return true;
}

// Persistent launches (ffn.hip).  occupancy: resident workgroups per compute
// unit of `kernel` at `threads` per workgroup (at least 1).  persistent_grid:
// compute units x occ of the current device, rounded down to a multiple of the
// XCD count, and at most xcd_grid(work).
int occupancy(const void* kernel, int threads);
unsigned persistent_grid(int occ, int64_t work);

// Launch the tile-table builder (defined in ffn.hip).
void launch_tile_map(const int32_t* offsets, int E, int BM, int64_t R, int64_t max_tiles, int4* tiles,
                     hipStream_t s);

// GEMM launchers (defined in gemm_bf16.hip / gemm_f32.hip).
int launch_ffn_bf16(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s);
int launch_ffn_f32(int kind, const FfnArgs& a, int64_t max_tiles, hipStream_t s);
int ffn_bf16_bm(int64_t R, int E);  // row-tile height for this workload
int ffn_f32_bm();

}  // namespace moe
