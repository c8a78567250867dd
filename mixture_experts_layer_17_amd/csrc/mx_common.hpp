// MXFP8 internals shared by the quantiser, the MX GEMMs and the FFN entry points.
#pragma once

#include "ffn_common.hpp"

namespace moe {

// E4M3 codes of four fp32 values, a in the low byte: round to nearest, ties to
// even, saturated to +-448, sign kept.  The clamp makes the saturation
// explicit; v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950) then rounds to nearest even,
// subnormals included.  For every fp32 input with |y| < 512, the range a
// block's scaled values lie in, this equals the integer definition (drop 20
// mantissa bits with ties to even; multiples of 2^-9 below 2^-6): all 2^31
// such inputs were compared on the device, and the tests check the rounding
// boundaries against the oracle.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Shared block exponent e = floor(log2(amax)) - 8, clamped to [-127, 127];
// -127 for an all-zero block.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax) & 0x7FFFFFFFu;
  int p;
  if (b >= 0x00800000u) {
    p = static_cast<int>(b >> 23) - 127;
  } else if (b != 0u) {
    p = (31 - __clz(static_cast<int>(b))) - 149;  // fp32 subnormal
  } else {
    return -127;
  }
  const int e = p - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an fp32 multiplier (e in [-127, 127]); exact for e >= -126 and for the
// values that can occur in a block with e = -127 (their scaled magnitudes stay
// below 2).
__device__ __forceinline__ float mx_inv_scale(int e) {
  const int n = -e;  // in [-127, 127]
  return n >= -126 ? __uint_as_float(static_cast<uint32_t>(n + 127) << 23) : __uint_as_float(0x00400000u);
}

// Launchers of the quantiser (mx.hip).  Scale layouts: the public one is
// row-major [nrows, nblk]; with `grouped` (the MX GEMM operands; nblk % 4 == 0)
// the scale of (row r, block b) is byte ((b/4) nrows + r) 4 + b%4, so a tile's
// scales for one K-step of 128 elements are one contiguous run of 32-bit words.
//  rows layout: blocks along the contiguous axis; q [rows, cols], scales of a [rows, cols/32] matrix
void launch_mx_rows(const void* src, int src_dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sc,
                    hipStream_t s, bool grouped);
//  column layout: blocks run down the rows, stored transposed: q [batch][cols][ldq], scales of a
//  [batch][cols][ldq/32] matrix (grouped: each batch's [cols, ldq/32] matrix grouped).  With seg (device,
//  nseg+1 offsets; batch 1) blocks restart at each segment; blk (device, nseg+1, or NULL) is the prefix sum
//  of the segments' 32-row block counts when the caller has it.
void launch_mx_cols(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols, const int32_t* seg,
                    int nseg, int64_t ldq, uint8_t* q, uint8_t* sc, hipStream_t s, bool grouped,
                    const int32_t* blk);
//  both layouts of a [batch, rows, cols] source from one read (no segments; rows % 128 == 0, cols % 128 == 0),
//  grouped scales: column layout qc [batch][cols][rows] (scales grouped per batch) and row layout
//  qr [batch][rows][cols] (scales of the [batch*rows, cols/32] matrix grouped).
void launch_mx_both(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols, uint8_t* qc,
                    uint8_t* sc, uint8_t* qr, uint8_t* scr, hipStream_t s);

// Token-axis length of the weight gradients' MX operands: every expert segment
// padded to 32 tokens, the total to a whole number of scale groups (128
// tokens) plus one zero group, so that a K-step starting mid-group never reads
// a group past the end.
inline int64_t mx_token_rows(int64_t R, int E) { return 128 * (cdiv(cdiv(R, 32) + E, 4) + 1); }

//  destination-major gather of an expert-major buffer's rows into both of its MX layouts: the rows layout
//  (codes qr [R, d], scales grouped over the R rows: word of (row, group G) at scr + 4 (G R + row)) and the
//  token-axis layout (as launch_mx_cols with segments and grouped scales: qt [d][ldq], ldq = mx_token_rows).
//  Expert row r holds source row perm_src[r] / k of src [T, d] (bf16), times gates[perm_src[r]] rounded to
//  bf16 when gates is not NULL; without perm_src (and gates) src is the expert-major buffer [R, d] itself;
//  rows_out [R, d] (bf16, may be NULL) receives the rows themselves.
//  seg: nseg + 1 segment offsets, blk: their 32-row block-count prefix (device).  d % 128 == 0.
void launch_mx_gather(const uint16_t* src, int64_t R, int d, int k, const int32_t* perm_src, const float* gates,
                      const int32_t* seg, const int32_t* blk, int nseg, uint16_t* rows_out, uint8_t* qr,
                      uint8_t* scr, uint8_t* qt, uint8_t* sct, hipStream_t s);

// MXFP8 expert FFN (gemm_mx.hip).
size_t mx_ffn_scratch_bytes(int64_t R, int E, int d, int f, int is_bwd);
int ffn_mx_bm(int64_t R, int E);  // row-tile height for this workload
//  wcache: NULL, or a weight cache built by mx_wcache_build for the same weights (then no weight is quantised).
//  x_mx / dy_mx: NULL, or X / dY already in the MX rows layout (codes [R, d], then at the next 256-byte boundary
//  the grouped scale words), as moe_dispatch_mx / moe_combine_bwd_mx write them.  x_mxt / dy_mxt: NULL, or X /
//  dY already in the token-axis layout (codes [d][mx_token_rows(R, E)], then at the next 256-byte boundary the
//  grouped scale words), as moe_dispatch_mx_tok / moe_combine_bwd_mx_tok write them.
int mx_ffn_fwd(const FfnArgs& a, int64_t max_tiles, const char* wcache, const uint8_t* x_mx, char* scratch,
               hipStream_t s);
int mx_ffn_bwd(const FfnArgs& a, int64_t max_tiles, const int32_t* mx_blk_offsets, const char* wcache,
               const uint8_t* dy_mx, const uint8_t* x_mxt, const uint8_t* dy_mxt, char* scratch, hipStream_t s);
size_t mx_wcache_bytes(int E, int d, int f);
void mx_wcache_build(const void* wg, const void* wu, const void* wd, int E, int d, int f, char* cache,
                     hipStream_t s);

}  // namespace moe
