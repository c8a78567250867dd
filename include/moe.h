/*
 * moe.h — C ABI of libmoe: one GPU's share of an MoE layer, forward and backward,
 * on AMD Instinct MI355X (gfx950).
 *
 * The method is the MoE training path of Ai2's "Introducing Olmo-core 3: open,
 * scalable training infrastructure for large MoE models", section "Scaling and
 * optimizing MoE training": tokens are routed to a few experts, routed rows are
 * written straight into the experts' input buffers (row-wise expert
 * parallelism), routing metadata stays on the GPU so the host never waits for
 * it, the many small expert products run as one grouped GEMM, and MXFP8 can
 * replace BF16 in the expert products.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer to caller-owned memory, row-major,
 *    16-byte aligned.  The library never allocates, frees, copies to the host or
 *    synchronises inside these calls; it keeps no per-call state.  Scratch memory
 *    comes from the caller as `ws` of at least the size the matching
 *    *_workspace() function returns (a pure function of the shape).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues kernels on it and returns; results are ready when the
 *    stream reaches them.  No device-derived value ever reaches the host.
 *  - Outputs are overwritten (never accumulated into), including zero gradients
 *    for experts that received no rows; the one exception is
 *    moe_router_logits_bwd with accumulate_dx = 1.  Outputs must not alias inputs.
 *  - Errors: arguments are validated on the host before anything is launched.
 *    Invalid values give MOE_EINVAL, valid but unimplemented shapes or types give
 *    MOE_EUNSUPPORTED, a too-small workspace gives MOE_EWORKSPACE; in these
 *    cases nothing is launched.  A failed launch gives MOE_EHIP.  Index arrays
 *    (topk_idx, offsets, perm_*) are trusted: they must come from
 *    moe_route_topk for the same T, E, k.  Non-finite inputs give unspecified
 *    (but memory-safe) results.
 *  - Determinism: identical inputs give identical output bits (no floating-point
 *    atomics; every reduction has a fixed order).
 *
 * Symbols: T tokens, d model width, E experts, k experts per token, f expert
 * hidden width, R = T*k routed rows.  Limits: 1 <= k <= 8, k <= E <= 256,
 * 0 <= T, R < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status;

/* Element / compute types.  Data-movement calls take MOE_F32 or MOE_BF16 (the
 * storage type).  The expert FFN takes all three: MOE_F32 (fp32 storage and
 * math), MOE_BF16 (bf16 storage, bf16 MFMA, fp32 accumulate), MOE_MXFP8 (bf16
 * storage and outputs; every expert GEMM runs on MX-scaled FP8 MFMA with
 * operands quantised on the device, fp32 accumulate). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 } moe_prec;

/* 4: moe_grouped_ffn_bwd takes x_mxt and dy_mxt; the token-axis MX calls. */
int moe_abi_version(void);
const char* moe_status_str(int status);

/* ---------------------------------------------------------------------------
 * Router.
 * ------------------------------------------------------------------------- */

/* Router logits l = x W_r (the routing step of "Scaling and optimizing MoE
 * training"; the pages give no router formula, the plain linear router is used).
 * x [T, d] and w_r [d, E] in `dtype` (MOE_F32 or MOE_BF16); logits [T, E] fp32,
 * fp32 accumulation.  d % 8 == 0. */
int moe_router_logits(const void* x, const void* w_r, int dtype, int64_t T, int32_t d, int32_t E,
                      float* logits, void* stream);

/* Backward of moe_router_logits: dx (+)= dlogits W_r^T and dw_r = x^T dlogits.
 * dlogits [T, E] fp32; dx [T, d] and dw_r [d, E] in `dtype`.  With
 * accumulate_dx = 1 the router term is added to dx (so it joins the output of
 * moe_dispatch_bwd); with 0 dx is overwritten.  dw_r is reduced over tokens in
 * a fixed order through the workspace. */
size_t moe_router_logits_bwd_workspace(int64_t T, int32_t d, int32_t E);
int moe_router_logits_bwd(const void* x, const void* w_r, int dtype, const float* dlogits, int64_t T,
                          int32_t d, int32_t E, void* dx, int accumulate_dx, void* dw_r, void* ws,
                          size_t ws_bytes, void* stream);

/* Top-k routing with the routing metadata built on the device ("Scaling and
 * optimizing MoE training": the metadata stays on the GPU; introduction: four
 * of 8 or 128 experts are chosen per token).
 *   logits [T, E] fp32 (input)
 *   topk_idx [T, k] int32: slot j = j-th expert under (logit descending, index
 *            ascending); -0.0 and +0.0 tie; a NaN logit ranks below every
 *            number (-inf included), NaNs among themselves by index
 *   gates [T, k] fp32: softmax over the k chosen logits (= softmax over all E,
 *            renormalised over the chosen set); NaN for every slot of a token
 *            whose chosen logits include a NaN or whose largest chosen logit
 *            is infinite (a chosen -inf below a finite largest gets gate 0)
 *   counts [E], offsets [E+1] int32: rows per expert and their exclusive prefix
 *            sum (offsets[E] = R)
 *   perm_src [R] int32: expert-buffer row -> flat slot t*k+j (rows of an expert
 *            are in token order)
 *   perm_dst [R] int32: flat slot t*k+j -> expert-buffer row
 *   mx_blk_offsets [E+1] int32 or NULL: prefix sum of ceil(counts/32), the
 *            32-row blocks per expert used by token-axis MX quantisation
 * Bit-exact and deterministic: no atomics decide any order. */
size_t moe_route_topk_workspace(int64_t T, int32_t E, int32_t k);
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                   float* gates, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                   int32_t* perm_dst, int32_t* mx_blk_offsets, void* ws, size_t ws_bytes,
                   void* stream);

/* moe_route_topk without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs and bits as moe_route_topk;
 * the scratch is a static 8 MiB device array that the library holds on each
 * GPU it runs on until the process ends (the current device's copy is used:
 * the stream must belong to the current device).  Limits: T*k <= 2^20 and
 * ceil(T/64)*E <= 2^20, else MOE_EWORKSPACE with nothing launched; MOE_EHIP
 * if the array's device address cannot be obtained.  Every byte of the scratch
 * is written before it is read, so nothing needs clearing between calls, but
 * all calls on one GPU share it: calls that overlap on one GPU (different
 * streams, or host threads) race and give undefined results. */
int moe_route_topk_noalloc(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                           float* gates, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                           int32_t* perm_dst, int32_t* mx_blk_offsets, void* stream);

/* Backward of the renormalised gates (the router is trained with the rest of
 * the layer in the MoE training path of "Scaling and optimizing MoE training";
 * the pages give no gradient formula, so this is the exact gradient of the
 * gates moe_route_topk computes): dlogits[t, S_j] = g_j (dg_j - sum_i g_i dg_i),
 * exactly zero for unselected experts (the renormalised gates do not depend on
 * them).  gates, dgates [T, k] fp32, topk_idx [T, k] from moe_route_topk;
 * dlogits [T, E] fp32, overwritten.  MOE_EINVAL / MOE_EUNSUPPORTED for bad
 * sizes or null pointers, nothing launched; T = 0 is a no-op. */
int moe_route_topk_bwd(const float* gates, const float* dgates, const int32_t* topk_idx, int64_t T,
                       int32_t E, int32_t k, float* dlogits, void* stream);

/* Load statistics of a routing ("Scaling to the trillion-parameter range":
 * a balance metric alone can be gamed, so the observable load is exported).
 * counts [E] int32 (from moe_route_topk), 1 <= E <= 256; stats [4] int32 on
 * the device, overwritten: {largest expert's rows, smallest expert's rows,
 * number of experts with no rows, total rows}.  MOE_EINVAL for a bad E or a
 * null pointer. */
int moe_route_stats(const int32_t* counts, int32_t E, int32_t* stats, void* stream);

/* ---------------------------------------------------------------------------
 * Row-wise dispatch and weighted combine ("Scaling and optimizing MoE
 * training": routed data goes directly into the experts' input buffers).
 * All in `dtype` (MOE_F32 or MOE_BF16), d % 8 == 0.
 * ------------------------------------------------------------------------- */

/* x_perm[perm_dst[t*k+j]] = x[t]: each token row is read once and written to
 * its k rows of the expert-major buffer.  x [T, d], x_perm [R, d]; exact copy. */
int moe_dispatch(const void* x, int dtype, int64_t T, int32_t d, int32_t k, const int32_t* perm_dst,
                 void* x_perm, void* stream);

/* dx[t] = sum_j dx_perm[perm_dst[t*k+j]] (fp32 sum in slot order). */
int moe_dispatch_bwd(const void* dx_perm, int dtype, int64_t T, int32_t d, int32_t k,
                     const int32_t* perm_dst, void* dx, void* stream);

/* out[t] = sum_j gates[t,j] * y_perm[perm_dst[t*k+j]] (fp32 sum in slot order).
 * y_perm [R, d] holds the unweighted expert outputs; out [T, d]. */
int moe_combine(const void* y_perm, int dtype, const float* gates, const int32_t* perm_dst,
                int64_t T, int32_t d, int32_t k, void* out, void* stream);

/* Backward of moe_combine for upstream gradient dout [T, d]:
 *   dy_perm[perm_dst[t*k+j]] = gates[t,j] * dout[t]          ([R, d], dtype)
 *   dgates[t,j] = <dout[t], y_perm[perm_dst[t*k+j]]>          ([T, k], fp32) */
int moe_combine_bwd(const void* dout, const void* y_perm, int dtype, const float* gates,
                    const int32_t* perm_dst, int64_t T, int32_t d, int32_t k, void* dy_perm,
                    float* dgates, void* stream);

/* MXFP8 data movement ("Scaling and optimizing MoE training": the MXFP8 gains
 * came from the expert FFN and from moving data between experts): the two
 * calls that write an expert-major buffer the MXFP8 FFN quantises along d
 * (X for the gate/up GEMM, dY for the down-projection's data gradient) also
 * write its MX rows layout, so the FFN skips that quantisation pass.
 * The MX buffer `*_mx` (caller-owned, moe_mx_act_bytes(R, d) bytes, R = T*k)
 * holds the E4M3 codes [R, d] (blocks of 32 along d, as mx_quantize axis 1),
 * then, at the next 256-byte boundary, the E8M0 bytes in grouped order: the
 * byte of (row r, block b) at ((b/4)*R + r)*4 + b%4.  Codes and scales are
 * bit-identical to mx_quantize of the bf16 buffer the same call writes.
 * bf16 only; d % 128 == 0 (else MOE_EUNSUPPORTED); otherwise as moe_dispatch /
 * moe_combine_bwd.  moe_mx_act_bytes returns 0 for invalid sizes. */
size_t moe_mx_act_bytes(int64_t rows, int32_t cols);
int moe_dispatch_mx(const void* x, int64_t T, int32_t d, int32_t k, const int32_t* perm_dst,
                    void* x_perm, void* x_mx, void* stream);
int moe_combine_bwd_mx(const void* dout, const void* y_perm, const float* gates, const int32_t* perm_dst,
                       int64_t T, int32_t d, int32_t k, void* dy_perm, float* dgates, void* dy_mx,
                       void* stream);

/* MXFP8 data movement with the token-axis layout ("Scaling and optimizing MoE
 * training": the MXFP8 gains came from the expert FFN and from moving data
 * between experts).  The weight gradients contract over each expert's tokens,
 * so the MXFP8 backward needs X and dY also quantised along the tokens, per
 * expert segment; these two calls write that layout together with the rows
 * layout of moe_dispatch_mx / moe_combine_bwd_mx, from one destination-major
 * pass that reads each expert row's token row directly, so the bf16 expert rows
 * need not be written at all (x_perm / dy_perm may be NULL; given, they receive
 * the same rows as moe_dispatch / moe_combine_bwd).
 * Token-axis layout of an expert-major [R, cols] buffer (the MX buffer `*_mxt`,
 * caller-owned, moe_mx_tok_bytes(R, E, cols) bytes): Rp = moe_mx_tok_rows(R, E)
 * padded token positions, expert e's 32-row blocks at positions
 * [32 mx_blk_offsets[e], 32 mx_blk_offsets[e+1]) (mx_blk_offsets from
 * moe_route_topk; a segment's last block zero-padded, positions past the last
 * segment zero); E4M3 codes [cols, Rp] (column c, position p at c Rp + p), then
 * at the next 256-byte boundary the E8M0 bytes, the byte of (column c, block b)
 * at ((b/4) cols + c) 4 + b%4.  Codes and scales are bit-identical to
 * mx_quantize(axis 0, seg_offsets = offsets) of the bf16 expert rows (scales
 * regrouped as stated).  The rows layout `*_mx` is as for moe_dispatch_mx.
 * moe_combine_bwd_mx_tok also writes dgates (as moe_combine_bwd); dY = gate x
 * dout is rounded to bf16 before it is encoded, as moe_combine_bwd stores it.
 * perm_src, offsets, mx_blk_offsets: from moe_route_topk for the same T, E, k.
 * bf16 only; d % 128 == 0 (else MOE_EUNSUPPORTED); 1 <= E <= 256; otherwise as
 * moe_dispatch / moe_combine_bwd.  moe_mx_tok_rows / _bytes return 0 for
 * invalid sizes. */
int64_t moe_mx_tok_rows(int64_t R, int32_t E);
size_t moe_mx_tok_bytes(int64_t R, int32_t E, int32_t cols);
int moe_dispatch_mx_tok(const void* x, int64_t T, int32_t d, int32_t k, int32_t E, const int32_t* perm_src,
                        const int32_t* offsets, const int32_t* mx_blk_offsets, void* x_perm, void* x_mx,
                        void* x_mxt, void* stream);
int moe_combine_bwd_mx_tok(const void* dout, const void* y_perm, const float* gates, const int32_t* perm_dst,
                           const int32_t* perm_src, const int32_t* offsets, const int32_t* mx_blk_offsets,
                           int64_t T, int32_t d, int32_t k, int32_t E, void* dy_perm, float* dgates, void* dy_mx,
                           void* dy_mxt, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped SwiGLU expert FFN ("Scaling and optimizing MoE training": the small
 * per-expert products run as one grouped GEMM; MXFP8 where it pays).
 * Rows of expert e are [offsets[e], offsets[e+1]) of the expert-major buffer
 * (device metadata from moe_route_topk; the host never reads it).
 *   w_gate, w_up [E, d, f], w_down [E, f, d]   (x @ W orientation)
 *   forward:  h_gate = X We_g, h_up = X We_u, a_act = silu(h_gate) * h_up,
 *             y_perm = a_act We_d  (unweighted; the gate is applied in combine)
 *   backward: dA = dY Wd^T, dh_up = dA silu(Hg), dh_gate = dA Hu s (1 + Hg (1 - s)),
 *             dx_perm = dh_gate Wg^T + dh_up Wu^T,
 *             dw_down = A^T dY, dw_gate = X^T dh_gate, dw_up = X^T dh_up
 *             (all experts written; zero for experts with no rows)
 * Storage: fp32 for MOE_F32, bf16 for MOE_BF16 and MOE_MXFP8.  h_gate, h_up,
 * a_act [R, f] are saved by the forward and read by the backward.
 * MOE_MXFP8 quantises every GEMM operand on the device to E4M3 with one E8M0
 * scale per 32 elements along that GEMM's contraction axis (as mx_quantize).
 * Limits: d % 64 == 0 and f % 64 == 0 (MOE_MXFP8: % 128).  mx_blk_offsets
 * (from moe_route_topk) is required by the MOE_MXFP8 backward, else ignored.
 * mx_wcache (MOE_MXFP8 only, else ignored; may be NULL): a cache built by
 * moe_mx_weight_cache_build from these same weights, E, d and f; with it the
 * call quantises no weight (w_gate/w_up/w_down are still passed and
 * validated); results are bit-identical to those without it.
 * x_mx (forward) / dy_mx (backward) (MOE_MXFP8 only, else MOE_EINVAL; may be
 * NULL): x_perm / dy_perm already in the MX rows layout written by
 * moe_dispatch_mx / moe_combine_bwd_mx (or the _tok calls) for the same buffer;
 * the call then does not quantise it again (bit-identical results).
 * x_mxt / dy_mxt (backward, MOE_MXFP8 only, else MOE_EINVAL; may be NULL): X / dY
 * in the token-axis layout of moe_dispatch_mx_tok / moe_combine_bwd_mx_tok, used
 * by the weight gradients instead of quantising x_perm / dy_perm along the
 * tokens (bit-identical results).  With MOE_MXFP8, x_perm may be NULL when the
 * forward has x_mx and the backward x_mxt, and dy_perm when the backward has
 * both dy_mx and dy_mxt. */
size_t moe_grouped_ffn_workspace(int64_t R, int32_t E, int32_t d, int32_t f, int prec, int is_bwd);
int moe_grouped_ffn_fwd(int64_t R, int32_t E, int32_t d, int32_t f, int prec, const int32_t* offsets,
                        const void* x_perm, const void* w_gate, const void* w_up, const void* w_down,
                        const void* mx_wcache, const void* x_mx, void* h_gate, void* h_up, void* a_act,
                        void* y_perm, void* ws, size_t ws_bytes, void* stream);
int moe_grouped_ffn_bwd(int64_t R, int32_t E, int32_t d, int32_t f, int prec, const int32_t* offsets,
                        const int32_t* mx_blk_offsets, const void* dy_perm, const void* x_perm,
                        const void* h_gate, const void* h_up, const void* a_act, const void* w_gate,
                        const void* w_up, const void* w_down, const void* mx_wcache, const void* dy_mx,
                        const void* x_mxt, const void* dy_mxt, void* dx_perm, void* dw_gate, void* dw_up,
                        void* dw_down, void* ws, size_t ws_bytes, void* stream);

/* Pre-quantised MXFP8 expert weights ("Scaling and optimizing MoE training":
 * converting into MXFP8 has a cost the savings must exceed).  Weights change
 * once per optimiser step, so a loop with several micro-batches per step can
 * quantise them once: the cache holds each of w_gate, w_up [E, d, f] and
 * w_down [E, f, d] (bf16) in both orientations the MXFP8 FFN uses (forward:
 * blocks along d for w_gate/w_up and along f for w_down; backward: blocks along
 * the last axis), each produced from a single read of the weight.
 * moe_mx_weight_cache_bytes(E, d, f) = 6 E d f (1 + 1/32) bytes plus alignment.
 * Layout (the FFN calls take the cache back unchanged; it is stated so that it
 * can be inspected or stored): six regions in the order w_gate, w_up, w_down
 * forward, then w_gate, w_up, w_down backward; each region is its E4M3 codes
 * (E d f bytes) and then its E8M0 scale bytes (E d f / 32), both parts starting
 * on a 256-byte boundary.  A forward region holds each expert's weight
 * quantised down its rows and stored transposed ([E, f, d] for w_gate/w_up,
 * [E, d, f] for w_down; blocks run along the last axis); with M the rows and
 * K the last axis of that stored form, the scale of expert e, row m, block b
 * is byte e M (K/32) + ((b/4) M + m) 4 + b%4.  A backward region keeps the
 * weight's own shape with blocks along its last axis, and the scale of expert
 * e, row m, block b is byte ((b/4) E M + e M + m) 4 + b%4.  The cache stays
 * valid while the weights are unchanged; building
 * again overwrites it.  Errors: MOE_EINVAL (null or unaligned pointer, bad E,
 * d, f), MOE_EUNSUPPORTED (d or f not a multiple of 128), MOE_EWORKSPACE
 * (cache_bytes too small); nothing is launched then. */
size_t moe_mx_weight_cache_bytes(int32_t E, int32_t d, int32_t f);
int moe_mx_weight_cache_build(const void* w_gate, const void* w_up, const void* w_down, int32_t E,
                              int32_t d, int32_t f, void* cache, size_t cache_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MXFP8 quantiser ("Scaling and optimizing MoE training" names MXFP8 and the
 * cost of converting into it; the format follows the public OCP MX v1.0 spec):
 * blocks of 32 consecutive elements along `axis`; scale exponent
 * e = floor(log2(max|v|)) - 8 clamped to [-127, 127] (all-zero block: -127),
 * stored as the E8M0 byte e + 127; elements v / 2^e rounded to nearest-even
 * E4M3 (bias 7), saturated to +-448, sign kept.
 *   src [batch, rows, cols] in src_dtype (MOE_F32 or MOE_BF16).
 *   axis 1: q [batch, rows, cols], scales [batch, rows, cols/32]; cols % 32 == 0.
 *   axis 0, seg_offsets NULL: blocks run down the rows and are stored
 *           contiguously, i.e. transposed: q [batch, cols, rows],
 *           scales [batch, cols, rows/32]; rows % 32 == 0.
 *   axis 0 with seg_offsets (device int32, nseg+1 prefix offsets of row
 *           segments, seg_offsets[nseg] = rows, 1 <= nseg <= 256; batch == 1):
 *           blocks restart at
 *           each segment and a segment's last block is zero-padded.  With
 *           B_s = sum_{s'<s} ceil(n_s'/32) and Rp = 32*(ceil(rows/32) + nseg),
 *           q is [cols, Rp] with segment s in columns [32 B_s, 32 B_{s+1}),
 *           scales [cols, Rp/32]; columns past 32 B_nseg are written as zero
 *           codes with scale byte 0.
 * cols % 8 == 0 for axis 0. */
int mx_quantize(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols,
                int32_t axis, const int32_t* seg_offsets, int32_t nseg, uint8_t* q,
                uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics: per-kernel timing for benchmarks and profiling (no page
 * defines it).  While enabled, every kernel the library launches is bracketed
 * by two HIP events recorded on the caller's stream; events come from a pool
 * that grows on first use, so enable it and run one warm-up pass before a timed
 * region.  moe_timing_enable(1) also discards earlier records; (0) stops.
 * moe_timing_report waits for the recorded events and writes one text line per
 * kernel name, "<name> <launches> <total_ms>\n", NUL-terminated, into buf
 * (MOE_EINVAL if len is too small), then discards the records.  Process-wide
 * state guarded by a mutex.
 * ------------------------------------------------------------------------- */
int moe_timing_enable(int on);
int moe_timing_report(char* buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
