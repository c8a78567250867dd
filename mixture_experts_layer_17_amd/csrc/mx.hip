// MXFP8 quantiser: bf16/fp32 -> E4M3 elements + one E8M0 scale per 32 elements.
//
// Olmo-core 3 announcement, "Scaling and optimizing MoE training": MXFP8 pays
// only when the savings exceed the cost of converting between formats, so the
// conversion is a pure HBM stream (read 2 bytes, write 1 + 1/32 per element).
// Format: the public OCP Microscaling (MX) v1.0 spec, FP8 E4M3 elements.
//
// Row layout (blocks along the contiguous axis): four lanes share one 32-element
// block, each lane converts 8 elements; amax is combined with two lane
// exchanges.  A wave instruction reads 1 KiB (bf16) and writes 512 bytes.
// Column layout (blocks down the rows, written transposed so each block's 32
// bytes are contiguous): one lane owns 16 bytes of columns for 32 rows; the 32
// row loads of a wave are 1 KiB each.  Blocks may restart at segment
// boundaries (expert segments of the token axis) with zero-padded tails.
#include "mx_common.hpp"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* o);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* o) {
  Elem<uint16_t>::unpack(*reinterpret_cast<const uint4*>(p), o);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* o) {
  Elem<float>::unpack(reinterpret_cast<const uint4*>(p)[0], o);
  Elem<float>::unpack(reinterpret_cast<const uint4*>(p)[1], o + 4);
}

template <typename T>
__global__ __launch_bounds__(256) void mx_rows_kernel(const T* __restrict__ src, int64_t nvec8,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  // nvec8 = rows * cols / 8; vector i covers elements [8i, 8i+8); block = i / 4.
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool ok = i < nvec8;
  float v[8];
  if (ok) {
    load8<T>(src + i * 8, v);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = mx_block_exponent(amax);
  const float inv = mx_inv_scale(e);
  if (!ok) return;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) lo |= e4m3_encode(v[j] * inv) << (8 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) hi |= e4m3_encode(v[4 + j] * inv) << (8 * j);
  reinterpret_cast<uint2*>(q)[i] = make_uint2(lo, hi);
  if ((i & 3) == 0) sc[i >> 2] = static_cast<uint8_t>(e + 127);
}

// j-th element (compile-time j after unrolling) of a 16-byte vector, as fp32.
template <typename T>
__device__ __forceinline__ float elem_of(const uint4& v, int j);
template <>
__device__ __forceinline__ float elem_of<uint16_t>(const uint4& v, int j) {
  const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
  return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float elem_of<float>(const uint4& v, int j) {
  return __uint_as_float(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w);
}

// One wave per (32-row block, 64*VEC columns); VEC columns per lane.
template <typename T>
__global__ __launch_bounds__(64) void mx_cols_kernel(const T* __restrict__ src, int64_t rows, int64_t cols,
                                                    const int32_t* __restrict__ seg, int nseg, int64_t ldq,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ int32_t s_off[kMaxE + 1];
  __shared__ int32_t s_blk[kMaxE + 1];
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.y;  // global 32-row block index
  const int64_t bz = blockIdx.z;
  int64_t r0, nvalid;
  if (seg) {
    for (int i = lane; i <= nseg; i += 64) s_off[i] = seg[i];
    __syncthreads();
    if (lane == 0) {
      int32_t run = 0;
      s_blk[0] = 0;
      for (int i = 0; i < nseg; ++i) {
        int32_t n = s_off[i + 1] - s_off[i];
        if (n < 0) n = 0;
        run += (n + 31) / 32;
        s_blk[i + 1] = run;
      }
    }
    __syncthreads();
    if (b >= s_blk[nseg]) {
      // padding past the last segment: written as zero codes with zero-block scales
      r0 = 0;
      nvalid = 0;
    } else {
      int lo = 0, hi = nseg;  // find s with s_blk[s] <= b < s_blk[s+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_blk[mid] <= b) lo = mid; else hi = mid;
      }
      r0 = s_off[lo] + (b - s_blk[lo]) * 32;
      const int64_t end = s_off[lo + 1] < rows ? s_off[lo + 1] : rows;
      nvalid = end - r0;
      if (nvalid > 32) nvalid = 32;
      if (nvalid < 0) nvalid = 0;
    }
  } else {
    r0 = b * 32;
    nvalid = 32;
  }
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 64 + lane) * VEC;
  if (c0 >= cols) return;
  const T* base = src + bz * rows * cols + r0 * cols + c0;
  uint4 raw[32];
#pragma unroll
  for (int r = 0; r < 32; ++r)
    raw[r] = r < nvalid ? *reinterpret_cast<const uint4*>(base + r * cols) : make_uint4(0, 0, 0, 0);
  uint8_t* qb = q + bz * cols * ldq;
  uint8_t* sb = sc + bz * cols * (ldq / 32);
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(elem_of<T>(raw[r], j)));
    const int e = mx_block_exponent(amax);
    const float inv = mx_inv_scale(e);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      w[k] = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[k] |= e4m3_encode(elem_of<T>(raw[4 * k + t], j) * inv) << (8 * t);
    }
    uint4* dst = reinterpret_cast<uint4*>(qb + (c0 + j) * ldq + b * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    sb[(c0 + j) * (ldq / 32) + b] = static_cast<uint8_t>(e + 127);
  }
}

}  // namespace

void launch_mx_rows(const void* src, int src_dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sc,
                    hipStream_t s) {
  const int64_t nvec8 = rows * cols / 8;
  if (nvec8 == 0) return;
  const dim3 grid(static_cast<unsigned>(cdiv(nvec8, 256)));
  if (src_dtype == MOE_F32)
    MOE_LAUNCH("mx_quantize_rows", mx_rows_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(src), nvec8, q, sc);
  else
    MOE_LAUNCH("mx_quantize_rows", mx_rows_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), nvec8, q,
                       sc);
}

void launch_mx_cols(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols, const int32_t* seg,
                    int nseg, int64_t ldq, uint8_t* q, uint8_t* sc, hipStream_t s) {
  const int vec = src_dtype == MOE_F32 ? 4 : 8;
  const int64_t nblk = seg ? cdiv(rows, 32) + nseg : rows / 32;
  if (nblk == 0 || cols == 0 || batch == 0) return;
  const dim3 grid(static_cast<unsigned>(cdiv(cols, 64 * vec)), static_cast<unsigned>(nblk),
                  static_cast<unsigned>(batch));
  if (src_dtype == MOE_F32)
    MOE_LAUNCH("mx_quantize_cols", mx_cols_kernel<float>, grid, dim3(64), 0, s, static_cast<const float*>(src), rows, cols, seg,
                       nseg, ldq, q, sc);
  else
    MOE_LAUNCH("mx_quantize_cols", mx_cols_kernel<uint16_t>, grid, dim3(64), 0, s, static_cast<const uint16_t*>(src), rows, cols,
                       seg, nseg, ldq, q, sc);
}

}  // namespace moe

using namespace moe;

extern "C" int mx_quantize(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols, int32_t axis,
                           const int32_t* seg_offsets, int32_t nseg, uint8_t* q, uint8_t* scales, void* stream) {
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_EINVAL;
  if (batch < 0 || rows < 0 || cols < 0 || (axis != 0 && axis != 1)) return MOE_EINVAL;
  if (batch * rows * cols == 0) return MOE_OK;
  if (!src || !q || !scales || !aligned16(src) || !aligned16(q)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (axis == 1) {
    if (seg_offsets || cols % 32) return MOE_EINVAL;
    launch_mx_rows(src, src_dtype, batch * rows, cols, q, scales, s);
    return launch_status();
  }
  if (cols % 8) return MOE_EINVAL;
  if (seg_offsets) {
    if (batch != 1 || nseg < 1 || nseg > kMaxE) return MOE_EINVAL;
    const int64_t ldq = 32 * (cdiv(rows, 32) + nseg);
    launch_mx_cols(src, src_dtype, 1, rows, cols, seg_offsets, nseg, ldq, q, scales, s);
  } else {
    if (rows % 32) return MOE_EINVAL;
    launch_mx_cols(src, src_dtype, batch, rows, cols, nullptr, 0, rows, q, scales, s);
  }
  return launch_status();
}
