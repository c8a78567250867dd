// Internal helpers shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// bf16 stored as raw uint16 bits; conversions are explicit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest, ties to even: the hardware conversion (v_cvt_pk_bf16_f32,
// two values per instruction on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

// Element type traits for the two storage types of the data-movement kernels.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* o) {
    return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                      __float_as_uint(o[3]));
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void unpack(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ uint4 pack(const float* o) {
    return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                      pack_bf16x2(o[6], o[7]));
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16(v));
  }
};

// Wave-wide sum (64 lanes), result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// The reciprocal is the hardware approximation (v_rcp_f32, about 1 ulp), not
// an IEEE division; exp(-z) overflowing to infinity gives 0 as it should.
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// ---------------------------------------------------------------------------
// Launch wrapper: optionally brackets each launch with timing events (timing.hip).
// ---------------------------------------------------------------------------
bool timing_on();
void timing_mark(const char* name, hipStream_t s, bool begin);

#define MOE_LAUNCH(name, kernel, grid, block, shmem, stream, ...)             \
  do {                                                                        \
    const bool moe_t_ = ::moe::timing_on();                                   \
    if (moe_t_) ::moe::timing_mark(name, stream, true);                       \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);      \
    if (moe_t_) ::moe::timing_mark(name, stream, false);                      \
  } while (0)

// ---------------------------------------------------------------------------
// Host-side helpers.
// ---------------------------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Zero-fill with a kernel (never hipMemsetAsync, so that callers may capture
// the calls in a HIP graph).  Each translation unit gets its own copy.
namespace {
__global__ __launch_bounds__(256) void zero_fill_kernel(uint8_t* __restrict__ p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n16) reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
  const size_t tail = bytes - n16 * 16;
  if (i < tail) p[n16 * 16 + i] = 0;
}
inline void launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return;
  const size_t n = bytes / 16 > 16 ? bytes / 16 : 16;
  MOE_LAUNCH("zero_fill", zero_fill_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<uint8_t*>(p), bytes);
}
}  // namespace

// Largest supported sizes.
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;

// 16-byte store with the non-temporal hint, for large outputs that no kernel
// reads soon: they stream to memory instead of being allocated (and filled) in
// the L2.  Measured faster for the dispatch rows and the GEMM epilogues, slower
// for the combine outputs, which keep ordinary stores.
// Read of a value the whole wave shares (tile tables, expert schedules) through
// the constant address space, so that the compiler issues a scalar load (counted
// by lgkmcnt): a vector load would sit in the vector memory counter behind the
// wave's earlier stores, and waiting for it would wait for them.  Only for data
// no kernel in flight writes.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}
__device__ __forceinline__ int4 ld_uniform(const int4* p) {
  typedef int i32x4_c __attribute__((ext_vector_type(4)));
  const i32x4_c v = *(const __attribute__((address_space(4))) i32x4_c*)p;
  return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store16_nt(void* p, const uint4& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

}  // namespace moe
