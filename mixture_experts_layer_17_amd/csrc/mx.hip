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
// bytes are contiguous): tiles of 4 blocks x 64 columns pass through LDS so
// that both the row reads and the transposed writes are whole 128-byte runs.
// Blocks may restart at segment boundaries (expert segments of the token axis)
// with zero-padded tails.
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

// Scale byte of (row r, block b) of a [nrows, nblk] scale matrix: row-major
// (the public layout) or, for the GEMM operands, grouped by four blocks (one
// K-step of the MX GEMMs): byte ((b/4) nrows + r) 4 + b%4, so that a tile's
// scale words for one K-step are contiguous.
__device__ __forceinline__ int64_t scale_index(bool grouped, int64_t r, int64_t b, int64_t nrows, int64_t nblk) {
  return grouped ? ((b >> 2) * nrows + r) * 4 + (b & 3) : r * nblk + b;
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
  const uint32_t lo = e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  const uint32_t hi = e4m3_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  reinterpret_cast<uint2*>(q)[i] = make_uint2(lo, hi);
  if ((i & 3) == 0) sc[i >> 2] = static_cast<uint8_t>(e + 127);
}

// Row layout with grouped scales: the same streaming order as mx_rows_kernel
// (vector i = elements [8i, 8i+8) of the flattened matrix); the 16 lanes of a
// group (128 elements, four blocks of one row) combine their scale bytes into
// the group's word, written at (G*nrows + r) for group G of row r.
template <typename T>
__global__ __launch_bounds__(256) void mx_rows_grouped_kernel(const T* __restrict__ src, uint32_t nvec8,
                                                             uint32_t nrows, uint32_t ngpr,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = i < nvec8;
  float v[8];
  if (ok) {
    load8<T>(src + static_cast<int64_t>(i) * 8, v);
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
  uint32_t sw = static_cast<uint32_t>(e + 127) << (8 * ((i >> 2) & 3));
  sw |= __shfl_xor(sw, 4, 64);
  sw |= __shfl_xor(sw, 8, 64);
  if (!ok) return;
  const uint32_t lo = e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  const uint32_t hi = e4m3_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  reinterpret_cast<uint2*>(q)[i] = make_uint2(lo, hi);
  if ((i & 15) == 0) {
    const uint32_t gg = i >> 4, r = gg / ngpr, G = gg - r * ngpr;
    reinterpret_cast<uint32_t*>(sc)[G * nrows + r] = sw;
  }
}

// Column layout: a workgroup takes 4 consecutive 32-row blocks (in block
// order; with segments each block has its own first row and valid rows) x 64
// columns.  Rows come in as 16-byte vectors into LDS; wave w quantises block w
// with one column per lane (32 values down the column); the 64 x 128 encoded
// bytes are staged in LDS and leave as whole 128-byte runs of output rows.
constexpr int kColW = 64;

// With BOTH (no segments), the same tile is also quantised along the columns:
// thread t encodes 32 consecutive elements of tile row t/2 into the row layout
// qr [batch, rows, cols], scr [batch, rows, cols/32] (one read of the source
// serves both orientations).
template <typename T, bool BOTH, bool GROUPED>
__global__ __launch_bounds__(256) void mx_cols_kernel(const T* __restrict__ src, int64_t batch, int64_t rows,
                                                     int64_t cols,
                                                     const int32_t* __restrict__ seg, const int32_t* __restrict__ blk,
                                                     int nseg, int64_t ldq,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                     uint8_t* __restrict__ qr, uint8_t* __restrict__ scr) {
  constexpr int VEC = 16 / sizeof(T);       // elements per 16-byte vector
  constexpr int VPR = kColW / VEC;          // vectors per tile row
  constexpr int LDT = kColW + VEC;          // padded tile row (16-byte aligned)
  __shared__ __attribute__((aligned(16))) T tile[128 * LDT];
  // encoded bytes, 4 blocks x 32 per output row.  Without BOTH they take the
  // tile's place once every read of it is done (less LDS per workgroup, more
  // workgroups per CU: measured faster); BOTH still reads the tile afterwards.
  __shared__ uint32_t obuf_own[BOTH ? kColW : 1][33];
  static_assert(kColW * 33 * 4 <= 128 * LDT * sizeof(T), "output staging fits the tile");
  uint32_t (*obuf)[33] = BOTH ? obuf_own : reinterpret_cast<uint32_t (*)[33]>(tile);
  __shared__ uint8_t osc[kColW][4];
  __shared__ int32_t s_off[kMaxE + 1];
  __shared__ int32_t s_blk[kMaxE + 1];
  __shared__ int64_t b_r0[4];
  __shared__ int b_nv[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Tile of this workgroup.  BOTH: the two 64-column tiles of each 128-column
  // span go to workgroups 8 ids apart, hence on the same XCD, so the two
  // 64-byte halves of each row-layout line meet in one L2 (consecutive ids
  // alternate over the 8 XCDs); the grid is flat, 16 ids per 8 spans.
  int64_t bx, by, bz;
  if constexpr (BOTH) {
    const int64_t gx = (cols + kColW - 1) / kColW, gy = (rows / 32 + 3) / 4;
    const int64_t L = blockIdx.x, P = (L >> 4) * 8 + (L & 7), half = (L >> 3) & 1;
    const int64_t spans = gx / 2;  // cols % 128 == 0
    bx = 2 * (P % spans) + half;
    by = (P / spans) % gy;
    bz = P / (spans * gy);
    if (bz >= batch) return;  // the flat grid's tail
  } else {
    bx = blockIdx.x;
    by = blockIdx.y;
    bz = blockIdx.z;
  }
  const int64_t nblk = seg ? ldq / 32 : rows / 32;
  const int64_t b0 = by * 4;
  if (seg) {
    // segment offsets and the prefix sum of their 32-row block counts: given
    // (blk), or an inclusive scan over one thread per segment
    static_assert(kMaxE == 256, "one thread per segment");
    for (int i = tid; i <= nseg; i += blockDim.x) s_off[i] = seg[i];
    if (blk) {
      for (int i = tid; i <= nseg; i += blockDim.x) s_blk[i] = blk[i];
    } else {
      __syncthreads();
      int32_t c = 0;
      if (tid < nseg) {
        const int32_t n = s_off[tid + 1] - s_off[tid];
        c = n > 0 ? (n + 31) / 32 : 0;
      }
      s_blk[tid + 1] = c;
      if (tid == 0) s_blk[0] = 0;
      __syncthreads();
      for (int o = 1; o < kMaxE; o <<= 1) {
        const int32_t v = tid >= o ? s_blk[tid + 1 - o] : 0;
        __syncthreads();
        s_blk[tid + 1] += v;
        __syncthreads();
      }
    }
    __syncthreads();
  }
  if (tid < 4) {
    const int64_t b = b0 + tid;
    int64_t r0 = 0, nv = 0;
    if (b < nblk) {
      if (!seg) {
        r0 = b * 32;
        nv = 32;
      } else if (b < s_blk[nseg]) {  // blocks past the last segment stay zero padding
        int lo = 0, hi = nseg;       // s with s_blk[s] <= b < s_blk[s+1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_blk[mid] <= b) lo = mid; else hi = mid;
        }
        r0 = s_off[lo] + (b - s_blk[lo]) * 32;
        const int64_t end = s_off[lo + 1] < rows ? s_off[lo + 1] : rows;
        nv = end - r0;
        if (nv > 32) nv = 32;
        if (nv < 0) nv = 0;
      }
    }
    b_r0[tid] = r0;
    b_nv[tid] = static_cast<int>(nv);
  }
  __syncthreads();
  const int64_t c0 = bx * kColW;
  const T* base = src + bz * rows * cols;
  for (int v = tid; v < 128 * VPR; v += blockDim.x) {
    const int tr = v / VPR, cv = v - tr * VPR;
    const int bi = tr >> 5, r = tr & 31;
    const int64_t col = c0 + cv * VEC;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < b_nv[bi] && col < cols) val = *reinterpret_cast<const uint4*>(base + (b_r0[bi] + r) * cols + col);
    *reinterpret_cast<uint4*>(tile + tr * LDT + cv * VEC) = val;
  }
  __syncthreads();
  {
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      v[r] = Elem<T>::load1(tile, (wave * 32 + r) * LDT + lane);
      amax = fmaxf(amax, fabsf(v[r]));
    }
    const int e = mx_block_exponent(amax);
    const float inv = mx_inv_scale(e);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = e4m3_pack4(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
    if constexpr (!BOTH) __syncthreads();  // the tile is read: obuf takes its place
#pragma unroll
    for (int k = 0; k < 8; ++k) obuf[lane][wave * 8 + k] = w[k];
    osc[lane][wave] = static_cast<uint8_t>(e + 127);
  }
  __syncthreads();
  uint8_t* qb = q + bz * cols * ldq;
  for (int c = tid; c < kColW * 8; c += blockDim.x) {
    const int oc = c >> 3, ch = c & 7;  // 16-byte chunk ch of output row oc (block ch / 2)
    if (c0 + oc < cols && b0 + (ch >> 1) < nblk) {
      const uint32_t* o = &obuf[oc][ch * 4];
      uint8_t* dst = qb + (c0 + oc) * ldq + b0 * 32 + ch * 16;
      // BOTH (the weight cache, read by later passes): streaming stores of whole lines (1876 -> 1817 us per step
      // for the three weights at E = 128; streaming stores of the row layout's half lines were slower, 1946)
      if constexpr (BOTH) store16_nt(dst, make_uint4(o[0], o[1], o[2], o[3]));
      else *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  uint8_t* sb = sc + bz * cols * (ldq / 32);
  if constexpr (GROUPED) {
    // the four blocks of this workgroup are one group: 64 consecutive scale words
    if (tid < kColW && c0 + tid < cols) {
      const uint32_t w = osc[tid][0] | (osc[tid][1] << 8) | (osc[tid][2] << 16) | (static_cast<uint32_t>(osc[tid][3]) << 24);
      reinterpret_cast<uint32_t*>(sb)[(b0 >> 2) * cols + c0 + tid] = w;
    }
  } else {
    const int oc = tid >> 2, j = tid & 3;
    if (c0 + oc < cols && b0 + j < nblk) sb[(c0 + oc) * (ldq / 32) + b0 + j] = osc[oc][j];
  }
  if constexpr (BOTH) {
    const int64_t batch_rows = batch * rows;
    // row layout: in each half of the tile, four lanes per tile row (16
    // columns each, two lanes per 32-element block), so that a store
    // instruction writes 16 whole 64-byte row segments
    const int qt = tid & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tr = h * 64 + (tid >> 2);
      const int64_t r = b0 * 32 + tr;
      float v[16];
      const T* tp = tile + tr * LDT + qt * 16;
#pragma unroll
      for (int u = 0; u < 16 / VEC; ++u) {
        const uint4 raw = *reinterpret_cast<const uint4*>(tp + u * VEC);
        float tmp[VEC];
        Elem<T>::unpack(raw, tmp);
#pragma unroll
        for (int j = 0; j < VEC; ++j) v[u * VEC + j] = tmp[j];
      }
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      const int e = mx_block_exponent(amax);
      const float inv = mx_inv_scale(e);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = e4m3_pack4(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
      // the row's two scale bytes (blocks c0/32 and c0/32 + 1, adjacent in both scale layouts) from lanes qt = 0, 2
      const uint32_t pair = static_cast<uint32_t>(e + 127) | (static_cast<uint32_t>(__shfl_xor(e, 2, 64) + 127) << 8);
      if (r < rows && c0 + qt * 16 < cols) {
        *reinterpret_cast<uint4*>(qr + (bz * rows + r) * cols + c0 + qt * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        if (qt == 0)
          *reinterpret_cast<uint16_t*>(scr + scale_index(GROUPED, bz * rows + r, c0 / 32, batch_rows, cols / 32)) =
              static_cast<uint16_t>(pair);
      }
    }
  }
}

// Destination-major gather of an expert-major buffer's rows into both MX
// layouts at once (launch_mx_gather; without a permutation, both layouts of an
// expert-major buffer from one read): a workgroup takes 4 consecutive 32-row
// blocks of the padded token axis (in block order, each block inside one expert
// segment) and NSUB consecutive 64-column subtiles of them.  Each tile row names
// its expert row and, through the routing's permutation, the token row it
// copies (times the slot's gate for dY, rounded to bf16 as the combine backward
// stores it); every subtile's loads are issued before the first is encoded,
// so a row's scattered pieces are in flight together.  A subtile is quantised
// down the tokens exactly as mx_cols_kernel does with segments, and along d
// into the rows layout as mx_cols_kernel's BOTH pass does (the workgroup writes
// whole 128-byte lines of it); padding rows are zero in the token layout and
// absent from the rows layout.
template <bool SCALED, int NSUB>
__global__ __launch_bounds__(256) void mx_gather_kernel(const uint16_t* __restrict__ src, int64_t R, int d, int k,
                                                       const int32_t* __restrict__ perm_src,
                                                       const float* __restrict__ gates,
                                                       const int32_t* __restrict__ seg, const int32_t* __restrict__ blk,
                                                       int nseg, int64_t ldq, uint16_t* __restrict__ rows_out,
                                                       uint8_t* __restrict__ qr, uint8_t* __restrict__ scr,
                                                       uint8_t* __restrict__ qt, uint8_t* __restrict__ sct) {
  constexpr int VEC = 8;               // bf16 elements per 16-byte vector
  constexpr int VPR = kColW / VEC;     // vectors per tile row
  constexpr int LDT = kColW + VEC;     // padded tile row
  constexpr int NV = 128 * VPR / 256;  // vectors per thread and subtile
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * LDT];
  __shared__ uint32_t obuf[kColW][33];
  __shared__ uint8_t osc[kColW][4];
  __shared__ int32_t s_off[kMaxE + 1];
  __shared__ int32_t s_blk[kMaxE + 1];
  __shared__ int64_t s_src[128];  // element offset of the tile row's token row in src; -1: padding
  __shared__ int64_t s_row[128];  // the tile row's expert row; -1: padding
  __shared__ float s_gate[128];
  __shared__ int64_t b_r0[4];
  __shared__ int b_nv[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gx = d / (kColW * NSUB), gy = ldq / 128;  // d % (64 NSUB) == 0, ldq % 128 == 0
  const int64_t bx = blockIdx.x % gx, by = blockIdx.x / gx;
  if (by >= gy) return;
  const int64_t nblk = ldq / 32;
  const int64_t b0 = by * 4;
  for (int i = tid; i <= nseg; i += blockDim.x) {
    s_off[i] = seg[i];
    s_blk[i] = blk[i];
  }
  __syncthreads();
  if (tid < 4) {
    const int64_t b = b0 + tid;
    int64_t r0 = 0, nv = 0;
    if (b < nblk && b < s_blk[nseg]) {  // blocks past the last segment stay zero padding
      int lo = 0, hi = nseg;            // s with s_blk[s] <= b < s_blk[s+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_blk[mid] <= b) lo = mid; else hi = mid;
      }
      r0 = s_off[lo] + (b - s_blk[lo]) * 32;
      const int64_t end = s_off[lo + 1] < R ? s_off[lo + 1] : R;
      nv = end - r0;
      if (nv > 32) nv = 32;
      if (nv < 0) nv = 0;
    }
    b_r0[tid] = r0;
    b_nv[tid] = static_cast<int>(nv);
  }
  __syncthreads();
  if (tid < 128) {
    const int bi = tid >> 5, r = tid & 31;
    int64_t row = -1, off = -1;
    float g = 0.f;
    if (r < b_nv[bi]) {
      row = b_r0[bi] + r;
      if (perm_src) {
        const int32_t slot = perm_src[row];
        off = static_cast<int64_t>(slot / k) * d;
        if constexpr (SCALED) g = gates[slot];
      } else {
        off = row * d;  // no permutation: src is the expert-major buffer itself
      }
    }
    s_row[tid] = row;
    s_src[tid] = off;
    s_gate[tid] = g;
  }
  __syncthreads();
  // vector i of this thread: tile row (tid + 256 i) / VPR, 16-byte column (tid + 256 i) % VPR
  auto load = [&](int64_t c0, uint4 (&out)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + 256 * i;
      const int tr = v / VPR, cv = v - tr * VPR;
      const int64_t off = s_src[tr];
      out[i] = off >= 0 ? *reinterpret_cast<const uint4*>(src + off + c0 + cv * VEC) : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 all[NSUB][NV];  // every subtile's loads in flight at once: a row's NSUB x 128 bytes together
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) load((bx * NSUB + sub) * kColW, all[sub]);
  // rows layout: the low half of each row's group word (blocks of the even subtile), stored whole, as one
  // 4-byte word, with the odd subtile's half (2-byte pieces were half-sector writes)
  uint32_t pend[2] = {0u, 0u};
  static_assert(NSUB % 2 == 0, "subtile pairs make whole scale groups");
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    const int64_t c0 = (bx * NSUB + sub) * kColW;
    uint4 cur[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) cur[i] = all[sub][i];
    __syncthreads();  // the previous subtile's reads of the tile and of obuf are done
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + 256 * i;
      const int tr = v / VPR, cv = v - tr * VPR;
      uint4 val = cur[i];
      if (s_src[tr] >= 0) {
        if constexpr (SCALED) {
          float f[VEC];
          Elem<uint16_t>::unpack(val, f);
          const float g = s_gate[tr];
#pragma unroll
          for (int j = 0; j < VEC; ++j) f[j] = g * f[j];
          val = Elem<uint16_t>::pack(f);
        }
        if (rows_out) *reinterpret_cast<uint4*>(rows_out + s_row[tr] * d + c0 + cv * VEC) = val;
      }
      *reinterpret_cast<uint4*>(tile + tr * LDT + cv * VEC) = val;
    }
    __syncthreads();
    {
      // down the tokens: wave w encodes block w, one column per lane
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        v[r] = Elem<uint16_t>::load1(tile, (wave * 32 + r) * LDT + lane);
        amax = fmaxf(amax, fabsf(v[r]));
      }
      const int e = mx_block_exponent(amax);
      const float inv = mx_inv_scale(e);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        obuf[lane][wave * 8 + q] =
            e4m3_pack4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
      osc[lane][wave] = static_cast<uint8_t>(e + 127);
    }
    __syncthreads();
    for (int c = tid; c < kColW * 8; c += blockDim.x) {
      const int oc = c >> 3, ch = c & 7;  // 16-byte chunk ch of output row oc (block ch / 2)
      if (b0 + (ch >> 1) < nblk) {
        const uint32_t* o = &obuf[oc][ch * 4];
        // streaming stores: the token layout is read by the weight gradients, not by the next kernel (four
        // launches 676 -> 652 us per step at E = 128)
        store16_nt(qt + (c0 + oc) * ldq + b0 * 32 + ch * 16, make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
    if (tid < kColW) {
      // the four blocks of this workgroup are one group: 64 consecutive scale words
      const uint32_t w =
          osc[tid][0] | (osc[tid][1] << 8) | (osc[tid][2] << 16) | (static_cast<uint32_t>(osc[tid][3]) << 24);
      reinterpret_cast<uint32_t*>(sct)[(b0 >> 2) * d + c0 + tid] = w;
    }
    // along d: four lanes per tile row (16 columns each, two lanes per 32-element block)
    const int qq = tid & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tr = h * 64 + (tid >> 2);
      const int64_t row = s_row[tr];
      float v[16];
      const uint16_t* tp = tile + tr * LDT + qq * 16;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float tmp[VEC];
        Elem<uint16_t>::unpack(*reinterpret_cast<const uint4*>(tp + u * VEC), tmp);
#pragma unroll
        for (int j = 0; j < VEC; ++j) v[u * VEC + j] = tmp[j];
      }
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      const int e = mx_block_exponent(amax);
      const float inv = mx_inv_scale(e);
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = e4m3_pack4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
      // the row's two scale bytes (blocks c0/32 and c0/32 + 1, one half of its group word) from lanes qq = 0, 2
      const uint32_t pair =
          static_cast<uint32_t>(e + 127) | (static_cast<uint32_t>(__shfl_xor(e, 2, 64) + 127) << 8);
      if (row >= 0) {
        *reinterpret_cast<uint4*>(qr + row * d + c0 + qq * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        if (qq == 0) {
          if ((sub & 1) == 0)
            pend[h] = pair;
          else
            *reinterpret_cast<uint32_t*>(scr + scale_index(true, row, (c0 - kColW) / 32, R, d / 32)) =
                pend[h] | (pair << 16);
        }
      }
    }
  }
}

}  // namespace

void launch_mx_rows(const void* src, int src_dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sc,
                    hipStream_t s, bool grouped) {
  const int64_t nvec8 = rows * cols / 8;
  if (nvec8 == 0) return;
  if (grouped) {
    // cols % 128 == 0; the vector count fits 32 bits for the FFN's operands
    const dim3 grid(static_cast<unsigned>(cdiv(nvec8, 256)));
    if (src_dtype == MOE_F32)
      MOE_LAUNCH("mx_quantize_rows", mx_rows_grouped_kernel<float>, grid, dim3(256), 0, s,
                 static_cast<const float*>(src), static_cast<uint32_t>(nvec8), static_cast<uint32_t>(rows),
                 static_cast<uint32_t>(cols / 128), q, sc);
    else
      MOE_LAUNCH("mx_quantize_rows", mx_rows_grouped_kernel<uint16_t>, grid, dim3(256), 0, s,
                 static_cast<const uint16_t*>(src), static_cast<uint32_t>(nvec8), static_cast<uint32_t>(rows),
                 static_cast<uint32_t>(cols / 128), q, sc);
    return;
  }
  const dim3 grid(static_cast<unsigned>(cdiv(nvec8, 256)));
  if (src_dtype == MOE_F32)
    MOE_LAUNCH("mx_quantize_rows", mx_rows_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(src),
               nvec8, q, sc);
  else
    MOE_LAUNCH("mx_quantize_rows", mx_rows_kernel<uint16_t>, grid, dim3(256), 0, s,
               static_cast<const uint16_t*>(src), nvec8, q, sc);
}

void launch_mx_cols(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols, const int32_t* seg,
                    int nseg, int64_t ldq, uint8_t* q, uint8_t* sc, hipStream_t s, bool grouped, const int32_t* blk) {
  const int64_t nblk = seg ? ldq / 32 : rows / 32;
  if (nblk == 0 || cols == 0 || batch == 0) return;
  const dim3 grid(static_cast<unsigned>(cdiv(cols, kColW)), static_cast<unsigned>(cdiv(nblk, 4)),
                  static_cast<unsigned>(batch));
  if (src_dtype == MOE_F32) {
    if (grouped)
      MOE_LAUNCH("mx_quantize_cols", (mx_cols_kernel<float, false, true>), grid, dim3(256), 0, s,
                 static_cast<const float*>(src), batch, rows, cols, seg, blk, nseg, ldq, q, sc, nullptr, nullptr);
    else
      MOE_LAUNCH("mx_quantize_cols", (mx_cols_kernel<float, false, false>), grid, dim3(256), 0, s,
                 static_cast<const float*>(src), batch, rows, cols, seg, blk, nseg, ldq, q, sc, nullptr, nullptr);
  } else {
    if (grouped)
      MOE_LAUNCH("mx_quantize_cols", (mx_cols_kernel<uint16_t, false, true>), grid, dim3(256), 0, s,
                 static_cast<const uint16_t*>(src), batch, rows, cols, seg, blk, nseg, ldq, q, sc, nullptr, nullptr);
    else
      MOE_LAUNCH("mx_quantize_cols", (mx_cols_kernel<uint16_t, false, false>), grid, dim3(256), 0, s,
                 static_cast<const uint16_t*>(src), batch, rows, cols, seg, blk, nseg, ldq, q, sc, nullptr, nullptr);
  }
}

void launch_mx_both(const void* src, int src_dtype, int64_t batch, int64_t rows, int64_t cols, uint8_t* qc,
                    uint8_t* sc, uint8_t* qr, uint8_t* scr, hipStream_t s) {
  const int64_t nblk = rows / 32;
  if (nblk == 0 || cols == 0 || batch == 0) return;
  // flat grid of tiles (see mx_cols_kernel), rounded up to whole runs of 16 ids
  const int64_t tiles = cdiv(cols, kColW) * cdiv(nblk, 4) * batch;
  const dim3 grid(static_cast<unsigned>(cdiv(tiles, 16) * 16));
  if (src_dtype == MOE_F32)
    MOE_LAUNCH("mx_quantize_both", (mx_cols_kernel<float, true, true>), grid, dim3(256), 0, s,
               static_cast<const float*>(src), batch, rows, cols, nullptr, nullptr, 0, rows, qc, sc, qr, scr);
  else
    MOE_LAUNCH("mx_quantize_both", (mx_cols_kernel<uint16_t, true, true>), grid, dim3(256), 0, s,
               static_cast<const uint16_t*>(src), batch, rows, cols, nullptr, nullptr, 0, rows, qc, sc, qr, scr);
}

void launch_mx_gather(const uint16_t* src, int64_t R, int d, int k, const int32_t* perm_src, const float* gates,
                      const int32_t* seg, const int32_t* blk, int nseg, uint16_t* rows_out, uint8_t* qr,
                      uint8_t* scr, uint8_t* qt, uint8_t* sct, hipStream_t s) {
  if (R == 0 || d == 0) return;
  const int64_t ldq = mx_token_rows(R, nseg);
  const bool four = d % (4 * kColW) == 0;  // four 64-column subtiles per workgroup, else two (d % 128 == 0)
  const dim3 grid(static_cast<unsigned>((d / (kColW * (four ? 4 : 2))) * (ldq / 128)));
#define MOE_GATHER(SC, NS)                                                                                         \
  MOE_LAUNCH("mx_gather", (mx_gather_kernel<SC, NS>), grid, dim3(256), 0, s, src, R, d, k, perm_src, gates, seg, \
             blk, nseg, ldq, rows_out, qr, scr, qt, sct)
  if (gates) {
    if (four) MOE_GATHER(true, 4); else MOE_GATHER(true, 2);
  } else {
    if (four) MOE_GATHER(false, 4); else MOE_GATHER(false, 2);
  }
#undef MOE_GATHER
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
    launch_mx_rows(src, src_dtype, batch * rows, cols, q, scales, s, false);
    return launch_status();
  }
  if (cols % 8) return MOE_EINVAL;
  if (seg_offsets) {
    if (batch != 1 || nseg < 1 || nseg > kMaxE) return MOE_EINVAL;
    const int64_t ldq = 32 * (cdiv(rows, 32) + nseg);
    launch_mx_cols(src, src_dtype, 1, rows, cols, seg_offsets, nseg, ldq, q, scales, s, false, nullptr);
  } else {
    if (rows % 32) return MOE_EINVAL;
    launch_mx_cols(src, src_dtype, batch, rows, cols, nullptr, 0, rows, q, scales, s, false, nullptr);
  }
  return launch_status();
}
