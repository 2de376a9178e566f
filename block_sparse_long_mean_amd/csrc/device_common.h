// device_common.h -- small device helpers shared by the kernels of libfp.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp_internal.h"

namespace fp {

// Work-item and work-group ids read straight from the hardware registers.
// HIP's threadIdx / blockIdx / gridDim and __syncthreads_or go through
// device-library functions that are not inlined into code built with IEEE
// mode off (their function attributes differ), and each such call costs a
// full register save around it; these builtins need none.
__device__ __forceinline__ int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int block_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two floats -> two OCP E4M3 codes packed in the low 16 bits (round to
// nearest even; inputs are kept inside +-448 by the callers).
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Four floats -> four OCP E4M3 codes in one dword (a, b in the low half, c, d
// in the high half), two conversions that each write one half of the word.
// The first one's other half is a placeholder that the second overwrites.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Four E4M3 codes (one dword) -> four floats.
__device__ __forceinline__ f32x4 e4m3x4_to_f32(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f32x4 r;
  r[0] = lo[0];
  r[1] = lo[1];
  r[2] = hi[0];
  r[3] = hi[1];
  return r;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = thread_x() & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Segment s -> (request b, kv head h, tile I) through the per-request segment
// offsets (binary search; segments are ordered request, kv head, tile).
struct SegCoord {
  int b, h;
  int64_t I;
  int L;        // key/value length of the request
  int Lq;       // query length (the queries are the last Lq positions)
  int off;      // position of the first query: L - Lq
  int64_t row0; // first Q row of the request
  int64_t kv0;  // first K/V row of the request (contiguous layout)
};

__device__ __forceinline__ SegCoord seg_coord(const Geo& g, int64_t s) {
  int lo = 0, hi = g.nreq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)g.seg_off[mid] <= s)
      lo = mid;
    else
      hi = mid - 1;
  }
  SegCoord c;
  c.b = lo;
  // 32-bit division: segment counts stay below 2^31 / 16 (checked on the
  // host), and a 64-bit division expands to ~140 scalar instructions
  const int local = (int)(s - g.seg_off[lo]);
  int nt = (g.seg_off[lo + 1] - g.seg_off[lo]) / g.hkv;
  if (nt < 1) nt = 1;
  c.h = local / nt;
  c.I = local - c.h * nt;
  c.row0 = g.cu_q[lo];
  c.Lq = g.cu_q[lo + 1] - g.cu_q[lo];
  c.kv0 = g.cu_kv[lo];
  c.L = g.cu_kv[lo + 1] - g.cu_kv[lo];
  c.off = c.L - c.Lq;
  return c;
}

// Tile geometry: valid packed rows, first/last (absolute) position, and the
// blocks of the first and last position.  Packed row r of the tile is query
// r >> log2g of the request, at position off + (r >> log2g).  A fresh prefill's
// tile never crosses a block edge (beta1 == beta); a chunk that starts inside a
// block can put one tile across two blocks, and both are its diagonal.
struct TileGeo {
  int nrows;
  int t0, t1, beta, beta1;
};

__device__ __forceinline__ TileGeo tile_geo(const Geo& g, const SegCoord& c) {
  TileGeo t;
  int64_t packed = (int64_t)c.Lq << g.log2g;
  int64_t r0 = c.I * kRows;
  int64_t r1 = r0 + kRows;
  if (r1 > packed) r1 = packed;
  t.nrows = (int)(r1 - r0);
  t.t0 = c.off + (int)(r0 >> g.log2g);
  t.t1 = c.off + (int)((r1 - 1) >> g.log2g);
  t.beta = t.t0 / kBlock;
  t.beta1 = t.t1 / kBlock;
  return t;
}

// Row of the K/V storage holding token j of request b ([V2] Eq. 22), or -1
// when the page table points outside the pool.
__device__ __forceinline__ int64_t kv_row(const Geo& g, const SegCoord& c, int j) {
  if (!g.page_table) return c.kv0 + j;
  int pg = j / g.page_size;
  int64_t page = g.page_table[(int64_t)c.b * g.max_pages + pg];
  int64_t slot = page * g.page_size + (j - pg * g.page_size);
  if (page < 0 || slot >= g.num_slots) return -1;
  return slot;
}

__device__ __forceinline__ int elem_bytes(int dtype) {
  return dtype == kF32 ? 4 : (dtype == kBF16 ? 2 : 1);
}

}  // namespace fp
