// qtile.h -- staging of one query tile (128 packed rows, PackGQA order) in
// LDS as bf16 MFMA operands; shared by the scoring and block-mass kernels.
#pragma once

#include "device_common.h"

namespace fp {

constexpr int kQPitch = kD + 8;  // bf16 elements per staged Q row (bank spread)

__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = thread_x() >> 6;
  __syncthreads();
  if ((thread_x() & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Stage the tile's 128 packed query rows as bf16 (hi, and lo for fp32 input).
template <int DT>
__device__ __forceinline__ void stage_q(const Geo& g, const SegCoord& c, const TileGeo& t,
                                        const void* q, uint16_t* qh, uint16_t* ql) {
  const int tid = thread_x();
  const int64_t r0 = c.I * kRows;
  // all of a thread's loads are issued before the first is used
  if constexpr (DT == kBF16) {
    uint4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = tid + 256 * k, r = i >> 4, ch = i & 15;
      w[k] = make_uint4(0, 0, 0, 0);
      if (r < t.nrows) {
        int64_t pr = r0 + r;
        int64_t row = c.row0 + (pr >> g.log2g);
        int head = c.h * g.g + (int)(pr & (g.g - 1));
        w[k] = *(const uint4*)((const uint16_t*)q + (row * g.hq + head) * kD + ch * 8);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = tid + 256 * k, r = i >> 4, ch = i & 15;
      *(uint4*)(qh + r * kQPitch + ch * 8) = w[k];
    }
  } else if constexpr (DT == kE4M3) {
    uint4 wv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + 256 * k, r = i >> 3, ch = i & 7;
      wv[k] = make_uint4(0, 0, 0, 0);
      if (r < t.nrows) {
        int64_t pr = r0 + r;
        int64_t row = c.row0 + (pr >> g.log2g);
        int head = c.h * g.g + (int)(pr & (g.g - 1));
        wv[k] = *(const uint4*)((const uint8_t*)q + (row * g.hq + head) * kD + ch * 16);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + 256 * k, r = i >> 3, ch = i & 7;
      const uint4 w = wv[k];
      uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      uint16_t o[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 f = e4m3x4_to_f32(ww[j]);  // exact in bf16
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * j + e] = f32_to_bf16_bits(f[e]);
      }
      uint4* dst = (uint4*)(qh + r * kQPitch + ch * 16);
      dst[0] = *(uint4*)&o[0];
      dst[1] = *(uint4*)&o[8];
    }
  } else {
    float4 wv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = tid + 256 * k, r = i >> 5, ch = i & 31;
      wv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < t.nrows) {
        int64_t pr = r0 + r;
        int64_t row = c.row0 + (pr >> g.log2g);
        int head = c.h * g.g + (int)(pr & (g.g - 1));
        wv[k] = *(const float4*)((const float*)q + (row * g.hq + head) * kD + ch * 4);
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = tid + 256 * k, r = i >> 5, ch = i & 31;
      const float4 w = wv[k];
      float f[4] = {w.x, w.y, w.z, w.w};
      uint16_t oh[4], ol[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oh[e] = f32_to_bf16_bits(f[e]);
        ol[e] = f32_to_bf16_bits(f[e] - bf16_bits_to_f32(oh[e]));
      }
      *(uint2*)(qh + r * kQPitch + ch * 4) = *(uint2*)oh;
      *(uint2*)(ql + r * kQPitch + ch * 4) = *(uint2*)ol;
    }
  }
}

}  // namespace fp
