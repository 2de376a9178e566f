// fp8_mfma_probe.hip -- test support: the E4M3 MFMA exactly as the attention
// kernel uses it for logits (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales,
// two chained MFMAs over a 128-wide contraction, the kernel's lane layout),
// on caller-given 32x128 tiles, so that a test can measure how far its fp32
// results sit from the exact sums.  Not part of libfp.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One 64-lane workgroup per tile: D[t][i][j] = sum_k A[t][i][k] * B[t][j][k]
// for E4M3 codes A, B [ntiles][32][128] and fp32 D [ntiles][32][32].
__global__ __launch_bounds__(64) void fp8_mfma_probe_kernel(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ B,
                                                            float* __restrict__ D, int ntiles) {
  const int tile = blockIdx.x;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const uint8_t* a = A + (size_t)tile * 32 * 128;
  const uint8_t* b = B + (size_t)tile * 32 * 128;
  f32x16 acc = {};
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    // lane (c, h) holds row c, contraction elements 64 m + 32 h .. +31
    const uint4* ap = (const uint4*)(a + c * 128 + 64 * m + 32 * h);
    const uint4* bp = (const uint4*)(b + c * 128 + 64 * m + 32 * h);
    const uint4 a0 = ap[0], a1 = ap[1], b0 = bp[0], b1 = bp[1];
    const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  }
  // register r of lane (c, h) is D[8 (r / 4) + 4 h + r % 4][c]
  float* d = D + (size_t)tile * 32 * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) d[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + c] = acc[r];
}

extern "C" int fp8_mfma_probe(const uint8_t* A, const uint8_t* B, float* D, int ntiles, void* stream) {
  if (ntiles < 0) return -1;
  if (ntiles == 0) return 0;
  fp8_mfma_probe_kernel<<<ntiles, 64, 0, (hipStream_t)stream>>>(A, B, D, ntiles);
  return (int)hipGetLastError();
}
