// mass.hip -- exact block attention mass of every (query tile, candidate
// block): the diagnostic that measures what the pooled-key selection keeps.
//
// FlashPrefill (V1) summary page, §3.1 "exact identification": every query of
// the tile against every visible key, the attention summed within each block
// and averaged over the tile's queries,
//   mass_J = (1/n) sum_r sum_{i in B_J, i <= t_r} exp(sigma q_r.k_i - LSE_r),
// with LSE_r the row's dense log-sum-exp (an input: fp_dense_attn's LSE).  For
// the blocks J < beta that every row sees whole, the mean surrogate that the
// correction of [V2] Eq. 6 substitutes (V1 §3.1's Psi_pool against Psi_sum),
//   sur_J = (1/n) sum_r 128 exp(sigma q_r.k_bar_J - LSE_r).
//
// One workgroup per segment; the tile's Q rows are staged once in LDS (A
// operand).  For the exact mass each wave takes whole blocks (four 32-key
// column tiles): K rows go straight from memory into the B operand, one
// v_mfma_f32_32x32x16_bf16 chain per 32 rows x 32 keys, then one exp2 per
// (row, key) against the row's LSE with the causal mask on the tiles that
// reach past the tile's first position.  Each lane owns one key column, so a
// block's sum is one wave reduction.  The surrogate reuses the scoring
// kernel's operands (k_bar split into bf16 hi + lo).  This is a diagnostic:
// it does the dense QK^T work (no P V), about half a dense attention call.
#include "device_common.h"
#include "qtile.h"

namespace fp {

namespace {

// B operand of K rows: lane (key column col, half) gets dims 16 ks + 8 half ..
// +8 of key `row` as bf16 (hi; lo for fp32 inputs).  `row` < 0 reads zeros.
template <int DT>
__device__ __forceinline__ void k_operand(const void* k, int64_t row, int hkv, int h, int half,
                                          bf16x8 (&bh)[8], bf16x8 (&bl)[8]) {
  if constexpr (DT == kBF16) {
    const uint16_t* p = (const uint16_t*)k + (row * hkv + h) * kD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bh[ks] = row >= 0 ? *(const bf16x8*)(p + 16 * ks) : bf16x8{};
  } else if constexpr (DT == kE4M3) {
    const uint8_t* p = (const uint8_t*)k + (row * hkv + h) * kD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint2 w = row >= 0 ? *(const uint2*)(p + 16 * ks) : make_uint2(0, 0);
      f32x4 a = e4m3x4_to_f32(w.x), b = e4m3x4_to_f32(w.y);  // exact in bf16
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (__bf16)a[e];
        o[4 + e] = (__bf16)b[e];
      }
      bh[ks] = o;
    }
  } else {
    const float* p = (const float*)k + (row * hkv + h) * kD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (row >= 0) {
        x0 = *(const float4*)(p + 16 * ks);
        x1 = *(const float4*)(p + 16 * ks + 4);
      }
      float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = (__bf16)f[e];
        lo[e] = (__bf16)(f[e] - (float)hi[e]);
      }
      bh[ks] = hi;
      bl[ks] = lo;
    }
  }
}

// Q rows 32 rt .. +31 x the 32 columns of the B operand; lane (col, half)
// gets column col, rows 32 rt + 8 (r / 4) + 4 half + r % 4 in element r.
template <int NQ, bool BLO>
__device__ __forceinline__ f32x16 qk_rows(const uint16_t* qh, const uint16_t* ql, int rt, int col, int half,
                                          const bf16x8 (&bh)[8], const bf16x8 (&bl)[8]) {
  f32x16 acc = f32x16{};
  const uint16_t* arow = qh + (rt * 32 + col) * kQPitch + 8 * half;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 a = *(const bf16x8*)(arow + ks * 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], acc, 0, 0, 0);
    if constexpr (BLO) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[ks], acc, 0, 0, 0);
    if constexpr (NQ == 2) {
      bf16x8 al = *(const bf16x8*)(ql + (rt * 32 + col) * kQPitch + 8 * half + ks * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh[ks], acc, 0, 0, 0);
    }
  }
  return acc;
}

}  // namespace

template <int DT>
__global__ __launch_bounds__(256) void block_mass_kernel(Geo g, MeansLayout ml, const void* __restrict__ q,
                                                         const void* __restrict__ k,
                                                         const float* __restrict__ lse,
                                                         const char* __restrict__ means,
                                                         float* __restrict__ mass, float* __restrict__ sur) {
  extern __shared__ __align__(16) char smem[];
  constexpr int NQ = DT == kF32 ? 2 : 1;
  uint16_t* qh = (uint16_t*)smem;
  uint16_t* ql = qh + kRows * kQPitch;
  float* lse2 = (float*)(smem + NQ * kRows * kQPitch * 2);  // row LSE in log2 units
  int* qpos = (int*)(lse2 + kRows);                           // row's query index (position - off)
  __shared__ int err_sh;

  const int64_t s = block_x();
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  const int lane = thread_x() & 63, wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int nc = t.beta1 + 1;
  const float dq = DT == kE4M3 ? g.descale[0] : 1.f;
  const float dk = DT == kE4M3 ? g.descale[1] : 1.f;
  const float l2e = 1.4426950408889634f;
  const float sl_k = g.scale * l2e * dq * dk;  // exact keys
  // the pooled means' scoring operands are stored already multiplied by
  // sigma log2 e (and c_q): their products are logits in log2 units
  const float inv_n = 1.f / (float)t.nrows;

  if (thread_x() == 0) err_sh = 0;
  if (thread_x() < kRows) {
    const int r = thread_x();
    float l = INFINITY;  // padding rows: exp2(x - inf) = 0
    int qi = 0;
    if (r < t.nrows) {
      const int64_t pr = c.I * kRows + r;
      qi = (int)(pr >> g.log2g);
      const int head = c.h * g.g + (int)(pr & (g.g - 1));
      l = lse[(c.row0 + qi) * g.hq + head] * l2e;
    }
    lse2[r] = l;
    qpos[r] = qi;
  }
  stage_q<DT>(g, c, t, q, qh, ql);
  __syncthreads();

  // exact mass: wave takes blocks J = wave, wave + 4, ...
  for (int J = wave; J < nc; J += 4) {
    float acc_sum = 0.f;
#pragma unroll 1
    for (int ct = 0; ct < 4; ++ct) {
      const int key0 = J * kBlock + ct * 32;
      if (key0 > t.t1) break;  // no row sees these keys
      const int key = key0 + col;
      int64_t row = -1;
      if (key <= t.t1) {
        row = kv_row(g, c, key);
        if (row < 0) atomicOr(&err_sh, kErrPage);
      }
      bf16x8 bh[8], bl[8];
      k_operand<DT>(k, row, g.hkv, c.h, half, bh, bl);
      const bool masked = key0 + 31 > t.t0;  // some key here lies past some row's position
      const int kq = key - c.off;             // visible to rows whose query index is >= kq
      float part = 0.f;
#pragma unroll 1
      for (int rt = 0; rt < 4; ++rt) {
        const f32x16 acc = qk_rows<NQ, DT == kF32>(qh, ql, rt, col, half, bh, bl);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int R = rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          float e = __builtin_amdgcn_exp2f(fmaf(acc[r], sl_k, -lse2[R]));
          if (masked && kq > qpos[R]) e = 0.f;
          part += e;
        }
      }
      if (row >= 0) acc_sum += part;
    }
    const float tot = wave_sum(acc_sum);
    if (lane == 0) mass[s * g.max_nj + J] = tot * inv_n;
  }
  for (int J = nc + thread_x(); J < g.max_nj; J += 256) mass[s * g.max_nj + J] = -1.f;

  if (sur) {
    // surrogate: 32-block column tiles of the pooled means, blocks J < beta
    const bf16x8* khi = (const bf16x8*)(means + ml.khi);
    const bf16x8* klo = (const bf16x8*)(means + ml.klo);
    const int64_t jt0 = g.blk_base[c.b] >> 5;
    const bf16x8* khs = khi + ((jt0 * g.hkv + c.h) * 8) * 64;
    const bf16x8* kls = klo + ((jt0 * g.hkv + c.h) * 8) * 64;
    const int64_t jstride = (int64_t)g.hkv * 8 * 64;
    for (int jt = wave; jt * 32 < t.beta; jt += 4) {
      bf16x8 bh[8], bl[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bh[ks] = khs[jt * jstride + ks * 64 + lane];
        bl[ks] = kls[jt * jstride + ks * 64 + lane];
      }
      float sum = 0.f;
#pragma unroll 1
      for (int rt = 0; rt < 4; ++rt) {
        const f32x16 acc = qk_rows<NQ, true>(qh, ql, rt, col, half, bh, bl);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int R = rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          sum += __builtin_amdgcn_exp2f(acc[r] - lse2[R]);
        }
      }
      sum += __shfl_xor(sum, 32, 64);
      const int J = jt * 32 + col;
      if (half == 0 && J < t.beta) sur[s * g.max_nj + J] = (float)kBlock * sum * inv_n;
    }
    for (int J = t.beta + thread_x(); J < g.max_nj; J += 256) sur[s * g.max_nj + J] = J < nc ? 0.f : -1.f;
  }
  __syncthreads();
  if (thread_x() == 0 && err_sh) atomicOr(&g.hdr->err, err_sh);
}

hipError_t launch_block_mass(const Geo& g, const MeansLayout& ml, const void* q, const void* k,
                             const float* lse, const char* means, float* mass, float* sur, hipStream_t st) {
  const int nq = g.dtype == kF32 ? 2 : 1;
  const size_t lds = (size_t)nq * kRows * kQPitch * 2 + kRows * 8;
  dim3 grid((unsigned)g.n_seg);
  {
    const void* fn = g.dtype == kBF16 ? (const void*)block_mass_kernel<kBF16>
                     : g.dtype == kF32 ? (const void*)block_mass_kernel<kF32>
                                       : (const void*)block_mass_kernel<kE4M3>;
    hipError_t e = set_lds_limit(fn, 2 * kRows * kQPitch * 2 + kRows * 8);
    if (e != hipSuccess) return e;
  }
  switch (g.dtype) {
    case kBF16:
      block_mass_kernel<kBF16><<<grid, 256, lds, st>>>(g, ml, q, k, lse, means, mass, sur);
      break;
    case kF32:
      block_mass_kernel<kF32><<<grid, 256, lds, st>>>(g, ml, q, k, lse, means, mass, sur);
      break;
    default:
      block_mass_kernel<kE4M3><<<grid, 256, lds, st>>>(g, ml, q, k, lse, means, mass, sur);
      break;
  }
  return hipGetLastError();
}

}  // namespace fp
