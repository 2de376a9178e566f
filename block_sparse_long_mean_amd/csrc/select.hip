// select.hip -- index stage after pooling: block scoring, alpha*max selection,
// CSR offsets and CSR expansion.
//
// Scoring ([V2] §3.1 Eq. 1-3, §3.3 Eq. 19-20).  One workgroup per segment
// (one PackGQA query tile of 128 packed rows of one KV head).  The tile's Q
// rows are staged once in LDS; every wave takes 32-block column tiles of the
// pooled keys and computes the 128x32 logit tile with bf16 MFMAs.  kbar is
// fp32, split into bf16 hi + lo (two MFMAs per step, ~16 significant bits)
// so that the normalised energies are accurate to ~1e-5 relative; fp32
// queries are split the same way (three MFMAs).  Each lane owns one block
// column and 64 of its 128 rows, so the per-block maximum m_J and the energy
// S_J = sum_r 2^(s_rJ log2 e - m_J) (the form of Eq. 1, in log2 units) need
// only one cross-lane exchange and no workgroup barrier; the final rescale
// E_J = S_J 2^(m_J - M) with M = max_J m_J is the step Eq. 20 describes.
// Selection keeps E_J >= alpha * max E or forced blocks, writes one bit per
// block and the segment's tile count; no energy array goes to HBM.
#include "device_common.h"
#include "qtile.h"

namespace fp {

template <int DT>
__global__ __launch_bounds__(256) void score_select_kernel(Geo g, MeansLayout ml, const void* __restrict__ q,
                                                           const char* __restrict__ means, float alpha,
                                                           int sink, int win, int32_t* __restrict__ counts,
                                                           uint32_t* __restrict__ bits,
                                                           float* __restrict__ energies) {
  extern __shared__ __align__(16) char smem[];
  constexpr int NQ = DT == kF32 ? 2 : 1;
  uint16_t* qh = (uint16_t*)smem;
  uint16_t* ql = qh + kRows * kQPitch;
  float* mJ = (float*)(smem + NQ * kRows * kQPitch * 2);
  float* SJ = mJ + g.max_nj;
  __shared__ float red[4];
  __shared__ int nsel_w[4];

  const int64_t s = blockIdx.x;
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const float sl = g.scale * 1.4426950408889634f * (DT == kE4M3 ? g.descale[0] : 1.f);
  const int nc = t.beta1 + 1;  // blocks holding a key visible to some row
  const int njt = (nc + 31) >> 5;
  const bf16x8* khi = (const bf16x8*)(means + ml.khi);
  const bf16x8* klo = (const bf16x8*)(means + ml.klo);
  const int64_t jt0 = g.blk_base[c.b] >> 5;
  const int half = lane >> 5, col = lane & 31;

  // the B operands (kbar hi, lo) of column tile jt: 32 blocks x 128 dims, the
  // segment's column tiles one fragment stride apart
  const bf16x8* khs = khi + ((jt0 * g.hkv + c.h) * 8) * 64;
  const bf16x8* kls = klo + ((jt0 * g.hkv + c.h) * 8) * 64;
  const int64_t jstride = (int64_t)g.hkv * 8 * 64;
  const int nrows = t.nrows;
  auto kb_load = [&](int jt, bf16x8 (&bh)[8], bf16x8 (&bl)[8]) {
    const bf16x8* ph = khs + jt * jstride;
    const bf16x8* pl = kls + jt * jstride;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bh[ks] = ph[ks * 64 + lane];
      bl[ks] = pl[ks * 64 + lane];
    }
  };
  // logits of the 128 rows x 32 blocks of column tile jt, 32 rows at a time;
  // per block (= lane column) the running maximum of the raw products (sl > 0)
  // and the sum of 2^(logit - max), logits in log2 units
  auto tile = [&](auto ragged_tag, int jt, const bf16x8 (&bh)[8], const bf16x8 (&bl)[8]) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    float m = -INFINITY, sum = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x16 acc = f32x16{};
      const uint16_t* arow = qh + (rt * 32 + col) * kQPitch + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 a = *(const bf16x8*)(arow + ks * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[ks], acc, 0, 0, 0);
        if constexpr (NQ == 2) {
          bf16x8 al = *(const bf16x8*)(ql + (rt * 32 + col) * kQPitch + 8 * half + ks * 16);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh[ks], acc, 0, 0, 0);
        }
      }
      // lane owns block column col, rows rt*32 + 8*(r/4) + 4*half + r%4; padding
      // rows of a ragged tile are masked out
      if constexpr (RAGGED) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nrows) acc[r] = -INFINITY;
      }
      float m0 = fmaxf(acc[0], fmaxf(acc[1], acc[2])), m1 = fmaxf(acc[8], fmaxf(acc[9], acc[10]));
      m0 = fmaxf(m0, fmaxf(acc[3], acc[4]));
      m1 = fmaxf(m1, fmaxf(acc[11], acc[12]));
      m0 = fmaxf(m0, fmaxf(acc[5], acc[6]));
      m1 = fmaxf(m1, fmaxf(acc[13], acc[14]));
      m0 = fmaxf(m0, fmaxf(acc[7], acc[15]));
      const float mn = fmaxf(m, fmaxf(m0, m1));
      const float msl = mn == -INFINITY ? 0.f : mn * sl;
      float s0 = sum * __builtin_amdgcn_exp2f(fmaf(m, sl, -msl)), s1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        s0 += __builtin_amdgcn_exp2f(fmaf(acc[r], sl, -msl));
        s1 += __builtin_amdgcn_exp2f(fmaf(acc[r + 1], sl, -msl));
      }
      sum = s0 + s1;
      m = mn;
    }
    // the other lane half holds the block's other 64 rows
    const float mo = __shfl_xor(m, 32, 64), so = __shfl_xor(sum, 32, 64);
    const float mx = fmaxf(m, mo) * sl;
    sum = sum * __builtin_amdgcn_exp2f(fmaf(m, sl, -mx)) + so * __builtin_amdgcn_exp2f(fmaf(mo, sl, -mx));
    const int J = jt * 32 + col;
    if (half == 0 && J < nc) {
      mJ[J] = mx;
      SJ[J] = sum;
    }
  };
  // one register set of operands per wave; the first column tile's load is in
  // flight while Q is staged
  bf16x8 bh[8], bl[8];
  if (wave < njt) kb_load(wave, bh, bl);
  stage_q<DT>(g, c, t, q, qh, ql);
  __syncthreads();
  auto sweep = [&](auto ragged_tag) {
    for (int jt = wave; jt < njt; jt += 4) {
      if (jt != wave) kb_load(jt, bh, bl);
      tile(ragged_tag, jt, bh, bl);
    }
  };
  if (nrows < kRows)
    sweep(std::true_type{});
  else
    sweep(std::false_type{});
  __syncthreads();

  // E_J = S_J 2^(m_J - M), M = max_J m_J; then keep E_J >= alpha max E or forced.
  float lm = -INFINITY;
  for (int J = threadIdx.x; J < nc; J += 256) lm = fmaxf(lm, mJ[J]);
  const float M = block_max(lm, red);
  float le = 0.f;
  for (int J = threadIdx.x; J < nc; J += 256) {
    float e = SJ[J] * __builtin_amdgcn_exp2f(mJ[J] - M);
    SJ[J] = e;
    le = fmaxf(le, e);
  }
  const float Emax = block_max(le, red);  // >= 1: the block attaining M has S >= 1
  const float thr = alpha * Emax;
  int nsel = 0;
  for (int base = wave * 64; base < nc; base += 256) {
    const int J = base + lane;
    const bool in = J < nc;
    const bool forced = J < sink || (J >= t.beta - win && J < t.beta) || J >= t.beta;
    const bool sel = in && (forced || SJ[J] >= thr);
    const uint64_t m = __ballot(sel);
    if (lane == 0) {
      int w0 = base >> 5;
      bits[s * g.words + w0] = (uint32_t)m;
      if (w0 + 1 < g.words) bits[s * g.words + w0 + 1] = (uint32_t)(m >> 32);
    }
    nsel += __popcll(m);
    if (energies && in) energies[s * g.max_nj + J] = SJ[J] / Emax;
  }
  if (energies)
    for (int J = nc + threadIdx.x; J < g.max_nj; J += 256) energies[s * g.max_nj + J] = -1.f;
  if (lane == 0) nsel_w[wave] = nsel;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = nsel_w[0] + nsel_w[1] + nsel_w[2] + nsel_w[3];
    // each kept block gives tiles 2J and 2J+1; the last block's second tile is
    // dropped when it starts after the tile's last position
    int trim = (int64_t)kTile * (2 * t.beta1 + 1) > t.t1 ? 1 : 0;
    counts[s] = 2 * tot - trim;
  }
}

// Exclusive prefix sum of the per-segment counts into cu[n+1], in two
// passes: 1024-entry blocks reduce to partial sums (scan_part_kernel), then
// every block rescans its entries on top of the sum of the partials before it.
__device__ __forceinline__ int block_excl_scan_1024(int x, int* sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  if (w == 0) {
    int v = lane < 16 ? sh[lane] : 0;
    int vi = wave_incl_scan(v);
    if (lane < 16) sh[16 + lane] = vi - v;
    if (lane == 15) sh[32] = vi;
  }
  __syncthreads();
  total = sh[32];
  const int r = sh[16 + w] + incl - x;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void scan_part_kernel(const int32_t* __restrict__ counts, int64_t n,
                                                         int32_t* __restrict__ part) {
  __shared__ int sh[40];
  const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  int total;
  block_excl_scan_1024(i < n ? counts[i] : 0, sh, total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void scan_final_kernel(const int32_t* __restrict__ counts, int64_t n,
                                                          const int32_t* __restrict__ part, int32_t* __restrict__ cu) {
  __shared__ int sh[40];
  __shared__ int base_sh;
  // offset of this block: sum of the partials before it (one wave)
  if (threadIdx.x < 64) {
    int acc = 0;
    for (int b = threadIdx.x; b < (int)blockIdx.x; b += 64) acc += part[b];
    acc = wave_sum_i(acc);
    if (threadIdx.x == 0) base_sh = acc;
  }
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  const int x = i < n ? counts[i] : 0;
  int total;
  const int ex = block_excl_scan_1024(x, sh, total);
  if (i < n) cu[i] = base_sh + ex;
  if (i == n - 1) cu[n] = base_sh + ex + x;
}

// One wave per segment: ballot + prefix count turn the selection bits into the
// ascending list of physical tile ids (logical block J -> tiles 2J, 2J+1).
__global__ __launch_bounds__(256) void expand_kernel(Geo g, const int32_t* __restrict__ cu,
                                                     const uint32_t* __restrict__ bits,
                                                     int32_t* __restrict__ idx, int64_t cap) {
  const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= g.n_seg) return;
  const int lane = threadIdx.x & 63;
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  const int64_t start = cu[s];
  const int nc = t.beta1 + 1;  // blocks holding a key visible to some row
  int o = 0;
  for (int base = 0; base < nc; base += 64) {
    const int J = base + lane;
    bool sel = false;
    if (J < nc) sel = (bits[s * g.words + (J >> 5)] >> (J & 31)) & 1u;
    const uint64_t m = __ballot(sel);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (sel) {
      int64_t pos = start + o + 2 * before;
      if (pos < cap) idx[pos] = 2 * J;
      if ((int64_t)kTile * (2 * J + 1) <= t.t1 && pos + 1 < cap) idx[pos + 1] = 2 * J + 1;
    }
    o += 2 * __popcll(m);
  }
}

hipError_t launch_score_select(const Geo& g, const MeansLayout& ml, const void* q, const char* means,
                               float alpha, int sink, int win, int32_t* counts, uint32_t* bits,
                               float* energies, hipStream_t st) {
  const int nq = g.dtype == kF32 ? 2 : 1;
  size_t lds = (size_t)nq * kRows * kQPitch * 2 + (size_t)g.max_nj * 8;
  dim3 grid((unsigned)g.n_seg);
  static bool attr_set[3] = {false, false, false};
  if (!attr_set[g.dtype]) {
    const void* fn = g.dtype == kBF16 ? (const void*)score_select_kernel<kBF16>
                     : g.dtype == kF32 ? (const void*)score_select_kernel<kF32>
                                       : (const void*)score_select_kernel<kE4M3>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       2 * kRows * kQPitch * 2 + kMaxBlocks * 8);
    if (e != hipSuccess) return e;
    attr_set[g.dtype] = true;
  }
  switch (g.dtype) {
    case kBF16:
      score_select_kernel<kBF16><<<grid, 256, lds, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                         energies);
      break;
    case kF32:
      score_select_kernel<kF32><<<grid, 256, lds, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                        energies);
      break;
    default:
      score_select_kernel<kE4M3><<<grid, 256, lds, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                         energies);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* counts, int64_t n, int32_t* cu, int32_t* part, hipStream_t st) {
  const unsigned nb = (unsigned)((n + 1023) / 1024);
  scan_part_kernel<<<nb, 1024, 0, st>>>(counts, n, part);
  scan_final_kernel<<<nb, 1024, 0, st>>>(counts, n, part, cu);
  return hipGetLastError();
}

hipError_t launch_expand(const Geo& g, const int32_t* cu, const uint32_t* bits, int32_t* idx, int64_t cap,
                         hipStream_t st) {
  expand_kernel<<<(unsigned)((g.n_seg + 3) / 4), 256, 0, st>>>(g, cu, bits, idx, cap);
  return hipGetLastError();
}

}  // namespace fp
