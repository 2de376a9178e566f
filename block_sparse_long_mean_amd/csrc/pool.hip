// pool.hip -- per-request metadata and block-mean pooling of K and V.
//
// Pooling ([V2] §3.2 Eq. 5, §3.4 index stage): kbar_J and vbar_J are the means
// of the keys / values of block J over the block's actual token count (E4M3
// inputs are descaled first).  The kernel is HBM-bound: every K/V byte is read
// once with 16-byte loads, 16 lanes per 256-byte key row, and summed in fp32.
// Besides the float means it writes the derived operands other kernels use:
// kbar split into bf16 hi + lo parts in MFMA B-operand order (scoring), and
// kbar/vbar in the input element type (mean-correction steps of attention).
#include "device_common.h"

namespace fp {

// One workgroup: exclusive scans of per-request segment counts and padded
// block counts.  Also clears the device error flag of the workspace.
__global__ __launch_bounds__(1024) void meta_kernel(Geo g) {
  __shared__ int64_t sseg[1024];
  __shared__ int64_t sblk[1024];
  const int tid = thread_x();
  const int per = (g.nreq + 1023) / 1024;
  const int lo = tid * per;
  const int hi = min(lo + per, g.nreq);
  int64_t ns = 0, nb = 0;
  // segments come from the query length, blocks from the key length
  for (int b = lo; b < hi; ++b) {
    int64_t Lq = g.cu_q[b + 1] - g.cu_q[b];
    int64_t L = g.cu_kv[b + 1] - g.cu_kv[b];
    ns += (int64_t)g.hkv * (((Lq << g.log2g) + kRows - 1) / kRows);
    nb += ((L + kBlock - 1) / kBlock + kChunk - 1) / kChunk * kChunk;
  }
  sseg[tid] = ns;
  sblk[tid] = nb;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int64_t a = tid >= o ? sseg[tid - o] : 0;
    int64_t c = tid >= o ? sblk[tid - o] : 0;
    __syncthreads();
    sseg[tid] += a;
    sblk[tid] += c;
    __syncthreads();
  }
  int64_t s0 = sseg[tid] - ns, b0 = sblk[tid] - nb;
  for (int b = lo; b < hi; ++b) {
    g.seg_off[b] = (int32_t)s0;
    g.blk_base[b] = (int32_t)b0;
    int64_t Lq = g.cu_q[b + 1] - g.cu_q[b];
    int64_t L = g.cu_kv[b + 1] - g.cu_kv[b];
    s0 += (int64_t)g.hkv * (((Lq << g.log2g) + kRows - 1) / kRows);
    b0 += ((L + kBlock - 1) / kBlock + kChunk - 1) / kChunk * kChunk;
  }
  if (tid == 1023) {
    g.seg_off[g.nreq] = (int32_t)sseg[1023];
    g.blk_base[g.nreq] = (int32_t)sblk[1023];
  }
  if (tid == 0) {
    g.hdr->err = 0;
    g.hdr->redo = 0;
  }
}

// 8 consecutive elements of a K/V row as floats.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float c, float* out) {
  if constexpr (DT == kBF16) {
    uint4 w = *(const uint4*)((const uint16_t*)base + elem);
    uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __builtin_bit_cast(float, ww[i] << 16);
      out[2 * i + 1] = __builtin_bit_cast(float, ww[i] & 0xffff0000u);
    }
  } else if constexpr (DT == kF32) {
    const float4* p = (const float4*)((const float*)base + elem);
    float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    uint2 w = *(const uint2*)((const uint8_t*)base + elem);
    f32x4 a = e4m3x4_to_f32(w.x), b = e4m3x4_to_f32(w.y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i] * c;
      out[4 + i] = b[i] * c;
    }
  }
}

// grid (padded block, kv head); 256 threads = 16 token groups x 16 column chunks.
template <int DT>
__global__ __launch_bounds__(256) void pool_kernel(Geo g, MeansLayout ml, const void* __restrict__ k,
                                                   const void* __restrict__ v, char* __restrict__ means) {
  __shared__ float red[2][16][kD];
  const int64_t gb = block_x();
  const int h = block_y();
  const int tid = thread_x();
  // request owning padded block gb
  int lo = 0, hi = g.nreq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)g.blk_base[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  SegCoord c;
  c.b = lo;
  c.h = h;
  c.I = 0;
  c.row0 = g.cu_q[lo];
  c.Lq = g.cu_q[lo + 1] - g.cu_q[lo];
  c.kv0 = g.cu_kv[lo];
  c.L = g.cu_kv[lo + 1] - g.cu_kv[lo];
  c.off = c.L - c.Lq;
  const int J = (int)(gb - g.blk_base[lo]);
  const int n = max(0, min(kBlock, c.L - J * kBlock));
  const float ck = DT == kE4M3 ? g.descale[1] : 1.f;
  const float cv = DT == kE4M3 ? g.descale[2] : 1.f;

  const bool vcols = DT == kE4M3 && g.vcols;  // V stored transposed: pooled below
  const int chunk = tid & 15, tg = tid >> 4;
  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
  for (int t = tg; t < n; t += 16) {
    int64_t row = kv_row(g, c, J * kBlock + t);
    if (row < 0) {
      atomicOr(&g.hdr->err, kErrPage);
      continue;
    }
    int64_t el = (row * g.hkv + h) * kD + chunk * 8;
    float a[8], b[8];
    load8<DT>(k, el, ck, a);
    if (!vcols) load8<DT>(v, el, cv, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sk[e] += a[e];
      if (!vcols) sv[e] += b[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][tg][chunk * 8 + e] = sk[e];
    red[1][tg][chunk * 8 + e] = sv[e];
  }
  __syncthreads();
  if (vcols) {
    // transposed V: thread (dim d, half hf) sums tokens 64 hf .. 64 hf + 63 of
    // the block, contiguous in dim d's row (16-byte pieces; the last piece is
    // masked past the block's n tokens); its partial replaces row hf of red[1]
    const int d = tid & 127, hf = tid >> 7;
    const int j0 = J * kBlock + 64 * hf;
    const int cnt = max(0, min(64, n - 64 * hf));
    float s = 0.f;
    if (cnt > 0) {
      int64_t rowb;  // byte offset of token j0 of dim d
      if (!g.page_table) {
        rowb = ((int64_t)h * kD + d) * g.vrow + c.kv0 + j0;
      } else {
        const int64_t page = g.page_table[(int64_t)c.b * g.max_pages + j0 / g.page_size];
        if (page < 0 || (page + 1) * g.page_size > g.num_slots) {
          atomicOr(&g.hdr->err, kErrPage);
          rowb = -1;
        } else {
          rowb = ((page * g.hkv + h) * kD + d) * g.page_size + j0 % g.page_size;
        }
      }
      if (rowb >= 0) {
        const uint8_t* p = (const uint8_t*)v + rowb;
        for (int c16 = 0; 16 * c16 < cnt; ++c16) {
          const uint4 w = *(const uint4*)(p + 16 * c16);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 f = e4m3x4_to_f32(ww[q4]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (16 * c16 + 4 * q4 + e < cnt) s += f[e];
          }
        }
      }
    }
    red[1][hf][d] = s * cv;
    __syncthreads();
  }
  const int which = tid >> 7, d = tid & 127;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += red[which][i][d];
  const float mean = n > 0 ? s / (float)n : 0.f;
  const int64_t row_el = (gb * g.hkv + h) * kD + d;
  float* f32out = (float*)(means + (which ? ml.vbar32 : ml.kbar32));
  f32out[row_el] = mean;
  // operand copy in the element type
  char* op = means + (which ? ml.vop : ml.kop);
  if constexpr (DT == kBF16) {
    ((uint16_t*)op)[row_el] = f32_to_bf16_bits(mean);
  } else if constexpr (DT == kF32) {
    ((float*)op)[row_el] = mean;
  } else {
    // transposed V: the correction operands of a 64-block chunk are [dim][block]
    const int64_t el = which && vcols ? (((gb >> 6) * g.hkv + h) * kD + d) * kChunk + (gb & 63) : row_el;
    const float x = fminf(448.f, fmaxf(-448.f, mean / (which ? cv : ck)));
    const uint32_t hi = f32x2_to_e4m3x2(x, 0.f);
    ((uint8_t*)op)[el] = (uint8_t)hi;
    if (which == 0) {
      // kbar/c_k = hi + lo/16: the part that the E4M3 code drops, scaled by 2^4
      // and rounded again, so that the correction logits carry ~8 significant
      // bits (the attention kernel multiplies lo back by 2^-4 through the MFMA's
      // operand scale)
      const float r = (x - e4m3x4_to_f32(hi)[0]) * 16.f;
      ((uint8_t*)(means + ml.klo8))[row_el] = (uint8_t)f32x2_to_e4m3x2(fminf(448.f, fmaxf(-448.f, r)), 0.f);
    }
  }
  // The scoring operands: kbar times sl = sigma log2 e (E4M3: also c_q, the
  // query scale), so that a query row's product with them is its logit in
  // log2 units, split as hi + lo in bf16 and stored in MFMA B-operand order:
  // [block/32][head][d/16][lane = block%32 + 32*((d%16)/8)][d%8]
  const float sl = g.scale * 1.4426950408889634f * (DT == kE4M3 ? g.descale[0] : 1.f);
  float hv = 0.f, lv = 0.f;
  if (which == 0) {
    const float ms = mean * sl;
    const uint16_t hb = f32_to_bf16_bits(ms);
    hv = bf16_bits_to_f32(hb);
    const uint16_t lb = f32_to_bf16_bits(ms - hv);
    lv = bf16_bits_to_f32(lb);
    int64_t jt = gb >> 5;
    int j = (int)(gb & 31);
    int ks = d >> 4, hh = (d >> 3) & 1, e = d & 7;
    int64_t o = (((jt * g.hkv + h) * 8 + ks) * 64 + j + 32 * hh) * 8 + e;
    ((uint16_t*)(means + ml.khi))[o] = hb;
    ((uint16_t*)(means + ml.klo))[o] = lb;
  }
  // |lo|_2 and |hi|_2 over the block's 128 dims (waves 0 and 1 hold K's
  // dims): scoring with hi alone is off from hi + lo by at most |q|_2 |lo|_2,
  // and no logit of hi alone exceeds |q|_2 |hi|_2 (Cauchy-Schwarz)
  __shared__ float lsq[2], hsq[2];
  const float la = wave_sum(lv * lv), ha = wave_sum(hv * hv);
  if ((tid & 63) == 0 && tid < 128) {
    lsq[tid >> 6] = la;
    hsq[tid >> 6] = ha;
  }
  __syncthreads();
  if (tid == 0) {
    ((float*)(means + ml.kbnd))[gb * g.hkv + h] = sqrtf(lsq[0] + lsq[1]);
    ((float*)(means + ml.knrm))[gb * g.hkv + h] = sqrtf(hsq[0] + hsq[1]);
  }
}

hipError_t launch_meta(const Geo& g, hipStream_t st) {
  meta_kernel<<<1, 1024, 0, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_pool(const Geo& g, const MeansLayout& ml, const void* k, const void* v, char* means,
                       hipStream_t st) {
  dim3 grid((unsigned)g.nb_pad, (unsigned)g.hkv);
  switch (g.dtype) {
    case kBF16: pool_kernel<kBF16><<<grid, 256, 0, st>>>(g, ml, k, v, means); break;
    case kF32: pool_kernel<kF32><<<grid, 256, 0, st>>>(g, ml, k, v, means); break;
    default: pool_kernel<kE4M3><<<grid, 256, 0, st>>>(g, ml, k, v, means); break;
  }
  return hipGetLastError();
}

}  // namespace fp
