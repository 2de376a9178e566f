// select.hip -- index stage after pooling: block scoring, alpha*max selection,
// CSR offsets and CSR expansion.
//
// Scoring ([V2] §3.1 Eq. 1-3, §3.3 Eq. 19-20).  One workgroup per segment
// (one PackGQA query tile of 128 packed rows of one KV head).  The tile's Q
// rows are staged once in LDS; every wave takes 32-block column tiles of the
// pooled keys and computes the 128x32 logit tile with bf16 MFMAs.  The pooled
// keys arrive multiplied by sigma log2 e (pooling does it), so the MFMA
// products are logits in log2 units, and split into bf16 hi + lo (~16
// significant bits, normalised energies accurate to ~1e-5 relative).  Each
// lane owns one block column and 64 of its 128 rows, so a block's energy
// S_J = sum_r 2^(x_rJ - c_J) (the form of Eq. 1, in log2 units, against a
// per-block reference c_J) needs only one cross-lane exchange and no
// workgroup barrier; E_J = S_J 2^(c_J - M) with a common M is the rescale that
// Eq. 20 describes.  Selection keeps E_J >= alpha * max E or forced blocks,
// writes one bit per block and the segment's tile count; no energy array goes
// to HBM unless the caller asks for it.
//
// Two kernels.  score_hi_kernel (bf16 / e4m3 queries, no energies requested)
// multiplies by hi alone and bounds what lo would add (Cauchy-Schwarz, per
// block); only the few blocks whose keep/drop decision or claim to the
// maximum the bound leaves open are scored again with hi + lo, so the kept set
// is that of hi + lo scoring.  A segment whose sums it cannot trust goes to a
// list instead.  score_exact_kernel scores every block with hi + lo (fp32
// queries: also q's lo part, three MFMAs) and writes the energies on request;
// it serves the calls that want energies, fp32 queries, and that list.
#include "device_common.h"
#include "qtile.h"

namespace fp {

// x of the lane in the other half that holds the same block column
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0-31 get lane + 32's x in r[1]; lanes 32-63 get lane - 32's in r[0]
  return __uint_as_float((thread_x() & 32) ? r[0] : r[1]);
}

// What both scoring kernels need of one segment.
struct ScoreSeg {
  int64_t s;
  TileGeo t;
  int nc;                // blocks holding a key visible to some row (J <= beta1)
  int njt;               // 32-block column tiles covering them
  const bf16x8* khs;     // hi B operands of the segment's first column tile
  const bf16x8* kls;     // lo B operands
  int64_t jstride;       // from one column tile's operands to the next (bf16x8 units)
  const float* knrm;     // |hi_J|_2 of block J at knrm[J * hkv]
  const float* kbnd;     // |lo_J|_2 of block J at kbnd[J * hkv]
};

__device__ __forceinline__ ScoreSeg score_seg(const Geo& g, const MeansLayout& ml, const char* means, int64_t s,
                                              SegCoord& c) {
  ScoreSeg z;
  z.s = s;
  c = seg_coord(g, s);
  z.t = tile_geo(g, c);
  z.nc = z.t.beta1 + 1;
  z.njt = (z.nc + 31) >> 5;
  const int64_t jt0 = g.blk_base[c.b] >> 5;
  z.khs = (const bf16x8*)(means + ml.khi) + ((jt0 * g.hkv + c.h) * 8) * 64;
  z.kls = (const bf16x8*)(means + ml.klo) + ((jt0 * g.hkv + c.h) * 8) * 64;
  z.jstride = (int64_t)g.hkv * 8 * 64;
  const int64_t b0 = (int64_t)g.blk_base[c.b] * g.hkv + c.h;
  z.knrm = (const float*)(means + ml.knrm) + b0;
  z.kbnd = (const float*)(means + ml.kbnd) + b0;
  return z;
}

// A operand of the staged tile: rows rt*32 + col, dims 16 ks + 8 half .. + 7
__device__ __forceinline__ bf16x8 q_op(const uint16_t* qs, int rt, int ks) {
  const int lane = thread_x() & 63;
  return *(const bf16x8*)(qs + (rt * 32 + (lane & 31)) * kQPitch + 8 * (lane >> 5) + ks * 16);
}

// Padding rows of a ragged tile: the lane's register r of row tile rt holds
// row rt*32 + 8*(r/4) + 4*half + r%4.
__device__ __forceinline__ void mask_rows(f32x16& v, int rt, int nrows) {
  const int half = (thread_x() >> 5) & 1;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nrows) v[r] = -INFINITY;
}

// Selection (Eq. 20 plus the forced blocks): keep J when forced or when
// SJ[J] >= thr; one bit per block, the segment's tile count (each kept block
// gives tiles 2J and 2J+1; the last block's second tile is dropped when it
// starts after the tile's last position).
__device__ __forceinline__ void write_selection(const Geo& g, const ScoreSeg& z, const float* SJ, float thr,
                                                int sink, int win, int32_t* counts, uint32_t* bits,
                                                int* nsel_w) {
  const int lane = thread_x() & 63, wave = thread_x() >> 6;
  const TileGeo& t = z.t;
  int nsel = 0;
  for (int base = wave * 64; base < z.nc; base += 256) {
    const int J = base + lane;
    const bool forced = J < sink || (J >= t.beta - win && J < t.beta) || J >= t.beta;
    const bool sel = J < z.nc && (forced || SJ[J] >= thr);
    const uint64_t m = __ballot(sel);
    if (lane == 0) {
      const int w0 = base >> 5;
      bits[z.s * g.words + w0] = (uint32_t)m;
      if (w0 + 1 < g.words) bits[z.s * g.words + w0 + 1] = (uint32_t)(m >> 32);
    }
    nsel += __popcll(m);
  }
  if (lane == 0) nsel_w[wave] = nsel;
  __syncthreads();
  if (thread_x() == 0) {
    const int tot = nsel_w[0] + nsel_w[1] + nsel_w[2] + nsel_w[3];
    const int trim = (int64_t)kTile * (2 * t.beta1 + 1) > t.t1 ? 1 : 0;
    counts[z.s] = 2 * tot - trim;
  }
}

// ---------------------------------------------------------------------------
// score_hi_kernel: hi-only sweep with per-block bounds (bf16 / e4m3 queries).
//
// The reference c_J = |q|max |hi_J|_2 (|q|max = max_r |q_r|_2, from the Gram
// matrix of the staged rows) is an upper bound of every hi-only logit of block
// J (Cauchy-Schwarz).  It enters as the MFMA's initial accumulator, so the
// products come out as x_rJ - c_J and each weight costs one exp and one add.
// With every weight <= 1 (up to rounding) no sum overflows.  Weights below
// 2^-126 may flush to zero: at most 127 of them lose less than 2^-119, which
// against a sum >= 2^-100 is below 2^-19 of it (far inside the decisions'
// margin).  A sum below 2^-100 sends the column tile through again with a
// lower reference; a block whose logits all lie more than 400 below its
// bound, or an infinite or NaN sum, sends the segment to the list for
// full-precision scoring.
template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void score_hi_kernel(
    Geo g, MeansLayout ml, const void* __restrict__ q, const char* __restrict__ means, float alpha, int sink,
    int win, int32_t* __restrict__ counts, uint32_t* __restrict__ bits, int32_t* __restrict__ redo) {
  extern __shared__ __align__(16) char smem[];
  uint16_t* qh = (uint16_t*)smem;
  float* lE = (float*)(smem + kRows * kQPitch * 2);  // log2 energies of the sweep
  float* SJ = lE + g.max_nj;                          // keep flags, then hi + lo energies
  int* flg = (int*)(SJ + g.max_nj);                   // blocks scored again with hi + lo
  __shared__ float qred[4], red[4];
  __shared__ float pm[4][32], ps[4][32];  // per-wave partial statistics of re-scored blocks
  __shared__ int nsel_w[4], nflag_sh, nunc_sh;

  SegCoord c;
  const ScoreSeg z = score_seg(g, ml, means, block_x(), c);
  const TileGeo& t = z.t;
  const int lane = thread_x() & 63, wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int nc = z.nc, njt = z.njt, nrows = t.nrows;

  // hi fragments of column tile jt and |hi|_2 of this lane's block
  auto load_hi = [&](int jt, bf16x8 (&bh)[8], float& kn) {
    const bf16x8* ph = z.khs + jt * z.jstride;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bh[ks] = ph[ks * 64 + lane];
    const int J = jt * 32 + col;
    kn = J < nc ? z.knrm[(int64_t)J * g.hkv] : 0.f;
  };
  // the first column tile's operands are in flight while Q is staged
  bf16x8 bh[8];
  float kn = 0.f;
  if (wave < njt) load_hi(wave, bh, kn);
  float kb4[4] = {0.f, 0.f, 0.f, 0.f};  // |lo_J|_2 of this thread's first four blocks
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int J = thread_x() + 256 * k;
    if (J < nc) kb4[k] = z.kbnd[(int64_t)J * g.hkv];
  }
  stage_q<DT>(g, c, t, q, qh, nullptr);
  __syncthreads();
  {
    // max_r |q_r|^2 of the wave's 32 rows: the largest entry of their Gram
    // matrix Q Q^T (off-diagonal entries are bounded by the diagonal ones);
    // the A and B fragments of Q Q^T are the same registers
    f32x16 gacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = q_op(qh, wave, ks);
      gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, gacc, 0, 0, 0);
    }
    float gm = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) gm = fmaxf(gm, gacc[r]);
    gm = wave_max(gm);
    if (lane == 0) qred[wave] = gm;
  }
  __syncthreads();
  const float qn = sqrtf(fmaxf(fmaxf(qred[0], qred[1]), fmaxf(qred[2], qred[3])));

  // Logits of the 128 rows x 32 blocks of the loaded column tile against
  // reference cref (block J for this lane's column), 32 rows at a time,
  // software-pipelined over the four row tiles: the MFMAs of row tile rt
  // (into one of two accumulators) are issued with the weights of row tile
  // rt - 1 in eight pieces between them; the A operands (Q rows) are read two
  // ahead.  Leaves lE_J = c_J + log2 S_J (or +inf) in lE.
  auto tile_hi = [&](auto ragged_tag, int J, const bf16x8 (&b)[8], float cref) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    // A sum below 2^-100 means every logit of the block lies more than 100
    // below the reference; the column tile is then computed again with that
    // block's reference lowered by 100 (no weight can exceed 1 against it),
    // up to three times (logits down to 400 below the bound).  The lane halves
    // holding one block see the same merged sum and lower their reference
    // together.
    for (int pass = 0;; ++pass) {
      f32x16 cinit;
#pragma unroll
      for (int r = 0; r < 16; ++r) cinit[r] = -cref;
      float s0 = 0.f, s1 = 0.f;
      auto weights = [&](int rt, f32x16& v, int k) __attribute__((always_inline)) {
        if (RAGGED && k == 0) mask_rows(v, rt, nrows);
        s0 += __builtin_amdgcn_exp2f(v[2 * k]);
        s1 += __builtin_amdgcn_exp2f(v[2 * k + 1]);
      };
      f32x16 acc[2];
      bf16x8 ring[2];
      ring[0] = q_op(qh, 0, 0);
      ring[1] = q_op(qh, 0, 1);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 a = ring[ks & 1];
          const int nrt = ks + 2 < 8 ? rt : rt + 1, nks = (ks + 2) & 7;
          if (nrt < 4) ring[ks & 1] = q_op(qh, nrt, nks);
          acc[rt & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[ks], ks == 0 ? cinit : acc[rt & 1], 0, 0, 0);
          if (rt > 0) weights(rt - 1, acc[(rt - 1) & 1], ks);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) weights(3, acc[1], k);
      const float sm = s0 + s1;
      const float tot = sm + other_half(sm);  // the other lane half holds the block's other 64 rows
      const bool low = !(tot >= 0x1p-100f);   // also NaN
      if (pass < 3 && __ballot(low && J < nc) != 0) {
        if (low) cref -= 100.f;
        continue;
      }
      if (half == 0 && J < nc) lE[J] = !low && tot < INFINITY ? cref + __builtin_amdgcn_logf(tot) : INFINITY;
      break;
    }
  };
  auto sweep = [&](auto ragged_tag) {
    for (int jt = wave; jt < njt; jt += 4) {
      if (jt != wave) load_hi(jt, bh, kn);
      tile_hi(ragged_tag, jt * 32 + col, bh, qn * kn);
    }
  };
  if (nrows < kRows)
    sweep(std::true_type{});
  else
    sweep(std::false_type{});
  __syncthreads();

  // lE_J's hi + lo value lies in [lE_J - d_J, lE_J + d_J], d_J = |q|max
  // |lo_J|_2 (with a margin for the rounding of the Gram entries and of the
  // logits, ~2^-16 relative each); max lE lies in [elo, ehi]
  const float dsc = qn * (1.f + 0.0005f) * (1.f + 0.0078125f);
  auto each_block = [&](auto&& body) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int J = thread_x() + 256 * k;
      if (J < nc) body(J, kb4[k]);
    }
    for (int J = thread_x() + 1024; J < nc; J += 256) body(J, z.kbnd[(int64_t)J * g.hkv]);
  };
  float lhi = -INFINITY, llo = -INFINITY, lmx = -INFINITY;
  bool bad = false;
  each_block([&](int J, float lb) {
    const float le = lE[J], d = dsc * lb;
    bad |= le == INFINITY;  // a sum the sweep does not trust (stored as +inf, never NaN)
    lhi = fmaxf(lhi, le + d);
    llo = fmaxf(llo, le - d);
    lmx = fmaxf(lmx, le);
  });
  lhi = wave_max(lhi);
  llo = wave_max(llo);
  lmx = wave_max(lmx);
  const bool wbad = __ballot(bad) != 0;
  if (lane == 0) {
    pm[0][wave] = lhi;
    pm[1][wave] = llo;
    pm[2][wave] = lmx;
    nsel_w[wave] = wbad;
  }
  if (thread_x() == 0) nflag_sh = nunc_sh = 0;
  __syncthreads();
  if ((nsel_w[0] | nsel_w[1] | nsel_w[2] | nsel_w[3]) != 0) {
    if (thread_x() == 0) redo[atomicAdd(&g.hdr->redo, 1)] = (int32_t)z.s;
    return;  // the whole workgroup: the flags are in LDS
  }
  const float ehi = fmaxf(fmaxf(pm[0][0], pm[0][1]), fmaxf(pm[0][2], pm[0][3]));
  const float elo = fmaxf(fmaxf(pm[1][0], pm[1][1]), fmaxf(pm[1][2], pm[1][3]));
  const float M = fmaxf(fmaxf(pm[2][0], pm[2][1]), fmaxf(pm[2][2], pm[2][3]));
  __syncthreads();  // pm and nsel_w are read before they are written again

  // In log2 units: keep when lE - d >= log2(alpha) + ehi, drop when
  // lE + d < log2(alpha) + elo, each with a margin of 1e-4 relative plus what
  // fp32 rounding of log energies of this size can add.  Decided blocks
  // become +inf (kept) or 0 (dropped); the others, and every block that may
  // hold the maximum, go to the list for hi + lo scoring
  const float lal = alpha > 0.f ? __builtin_amdgcn_logf(alpha) : -INFINITY;
  const float mrg = 1.4426e-4f + fmaxf(fabsf(ehi), fabsf(elo)) * 0x1p-20f;  // log2(1 + 1e-4) + rounding
  auto forced_block = [&](int J) { return J < sink || (J >= t.beta - win && J < t.beta) || J >= t.beta; };
  each_block([&](int J, float lb) {
    const float le = lE[J], d = dsc * lb;
    const float up = le + d + mrg, dn = le - d;
    const bool keep = dn >= lal + ehi + mrg, drop = up < lal + elo;
    const bool maxc = up >= elo;
    const bool unc = !forced_block(J) && !keep && !drop;
    if (unc) atomicAdd(&nunc_sh, 1);
    if (unc || maxc) flg[atomicAdd(&nflag_sh, 1)] = J;
    SJ[J] = keep ? INFINITY : 0.f;
  });
  __syncthreads();
  // nothing undecided: the bounds alone give the kept set
  const int nflag = nunc_sh > 0 ? nflag_sh : 0;
  // hi + lo scoring of the listed blocks, 32 at a time, wave w taking rows
  // 32w..32w+31; the four partial (max, sum) pairs are merged per block
  for (int g0 = 0; g0 < nflag; g0 += 32) {
    const int J = flg[min(g0 + col, nflag - 1)];
    bf16x8 gh[8], gl[8];
    const int64_t o = (int64_t)(J >> 5) * z.jstride + (J & 31) + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      gh[ks] = z.khs[o + ks * 64];
      gl[ks] = z.kls[o + ks * 64];
    }
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = q_op(qh, wave, ks);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gh[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gl[ks], acc, 0, 0, 0);
    }
    mask_rows(acc, wave, nrows);
    float m = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[r]);
    const float mo = fmaxf(m, other_half(m));  // the wave's 32 rows of the block
    const float mref = mo == -INFINITY ? 0.f : mo;
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(acc[r] - mref);
    sum += other_half(sum);
    if (half == 0) {
      pm[wave][col] = mo;
      ps[wave][col] = sum;
    }
    __syncthreads();
    if (wave == 0 && half == 0 && g0 + col < nflag) {
      const float mx = fmaxf(fmaxf(pm[0][col], pm[1][col]), fmaxf(pm[2][col], pm[3][col]));
      float st = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) st += ps[w][col] * __builtin_amdgcn_exp2f(pm[w][col] - mx);
      // E_J relative to 2^M, M the largest lE (any common reference serves);
      // the maximum is among the listed blocks
      SJ[J] = st * __builtin_amdgcn_exp2f(mx - M);
    }
    __syncthreads();
  }
  // Decided blocks hold +inf (kept) or 0 (dropped): with none re-scored the
  // threshold only has to separate those two
  float thr = INFINITY;
  if (nflag > 0) {
    float le = 0.f;
    for (int i = thread_x(); i < nflag; i += 256) le = fmaxf(le, SJ[flg[i]]);
    thr = alpha * block_max(le, red);
  }
  write_selection(g, z, SJ, thr, sink, win, counts, bits, nsel_w);
}

// ---------------------------------------------------------------------------
// score_exact_kernel: every block with hi + lo.  LIST: the segments of the
// list that score_hi_kernel left (count in the workspace header), a
// grid-stride loop over them; otherwise segment = workgroup.
//
// Per column tile: logits of the 128 rows x 32 blocks (block J for this
// lane's column), 32 rows at a time; per block the running maximum m of the
// logits and the sum of 2^(logit - m).  Software-pipelined over the four row
// tiles: the MFMAs of row tile rt (into one of two accumulators) are issued
// with the statistics of row tile rt - 1 in eight pieces between them, and the
// A operands (Q rows) are read two ahead.
template <int DT, bool LIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void score_exact_kernel(
    Geo g, MeansLayout ml, const void* __restrict__ q, const char* __restrict__ means, float alpha, int sink,
    int win, int32_t* __restrict__ counts, uint32_t* __restrict__ bits, float* __restrict__ energies,
    const int32_t* __restrict__ redo, int nwg) {
  extern __shared__ __align__(16) char smem[];
  constexpr int NQ = DT == kF32 ? 2 : 1;
  uint16_t* qh = (uint16_t*)smem;
  uint16_t* ql = qh + kRows * kQPitch;
  float* mJ = (float*)(smem + NQ * kRows * kQPitch * 2);
  float* SJ = mJ + g.max_nj;
  __shared__ float red[4];
  __shared__ int nsel_w[4];
  const int lane = thread_x() & 63, wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int64_t nwork = LIST ? (int64_t)g.hdr->redo : g.n_seg;

  for (int64_t i = block_x(); i < nwork; i += nwg) {  // nwg: the grid's workgroup count
    const int64_t s = LIST ? (int64_t)redo[i] : i;
    SegCoord c;
    const ScoreSeg z = score_seg(g, ml, means, s, c);
    const TileGeo& t = z.t;
    const int nc = z.nc, njt = z.njt, nrows = t.nrows;

    auto tile = [&](auto ragged_tag, int J, const bf16x8 (&bh)[8], const bf16x8 (&bl)[8]) {
      constexpr bool RAGGED = decltype(ragged_tag)::value;
      float m = -INFINITY, sum = 0.f;
      auto mm = [&](int rt, int ks, const bf16x8 a, f32x16& ac) __attribute__((always_inline)) {
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], ks == 0 ? f32x16{} : ac, 0, 0, 0);
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[ks], ac, 0, 0, 0);
        if constexpr (NQ == 2) ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_op(ql, rt, ks), bh[ks], ac, 0, 0, 0);
      };
      // statistics of row tile rt (logits v), piece k of 8: the maximum, the
      // rescale of the running sum, then 16 weights (two sums)
      float mn = 0.f, mref = 0.f, s0 = 0.f, s1 = 0.f;
      auto stat = [&](int rt, f32x16& v, int k) __attribute__((always_inline)) {
        if (k == 0) {
          if constexpr (RAGGED) mask_rows(v, rt, nrows);
          float m0 = fmaxf(v[0], fmaxf(v[1], v[2])), m1 = fmaxf(v[8], fmaxf(v[9], v[10]));
          m0 = fmaxf(m0, fmaxf(v[3], v[4]));
          m1 = fmaxf(m1, fmaxf(v[11], v[12]));
          m0 = fmaxf(m0, fmaxf(v[5], v[6]));
          m1 = fmaxf(m1, fmaxf(v[13], v[14]));
          m0 = fmaxf(m0, fmaxf(v[7], v[15]));
          mn = fmaxf(m, fmaxf(m0, m1));
          mref = mn == -INFINITY ? 0.f : mn;
        } else if (k == 1) {
          s0 = sum * __builtin_amdgcn_exp2f(m - mref);
          s1 = 0.f;
        } else {
          // pieces 2-7: weights 0-2, 3-5, 6-8, 9-11, 12-13, 14-15
          const int r0 = k < 6 ? 3 * (k - 2) : 12 + 2 * (k - 6), r1 = k < 6 ? r0 + 3 : r0 + 2;
#pragma unroll
          for (int r = r0; r < r1; ++r) {
            const float e = __builtin_amdgcn_exp2f(v[r] - mref);
            if (r & 1)
              s1 += e;
            else
              s0 += e;
          }
          if (k == 7) {
            sum = s0 + s1;
            m = mn;
          }
        }
      };
      f32x16 acc[2];
      bf16x8 ring[2];
      ring[0] = q_op(qh, 0, 0);
      ring[1] = q_op(qh, 0, 1);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 a = ring[ks & 1];
          const int nrt = ks + 2 < 8 ? rt : rt + 1, nks = (ks + 2) & 7;
          if (nrt < 4) ring[ks & 1] = q_op(qh, nrt, nks);
          mm(rt, ks, a, acc[rt & 1]);
          if (rt > 0) stat(rt - 1, acc[(rt - 1) & 1], ks);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) stat(3, acc[1], k);
      // the other lane half holds the block's other 64 rows
      const float mo = other_half(m), so = other_half(sum);
      const float mx = fmaxf(m, mo);
      const float mu = mx == -INFINITY ? 0.f : mx;
      sum = sum * __builtin_amdgcn_exp2f(m - mu) + so * __builtin_amdgcn_exp2f(mo - mu);
      if (half == 0 && J < nc) {
        mJ[J] = mx;
        SJ[J] = sum;
      }
    };
    // the wave's first column tile is in flight while Q is staged
    bf16x8 bh[8], bl[8];
    auto load = [&](int jt) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bh[ks] = z.khs[jt * z.jstride + ks * 64 + lane];
        bl[ks] = z.kls[jt * z.jstride + ks * 64 + lane];
      }
    };
    if (wave < njt) load(wave);
    stage_q<DT>(g, c, t, q, qh, ql);
    __syncthreads();
    auto sweep = [&](auto ragged_tag) {
      for (int jt = wave; jt < njt; jt += 4) {
        if (jt != wave) load(jt);
        tile(ragged_tag, jt * 32 + col, bh, bl);
      }
    };
    if (nrows < kRows)
      sweep(std::true_type{});
    else
      sweep(std::false_type{});
    __syncthreads();
    // E_J = S_J 2^(m_J - M), M = max_J m_J; then keep E_J >= alpha max E or forced
    float lm = -INFINITY;
    for (int J = thread_x(); J < nc; J += 256) lm = fmaxf(lm, mJ[J]);
    const float M = block_max(lm, red);
    float le = 0.f;
    for (int J = thread_x(); J < nc; J += 256) {
      const float e = SJ[J] * __builtin_amdgcn_exp2f(mJ[J] - M);
      SJ[J] = e;
      le = fmaxf(le, e);
    }
    const float Emax = block_max(le, red);  // >= 1: the block attaining M has S >= 1
    if (energies) {
      for (int J = thread_x(); J < nc; J += 256) energies[s * g.max_nj + J] = SJ[J] / Emax;
      for (int J = nc + thread_x(); J < g.max_nj; J += 256) energies[s * g.max_nj + J] = -1.f;
    }
    write_selection(g, z, SJ, alpha * Emax, sink, win, counts, bits, nsel_w);
    __syncthreads();  // LDS is reused by the next segment
  }
}

// Exclusive prefix sum of the per-segment counts into cu[n+1], in two
// passes: 1024-entry blocks reduce to partial sums (scan_part_kernel), then
// every block rescans its entries on top of the sum of the partials before it.
__device__ __forceinline__ int block_excl_scan_1024(int x, int* sh, int& total) {
  const int lane = thread_x() & 63, w = thread_x() >> 6;
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
  const int64_t i = (int64_t)block_x() * 1024 + thread_x();
  int total;
  block_excl_scan_1024(i < n ? counts[i] : 0, sh, total);
  if (thread_x() == 0) part[block_x()] = total;
}

__global__ __launch_bounds__(1024) void scan_final_kernel(const int32_t* __restrict__ counts, int64_t n,
                                                          const int32_t* __restrict__ part, int32_t* __restrict__ cu) {
  __shared__ int sh[40];
  __shared__ int base_sh;
  // offset of this block: sum of the partials before it (one wave)
  if (thread_x() < 64) {
    int acc = 0;
    for (int b = thread_x(); b < (int)block_x(); b += 64) acc += part[b];
    acc = wave_sum_i(acc);
    if (thread_x() == 0) base_sh = acc;
  }
  __syncthreads();
  const int64_t i = (int64_t)block_x() * 1024 + thread_x();
  const int x = i < n ? counts[i] : 0;
  int total;
  const int ex = block_excl_scan_1024(x, sh, total);
  if (i < n) cu[i] = base_sh + ex;
  if (i == n - 1) cu[n] = base_sh + ex + x;
}

// One wave per segment: ballot + prefix count turn the selection bits into the
// ascending list of physical tile ids (logical block J -> tiles 2J, 2J+1).
// The segment's bit words are loaded once, one per lane (64 words = 2048
// blocks per load), and handed to the lanes of each 64-block step by a
// cross-lane permute, so that the steps do not wait on memory one by one.
__global__ __launch_bounds__(256) void expand_kernel(Geo g, const int32_t* __restrict__ cu,
                                                     const uint32_t* __restrict__ bits,
                                                     int32_t* __restrict__ idx, int64_t cap) {
  const int64_t s = (int64_t)block_x() * 4 + (thread_x() >> 6);
  if (s >= g.n_seg) return;
  const int lane = thread_x() & 63;
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  const int64_t start = cu[s];
  const int nc = t.beta1 + 1;  // blocks holding a key visible to some row
  const int nw = (nc + 31) >> 5;
  int o = 0;
  uint32_t wd = 0;
  for (int base = 0; base < nc; base += 64) {
    const int w0 = base >> 5;  // first word of this step
    if ((w0 & 63) == 0) wd = w0 + lane < nw ? bits[s * g.words + w0 + lane] : 0u;
    const int J = base + lane;
    // word (J >> 5) sits in lane (J >> 5) & 63 of this word group
    const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(((w0 & 63) + (lane >> 5)) << 2, (int)wd);
    const bool sel = J < nc && ((w >> (J & 31)) & 1u);
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
                               float* energies, int32_t* redo, hipStream_t st) {
  const size_t q1 = (size_t)kRows * kQPitch * 2;  // one staged tile (bf16)
  const dim3 grid((unsigned)g.n_seg);
  if (g.dtype != kF32 && !energies) {
    // hi-only scoring, then full precision for the segments it listed
    const void* fa = g.dtype == kBF16 ? (const void*)score_hi_kernel<kBF16> : (const void*)score_hi_kernel<kE4M3>;
    const void* fb = g.dtype == kBF16 ? (const void*)score_exact_kernel<kBF16, true>
                                      : (const void*)score_exact_kernel<kE4M3, true>;
    hipError_t e = set_lds_limit(fa, q1 + (size_t)kMaxBlocks * 12);
    if (e == hipSuccess) e = set_lds_limit(fb, q1 + (size_t)kMaxBlocks * 8);
    if (e != hipSuccess) return e;
    const size_t la = q1 + (size_t)g.max_nj * 12, lb = q1 + (size_t)g.max_nj * 8;
    const dim3 gl((unsigned)std::min<int64_t>(g.n_seg, 256));  // the list is usually empty
    if (g.dtype == kBF16) {
      score_hi_kernel<kBF16><<<grid, 256, la, st>>>(g, ml, q, means, alpha, sink, win, counts, bits, redo);
      score_exact_kernel<kBF16, true><<<gl, 256, lb, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                            nullptr, redo, (int)gl.x);
    } else {
      score_hi_kernel<kE4M3><<<grid, 256, la, st>>>(g, ml, q, means, alpha, sink, win, counts, bits, redo);
      score_exact_kernel<kE4M3, true><<<gl, 256, lb, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                            nullptr, redo, (int)gl.x);
    }
    return hipGetLastError();
  }
  const int nq = g.dtype == kF32 ? 2 : 1;
  const void* fn = g.dtype == kBF16 ? (const void*)score_exact_kernel<kBF16, false>
                   : g.dtype == kF32 ? (const void*)score_exact_kernel<kF32, false>
                                     : (const void*)score_exact_kernel<kE4M3, false>;
  hipError_t e = set_lds_limit(fn, nq * q1 + (size_t)kMaxBlocks * 8);
  if (e != hipSuccess) return e;
  const size_t lds = nq * q1 + (size_t)g.max_nj * 8;
  switch (g.dtype) {
    case kBF16:
      score_exact_kernel<kBF16, false><<<grid, 256, lds, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                               energies, nullptr, (int)grid.x);
      break;
    case kF32:
      score_exact_kernel<kF32, false><<<grid, 256, lds, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                              energies, nullptr, (int)grid.x);
      break;
    default:
      score_exact_kernel<kE4M3, false><<<grid, 256, lds, st>>>(g, ml, q, means, alpha, sink, win, counts, bits,
                                                               energies, nullptr, (int)grid.x);
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
