// select.hip -- index stage after pooling: block scoring, alpha*max selection,
// CSR offsets and CSR expansion.
//
// Scoring ([V2] §3.1 Eq. 1-3, §3.3 Eq. 19-20).  One workgroup per segment
// (one PackGQA query tile of 128 packed rows of one KV head).  The tile's Q
// rows are staged once in LDS; every wave takes 32-block column tiles of the
// pooled keys and computes the 128x32 logit tile with bf16 MFMAs.  kbar is
// fp32, split into bf16 hi + lo (~16 significant bits, normalised energies
// accurate to ~1e-5 relative).  The sweep multiplies by hi alone and bounds
// what lo would add (Cauchy-Schwarz, per block); only the few blocks whose
// keep/drop decision or claim to the maximum the bound leaves open are
// scored again with hi + lo, so the kept set is that of hi + lo scoring.
// With energies requested, and for fp32 queries (split the same way, three
// MFMAs), every block is scored with hi + lo.  Each lane owns one block
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DT == kF32 ? 2 : 3))) void score_select_kernel(Geo g, MeansLayout ml, const void* __restrict__ q,
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
  int* flg = (int*)(SJ + g.max_nj);  // blocks scored again with hi + lo
  __shared__ float red[4], qred[4];
  __shared__ int nsel_w[4], nflag_sh, nunc_sh;
  __shared__ float pm[4][32], ps[4][32];  // per-wave partial statistics of re-scored blocks

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
  // B operand fragments (hi, and lo when EXACT) of column tile jt
  auto kb_load = [&](auto exact_tag, int jt, bf16x8 (&bh)[8], bf16x8 (&bl)[8]) {
    constexpr bool EXACT = decltype(exact_tag)::value;
    const bf16x8* ph = khs + jt * jstride;
    const bf16x8* pl = kls + jt * jstride;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bh[ks] = ph[ks * 64 + lane];
      if constexpr (EXACT) bl[ks] = pl[ks * 64 + lane];
    }
  };
  // hi and lo fragments of block J for this lane's column (a gathered tile)
  auto kb_gather = [&](int J, bf16x8 (&bh)[8], bf16x8 (&bl)[8]) {
    const int64_t o = (int64_t)(J >> 5) * jstride + (J & 31) + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bh[ks] = khs[o + ks * 64];
      bl[ks] = kls[o + ks * 64];
    }
  };
  // logits of the 128 rows x 32 blocks whose operands are loaded (block J for
  // this lane's column), 32 rows at a time; per block the running maximum of
  // the raw products (sl > 0) and the sum of 2^(logit - max), logits in log2
  // units; EXACT uses kbar = hi + lo, otherwise hi alone.  Software-pipelined
  // over the four row tiles: the MFMAs of row tile rt (into one of two
  // accumulators) are issued with the statistics of row tile rt - 1 in eight
  // pieces between them, and the A operands (Q rows) are read two ahead.
  auto tile = [&](auto ragged_tag, auto exact_tag, int J, bool store, const bf16x8 (&bh)[8],
                  const bf16x8 (&bl)[8]) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    constexpr bool EXACT = decltype(exact_tag)::value;
    float m = -INFINITY, sum = 0.f;
    auto qa = [&](int rt, int ks) __attribute__((always_inline)) -> bf16x8 {
      return *(const bf16x8*)(qh + (rt * 32 + col) * kQPitch + 8 * half + ks * 16);
    };
    auto mm = [&](int rt, int ks, const bf16x8 a, f32x16& ac) __attribute__((always_inline)) {
      ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], ks == 0 ? f32x16{} : ac, 0, 0, 0);
      if constexpr (EXACT) {
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[ks], ac, 0, 0, 0);
        if constexpr (NQ == 2) {
          const bf16x8 al = *(const bf16x8*)(ql + (rt * 32 + col) * kQPitch + 8 * half + ks * 16);
          ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh[ks], ac, 0, 0, 0);
        }
      }
    };
    // statistics of row tile rt (logits v), piece k of 8: the maximum, the
    // rescale of the running sum, then 16 weights (two sums)
    float mn = 0.f, msl = 0.f, s0 = 0.f, s1 = 0.f;
    auto stat = [&](int rt, f32x16& v, int k) __attribute__((always_inline)) {
      if (k == 0) {
        // lane owns block column col, rows rt*32 + 8*(r/4) + 4*half + r%4;
        // padding rows of a ragged tile are masked out
        if constexpr (RAGGED) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nrows) v[r] = -INFINITY;
        }
        float m0 = fmaxf(v[0], fmaxf(v[1], v[2])), m1 = fmaxf(v[8], fmaxf(v[9], v[10]));
        m0 = fmaxf(m0, fmaxf(v[3], v[4]));
        m1 = fmaxf(m1, fmaxf(v[11], v[12]));
        m0 = fmaxf(m0, fmaxf(v[5], v[6]));
        m1 = fmaxf(m1, fmaxf(v[13], v[14]));
        m0 = fmaxf(m0, fmaxf(v[7], v[15]));
        mn = fmaxf(m, fmaxf(m0, m1));
        msl = mn == -INFINITY ? 0.f : mn * sl;
      } else if (k == 1) {
        s0 = sum * __builtin_amdgcn_exp2f(fmaf(m, sl, -msl));
        s1 = 0.f;
      } else {
        // pieces 2-7: weights 0-2, 3-5, 6-8, 9-11, 12-13, 14-15
        const int r0 = k < 6 ? 3 * (k - 2) : 12 + 2 * (k - 6), r1 = k < 6 ? r0 + 3 : r0 + 2;
#pragma unroll
        for (int r = r0; r < r1; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(v[r], sl, -msl));
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
    // hi alone: the lane's reference c (log2 units) is the maximum of its 16
    // rows in row tile 0 and stays fixed for the other 48 rows, so those need
    // no maximum and no rescale.  A later row that exceeds c by more than the
    // fp32 range makes the sum infinite, which the caller detects (the segment
    // is then scored again with hi + lo).  Terms more than 126 below c, which
    // underflow, are below 2^-126 of the sum (>= 1, from the row that set c).
    float cref = 0.f, cmax = -INFINITY;
    auto stat_hi = [&](int rt, f32x16& v, int k) __attribute__((always_inline)) {
      if (RAGGED && k == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nrows) v[r] = -INFINITY;
      }
      if (rt == 0 && k == 0) {
        float m0 = fmaxf(v[0], fmaxf(v[1], v[2])), m1 = fmaxf(v[8], fmaxf(v[9], v[10]));
        m0 = fmaxf(m0, fmaxf(v[3], v[4]));
        m1 = fmaxf(m1, fmaxf(v[11], v[12]));
        m0 = fmaxf(m0, fmaxf(v[5], v[6]));
        m1 = fmaxf(m1, fmaxf(v[13], v[14]));
        m0 = fmaxf(m0, fmaxf(v[7], v[15]));
        const float mm0 = fmaxf(m0, m1);
        cmax = mm0 * sl;
        cref = mm0 == -INFINITY ? 0.f : cmax;
        return;
      }
      // row tile 0 spreads its 16 weights over pieces 1-7 (the last takes
      // four), the others two per piece over 0-7
      const int r0 = rt == 0 ? 2 * k - 2 : 2 * k;
      const int r1 = rt == 0 ? (k == 7 ? 16 : 2 * k) : 2 * k + 2;
#pragma unroll
      for (int r = r0; r < r1; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(v[r], sl, -cref));
        if (r & 1)
          s1 += e;
        else
          s0 += e;
      }
    };
    auto st = [&](int rt, f32x16& v, int k) __attribute__((always_inline)) {
      if constexpr (EXACT)
        stat(rt, v, k);
      else
        stat_hi(rt, v, k);
    };
    f32x16 acc[2];
    bf16x8 ring[2];
    ring[0] = qa(0, 0);
    ring[1] = qa(0, 1);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = ring[ks & 1];
        const int nrt = ks + 2 < 8 ? rt : rt + 1, nks = (ks + 2) & 7;
        if (nrt < 4) ring[ks & 1] = qa(nrt, nks);
        mm(rt, ks, a, acc[rt & 1]);
        if (rt > 0) st(rt - 1, acc[(rt - 1) & 1], ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) st(3, acc[1], k);
    // the other lane half holds the block's other 64 rows
    if constexpr (EXACT) {
      const float mo = __shfl_xor(m, 32, 64), so = __shfl_xor(sum, 32, 64);
      const float mx = fmaxf(m, mo) * sl;
      sum = sum * __builtin_amdgcn_exp2f(fmaf(m, sl, -mx)) + so * __builtin_amdgcn_exp2f(fmaf(mo, sl, -mx));
      if (half == 0 && store) {
        mJ[J] = mx;
        SJ[J] = sum;
      }
    } else {
      // row 0 is valid, so half 0's reference is finite; the merged sum is
      // >= 1 and its log2 is the block's energy in log2 units.  A half's sum
      // is finite or +inf (never NaN); an infinite one is passed on as
      // lE = +inf before the merge could form inf * 0
      const float sm = s0 + s1;
      const float co = __shfl_xor(cmax, 32, 64), so = __shfl_xor(sm, 32, 64);
      const float mx = fmaxf(cmax, co);
      const float tot = sm * __builtin_amdgcn_exp2f(cmax - mx) + so * __builtin_amdgcn_exp2f(co - mx);
      const bool ovf = sm == INFINITY || so == INFINITY;
      if (half == 0 && store) mJ[J] = ovf ? INFINITY : mx + __builtin_amdgcn_logf(tot);
    }
  };
  // The sweep multiplies by kbar's hi part alone.  Its logits are off from
  // the hi + lo ones by at most sl * max_r |q_r|_2 * |lo_J|_2 per block
  // (Cauchy-Schwarz; d_J below), so a block's energy is known within a factor
  // 2^(+-d_J); blocks whose keep/drop decision that interval leaves open, and
  // the blocks that may hold the maximum, are scored again with hi + lo.  The
  // kept set is that of hi + lo scoring.  Every block is scored with hi + lo
  // when energies are wanted, for fp32 queries, and for tiles with at most
  // two column tiles (where the bound's fixed cost outweighs the halved sweep).
  const bool exact = NQ == 2 || energies != nullptr || njt <= 2;
  // one register set of operands per wave; the first column tile's load is in
  // flight while Q is staged
  bf16x8 bh[8], bl[8];
  if (wave < njt) {
    if (exact)
      kb_load(std::true_type{}, wave, bh, bl);
    else
      kb_load(std::false_type{}, wave, bh, bl);
  }
  // |lo_J|_2 of this thread's first four blocks, loaded ahead of the sweep
  const float* kbnd = (const float*)(means + ml.kbnd) + (int64_t)g.blk_base[c.b] * g.hkv + c.h;
  float kb4[4] = {0.f, 0.f, 0.f, 0.f};
  if (!exact) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int J = threadIdx.x + 256 * k;
      if (J < nc) kb4[k] = kbnd[(int64_t)J * g.hkv];
    }
  }
  stage_q<DT>(g, c, t, q, qh, ql);
  __syncthreads();
  if (!exact) {
    // max_r |q_r|^2 of the wave's 32 rows: the largest entry of their Gram
    // matrix Q Q^T (off-diagonal entries are bounded by the diagonal ones);
    // the A and B fragments of Q Q^T are the same registers
    f32x16 gacc = f32x16{};
    const uint16_t* arow = qh + (wave * 32 + col) * kQPitch + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = *(const bf16x8*)(arow + ks * 16);
      gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, gacc, 0, 0, 0);
    }
    float gm = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) gm = fmaxf(gm, gacc[r]);
    gm = wave_max(gm);
    if (lane == 0) qred[wave] = gm;  // read after the sweep's barrier
  }
  // the column tiles of the wave; the first one's operands are already loaded
  // unless `reload`
  auto sweep = [&](auto ragged_tag, auto exact_tag, bool reload) {
    for (int jt = wave; jt < njt; jt += 4) {
      if (jt != wave || reload) kb_load(exact_tag, jt, bh, bl);
      tile(ragged_tag, exact_tag, jt * 32 + col, jt * 32 + col < nc, bh, bl);
    }
  };
  auto sweep_exact = [&](bool reload) {
    if (nrows < kRows)
      sweep(std::true_type{}, std::true_type{}, reload);
    else
      sweep(std::false_type{}, std::true_type{}, reload);
    __syncthreads();
  };
  auto forced_block = [&](int J) { return J < sink || (J >= t.beta - win && J < t.beta) || J >= t.beta; };
  // blocks of this thread, J = threadIdx.x + 256 k, with |lo_J|_2
  auto each_block = [&](auto&& body) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int J = threadIdx.x + 256 * k;
      if (J < nc) body(J, kb4[k]);
    }
    for (int J = threadIdx.x + 1024; J < nc; J += 256) body(J, kbnd[(int64_t)J * g.hkv]);
  };
  // The hi-only sweep leaves lE_J = log2 of block J's energy (relative to an
  // arbitrary common reference) in mJ; its hi + lo value lies in
  // [lE_J - d_J, lE_J + d_J].  A segment where a sum overflowed is scored
  // again with hi + lo.
  bool redo = false;
  float ehi = 0.f, elo = 0.f, dsc = 0.f, M = 0.f;
  if (!exact) {
    if (nrows < kRows)
      sweep(std::true_type{}, std::false_type{}, false);
    else
      sweep(std::false_type{}, std::false_type{}, false);
    __syncthreads();
    const float q2 = sqrtf(fmaxf(fmaxf(qred[0], qred[1]), fmaxf(qred[2], qred[3])) * (1.f + 0.001f));
    dsc = sl * q2 * (1.f + 0.0078125f);
    // max lE lies in [elo, ehi]: one two-value workgroup maximum
    float lhi = -INFINITY, llo = -INFINITY, lmx = -INFINITY;
    bool ovf = false;
    each_block([&](int J, float lb) {
      const float le = mJ[J], d = dsc * lb;
      if (le == INFINITY) ovf = true;  // a sum overflowed (the tile stores +inf, never NaN)
      lhi = fmaxf(lhi, le + d);
      llo = fmaxf(llo, le - d);
      lmx = fmaxf(lmx, le);
    });
    lhi = wave_max(lhi);
    llo = wave_max(llo);
    lmx = wave_max(lmx);
    const bool wovf = __ballot(ovf) != 0;
    if (lane == 0) {
      pm[0][wave] = lhi;
      pm[1][wave] = llo;
      pm[2][wave] = lmx;
      nsel_w[wave] = wovf;
    }
    if (threadIdx.x == 0) nflag_sh = nunc_sh = 0;
    __syncthreads();
    ehi = fmaxf(fmaxf(pm[0][0], pm[0][1]), fmaxf(pm[0][2], pm[0][3]));
    elo = fmaxf(fmaxf(pm[1][0], pm[1][1]), fmaxf(pm[1][2], pm[1][3]));
    M = fmaxf(fmaxf(pm[2][0], pm[2][1]), fmaxf(pm[2][2], pm[2][3]));
    redo = (nsel_w[0] | nsel_w[1] | nsel_w[2] | nsel_w[3]) != 0;
    if (redo) __syncthreads();  // pm and nsel_w are read before they are written again
  }
  if (exact || redo) sweep_exact(redo);

  float thr;
  if (exact || redo) {
    // E_J = S_J 2^(m_J - M), M = max_J m_J; then keep E_J >= alpha max E or forced
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
    thr = alpha * Emax;
    if (energies) {
      for (int J = threadIdx.x; J < nc; J += 256) energies[s * g.max_nj + J] = SJ[J] / Emax;
      for (int J = nc + threadIdx.x; J < g.max_nj; J += 256) energies[s * g.max_nj + J] = -1.f;
    }
  } else {
    // In log2 units: keep when lE - d >= log2(alpha) + ehi, drop when
    // lE + d < log2(alpha) + elo, each with a margin of 1e-4 relative plus
    // what fp32 rounding of log energies of this size can add.  Decided
    // blocks become +inf (kept) or 0 (dropped); the others, and every block
    // that may hold the maximum, go to the list for hi + lo scoring
    const float lal = alpha > 0.f ? __builtin_amdgcn_logf(alpha) : -INFINITY;
    const float mrg = 1.4426e-4f + fmaxf(fabsf(ehi), fabsf(elo)) * 0x1p-20f;  // log2(1 + 1e-4) + rounding
    each_block([&](int J, float lb) {
      const float le = mJ[J], d = dsc * lb;
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
      kb_gather(J, bh, bl);
      f32x16 acc = f32x16{};
      const uint16_t* arow = qh + (wave * 32 + col) * kQPitch + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = *(const bf16x8*)(arow + ks * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (wave * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nrows) acc[r] = -INFINITY;
      float m = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[r]);
      const float mo = fmaxf(m, __shfl_xor(m, 32, 64));  // the wave's 32 rows of the block
      const float msl = mo == -INFINITY ? 0.f : mo * sl;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], sl, -msl));
      sum += __shfl_xor(sum, 32, 64);
      if (half == 0) {
        pm[wave][col] = mo;
        ps[wave][col] = sum;
      }
      __syncthreads();
      if (wave == 0 && half == 0 && g0 + col < nflag) {
        const float mx = fmaxf(fmaxf(pm[0][col], pm[1][col]), fmaxf(pm[2][col], pm[3][col])) * sl;
        float st = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) st += ps[w][col] * __builtin_amdgcn_exp2f(fmaf(pm[w][col], sl, -mx));
        mJ[J] = mx;
        SJ[J] = st;
      }
      __syncthreads();
    }
    // hi + lo energies E_J = S_J 2^(m_J - M) of the listed blocks, M the
    // largest lE (any common reference serves); the maximum is among them.
    // Decided blocks hold +inf (kept) or 0 (dropped): with none re-scored the
    // threshold only has to separate those two
    thr = INFINITY;
    if (nflag > 0) {
      float le = 0.f;
      for (int i = threadIdx.x; i < nflag; i += 256) {
        const int J = flg[i];
        const float e = SJ[J] * __builtin_amdgcn_exp2f(mJ[J] - M);
        SJ[J] = e;
        le = fmaxf(le, e);
      }
      thr = alpha * block_max(le, red);
    }
  }
  int nsel = 0;
  for (int base = wave * 64; base < nc; base += 256) {
    const int J = base + lane;
    const bool in = J < nc;
    const bool sel = in && (forced_block(J) || SJ[J] >= thr);
    const uint64_t m = __ballot(sel);
    if (lane == 0) {
      int w0 = base >> 5;
      bits[s * g.words + w0] = (uint32_t)m;
      if (w0 + 1 < g.words) bits[s * g.words + w0 + 1] = (uint32_t)(m >> 32);
    }
    nsel += __popcll(m);
  }
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
  // per block: m_J and S_J, and (bf16 / e4m3: hi-only scoring) the re-score list
  const int per_blk = nq == 2 ? 8 : 12;
  size_t lds = (size_t)nq * kRows * kQPitch * 2 + (size_t)g.max_nj * per_blk;
  dim3 grid((unsigned)g.n_seg);
  {
    const void* fn = g.dtype == kBF16 ? (const void*)score_select_kernel<kBF16>
                     : g.dtype == kF32 ? (const void*)score_select_kernel<kF32>
                                       : (const void*)score_select_kernel<kE4M3>;
    hipError_t e = set_lds_limit(fn, nq * kRows * kQPitch * 2 + kMaxBlocks * per_blk);
    if (e != hipSuccess) return e;
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
