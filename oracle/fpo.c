/*
 * fpo.c -- the oracle: a plain, slow, fp64 CPU statement of what the
 * FlashPrefill V2 block-sparse prefill path computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP path and must never be used to
 * produce a product result.
 *
 * Sources (cited by page title and section/equation):
 *   [V2]  "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context
 *         LLM Serving" (arXiv 2608.19758).
 *   [V1]  "FlashPrefill: Instantaneous Pattern Discovery and Thresholding for
 *         Ultra-Fast Long-Context Prefilling" (summary page), sections 3.1-3.4.
 *   [OCP] OCP 8-bit floating point specification, E4M3 ("FN") encoding.
 *
 * Everything is computed in double precision, one row / one block at a time,
 * in the order the pages state it.  Readings taken where the pages leave a
 * step open are marked READING where they are applied.
 *
 * Conventions shared with every caller (they are definitions of the problem,
 * not of the GPU path):
 *   - q is [total_q, hq, d] ragged by cu[]; k and v are [total_kv, hkv, d]
 *     ragged by cu_kv[] (NULL: by cu[]) (contiguous; paged inputs are de-paged
 *     by the caller with [V2] Eq. 22).
 *   - a request has L_kv keys and L_q <= L_kv queries, which are its last L_q
 *     positions: query i sits at position off + i, off = L_kv - L_q (a prefill
 *     chunk after a cached prefix, the index re-run for every chunk: [V2] §4.3
 *     "Compatibility with Chunked Prefill"; off = 0 for a fresh prefill).
 *   - packed row r of KV head h is query floor(r/g), at position
 *     off + floor(r/g), of query head h*g + (r mod g)     ([V2] §3.3 Eq. 12-13)
 *   - a query tile is R consecutive packed rows of one (request, KV head);
 *     segments are ordered (request, KV head, tile).      ([V2] §3.3 Eq. 17)
 *   - blocks are B tokens, physical tiles are P tokens.   ([V2] §3.3 impl. details)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { FPO_F32 = 0, FPO_BF16 = 1, FPO_E4M3 = 2 };

typedef struct {
  int32_t num_reqs, hq, hkv, d;
  const int64_t* cu;  /* [num_reqs+1] row offsets into q/k/v */
  int32_t dtype;      /* FPO_* */
  double cq, ck, cv;  /* per-tensor descales for E4M3 ([V2] §3.3 Eq. 15); 1 otherwise */
  const void* q;
  const void* k;
  const void* v;
  double scale;       /* softmax scale sigma = 1/sqrt(d) */
  int32_t block;      /* B, selection block size */
  int32_t rows;       /* R, packed rows per query tile */
  int32_t phys;       /* P, physical key tile */
  const int64_t* cu_kv; /* [num_reqs+1] row offsets into k/v, or NULL: the same as cu */
} fpo_problem;

/* ------------------------------------------------------------------ */
/* element decoding                                                     */
/* ------------------------------------------------------------------ */

/* [OCP] E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; there is no infinity.
 * The largest finite value is 2^8 * 1.75 = 448. */
double fpo_e4m3_decode(uint8_t x) {
  int sign = (x >> 7) & 1;
  int e = (x >> 3) & 15;
  int m = x & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Round-to-nearest-even into E4M3, saturating at +-448.  The non-negative
 * finite codes 0x00..0x7e decode to strictly increasing values, so the code
 * below |x| is found by bisection over the codes; of it and the next code the
 * nearer wins, a tie going to the even mantissa (the code's low bit). */
double fpo_e4m3_round(double x) {
  double ax = fabs(x);
  if (ax >= 448.0) return x < 0 ? -448.0 : 448.0;
  int lo = 0, hi = 126; /* decode(lo) <= ax < decode(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (fpo_e4m3_decode((uint8_t)mid) <= ax)
      lo = mid;
    else
      hi = mid;
  }
  double a = fpo_e4m3_decode((uint8_t)lo), b = fpo_e4m3_decode((uint8_t)hi);
  double best;
  if (ax - a < b - ax)
    best = a;
  else if (ax - a > b - ax)
    best = b;
  else
    best = (lo & 1) == 0 ? a : b;
  return x < 0 ? -best : best;
}

/* The two E4M3 values around |x| < 448 (lo <= |x| < hi), by the same bisection. */
static void e4m3_bracket(double ax, double* lo_v, double* hi_v) {
  int lo = 0, hi = 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (fpo_e4m3_decode((uint8_t)mid) <= ax)
      lo = mid;
    else
      hi = mid;
  }
  *lo_v = fpo_e4m3_decode((uint8_t)lo);
  *hi_v = fpo_e4m3_decode((uint8_t)hi);
}

static double bf16_decode(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static double elem(const void* base, int dtype, size_t i, double c) {
  switch (dtype) {
    case FPO_F32: return (double)((const float*)base)[i];
    case FPO_BF16: return bf16_decode(((const uint16_t*)base)[i]);
    case FPO_E4M3: return c * fpo_e4m3_decode(((const uint8_t*)base)[i]);
  }
  return NAN;
}

/* Load one vector of length d. */
static void load_q(const fpo_problem* p, int64_t row, int head, double* out) {
  size_t base = ((size_t)row * p->hq + head) * p->d;
  for (int i = 0; i < p->d; ++i) out[i] = elem(p->q, p->dtype, base + i, p->cq);
}
static void load_k(const fpo_problem* p, int64_t row, int head, double* out) {
  size_t base = ((size_t)row * p->hkv + head) * p->d;
  for (int i = 0; i < p->d; ++i) out[i] = elem(p->k, p->dtype, base + i, p->ck);
}
static void load_v(const fpo_problem* p, int64_t row, int head, double* out) {
  size_t base = ((size_t)row * p->hkv + head) * p->d;
  for (int i = 0; i < p->d; ++i) out[i] = elem(p->v, p->dtype, base + i, p->cv);
}

static double dot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

static double absdot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += fabs(a[i] * b[i]);
  return s;
}

/* ------------------------------------------------------------------ */
/* geometry                                                             */
/* ------------------------------------------------------------------ */

/* key/value length L_kv, query length L_q, first query position and first
 * K/V row of request b */
static int64_t req_len(const fpo_problem* p, int b) {
  const int64_t* c = p->cu_kv ? p->cu_kv : p->cu;
  return c[b + 1] - c[b];
}
static int64_t q_len(const fpo_problem* p, int b) { return p->cu[b + 1] - p->cu[b]; }
static int64_t q_off(const fpo_problem* p, int b) { return req_len(p, b) - q_len(p, b); }
static int64_t kv_start(const fpo_problem* p, int b) { return p->cu_kv ? p->cu_kv[b] : p->cu[b]; }
static int group(const fpo_problem* p) { return p->hq / p->hkv; }

int64_t fpo_blocks_in_req(const fpo_problem* p, int b) {
  return (req_len(p, b) + p->block - 1) / p->block;
}

/* first block of request b in the concatenated block list */
int64_t fpo_block_offset(const fpo_problem* p, int b) {
  int64_t off = 0;
  for (int i = 0; i < b; ++i) off += fpo_blocks_in_req(p, i);
  return off;
}

int64_t fpo_tiles_in_req(const fpo_problem* p, int b) {
  int64_t packed = (int64_t)group(p) * q_len(p, b);
  return (packed + p->rows - 1) / p->rows;
}

int64_t fpo_num_segments(const fpo_problem* p) {
  int64_t n = 0;
  for (int b = 0; b < p->num_reqs; ++b) n += (int64_t)p->hkv * fpo_tiles_in_req(p, b);
  return n;
}

/* Segment s -> (request, kv head, tile); segments are ordered (b, h, I). */
void fpo_segment_coords(const fpo_problem* p, int64_t s, int32_t* b_out, int32_t* h_out,
                        int64_t* i_out) {
  for (int b = 0; b < p->num_reqs; ++b) {
    int64_t nt = fpo_tiles_in_req(p, b);
    int64_t nb = (int64_t)p->hkv * nt;
    if (s < nb) {
      *b_out = b;
      *h_out = (int32_t)(s / nt);
      *i_out = s % nt;
      return;
    }
    s -= nb;
  }
  *b_out = -1;
  *h_out = -1;
  *i_out = -1;
}

/* Tile I of (b, h): packed rows [I*R, min((I+1)R, g*L_q)), first/last position
 * t0/t1 (off included) and its block beta = floor(t0/B) ([V2] §3.3 Eq. 13).
 * Returns the number of valid rows. */
int fpo_tile_info(const fpo_problem* p, int b, int64_t I, int64_t* t0, int64_t* t1,
                  int64_t* beta) {
  int g = group(p);
  int64_t packed = (int64_t)g * q_len(p, b);
  int64_t r0 = I * p->rows;
  int64_t r1 = r0 + p->rows;
  if (r1 > packed) r1 = packed;
  *t0 = q_off(p, b) + r0 / g;
  *t1 = q_off(p, b) + (r1 - 1) / g;
  *beta = *t0 / p->block;
  return (int)(r1 - r0);
}

/* ------------------------------------------------------------------ */
/* block mean pooling ([V2] §3.2 Eq. 5; §3.4 pipeline)                  */
/* ------------------------------------------------------------------ */

/* k_bar_J = (1/|B_J|) sum_{i in B_J} k_i, v_bar likewise, |B_J| = the actual
 * number of tokens in block J (the last block of a request may be short).
 * Output layout: [total_blocks][hkv][d], blocks concatenated by request. */
void fpo_pool_all(const fpo_problem* p, double* kbar, double* vbar) {
  int64_t nblk_total = fpo_block_offset(p, p->num_reqs);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t gb = 0; gb < nblk_total; ++gb) {
    int b = 0;
    int64_t J = gb;
    while (J >= fpo_blocks_in_req(p, b)) J -= fpo_blocks_in_req(p, b++);
    int64_t L = req_len(p, b);
    int64_t lo = J * p->block, hi = lo + p->block;
    if (hi > L) hi = L;
    double n = (double)(hi - lo);
    double* kv = (double*)malloc(sizeof(double) * p->d);
    for (int h = 0; h < p->hkv; ++h) {
      double* ko = kbar + ((size_t)gb * p->hkv + h) * p->d;
      double* vo = vbar + ((size_t)gb * p->hkv + h) * p->d;
      for (int i = 0; i < p->d; ++i) ko[i] = vo[i] = 0.0;
      for (int64_t t = lo; t < hi; ++t) {
        load_k(p, kv_start(p, b) + t, h, kv);
        for (int i = 0; i < p->d; ++i) ko[i] += kv[i];
        load_v(p, kv_start(p, b) + t, h, kv);
        for (int i = 0; i < p->d; ++i) vo[i] += kv[i];
      }
      for (int i = 0; i < p->d; ++i) {
        ko[i] /= n;
        vo[i] /= n;
      }
    }
    free(kv);
  }
}

/* pooled row of block J of request b (whose first block is blk0) */
static const double* kbar_row(const fpo_problem* p, const double* kbar, int64_t blk0, int h,
                              int64_t J) {
  return kbar + ((size_t)(blk0 + J) * p->hkv + h) * p->d;
}

/* ------------------------------------------------------------------ */
/* block energies of one tile ([V2] §3.1 Eq. 1-3, §3.3 Eq. 19-20)        */
/* ------------------------------------------------------------------ */

/* Candidate blocks are J in [0, beta1], beta1 = floor(t1/B) the block of the
 * tile's last position, the diagonal blocks included and scored with their full
 * pooled means (READING: the causal constraint of [V2] Eq. 3 and
 * thresh = alpha * max_{J <= I} of [V1] §3.4).  A fresh prefill's tile lies in
 * one block (beta1 = beta); a chunk whose first position is not a multiple of
 * R/g can put a tile across blocks beta and beta + 1 (READING, chunked prefill
 * of [V2] §4.3: every block holding a key visible to some row of the tile is a
 * candidate).  The logit carries the softmax
 * scale sigma as in [V2] Eq. 5 and Eq. 19 (READING: [V2] Eq. 1 omits it).
 *
 * form 0 -- direct: s_rJ = sigma q_r.k_bar_J, M = max_{r,J} s_rJ,
 *           E_J = sum_r exp(s_rJ - M).
 * form 1 -- [V2] Eq. 1-2 ([V1] §3.2): per-block max m_J over the tile rows,
 *           S_J = sum_r exp(s_rJ - m_J), global M = max_J m_J,
 *           E_J = S_J * exp(m_J - M).  Eq. 2's normalising sum and epsilon
 *           cancel in the ratio of Eq. 3 and are not formed.
 * form 2 -- [V2] Eq. 19-20: blocks visited in chunks of 64 with a running
 *           log2-domain maximum M; E_J = sum_r 2^(s_rJ log2 e - M) with the
 *           chunk's M stored as M_c; finally E_J <- E_J 2^(M_c - M_final).
 *
 * All forms return e_J = E_J / max_J' E_J' in (0, 1] (the normalised energy
 * that [V2] Eq. 3 / Eq. 20 compare against alpha).  Returns beta1 + 1. */
int64_t fpo_score_tile(const fpo_problem* p, const double* kbar, int b, int h, int64_t I,
                       int form, double* e_out) {
  int g = group(p);
  int64_t t0, t1, beta;
  int nrows = fpo_tile_info(p, b, I, &t0, &t1, &beta);
  int64_t nc = t1 / p->block + 1;
  int d = p->d;
  double* qv = (double*)malloc(sizeof(double) * (size_t)nrows * d);
  double* s = (double*)malloc(sizeof(double) * (size_t)nrows * nc);
  for (int r = 0; r < nrows; ++r) {
    int64_t pr = I * p->rows + r;
    load_q(p, p->cu[b] + pr / g, h * g + (int)(pr % g), qv + (size_t)r * d); /* query pr/g */
  }
  int64_t blk0 = fpo_block_offset(p, b);
  for (int r = 0; r < nrows; ++r)
    for (int64_t J = 0; J < nc; ++J)
      s[(size_t)r * nc + J] = p->scale * dot(qv + (size_t)r * d, kbar_row(p, kbar, blk0, h, J), d);

  if (form == 0) {
    double M = -INFINITY;
    for (size_t i = 0; i < (size_t)nrows * nc; ++i)
      if (s[i] > M) M = s[i];
    for (int64_t J = 0; J < nc; ++J) {
      double E = 0.0;
      for (int r = 0; r < nrows; ++r) E += exp(s[(size_t)r * nc + J] - M);
      e_out[J] = E;
    }
  } else if (form == 1) {
    double* m = (double*)malloc(sizeof(double) * nc);
    double Mi = -INFINITY;
    for (int64_t J = 0; J < nc; ++J) {
      m[J] = -INFINITY;
      for (int r = 0; r < nrows; ++r)
        if (s[(size_t)r * nc + J] > m[J]) m[J] = s[(size_t)r * nc + J];
      if (m[J] > Mi) Mi = m[J];
    }
    for (int64_t J = 0; J < nc; ++J) {
      double S = 0.0;
      for (int r = 0; r < nrows; ++r) S += exp(s[(size_t)r * nc + J] - m[J]);
      e_out[J] = S * exp(m[J] - Mi);
    }
    free(m);
  } else {
    const double LOG2E = 1.0 / log(2.0);
    const int64_t CH = 64;
    int64_t nchunks = (nc + CH - 1) / CH;
    double* Mc = (double*)malloc(sizeof(double) * nchunks);
    double M = -INFINITY;
    for (int64_t c = 0; c < nchunks; ++c) {
      int64_t j0 = c * CH, j1 = j0 + CH < nc ? j0 + CH : nc;
      double Mt = -INFINITY;
      for (int r = 0; r < nrows; ++r)
        for (int64_t J = j0; J < j1; ++J)
          if (s[(size_t)r * nc + J] * LOG2E > Mt) Mt = s[(size_t)r * nc + J] * LOG2E;
      if (Mt > M) M = Mt;
      Mc[c] = M;
      for (int64_t J = j0; J < j1; ++J) {
        double E = 0.0;
        for (int r = 0; r < nrows; ++r) E += exp2(s[(size_t)r * nc + J] * LOG2E - M);
        e_out[J] = E;
      }
    }
    for (int64_t J = 0; J < nc; ++J) e_out[J] *= exp2(Mc[J / CH] - M);
    free(Mc);
  }
  double Emax = 0.0;
  for (int64_t J = 0; J < nc; ++J)
    if (e_out[J] > Emax) Emax = e_out[J];
  for (int64_t J = 0; J < nc; ++J) e_out[J] /= Emax;
  free(qv);
  free(s);
  return nc;
}

/* ------------------------------------------------------------------ */
/* max-based threshold with forced blocks ([V2] Eq. 3, Eq. 20)          */
/* ------------------------------------------------------------------ */

/* Keep J iff e_J >= alpha (inclusive), or J is a sink block (J < n_sink), a
 * window block (the n_win blocks just before beta), or a diagonal block
 * J >= beta, i.e. one holding a position of the tile ([V2] §3.1 "Max-based
 * Dynamic Thresholding"; defaults in §4.1).  The candidates are J < nc.
 * ambig[J] marks unforced blocks with |e_J - alpha| <= 1e-4 alpha, where two
 * correct implementations may legitimately disagree. */
void fpo_select_tile(const double* e, int64_t nc, int64_t beta, double alpha, int n_sink,
                     int n_win, uint8_t* sel, uint8_t* ambig) {
  for (int64_t J = 0; J < nc; ++J) {
    int forced = (J < n_sink) || (J >= beta - n_win && J < beta) || (J >= beta);
    sel[J] = (uint8_t)(forced || e[J] >= alpha);
    if (ambig) ambig[J] = (uint8_t)(!forced && fabs(e[J] - alpha) <= 1e-4 * alpha);
  }
}

/* ------------------------------------------------------------------ */
/* CSR segment ([V2] §3.3 Eq. 17; logical-to-physical expansion, §3.4)   */
/* ------------------------------------------------------------------ */

/* Each selected logical block J becomes the B/P physical tiles J*(B/P)+k, in
 * ascending order.  READING: a tile p whose first key P*p lies after the
 * tile's last position t1 holds no visible key for any row and is dropped. */
int64_t fpo_csr_tile(const uint8_t* sel, int64_t nc, int64_t t1, int phys, int block,
                     int32_t* out) {
  int64_t n = 0;
  int per = block / phys;
  for (int64_t J = 0; J < nc; ++J) {
    if (!sel[J]) continue;
    for (int k = 0; k < per; ++k) {
      int64_t tile = J * per + k;
      if (tile * phys > t1) continue;
      if (out) out[n] = (int32_t)tile;
      ++n;
    }
  }
  return n;
}

/* Whole-problem index: cu[n_seg+1] (exclusive prefix sum in segment order)
 * and idx.  e_out / ambig_out (optional) are [n_seg][max_nc] with max_nc at
 * least the largest beta1+1, padded with -1 / 0.  Returns the number of idx entries, or
 * -1 if cap is too small. */
int64_t fpo_select_all(const fpo_problem* p, const double* kbar, double alpha, int n_sink,
                       int n_win, int form, int32_t* cu, int32_t* idx, int64_t cap,
                       double* e_out, uint8_t* ambig_out, int64_t max_nc) {
  int64_t nseg = fpo_num_segments(p);
  int64_t* counts = (int64_t*)malloc(sizeof(int64_t) * (nseg + 1));
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t s = 0; s < nseg; ++s) {
    int32_t b, h;
    int64_t I, t0, t1, beta;
    fpo_segment_coords(p, s, &b, &h, &I);
    fpo_tile_info(p, b, I, &t0, &t1, &beta);
    int64_t nc = t1 / p->block + 1;
    double* e = (double*)malloc(sizeof(double) * nc);
    uint8_t* sel = (uint8_t*)malloc(nc);
    uint8_t* amb = (uint8_t*)malloc(nc);
    fpo_score_tile(p, kbar, b, h, I, form, e);
    fpo_select_tile(e, nc, beta, alpha, n_sink, n_win, sel, amb);
    counts[s] = fpo_csr_tile(sel, nc, t1, p->phys, p->block, NULL);
    if (e_out)
      for (int64_t J = 0; J < max_nc; ++J) e_out[s * max_nc + J] = J < nc ? e[J] : -1.0;
    if (ambig_out)
      for (int64_t J = 0; J < max_nc; ++J) ambig_out[s * max_nc + J] = J < nc ? amb[J] : 0;
    free(e);
    free(sel);
    free(amb);
  }
  int64_t total = 0;
  for (int64_t s = 0; s < nseg; ++s) {
    int64_t c = counts[s];
    counts[s] = total;
    total += c;
  }
  counts[nseg] = total;
  for (int64_t s = 0; s <= nseg; ++s) cu[s] = (int32_t)counts[s];
  if (total > cap) {
    free(counts);
    return -1;
  }
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t s = 0; s < nseg; ++s) {
    int32_t b, h;
    int64_t I, t0, t1, beta;
    fpo_segment_coords(p, s, &b, &h, &I);
    fpo_tile_info(p, b, I, &t0, &t1, &beta);
    int64_t nc = t1 / p->block + 1;
    double* e = (double*)malloc(sizeof(double) * nc);
    uint8_t* sel = (uint8_t*)malloc(nc);
    fpo_score_tile(p, kbar, b, h, I, form, e);
    fpo_select_tile(e, nc, beta, alpha, n_sink, n_win, sel, NULL);
    fpo_csr_tile(sel, nc, t1, p->phys, p->block, idx + counts[s]);
    free(e);
    free(sel);
  }
  free(counts);
  return total;
}

/* Index of a list of segments (OpenMP over the list): scoring, selection and
 * CSR expansion of segs[n] into lists + n * stride (stride >= 2 * the
 * segment's candidate count), its length into counts[n]. */
void fpo_select_list(const fpo_problem* p, const double* kbar, double alpha, int n_sink, int n_win,
                     int form, int64_t nlist, const int64_t* segs, int64_t stride, int32_t* lists,
                     int32_t* counts) {
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t n = 0; n < nlist; ++n) {
    int32_t b, h;
    int64_t I, t0, t1, beta;
    fpo_segment_coords(p, segs[n], &b, &h, &I);
    fpo_tile_info(p, b, I, &t0, &t1, &beta);
    int64_t nc = t1 / p->block + 1;
    double* e = (double*)malloc(sizeof(double) * nc);
    uint8_t* sel = (uint8_t*)malloc(nc);
    fpo_score_tile(p, kbar, b, h, I, form, e);
    fpo_select_tile(e, nc, beta, alpha, n_sink, n_win, sel, NULL);
    counts[n] = (int32_t)fpo_csr_tile(sel, nc, t1, p->phys, p->block, NULL);
    if (counts[n] <= stride) fpo_csr_tile(sel, nc, t1, p->phys, p->block, lists + n * stride);
    free(e);
    free(sel);
  }
}

/* ------------------------------------------------------------------ */
/* attention of one tile with mean correction ([V2] §3.2 Eq. 4-6)       */
/* ------------------------------------------------------------------ */

/* For every valid row r of tile I (position t = floor(r/g)):
 *   exact tokens  T = { i <= t : floor(i/P) in idx }
 *   selected blocks S = { floor(p P / B) : p in idx }
 *   corrected blocks C = { J < beta : J not in S } when correction is on:
 *     the blocks fully visible to every row of the tile ([V2] §3.2
 *     "Implementation"); each stands for |B_J| = B tokens.
 *   logits a_i = sigma q.k_i (i in T), c_J = sigma q.k_bar_J + ln|B_J| (J in C)
 *   O = (sum_T e^{a_i-m} v_i + sum_C e^{c_J-m} v_bar_J) / (sum_T e^{a_i-m} + sum_C e^{c_J-m})
 *   LSE = m + ln(denominator), m = max of all logits.
 * p8 != 0 is an order-free diagnostic of [V2] Eq. 15: every weight e^{a-m},
 * m the FINAL row maximum, is multiplied by 2^8 and rounded to E4M3 before
 * both sums, and LSE subtracts ln 2^8.  Eq. 15 itself rounds against the
 * running maximum: fpo_attend_tile_eq15 below.
 * out is [R][d], lse is [R]; rows past the end of the request are zeroed. */
void fpo_attend_tile(const fpo_problem* p, const double* kbar, const double* vbar, int b,
                     int h, int64_t I, const int32_t* idx, int64_t T, int correction, int p8,
                     double* out, double* lse) {
  int g = group(p), d = p->d;
  int64_t t0, t1, beta;
  int nrows = fpo_tile_info(p, b, I, &t0, &t1, &beta);
  int64_t L = req_len(p, b);
  int64_t nblk = fpo_blocks_in_req(p, b);
  int64_t blk0 = fpo_block_offset(p, b);
  uint8_t* in_s = (uint8_t*)calloc((size_t)nblk, 1);
  for (int64_t t = 0; t < T; ++t) {
    int64_t J = (int64_t)idx[t] * p->phys / p->block;
    if (J >= 0 && J < nblk) in_s[J] = 1;
  }
  double* qv = (double*)malloc(sizeof(double) * d);
  double* kv = (double*)malloc(sizeof(double) * d);
  double* vv = (double*)malloc(sizeof(double) * d);
  double* num = (double*)malloc(sizeof(double) * d);
  for (int r = 0; r < p->rows; ++r) {
    double* o = out + (size_t)r * d;
    if (r >= nrows) {
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      if (lse) lse[r] = 0.0;
      continue;
    }
    int64_t pr = I * p->rows + r;
    int64_t t = q_off(p, b) + pr / g; /* position of the row's query */
    load_q(p, p->cu[b] + pr / g, h * g + (int)(pr % g), qv);
    /* pass 1: the row maximum over every logit that enters the softmax */
    double m = -INFINITY;
    for (int64_t e = 0; e < T; ++e)
      for (int64_t i = (int64_t)idx[e] * p->phys; i < ((int64_t)idx[e] + 1) * p->phys; ++i) {
        if (i > t || i >= L) continue;
        load_k(p, kv_start(p, b) + i, h, kv);
        double a = p->scale * dot(qv, kv, d);
        if (a > m) m = a;
      }
    if (correction)
      for (int64_t J = 0; J < beta; ++J) {
        if (in_s[J]) continue;
        double c = p->scale * dot(qv, kbar_row(p, kbar, blk0, h, J), d) + log((double)p->block);
        if (c > m) m = c;
      }
    /* pass 2: numerator and denominator of [V2] Eq. 6 */
    double den = 0.0;
    for (int i = 0; i < d; ++i) num[i] = 0.0;
    for (int64_t e = 0; e < T; ++e)
      for (int64_t i = (int64_t)idx[e] * p->phys; i < ((int64_t)idx[e] + 1) * p->phys; ++i) {
        if (i > t || i >= L) continue;
        load_k(p, kv_start(p, b) + i, h, kv);
        load_v(p, kv_start(p, b) + i, h, vv);
        double w = exp(p->scale * dot(qv, kv, d) - m);
        if (p8) w = fpo_e4m3_round(256.0 * w);
        den += w;
        for (int j = 0; j < d; ++j) num[j] += w * vv[j];
      }
    if (correction)
      for (int64_t J = 0; J < beta; ++J) {
        if (in_s[J]) continue;
        const double* kb = kbar_row(p, kbar, blk0, h, J);
        const double* vb = kbar_row(p, vbar, blk0, h, J);
        double w = exp(p->scale * dot(qv, kb, d) + log((double)p->block) - m);
        if (p8) w = fpo_e4m3_round(256.0 * w);
        den += w;
        for (int j = 0; j < d; ++j) num[j] += w * vb[j];
      }
    for (int j = 0; j < d; ++j) o[j] = num[j] / den;
    if (lse) lse[r] = m + log(den) - (p8 ? log(256.0) : 0.0);
  }
  free(in_s);
  free(qv);
  free(kv);
  free(vv);
  free(num);
}

/* [V2] §3.3 Eq. 15 as printed: the online softmax visited step by step, each
 * E4M3 weight rounded against the RUNNING row maximum m.
 *
 * Steps, in the order the pages give them: the listed tiles backwards
 * (n_t = idx[T - 1 - t], Eq. 17), then the correction chunks appended after
 * them (Algorithm 1, step 9); a chunk is 64 consecutive blocks (READING: the
 * chunk width is not printed) and holds the corrected blocks of its range.
 * W = T + ceil(beta/64) steps in all when correction is on, T otherwise.
 * Under KV splitting, split u of U takes steps [u ceil(W/U), (u+1) ceil(W/U))
 * of that sequence (Eq. 18's count partition; READING: the correction chunks
 * count as steps like the listed tiles) and starts with its own maximum; the
 * splits are merged exactly by their log-sum-exp.
 *
 * Per row and split, for each step with member logits x (keys i <= t of the
 * tile: a_i = sigma q.k_i; corrected blocks of the chunk: c_J = sigma q.k_bar_J
 * + ln|B_J|, values v_i / v_bar_J):
 *   m_new = max(m, max x);  acc *= e^{m - m_new};  den *= e^{m - m_new}
 *   P_x   = round_e4m3(2^8 e^{x - m_new})   (round = 0: 2^8 e^{x - m_new})
 *   acc  += sum P_x v_x;  den += sum P_x;  m = m_new
 * so a weight is rounded once, at the maximum of its own step; later rescales
 * act on the sums, not on rounded weights.  O = acc / den and LSE = m +
 * ln(den) - ln 2^8, with the splits merged first.  round = 0 is the same
 * recurrence with no rounding, which must reproduce fpo_attend_tile's exact
 * rows (the recurrence, the rescales and the split merge are exact in exact
 * arithmetic).  nsplit >= 1.  out is [R][d], lse is [R].
 *
 * Rounding ties (allow, lallow: optional [R]).  An implementation forms each
 * logit with some error; take it to be at most logit_err times the logit's
 * sum of absolute products, A = sigma sum_i |q_i k_i| (the same for a mean,
 * without its ln|B_J|).  A weight 2^8 e^{x - m} is then known only up to a
 * factor e^{+-delta}, delta = logit_err (A_x + A_m) with A_m that of the
 * logit that set the running maximum m; when that interval holds the midpoint
 * between the weight's two E4M3 neighbours, both roundings are valid.  For
 * each row, allow bounds how far the output can move (max-abs over the row)
 * and lallow how far the LSE can move if every such weight took its other
 * rounding:
 *   S  = sum over tied weights of f s_i,  SV = sum of f s_i |v_i|_inf
 *   allow = (SV + S |O|_inf) / (D - S),  lallow = -ln(1 - S / D)
 * with s_i the gap between the neighbours, f the weight's rescale factor into
 * the merged sums and D the merged denominator (a first-order bound that holds
 * while S < D; +inf otherwise).  Both are 0 when round = 0 or logit_err = 0. */
void fpo_attend_tile_eq15(const fpo_problem* p, const double* kbar, const double* vbar, int b,
                          int h, int64_t I, const int32_t* idx, int64_t T, int correction,
                          int round, int nsplit, double logit_err, double* out, double* lse,
                          double* allow, double* lallow) {
  int g = group(p), d = p->d;
  int64_t t0, t1, beta;
  int nrows = fpo_tile_info(p, b, I, &t0, &t1, &beta);
  int64_t L = req_len(p, b);
  int64_t nblk = fpo_blocks_in_req(p, b);
  int64_t blk0 = fpo_block_offset(p, b);
  const int64_t CH = 64;
  int64_t nch = correction ? (beta + CH - 1) / CH : 0;
  int64_t W = T + nch;
  if (nsplit < 1) nsplit = 1;
  int64_t per = (W + nsplit - 1) / nsplit;
  uint8_t* in_s = (uint8_t*)calloc((size_t)(nblk > 0 ? nblk : 1), 1);
  for (int64_t e = 0; e < T; ++e) {
    int64_t J = (int64_t)idx[e] * p->phys / p->block;
    if (J >= 0 && J < nblk) in_s[J] = 1;
  }
  double* qv = (double*)malloc(sizeof(double) * d);
  double* kv = (double*)malloc(sizeof(double) * d);
  double* vv = (double*)malloc(sizeof(double) * d);
  double* acc = (double*)malloc(sizeof(double) * d);
  double* tot = (double*)malloc(sizeof(double) * d);
  /* logits and values of one step's members */
  int64_t cap = p->phys > CH ? p->phys : CH;
  double* x = (double*)malloc(sizeof(double) * cap);
  double* xa = (double*)malloc(sizeof(double) * cap); /* sigma sum |q_i k_i| of each logit */
  double* xv = (double*)malloc(sizeof(double) * cap * d);
  double* m_u = (double*)malloc(sizeof(double) * nsplit);
  double* den_u = (double*)malloc(sizeof(double) * nsplit);
  double* ts_u = (double*)malloc(sizeof(double) * nsplit);  /* tied gaps, in split u's scale */
  double* tsv_u = (double*)malloc(sizeof(double) * nsplit); /* tied gaps times |v|_inf */
  double* acc_u = (double*)malloc(sizeof(double) * nsplit * d);
  for (int r = 0; r < p->rows; ++r) {
    double* o = out + (size_t)r * d;
    if (r >= nrows) {
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      if (lse) lse[r] = 0.0;
      if (allow) allow[r] = 0.0;
      if (lallow) lallow[r] = 0.0;
      continue;
    }
    int64_t pr = I * p->rows + r;
    int64_t t = q_off(p, b) + pr / g; /* position of the row's query */
    load_q(p, p->cu[b] + pr / g, h * g + (int)(pr % g), qv);
    for (int u = 0; u < nsplit; ++u) {
      double m = -INFINITY, am = 0.0, den = 0.0, ts = 0.0, tsv = 0.0; /* am: A of the maximum */
      for (int i = 0; i < d; ++i) acc[i] = 0.0;
      int64_t s0 = (int64_t)u * per, s1 = s0 + per;
      if (s0 > W) s0 = W;
      if (s1 > W) s1 = W;
      for (int64_t st = s0; st < s1; ++st) {
        /* the step's members */
        int64_t n = 0;
        if (st < T) {
          int64_t tile = idx[T - 1 - st];
          for (int64_t i = tile * p->phys; i < (tile + 1) * p->phys; ++i) {
            if (i > t || i >= L) continue;
            load_k(p, kv_start(p, b) + i, h, kv);
            load_v(p, kv_start(p, b) + i, h, xv + (size_t)n * d);
            xa[n] = p->scale * absdot(qv, kv, d);
            x[n++] = p->scale * dot(qv, kv, d);
          }
        } else {
          int64_t ch = st - T;
          for (int64_t J = ch * CH; J < (ch + 1) * CH && J < beta; ++J) {
            if (in_s[J]) continue;
            const double* vb = kbar_row(p, vbar, blk0, h, J);
            for (int i = 0; i < d; ++i) xv[(size_t)n * d + i] = vb[i];
            xa[n] = p->scale * absdot(qv, kbar_row(p, kbar, blk0, h, J), d);
            x[n++] = p->scale * dot(qv, kbar_row(p, kbar, blk0, h, J), d) + log((double)p->block);
          }
        }
        if (n == 0) continue;
        double mx = -INFINITY, amx = 0.0;
        for (int64_t j = 0; j < n; ++j)
          if (x[j] > mx) {
            mx = x[j];
            amx = xa[j];
          }
        if (mx > m) {
          am = amx;
          double f = m == -INFINITY ? 0.0 : exp(m - mx);
          den *= f;
          ts *= f;
          tsv *= f;
          for (int i = 0; i < d; ++i) acc[i] *= f;
          m = mx;
        }
        for (int64_t j = 0; j < n; ++j) {
          double w = 256.0 * exp(x[j] - m);
          if (round) {
            if (logit_err > 0.0 && w < 448.0) {
              double lo, hi;
              e4m3_bracket(w, &lo, &hi);
              double mid = 0.5 * (lo + hi), delta = logit_err * (xa[j] + am);
              if (fabs(log(w / mid)) <= delta) {
                double vmax = 0.0;
                for (int i = 0; i < d; ++i)
                  if (fabs(xv[(size_t)j * d + i]) > vmax) vmax = fabs(xv[(size_t)j * d + i]);
                ts += hi - lo;
                tsv += (hi - lo) * vmax;
              }
            }
            w = fpo_e4m3_round(w);
          }
          den += w;
          for (int i = 0; i < d; ++i) acc[i] += w * xv[(size_t)j * d + i];
        }
      }
      m_u[u] = m;
      den_u[u] = den;
      ts_u[u] = ts;
      tsv_u[u] = tsv;
      for (int i = 0; i < d; ++i) acc_u[(size_t)u * d + i] = acc[i];
    }
    /* merge the splits by their maxima */
    double M = -INFINITY;
    for (int u = 0; u < nsplit; ++u)
      if (m_u[u] > M) M = m_u[u];
    double D = 0.0, S = 0.0, SV = 0.0;
    for (int i = 0; i < d; ++i) tot[i] = 0.0;
    for (int u = 0; u < nsplit; ++u) {
      if (m_u[u] == -INFINITY) continue;
      double f = exp(m_u[u] - M);
      D += f * den_u[u];
      S += f * ts_u[u];
      SV += f * tsv_u[u];
      for (int i = 0; i < d; ++i) tot[i] += f * acc_u[(size_t)u * d + i];
    }
    double omax = 0.0;
    for (int i = 0; i < d; ++i) {
      o[i] = tot[i] / D;
      if (fabs(o[i]) > omax) omax = fabs(o[i]);
    }
    if (lse) lse[r] = M + log(D) - log(256.0);
    if (allow) allow[r] = S == 0.0 ? 0.0 : S < D ? (SV + S * omax) / (D - S) : INFINITY;
    if (lallow) lallow[r] = S == 0.0 ? 0.0 : S < D ? -log(1.0 - S / D) : INFINITY;
  }
  free(in_s);
  free(qv);
  free(kv);
  free(vv);
  free(acc);
  free(tot);
  free(x);
  free(xa);
  free(xv);
  free(m_u);
  free(den_u);
  free(ts_u);
  free(tsv_u);
  free(acc_u);
}

/* Dense causal softmax attention of the same rows ([V2] §3.2 Eq. 4 left). */
void fpo_dense_tile(const fpo_problem* p, int b, int h, int64_t I, double* out, double* lse) {
  int g = group(p), d = p->d;
  int64_t t0, t1, beta;
  int nrows = fpo_tile_info(p, b, I, &t0, &t1, &beta);
  double* qv = (double*)malloc(sizeof(double) * d);
  double* kv = (double*)malloc(sizeof(double) * d);
  double* vv = (double*)malloc(sizeof(double) * d);
  double* num = (double*)malloc(sizeof(double) * d);
  for (int r = 0; r < p->rows; ++r) {
    double* o = out + (size_t)r * d;
    if (r >= nrows) {
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      if (lse) lse[r] = 0.0;
      continue;
    }
    int64_t pr = I * p->rows + r;
    int64_t t = q_off(p, b) + pr / g; /* position of the row's query */
    load_q(p, p->cu[b] + pr / g, h * g + (int)(pr % g), qv);
    double m = -INFINITY;
    for (int64_t i = 0; i <= t; ++i) {
      load_k(p, kv_start(p, b) + i, h, kv);
      double a = p->scale * dot(qv, kv, d);
      if (a > m) m = a;
    }
    double den = 0.0;
    for (int i = 0; i < d; ++i) num[i] = 0.0;
    for (int64_t i = 0; i <= t; ++i) {
      load_k(p, kv_start(p, b) + i, h, kv);
      load_v(p, kv_start(p, b) + i, h, vv);
      double w = exp(p->scale * dot(qv, kv, d) - m);
      den += w;
      for (int j = 0; j < d; ++j) num[j] += w * vv[j];
    }
    for (int j = 0; j < d; ++j) o[j] = num[j] / den;
    if (lse) lse[r] = m + log(den);
  }
  free(qv);
  free(kv);
  free(vv);
  free(num);
}

/* Batch drivers over a list of segment ids (OpenMP over segments).
 * mode 0: sparse with the given CSR (cu, idx indexed by segment id);
 * mode 1: dense.  out is [nlist][R][d], lse is [nlist][R]. */
void fpo_attend_list(const fpo_problem* p, const double* kbar, const double* vbar,
                     int64_t nlist, const int64_t* segs, const int32_t* cu, const int32_t* idx,
                     int mode, int correction, int p8, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < nlist; ++n) {
    int32_t b, h;
    int64_t I;
    fpo_segment_coords(p, segs[n], &b, &h, &I);
    double* o = out + (size_t)n * p->rows * p->d;
    double* l = lse ? lse + (size_t)n * p->rows : NULL;
    if (mode == 1)
      fpo_dense_tile(p, b, h, I, o, l);
    else
      fpo_attend_tile(p, kbar, vbar, b, h, I, idx + cu[segs[n]], cu[segs[n] + 1] - cu[segs[n]],
                      correction, p8, o, l);
  }
}

/* [V2] Eq. 15 rows of a list of segments (OpenMP over segments): cu, idx
 * indexed by segment id as above; nsplit[n] (NULL: 1) is the split count of
 * the n-th listed segment; allow / lallow ([nlist][R], optional) as in
 * fpo_attend_tile_eq15. */
void fpo_attend_list_eq15(const fpo_problem* p, const double* kbar, const double* vbar,
                          int64_t nlist, const int64_t* segs, const int32_t* cu, const int32_t* idx,
                          int correction, int round, const int32_t* nsplit, double logit_err,
                          double* out, double* lse, double* allow, double* lallow) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < nlist; ++n) {
    int32_t b, h;
    int64_t I;
    fpo_segment_coords(p, segs[n], &b, &h, &I);
    fpo_attend_tile_eq15(p, kbar, vbar, b, h, I, idx + cu[segs[n]], cu[segs[n] + 1] - cu[segs[n]],
                         correction, round, nsplit ? nsplit[n] : 1, logit_err,
                         out + (size_t)n * p->rows * p->d, lse ? lse + (size_t)n * p->rows : NULL,
                         allow ? allow + (size_t)n * p->rows : NULL,
                         lallow ? lallow + (size_t)n * p->rows : NULL);
  }
}

/* ------------------------------------------------------------------ */
/* exact block attention mass (the selection-recall diagnostic)         */
/* ------------------------------------------------------------------ */

/* [V1] §3.1 "exact identification": every query of the tile is scored
 * against every visible key, the per-query attention is summed within each
 * block and then averaged over the tile's queries ("secondary averaging"):
 *   mass_J = (1/n) sum_r sum_{i in B_J, i <= t_r} exp(sigma q_r.k_i - LSE_r),
 * LSE_r the row's dense log-sum-exp, n the tile's valid rows, so that
 * sum_J mass_J = 1.  For the blocks J < beta that every row sees whole, the
 * mean surrogate the correction substitutes ([V2] Eq. 6; [V1] §3.1's
 * Psi_pool = exp(q.k_bar) against Psi_sum, the AM-GM pair) is
 *   sur_J = (1/n) sum_r |B_J| exp(sigma q_r.k_bar_J - LSE_r)  (0 for J >= beta),
 * so sur_J <= mass_J.  Returns nc = beta1 + 1, the candidate count; both
 * arrays hold nc entries. */
int64_t fpo_block_mass_tile(const fpo_problem* p, const double* kbar, int b, int h, int64_t I,
                            double* mass, double* sur) {
  int g = group(p), d = p->d;
  int64_t t0, t1, beta;
  int nrows = fpo_tile_info(p, b, I, &t0, &t1, &beta);
  int64_t nc = t1 / p->block + 1;
  int64_t blk0 = fpo_block_offset(p, b);
  double* qv = (double*)malloc(sizeof(double) * d);
  double* kv = (double*)malloc(sizeof(double) * d);
  double* a = (double*)malloc(sizeof(double) * (size_t)(t1 + 1));
  for (int64_t J = 0; J < nc; ++J) mass[J] = sur[J] = 0.0;
  for (int r = 0; r < nrows; ++r) {
    int64_t pr = I * p->rows + r;
    int64_t t = q_off(p, b) + pr / g;
    load_q(p, p->cu[b] + pr / g, h * g + (int)(pr % g), qv);
    double m = -INFINITY;
    for (int64_t i = 0; i <= t; ++i) {
      load_k(p, kv_start(p, b) + i, h, kv);
      a[i] = p->scale * dot(qv, kv, d);
      if (a[i] > m) m = a[i];
    }
    double den = 0.0;
    for (int64_t i = 0; i <= t; ++i) den += exp(a[i] - m);
    double lse = m + log(den);
    for (int64_t i = 0; i <= t; ++i) mass[i / p->block] += exp(a[i] - lse);
    for (int64_t J = 0; J < beta; ++J)
      sur[J] += (double)p->block *
                exp(p->scale * dot(qv, kbar_row(p, kbar, blk0, h, J), d) - lse);
  }
  for (int64_t J = 0; J < nc; ++J) {
    mass[J] /= nrows;
    sur[J] /= nrows;
  }
  free(qv);
  free(kv);
  free(a);
  return nc;
}

/* mass / sur of a list of segments, [nlist][max_nc], padded with -1. */
void fpo_block_mass_list(const fpo_problem* p, const double* kbar, int64_t nlist, const int64_t* segs,
                         int64_t max_nc, double* mass, double* sur) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < nlist; ++n) {
    int32_t b, h;
    int64_t I;
    fpo_segment_coords(p, segs[n], &b, &h, &I);
    double* mo = mass + (size_t)n * max_nc;
    double* so = sur + (size_t)n * max_nc;
    int64_t nc = fpo_block_mass_tile(p, kbar, b, h, I, mo, so);
    for (int64_t J = nc; J < max_nc; ++J) mo[J] = so[J] = -1.0;
  }
}

int fpo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
