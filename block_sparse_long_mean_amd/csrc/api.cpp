// api.cpp -- the C ABI of libfp.so (declared in include/fp.h): argument
// validation, buffer layouts, and the launch sequence of each entry point.
// Host-only code; every step of the computation runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "../../include/fp.h"
#include "fp_internal.h"

using namespace fp;

namespace fp {

hipError_t set_lds_limit(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;  // (kernel, device) pairs already raised
  std::lock_guard<std::mutex> lk(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}

}  // namespace fp

namespace {

thread_local std::string g_last_error;

fp_status fail(fp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Host view of the batch, derived from the host copies of the offsets.
struct HostGeo {
  int64_t total = 0, total_kv = 0, n_seg = 0, nb_pad = 0, idx_cap = 0;
  int64_t step_cap = 0;  // most attention steps the scheduler can count (int32 prefix sums)
  int32_t max_len = 0, max_nj = 1, words = 1, g = 1, log2g = 0;  // max_len: longest K/V sequence
};

fp_status validate_problem(const fp_problem* p, HostGeo* hg) {
  if (!p) return fail(FP_ERR_INVALID_ARG, "problem is NULL");
  if (p->num_reqs < 1) return fail(FP_ERR_INVALID_ARG, "num_reqs must be >= 1 (got %d)", p->num_reqs);
  if (p->num_heads_kv < 1 || p->num_heads_q < 1)
    return fail(FP_ERR_INVALID_ARG, "head counts must be >= 1");
  if (p->num_heads_q % p->num_heads_kv)
    return fail(FP_ERR_INVALID_ARG, "num_heads_q (%d) is not a multiple of num_heads_kv (%d)", p->num_heads_q,
                p->num_heads_kv);
  const int g = p->num_heads_q / p->num_heads_kv;
  if ((g & (g - 1)) || g > kRows)
    return fail(FP_ERR_UNSUPPORTED, "group size %d must be a power of two <= %d", g, kRows);
  if (p->head_dim != kD) return fail(FP_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", kD, p->head_dim);
  if (!p->cu_seqlens_q || !p->cu_seqlens_q_host)
    return fail(FP_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_q_host are required");
  if (p->dtype != FP_F32 && p->dtype != FP_BF16 && p->dtype != FP_E4M3)
    return fail(FP_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->dtype == FP_E4M3 && !p->descale) return fail(FP_ERR_INVALID_ARG, "E4M3 inputs need descale[3]");
  if (p->v_layout != FP_V_ROWS && p->v_layout != FP_V_COLS)
    return fail(FP_ERR_INVALID_ARG, "unknown v_layout %d", p->v_layout);
  if (p->v_layout == FP_V_COLS && p->dtype != FP_E4M3)
    return fail(FP_ERR_UNSUPPORTED, "column-major V is an E4M3 layout");
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale >= 0.f))
    return fail(FP_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  const int32_t* cu = p->cu_seqlens_q_host;
  if ((p->cu_seqlens_kv == nullptr) != (p->cu_seqlens_kv_host == nullptr))
    return fail(FP_ERR_INVALID_ARG, "cu_seqlens_kv and cu_seqlens_kv_host are given together or not at all");
  const int32_t* ckv = p->cu_seqlens_kv_host ? p->cu_seqlens_kv_host : cu;
  if (cu[0] != 0) return fail(FP_ERR_INVALID_ARG, "cu_seqlens_q_host[0] must be 0");
  if (ckv[0] != 0) return fail(FP_ERR_INVALID_ARG, "cu_seqlens_kv_host[0] must be 0");
  hg->g = g;
  while ((1 << hg->log2g) < g) ++hg->log2g;
  int64_t max_len = 0;
  for (int b = 0; b < p->num_reqs; ++b) {
    const int64_t Lq = (int64_t)cu[b + 1] - cu[b];
    const int64_t L = (int64_t)ckv[b + 1] - ckv[b];
    if (Lq < 0) return fail(FP_ERR_INVALID_ARG, "cu_seqlens_q_host decreases at request %d", b);
    if (L < Lq)
      return fail(FP_ERR_INVALID_ARG, "request %d has %lld keys for %lld queries (needs L_kv >= L_q)", b,
                  (long long)L, (long long)Lq);
    if (L > (int64_t)kMaxBlocks * kBlock)
      return fail(FP_ERR_UNSUPPORTED, "request %d has %lld tokens; the limit is %d", b, (long long)L,
                  kMaxBlocks * kBlock);
    max_len = std::max(max_len, L);
    const int64_t off = L - Lq;  // position of the request's first query
    const int64_t nt = ((Lq << hg->log2g) + kRows - 1) / kRows;
    hg->n_seg += (int64_t)p->num_heads_kv * nt;
    const int64_t nj = (L + kBlock - 1) / kBlock;
    hg->nb_pad += (nj + kChunk - 1) / kChunk * kChunk;
    // worst-case CSR: every causal tile of every segment; worst-case step count
    // of the scheduler: a listed count clamped to both tiles of every candidate
    // block, plus every correction chunk
    for (int64_t I = 0; I < nt; ++I) {
      int64_t r0 = I * kRows;
      int64_t r1 = std::min((I + 1) * kRows, Lq << hg->log2g);
      int64_t t0 = off + (r0 >> hg->log2g);
      int64_t t1 = off + ((r1 - 1) >> hg->log2g);
      hg->idx_cap += (int64_t)p->num_heads_kv * (t1 / kTile + 1);
      hg->step_cap += (int64_t)p->num_heads_kv * (2 * (t1 / kBlock + 1) + (t0 / kBlock + kChunk - 1) / kChunk);
    }
  }
  hg->total = cu[p->num_reqs];
  hg->total_kv = ckv[p->num_reqs];
  if (hg->total > INT32_MAX / 2) return fail(FP_ERR_UNSUPPORTED, "total_q too large");
  if (hg->n_seg > INT32_MAX / 16 || hg->idx_cap > INT32_MAX)
    return fail(FP_ERR_UNSUPPORTED, "too many segments for int32 CSR offsets");
  if (hg->step_cap > INT32_MAX)
    return fail(FP_ERR_UNSUPPORTED, "up to %lld attention steps: too many for the scheduler's int32 sums",
                (long long)hg->step_cap);
  hg->max_len = (int32_t)max_len;
  hg->max_nj = (int32_t)std::max<int64_t>(1, (max_len + kBlock - 1) / kBlock);
  hg->words = (hg->max_nj + 31) / 32 + 1;
  // K/V rows are addressed through 32-bit buffer offsets (one KV head's rows of
  // a request, or of the whole page pool), which must stay below 4 GiB; a
  // request's last 64-key tile may reach up to 63 rows past its end
  const uint64_t rowstride = (uint64_t)p->num_heads_kv * kD * (p->dtype == FP_F32 ? 4 : p->dtype == FP_BF16 ? 2 : 1);
  const uint64_t kv_span =
      (uint64_t)(p->page_table ? std::max<int64_t>(p->num_pool_slots, 1) : max_len + kTile) * rowstride;
  if (kv_span >= 0xfffff000ull)
    return fail(FP_ERR_UNSUPPORTED, "K/V span of %llu bytes per head exceeds the 4 GiB addressing range",
                (unsigned long long)kv_span);
  if (p->page_table) {
    if (p->page_size < 1) return fail(FP_ERR_INVALID_ARG, "page_size must be >= 1");
    if ((int64_t)p->max_pages_per_req * p->page_size < max_len)
      return fail(FP_ERR_INVALID_ARG, "max_pages_per_req * page_size (%lld) < longest request (%lld)",
                  (long long)p->max_pages_per_req * p->page_size, (long long)max_len);
    if (p->num_pool_slots < 1) return fail(FP_ERR_INVALID_ARG, "num_pool_slots must be >= 1");
  }
  if (p->v_layout == FP_V_COLS) {
    if (p->page_table && (p->page_size % kTile || p->num_pool_slots % p->page_size))
      return fail(FP_ERR_UNSUPPORTED, "column-major paged V needs a page size that is a multiple of %d and "
                  "num_pool_slots a multiple of it", kTile);
    // a head's transposed values are addressed through one 32-bit buffer range
    if (!p->page_table && (uint64_t)kD * (uint64_t)hg->total_kv >= 0xfffff000ull)
      return fail(FP_ERR_UNSUPPORTED, "column-major V of %lld rows exceeds the 4 GiB addressing range",
                  (long long)hg->total_kv);
    // 16-byte pieces of a transposed row are loaded whole: rows start 16-aligned
    if (!p->page_table) {
      for (int b = 0; b <= p->num_reqs; ++b)
        if (ckv[b] % 16)
          return fail(FP_ERR_UNSUPPORTED, "contiguous column-major V needs every K/V offset to be a "
                      "multiple of 16 (offset %d of request %d)", ckv[b], b);
    }
  }
  return FP_OK;
}

fp_status validate_params(const fp_select_params* sp) {
  if (!sp) return fail(FP_ERR_INVALID_ARG, "select params are NULL");
  if (!(std::isfinite(sp->alpha) && sp->alpha >= 0.f))
    return fail(FP_ERR_INVALID_ARG, "alpha must be finite and >= 0");
  if (sp->block_size != kBlock) return fail(FP_ERR_UNSUPPORTED, "block_size must be %d", kBlock);
  if (sp->sink_blocks < 0 || sp->window_blocks < 0)
    return fail(FP_ERR_INVALID_ARG, "sink_blocks and window_blocks must be >= 0");
  return FP_OK;
}

int elem_size(int dtype) { return dtype == FP_F32 ? 4 : (dtype == FP_BF16 ? 2 : 1); }

MeansLayout means_layout(const fp_problem* p, const HostGeo& hg) {
  MeansLayout m{};
  const size_t rows = (size_t)hg.nb_pad * p->num_heads_kv * kD;
  size_t o = 0;
  m.kbar32 = o; o = align256(o + rows * 4);
  m.vbar32 = o; o = align256(o + rows * 4);
  m.khi = o; o = align256(o + rows * 2);
  m.klo = o; o = align256(o + rows * 2);
  m.kop = o; o = align256(o + rows * elem_size(p->dtype));
  m.vop = o; o = align256(o + rows * elem_size(p->dtype));
  m.klo8 = o; o = align256(o + (p->dtype == FP_E4M3 ? rows : 0));
  m.kbnd = o; o = align256(o + (size_t)hg.nb_pad * p->num_heads_kv * 4);
  m.knrm = o; o = align256(o + (size_t)hg.nb_pad * p->num_heads_kv * 4);
  m.total = o;
  return m;
}

std::mutex g_dev_mu;
std::vector<int> g_cu_count;

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_cu_count.size() <= dev) g_cu_count.resize(dev + 1, 0);
  if (!g_cu_count[dev]) {
    hipDeviceProp_t prop;
    g_cu_count[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess ? prop.multiProcessorCount : 256;
  }
  return g_cu_count[dev];
}

SplitPolicy split_policy(const fp_problem* p, const HostGeo& hg) {
  SplitPolicy sp;
  const int64_t slots = (int64_t)device_cus() * attn_wgs_per_cu(p->dtype);
  int64_t u = hg.n_seg > 0 ? (4 * slots + hg.n_seg - 1) / hg.n_seg : 1;
  sp.umax = (int32_t)std::max<int64_t>(1, std::min<int64_t>(16, u));
  sp.min_split = 4;
  // FP_MAX_SPLITS caps the split count of a segment (1 disables KV splitting)
  if (const char* e = std::getenv("FP_MAX_SPLITS")) {
    const int cap = std::atoi(e);
    if (cap >= 1) sp.umax = std::min<int32_t>(sp.umax, std::min(cap, 16));
  }
  return sp;
}

// with_select: the selection bitmasks of fp_select (the attention calls never
// touch them, so a layout for attention alone leaves them out).
WsLayout ws_layout(const fp_problem* p, const HostGeo& hg, const SplitPolicy& sp, bool with_select = true) {
  WsLayout w{};
  size_t o = 0;
  w.umax = sp.umax;
  w.hdr = o; o = align256(o + sizeof(WsHeader));
  w.seg_off = o; o = align256(o + (size_t)(p->num_reqs + 1) * 4);
  w.blk_base = o; o = align256(o + (size_t)(p->num_reqs + 1) * 4);
  w.counts = o; o = align256(o + (size_t)hg.n_seg * 4);
  w.scan_part = o; o = align256(o + (size_t)((hg.n_seg + 1023) / 1024 + 1) * 4);
  w.bits = o; o = align256(o + (with_select ? (size_t)hg.n_seg * hg.words * 4 : 0));
  w.redo = o; o = align256(o + (with_select ? (size_t)hg.n_seg * 4 : 0));
  w.work = o; o = align256(o + (size_t)hg.n_seg * 4);
  w.wscan = o; o = align256(o + (size_t)(hg.n_seg + 1) * 4);
  w.uscan = o; o = align256(o + (size_t)(hg.n_seg + 1) * 4);
  w.units = o; o = align256(o + (size_t)hg.n_seg * sp.umax * sizeof(UnitRec));
  w.part_o = o; o = align256(o + (sp.umax > 1 ? (size_t)hg.n_seg * sp.umax * kRows * kD * 4 : 0));
  w.part_ml = o; o = align256(o + (sp.umax > 1 ? (size_t)hg.n_seg * sp.umax * 2 * kRows * 4 : 0));
  w.total = o;
  return w;
}

Geo make_geo(const fp_problem* p, const HostGeo& hg, char* ws, const WsLayout& wl) {
  Geo g{};
  g.cu_q = p->cu_seqlens_q;
  g.cu_kv = p->cu_seqlens_kv ? p->cu_seqlens_kv : p->cu_seqlens_q;
  g.page_table = p->page_table;
  g.num_slots = p->page_table ? p->num_pool_slots : 0;
  g.page_size = p->page_table ? p->page_size : 1;
  g.max_pages = p->page_table ? p->max_pages_per_req : 0;
  g.nreq = p->num_reqs;
  g.hq = p->num_heads_q;
  g.hkv = p->num_heads_kv;
  g.g = hg.g;
  g.log2g = hg.log2g;
  g.dtype = p->dtype;
  g.descale = p->descale;
  g.vcols = p->v_layout == FP_V_COLS ? 1 : 0;
  g.vrow = p->page_table ? p->page_size : hg.total_kv;
  g.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.f / std::sqrt((float)p->head_dim);
  g.max_nj = hg.max_nj;
  g.words = hg.words;
  g.n_seg = hg.n_seg;
  g.nb_pad = hg.nb_pad;
  g.hdr = (WsHeader*)(ws + wl.hdr);
  g.seg_off = (int32_t*)(ws + wl.seg_off);
  g.blk_base = (int32_t*)(ws + wl.blk_base);
  return g;
}

#define FP_LAUNCH(call)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) return fail(FP_ERR_LAUNCH, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

struct Prepared {
  HostGeo hg;
  MeansLayout ml;
  SplitPolicy sp;
  WsLayout wl;
  Geo g;
};

fp_status prepare(const fp_problem* p, void* ws, size_t ws_bytes, Prepared* pr) {
  fp_status s = validate_problem(p, &pr->hg);
  if (s != FP_OK) return s;
  pr->ml = means_layout(p, pr->hg);
  pr->sp = split_policy(p, pr->hg);
  pr->wl = ws_layout(p, pr->hg, pr->sp);
  if (!ws) return fail(FP_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < pr->wl.total)
    return fail(FP_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, pr->wl.total);
  pr->g = make_geo(p, pr->hg, (char*)ws, pr->wl);
  return FP_OK;
}

}  // namespace

extern "C" {

const char* fp_last_error(void) { return g_last_error.c_str(); }

const char* fp_status_string(fp_status s) {
  switch (s) {
    case FP_OK: return "ok";
    case FP_ERR_INVALID_ARG: return "invalid argument";
    case FP_ERR_UNSUPPORTED: return "unsupported";
    case FP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FP_ERR_CAPACITY_TOO_SMALL: return "idx capacity too small";
    case FP_ERR_LAUNCH: return "kernel launch failed";
    case FP_ERR_DEVICE: return "device reported malformed input";
  }
  return "unknown status";
}

fp_status fp_query_sizes(const fp_problem* prob, const fp_select_params* params, fp_sizes* out) {
  if (!out) return fail(FP_ERR_INVALID_ARG, "out is NULL");
  HostGeo hg;
  fp_status s = validate_problem(prob, &hg);
  if (s != FP_OK) return s;
  if (params && (s = validate_params(params)) != FP_OK) return s;
  const SplitPolicy sp = split_policy(prob, hg);
  out->n_segments = hg.n_seg;
  out->idx_capacity = hg.idx_cap;
  out->means_bytes = means_layout(prob, hg).total;
  out->workspace_bytes = ws_layout(prob, hg, sp).total;
  out->max_blocks = hg.max_nj;
  return FP_OK;
}

int64_t fp_block_base(const fp_problem* prob, int32_t b) {
  if (!prob || !prob->cu_seqlens_q_host || b < 0 || b >= prob->num_reqs) return -1;
  const int32_t* ckv = prob->cu_seqlens_kv_host ? prob->cu_seqlens_kv_host : prob->cu_seqlens_q_host;
  int64_t base = 0;
  for (int i = 0; i < b; ++i) {
    int64_t L = (int64_t)ckv[i + 1] - ckv[i];
    base += ((L + kBlock - 1) / kBlock + kChunk - 1) / kChunk * kChunk;
  }
  return base;
}

fp_status fp_pool(const fp_problem* prob, const void* k, const void* v, void* means, void* ws, size_t ws_bytes,
                  void* stream) {
  Prepared pr;
  fp_status s = prepare(prob, ws, ws_bytes, &pr);
  if (s != FP_OK) return s;
  if (!k || !v || !means) return fail(FP_ERR_INVALID_ARG, "k, v and means are required");
  if (pr.hg.total_kv == 0) return FP_OK;
  hipStream_t st = (hipStream_t)stream;
  FP_LAUNCH(launch_meta(pr.g, st));
  FP_LAUNCH(launch_pool(pr.g, pr.ml, k, v, (char*)means, st));
  return FP_OK;
}

fp_status fp_select(const fp_problem* prob, const fp_select_params* params, const void* q, const void* k,
                    const void* v, int32_t* cu, int32_t* idx, int64_t idx_capacity, void* means,
                    float* energies, void* ws, size_t ws_bytes, void* stream) {
  Prepared pr;
  fp_status s = prepare(prob, ws, ws_bytes, &pr);
  if (s != FP_OK) return s;
  if ((s = validate_params(params)) != FP_OK) return s;
  if (!q || !k || !v || !cu || !idx || !means)
    return fail(FP_ERR_INVALID_ARG, "q, k, v, cu, idx and means are required");
  if (idx_capacity < pr.hg.idx_cap)
    return fail(FP_ERR_CAPACITY_TOO_SMALL, "idx holds %lld entries, needs %lld", (long long)idx_capacity,
                (long long)pr.hg.idx_cap);
  if (pr.hg.total == 0) return FP_OK;
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  int32_t* counts = (int32_t*)(wsb + pr.wl.counts);
  uint32_t* bits = (uint32_t*)(wsb + pr.wl.bits);
  FP_LAUNCH(launch_meta(pr.g, st));
  FP_LAUNCH(launch_pool(pr.g, pr.ml, k, v, (char*)means, st));
  FP_LAUNCH(launch_score_select(pr.g, pr.ml, q, (const char*)means, params->alpha, params->sink_blocks,
                                params->window_blocks, counts, bits, energies, (int32_t*)(wsb + pr.wl.redo), st));
  FP_LAUNCH(launch_scan(counts, pr.hg.n_seg, cu, (int32_t*)(wsb + pr.wl.scan_part), st));
  FP_LAUNCH(launch_expand(pr.g, cu, bits, idx, idx_capacity, st));
  return FP_OK;
}

// The attention launch sequence on a prepared problem.  Every workspace word
// it reads is written earlier in the same sequence (metadata, scheduler sums,
// counters, unit list), so the workspace needs no clearing between calls.
static fp_status launch_attention(const fp_problem* prob, Prepared& pr, const void* q, const void* k, const void* v,
                                  const int32_t* cu, const int32_t* idx, const void* means, int dense,
                                  int correction, void* out, float* lse, void* ws, void* stream) {
  if (pr.hg.total == 0) return FP_OK;
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const int grid = device_cus() * attn_wgs_per_cu(prob->dtype);
  FP_LAUNCH(launch_meta(pr.g, st));
  FP_LAUNCH(launch_sched(pr.g, pr.wl, wsb, cu, dense, correction, pr.sp, st));
  FP_LAUNCH(launch_attn(pr.g, pr.wl, wsb, pr.ml, q, k, v, cu, idx, (const char*)means, dense, correction, out,
                        lse, grid, st));
  if (pr.sp.umax > 1) FP_LAUNCH(launch_combine(pr.g, pr.wl, wsb, out, lse, st));
  return FP_OK;
}

static fp_status run_attn(const fp_problem* prob, const void* q, const void* k, const void* v, const int32_t* cu,
                          const int32_t* idx, const void* means, int dense, int correction, void* out,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  Prepared pr;
  fp_status s = prepare(prob, ws, ws_bytes, &pr);
  if (s != FP_OK) return s;
  if (!q || !k || !v || !out) return fail(FP_ERR_INVALID_ARG, "q, k, v and out are required");
  if (!dense && (!cu || !idx || !means)) return fail(FP_ERR_INVALID_ARG, "cu, idx and means are required");
  return launch_attention(prob, pr, q, k, v, cu, idx, means, dense, correction, out, lse, ws, stream);
}

// ---- scratch of the no-allocation entry point ----------------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the device
// address that hipGetSymbolAddress returns for the current device, taken once
// per device and kept in the table below.
constexpr size_t kStaticScratchBytes = FP_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static std::vector<void*> g_scratch_ptr;  // per device: scratch's address there, or null until first use

static fp_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(FP_ERR_LAUNCH, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FP_ERR_LAUNCH, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FP_OK;
}

fp_status fp_sparse_attn(const fp_problem* prob, const fp_select_params* params, const void* q, const void* k,
                         const void* v, const int32_t* cu, const int32_t* idx, const void* means,
                         int32_t mean_correction, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  fp_status s = validate_params(params);
  if (s != FP_OK) return s;
  return run_attn(prob, q, k, v, cu, idx, means, 0, mean_correction ? 1 : 0, out, lse, ws, ws_bytes, stream);
}

fp_status fp_sparse_attn_static(const fp_problem* prob, const fp_select_params* params, const void* q,
                                const void* k, const void* v, const int32_t* cu, const int32_t* idx,
                                const void* means, int32_t mean_correction, void* out, float* lse, void* stream) {
  fp_status s = validate_params(params);
  if (s != FP_OK) return s;
  Prepared pr;
  if ((s = validate_problem(prob, &pr.hg)) != FP_OK) return s;
  if (!q || !k || !v || !out || !cu || !idx || !means)
    return fail(FP_ERR_INVALID_ARG, "q, k, v, out, cu, idx and means are required");
  pr.ml = means_layout(prob, pr.hg);
  pr.sp.umax = 1;  // no KV splitting: no split partials in the scratch
  pr.sp.min_split = 4;
  pr.wl = ws_layout(prob, pr.hg, pr.sp, /*with_select=*/false);
  if (pr.wl.total > kStaticScratchBytes)
    return fail(FP_ERR_WORKSPACE_TOO_SMALL, "this problem needs %zu bytes of scratch; the static scratch holds %zu",
                pr.wl.total, kStaticScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != FP_OK) return s;
  pr.g = make_geo(prob, pr.hg, (char*)ws, pr.wl);
  return launch_attention(prob, pr, q, k, v, cu, idx, means, 0, mean_correction ? 1 : 0, out, lse, ws, stream);
}

fp_status fp_dense_attn(const fp_problem* prob, const void* q, const void* k, const void* v, void* out,
                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  return run_attn(prob, q, k, v, nullptr, nullptr, nullptr, 1, 0, out, lse, ws, ws_bytes, stream);
}

fp_status fp_block_mass(const fp_problem* prob, const void* q, const void* k, const float* lse,
                        const void* means, float* mass, float* surrogate, void* ws, size_t ws_bytes,
                        void* stream) {
  Prepared pr;
  fp_status s = prepare(prob, ws, ws_bytes, &pr);
  if (s != FP_OK) return s;
  if (!q || !k || !lse || !mass) return fail(FP_ERR_INVALID_ARG, "q, k, lse and mass are required");
  if (surrogate && !means) return fail(FP_ERR_INVALID_ARG, "the surrogate needs the pooled means");
  if (pr.hg.total == 0) return FP_OK;
  hipStream_t st = (hipStream_t)stream;
  FP_LAUNCH(launch_meta(pr.g, st));
  FP_LAUNCH(launch_block_mass(pr.g, pr.ml, q, k, lse, (const char*)means, mass, surrogate, st));
  return FP_OK;
}

fp_status fp_read_device_error(void* ws, void* stream, int32_t* flag) {
  if (!ws || !flag) return fail(FP_ERR_INVALID_ARG, "ws and flag are required");
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return fail(FP_ERR_LAUNCH, "stream synchronisation failed");
  int32_t f = 0;
  if (hipMemcpy(&f, ws, sizeof f, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(FP_ERR_LAUNCH, "reading the error flag failed");
  const int32_t zero = 0;
  if (hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
    return fail(FP_ERR_LAUNCH, "clearing the error flag failed");
  *flag = f;
  if (f) return fail(FP_ERR_DEVICE, "device flagged malformed input (bits 0x%x)", f);
  return FP_OK;
}

}  // extern "C"
