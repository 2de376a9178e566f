// fp_internal.h -- types and launchers shared by the HIP translation units of
// libfp.so.  Nothing here is part of the public ABI (include/fp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp {

// Fixed geometry of the method ([V2] §3.3 implementation details, §4.1):
// head dimension 128, selection block 128 tokens, physical key tile 64 tokens,
// query tile 128 packed rows.
constexpr int kD = 128;
constexpr int kBlock = 128;
constexpr int kTile = 64;
constexpr int kRows = 128;
constexpr int kChunk = 64;        // blocks per correction chunk / padding unit of the means
constexpr int kMaxBlocks = 8192;  // longest request: 8192 blocks = 1,048,576 tokens
constexpr int kXcds = 8;          // accelerator dies of an MI355X, each with its own L2

enum Dtype : int32_t { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

// Device error flag bits (workspace header word 0).
constexpr int32_t kErrPage = 1;
constexpr int32_t kErrIdx = 2;

// Workspace header words.
struct WsHeader {
  int32_t err;
  int32_t total_units;
  int32_t xcd_start[kXcds];    // first unit of each XCD's range (the next range's start ends it)
  int32_t redo;                // segments the hi-only scoring left for full precision
  int32_t pad[32 - 3 - kXcds];
  // units taken from each XCD's range, one 128-byte line apiece: atomics on
  // one line are serialised by the memory-side atomic unit
  int32_t xcd_counter[kXcds][32];
};

// Everything a kernel needs to walk the batch.  Passed by value.
struct Geo {
  const int32_t* cu_q;        // [nreq+1] query rows
  const int32_t* cu_kv;       // [nreq+1] key/value offsets (== cu_q for a fresh prefill)
  const int32_t* page_table;  // nullable
  int64_t num_slots;
  int32_t page_size;
  int32_t max_pages;
  int32_t nreq, hq, hkv, g, log2g;
  int32_t dtype;
  const float* descale;       // [3] for E4M3
  int32_t vcols;              // V stored transposed (E4M3): a head's values are rows of vrow bytes
  int64_t vrow;               // bytes from one dim's row of V^T to the next (total_kv, or page size)
  float scale;                // sigma
  int32_t max_nj;             // largest candidate-block count of a segment
  int32_t words;              // selection bitmask words per segment
  int64_t n_seg;
  int64_t nb_pad;             // padded block count of the means arrays
  // workspace views
  WsHeader* hdr;
  int32_t* seg_off;           // [nreq+1] first segment of each request
  int32_t* blk_base;          // [nreq+1] first (padded) block of each request
};

// Layout of the pooled-statistics buffer (byte offsets).
struct MeansLayout {
  size_t kbar32, vbar32;  // float [nb_pad][hkv][128]
  size_t khi, klo;        // bf16 hi + lo of kbar * sl (sl: sigma log2 e, times c_q for E4M3),
                          // MFMA B-operand order: [nb_pad/32][hkv][8][64][8]
  size_t kop, vop;        // element dtype, [nb_pad][hkv][128]: operands of correction steps
  size_t klo8;            // E4M3 only, [nb_pad][hkv][128]: kbar/c_k - kop, times 16, as E4M3
  size_t kbnd;            // float [nb_pad][hkv]: |lo|_2 over the dims (bounds the lo products)
  size_t knrm;            // float [nb_pad][hkv]: |hi|_2 over the dims (scoring's per-block reference)
  size_t total;
};

// One attention work unit as the scheduler writes it: everything a unit needs
// to start, in one 64-byte record (a single load instead of a chain of
// dependent lookups of segment offsets and CSR bounds).
struct UnitRec {
  int32_t s;          // segment
  int32_t split_ns;   // split | nsplit << 16
  int32_t seg0, T;    // CSR offset and listed tile count (sparse)
  int32_t b, h, I;    // request, kv head, query tile
  int32_t L, Lq, off; // key length, query length, first query position
  int32_t row0, kv0;  // first Q row, first K/V row (contiguous)
  int32_t blk_base;   // first (padded) block of the request
  int32_t pad[3];
};

// Layout of the workspace (byte offsets).
struct WsLayout {
  size_t hdr, seg_off, blk_base, counts, scan_part, bits, redo, work, wscan, uscan, units, part_o, part_ml, total;
  int32_t umax;           // largest split count of one segment
};

struct SplitPolicy {
  int32_t umax;
  int32_t min_split;      // fewest iterations a split unit gets
};

// --- launchers (each returns hipSuccess or the launch error) ---
hipError_t launch_meta(const Geo& g, hipStream_t st);
hipError_t launch_pool(const Geo& g, const MeansLayout& ml, const void* k, const void* v,
                       char* means, hipStream_t st);
hipError_t launch_score_select(const Geo& g, const MeansLayout& ml, const void* q, const char* means,
                               float alpha, int sink, int win, int32_t* counts, uint32_t* bits,
                               float* energies, int32_t* redo, hipStream_t st);
hipError_t launch_scan(const int32_t* counts, int64_t n, int32_t* cu, int32_t* part, hipStream_t st);
hipError_t launch_expand(const Geo& g, const int32_t* cu, const uint32_t* bits, int32_t* idx,
                         int64_t cap, hipStream_t st);
hipError_t launch_sched(const Geo& g, const WsLayout& wl, char* ws, const int32_t* cu,
                        int dense, int correction, const SplitPolicy& sp, hipStream_t st);
hipError_t launch_attn(const Geo& g, const WsLayout& wl, char* ws, const MeansLayout& ml,
                       const void* q, const void* k, const void* v, const int32_t* cu,
                       const int32_t* idx, const char* means, int dense, int correction,
                       void* out, float* lse, int grid, hipStream_t st);
hipError_t launch_block_mass(const Geo& g, const MeansLayout& ml, const void* q, const void* k,
                             const float* lse, const char* means, float* mass, float* sur, hipStream_t st);
hipError_t launch_combine(const Geo& g, const WsLayout& wl, char* ws, void* out, float* lse,
                          hipStream_t st);

int attn_wgs_per_cu(int dtype);

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per
// (kernel, device); safe to call from several host threads.
hipError_t set_lds_limit(const void* fn, int bytes);

}  // namespace fp
