// sched.hip -- work list of the persistent attention kernel.
//
// [V2] §3.3 "Sparsity-Aware Load Balancing": the cost of a query tile is its
// step count W = T (listed tiles) + C (mean-correction chunks); splits are
// always admitted, each split getting an equal share of the steps by count
// (Eq. 18).
//
// MI355X layout.  Each of the 8 XCDs has its own L2, and neighbouring query
// tiles of one KV head share most of their key tiles (sink, window, diagonal,
// the same clusters).  The segment list (ordered request, KV head, tile) is
// therefore cut into 8 contiguous ranges of equal total work, range x served
// by the workgroups of XCD x (workgroups are dispatched to XCDs round-robin by
// id) through that XCD's atomic counter, each range walked from its end:
// later tiles carry more candidate blocks and correction chunks, so this is
// close to heaviest-first while the tiles in flight on one XCD stay
// neighbours.  A workgroup whose range is exhausted takes units from the
// other ranges.  Units of a segment with U splits
// are contiguous; outputs do not depend on which workgroup runs a unit
// (splits are merged in split order).
#include "device_common.h"

namespace fp {

__device__ __forceinline__ void seg_work(const Geo& g, const int32_t* cu, int64_t s, int dense,
                                         int correction, const SplitPolicy& sp, int& U, int& W) {
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  if (dense) {
    W = t.t1 / kTile + 1;
  } else {
    int T = cu[s + 1] - cu[s];
    T = max(0, min(T, 2 * (t.beta1 + 1)));
    W = T + (correction ? (t.beta + kChunk - 1) / kChunk : 0);
  }
  W = max(W, 1);
  U = min(sp.umax, max(1, (W + sp.min_split - 1) / sp.min_split));
}

__global__ __launch_bounds__(256) void sched_count_kernel(Geo g, const int32_t* __restrict__ cu, int dense,
                                                          int correction, SplitPolicy sp, int32_t* work,
                                                          int32_t* nsplit) {
  const int64_t s = (int64_t)block_x() * 256 + thread_x();
  if (s >= g.n_seg) return;
  int U, W;
  seg_work(g, cu, s, dense, correction, sp, U, W);
  nsplit[s] = U;
  work[s] = W;
}

// wscan / uscan: exclusive prefix sums of work and split counts ([n_seg + 1]).
__global__ __launch_bounds__(256) void sched_place_kernel(Geo g, const int32_t* __restrict__ wscan,
                                                          const int32_t* __restrict__ uscan,
                                                          const int32_t* __restrict__ nsplit,
                                                          const int32_t* __restrict__ cu, UnitRec* units) {
  const int64_t s = (int64_t)block_x() * 256 + thread_x();
  const int64_t n = g.n_seg;
  const int64_t wtot = max(1, wscan[n]);
  if (block_x() == 0 && thread_x() < kXcds) g.hdr->xcd_counter[thread_x()][0] = 0;
  if (s == 0) g.hdr->total_units = uscan[n];
  if (s >= n) return;
  const int x = (int)min<int64_t>(kXcds - 1, (int64_t)wscan[s] * kXcds / wtot);
  const int xp = s > 0 ? (int)min<int64_t>(kXcds - 1, (int64_t)wscan[s - 1] * kXcds / wtot) : -1;
  // the first segment of range x (and of every empty range before it) opens it
  for (int y = xp + 1; y <= x; ++y) g.hdr->xcd_start[y] = uscan[s];
  // ranges after the last segment's are empty
  if (s == n - 1)
    for (int y = x + 1; y < kXcds; ++y) g.hdr->xcd_start[y] = uscan[n];
  const int U = nsplit[s];
  const int base = uscan[s];
  const SegCoord c = seg_coord(g, s);
  UnitRec r{};
  r.s = (int32_t)s;
  r.seg0 = cu ? cu[s] : 0;
  r.T = cu ? cu[s + 1] - cu[s] : 0;
  r.b = c.b;
  r.h = c.h;
  r.I = (int32_t)c.I;
  r.L = c.L;
  r.Lq = c.Lq;
  r.off = c.off;
  r.row0 = (int32_t)c.row0;
  r.kv0 = (int32_t)c.kv0;
  r.blk_base = g.blk_base[c.b];
  for (int u = 0; u < U; ++u) {
    r.split_ns = u | (U << 16);
    units[base + u] = r;
  }
}

hipError_t launch_sched(const Geo& g, const WsLayout& wl, char* ws, const int32_t* cu, int dense,
                        int correction, const SplitPolicy& sp, hipStream_t st) {
  int32_t* nsplit = (int32_t*)(ws + wl.counts);
  int32_t* work = (int32_t*)(ws + wl.work);
  int32_t* wscan = (int32_t*)(ws + wl.wscan);
  int32_t* uscan = (int32_t*)(ws + wl.uscan);
  int32_t* part = (int32_t*)(ws + wl.scan_part);
  UnitRec* units = (UnitRec*)(ws + wl.units);
  const unsigned nb = (unsigned)((g.n_seg + 255) / 256);
  sched_count_kernel<<<nb, 256, 0, st>>>(g, cu, dense, correction, sp, work, nsplit);
  hipError_t e = launch_scan(work, g.n_seg, wscan, part, st);
  if (e != hipSuccess) return e;
  e = launch_scan(nsplit, g.n_seg, uscan, part, st);
  if (e != hipSuccess) return e;
  sched_place_kernel<<<nb, 256, 0, st>>>(g, wscan, uscan, nsplit, dense ? nullptr : cu, units);
  return hipGetLastError();
}

}  // namespace fp
