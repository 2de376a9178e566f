// sched.hip -- work list of the persistent attention kernel.
//
// [V2] §3.3 "Sparsity-Aware Load Balancing": the cost of a query tile is its
// step count W = T (listed tiles) + C (mean-correction chunks); splits are
// always admitted, each split getting an equal share of the steps by count
// (Eq. 18), and work is issued heaviest first.  Here the split count of a
// segment is U = min(Umax, ceil(W / min_split)), with Umax chosen on the host
// from the segment count and the machine's workgroup slots, and the units are
// placed in descending order of their step count with a bucketed counting
// sort (device-side histogram, descending exclusive scan, atomic scatter).
// The order inside a bucket is unspecified; outputs do not depend on it
// because every unit computes the same thing wherever it runs and splits are
// merged in split order.
#include "device_common.h"

namespace fp {

__device__ __forceinline__ void seg_work(const Geo& g, const int32_t* cu, int64_t s, int dense,
                                         int correction, const SplitPolicy& sp, int& U, int& key) {
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  int W;
  if (dense) {
    W = t.t1 / kTile + 1;
  } else {
    int T = cu[s + 1] - cu[s];
    T = max(0, min(T, 2 * (t.beta + 1)));
    W = T + (correction ? (t.beta + kChunk - 1) / kChunk : 0);
  }
  U = min(sp.umax, max(1, (W + sp.min_split - 1) / sp.min_split));
  const int per = (W + U - 1) / U;
  key = min(per, kBuckets - 1);
}

__global__ __launch_bounds__(256) void sched_zero_kernel(int32_t* hist) {
  for (int i = threadIdx.x + blockIdx.x * 256; i < kBuckets; i += 256 * gridDim.x) hist[i] = 0;
}

// Lanes of a wave that share a bucket are served by one atomic: the lowest
// such lane adds their total, and each lane gets its own offset from a
// masked prefix sum.  Returns the lane's base (scatter) or 0 (count).
__device__ __forceinline__ int bucket_add(int32_t* ctr, bool active, int key, int amount) {
  int base_out = 0;
  uint64_t pending = __ballot(active);
  const int lane = threadIdx.x & 63;
  while (pending) {
    const int leader = __ffsll((long long)pending) - 1;
    const int lkey = __shfl(key, leader, 64);
    const bool mine = active && key == lkey && ((pending >> lane) & 1ull);
    const int contrib = mine ? amount : 0;
    const int incl = wave_incl_scan(contrib);
    const int total = __shfl(incl, 63, 64);
    int base = 0;
    if (lane == leader) base = atomicAdd(&ctr[lkey], total);
    base = __shfl(base, leader, 64);
    if (mine) base_out = base + incl - contrib;
    pending &= ~__ballot(mine);
  }
  return base_out;
}

__global__ __launch_bounds__(256) void sched_count_kernel(Geo g, const int32_t* __restrict__ cu, int dense,
                                                          int correction, SplitPolicy sp, int32_t* hist,
                                                          int32_t* nsplit) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool active = s < g.n_seg;
  int U = 0, key = 0;
  if (active) {
    seg_work(g, cu, s, dense, correction, sp, U, key);
    nsplit[s] = U;
  }
  bucket_add(hist, active, key, U);
}

// Descending exclusive scan of the bucket histogram (one workgroup).
__global__ __launch_bounds__(1024) void sched_scan_kernel(Geo g, const int32_t* __restrict__ hist,
                                                          int32_t* cursor) {
  __shared__ int32_t part[1024];
  constexpr int per = kBuckets / 1024;
  const int tid = threadIdx.x;
  // thread tid owns buckets (in descending key order) tid*per .. tid*per+per-1
  int loc = 0;
  for (int i = 0; i < per; ++i) loc += hist[kBuckets - 1 - (tid * per + i)];
  part[tid] = loc;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int a = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += a;
    __syncthreads();
  }
  int run = part[tid] - loc;
  for (int i = 0; i < per; ++i) {
    const int key = kBuckets - 1 - (tid * per + i);
    cursor[key] = run;
    run += hist[key];
  }
  if (tid == 1023) {
    g.hdr->total_units = part[1023];
    g.hdr->work_counter = 0;
  }
}

__global__ __launch_bounds__(256) void sched_scatter_kernel(Geo g, const int32_t* __restrict__ cu, int dense,
                                                            int correction, SplitPolicy sp, int32_t* cursor,
                                                            int2* units) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool active = s < g.n_seg;
  int U = 0, key = 0;
  if (active) seg_work(g, cu, s, dense, correction, sp, U, key);
  const int base = bucket_add(cursor, active, key, U);
  if (active)
    for (int u = 0; u < U; ++u) units[base + u] = make_int2((int)s, u | (U << 16));
}

hipError_t launch_sched(const Geo& g, const WsLayout& wl, char* ws, const int32_t* cu, int dense,
                        int correction, const SplitPolicy& sp, hipStream_t st) {
  int32_t* hist = (int32_t*)(ws + wl.hist);
  int32_t* cursor = (int32_t*)(ws + wl.cursor);
  int32_t* nsplit = (int32_t*)(ws + wl.counts);
  int2* units = (int2*)(ws + wl.units);
  const unsigned nb = (unsigned)((g.n_seg + 255) / 256);
  sched_zero_kernel<<<kBuckets / 256, 256, 0, st>>>(hist);
  sched_count_kernel<<<nb, 256, 0, st>>>(g, cu, dense, correction, sp, hist, nsplit);
  sched_scan_kernel<<<1, 1024, 0, st>>>(g, hist, cursor);
  sched_scatter_kernel<<<nb, 256, 0, st>>>(g, cu, dense, correction, sp, cursor, units);
  return hipGetLastError();
}

}  // namespace fp
