// attn.hip -- attention stage: persistent MFMA flash attention over the CSR
// index with mean-correction steps, the dense causal baseline on the same
// mainloop, and the combine of KV splits.
//
// Method ([V2] §3.2 Eq. 6, §3.3): for each query tile (128 PackGQA rows of one
// KV head, Eq. 12-13) the listed 64-key tiles are visited backwards
// (n_t = idx[cu + T - 1 - t], Eq. 17) with an online softmax; every block
// J < beta that no listed tile covers is then folded in as one extra step
// whose "keys" are pooled means: logit sigma q.kbar_J + ln 128, value
// vbar_J ([V2] §3.2 "Implementation"), 64 blocks per step, blocks that are
// selected or not fully visible masked out.  Under KV splitting a unit takes
// the contiguous count range [u ceil(W/U), (u+1) ceil(W/U)) of its W steps
// (Eq. 18) and partial results are merged by log-sum-exp in split order.
//
// MI355X mapping.  A workgroup is 4 waves x 32 query rows.  Logits are
// computed transposed, S^T = K Q^T (A = K tile from LDS, B = the wave's Q rows
// held in registers), so each lane owns one query row: row max and row sum
// are in-lane plus one exchange with lane^32, and the probabilities land in
// exactly the register layout of the B operand of O^T += V^T P^T.  K and V
// tiles travel HBM -> LDS by buffer DMA (bf16, e4m3; through the page table,
// [V2] Eq. 22, per tile or per row) into double-buffered LDS, one or two
// steps ahead; V^T operands are read with the LDS transpose loads (or, for a
// V stored transposed, directly).  fp32 stages K/V through registers.  bf16
// runs a software pipeline across steps (the softmax of one step in pieces
// between the MFMAs of its neighbours); e4m3 and fp32 take one step at a
// time.  The persistent grid takes its work units from a list that the
// scheduler cuts into work-balanced ranges, one per XCD, each served through
// an atomic counter of its own.  bf16: v_mfma_f32_32x32x16_bf16; e4m3:
// v_mfma_scale_f32_32x32x64_f8f6f4 with P quantised as e4m3(2^8 e^{s-m})
// ([V2] Eq. 15); fp32: v_mfma_f32_32x32x2f32.
#include "device_common.h"

namespace fp {

template <int DT>
struct Tr;
template <>
struct Tr<kBF16> {
  static constexpr int KPL = 8;  // contraction elements per lane per MFMA
  static constexpr int EB = 2;
  using Op = bf16x8;
};
template <>
struct Tr<kE4M3> {
  static constexpr int KPL = 32;
  static constexpr int EB = 1;
  using Op = i32x8;
};
template <>
struct Tr<kF32> {
  static constexpr int KPL = 1;
  static constexpr int EB = 4;
  using Op = float;
};

// One MFMA operand (KPL elements) from LDS, read in 16-byte pieces.
template <int DT>
__device__ __forceinline__ typename Tr<DT>::Op lds_op(const char* p) {
  if constexpr (DT == kBF16) {
    return __builtin_bit_cast(bf16x8, *(const uint4*)p);
  } else if constexpr (DT == kE4M3) {
    uint4 a = ((const uint4*)p)[0], b = ((const uint4*)p)[1];
    i32x8 r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
  } else {
    return *(const float*)p;
  }
}

// e4m3 with the A operand scaled by 2^-4 (E8M0 exponent 123): the lo part of
// the pooled keys, stored 16 times larger than it stands for
__device__ __forceinline__ f32x16 mma_lo8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 123, 0, 127);
}

template <int DT>
__device__ __forceinline__ f32x16 mma(typename Tr<DT>::Op a, typename Tr<DT>::Op b, f32x16 c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else if constexpr (DT == kE4M3)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  else
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// bf16 staging of the pipelined mainloop: rows padded instead of swizzled, so
// that every MFMA operand address is a per-lane base plus an immediate.
// K rows take 272 bytes (17 slots of 16 B: the 16-lane passes of the
// 128-bit operand reads, rows r..r+15 at one chunk, fall on distinct bank
// groups), V rows 320 bytes (20 slots: the 4 rows x 64 bytes that a pass of
// transpose reads touches fall on disjoint banks).  A DMA instruction fills
// 64 consecutive slots; the lane of a pad slot fetches a duplicate chunk.
struct PipeL {
  static constexpr int KSL = 17, VSL = 20;            // 16-byte slots per K / V row
  static constexpr int KP = 16 * KSL, VP = 16 * VSL;  // row pitches (bytes)
  static constexpr int KB = 64 * KP, VB = 64 * VP;    // one staged tile
  static constexpr int NK = 64 * KSL / 64, NV = 64 * VSL / 64;  // DMA instructions per tile
  static constexpr int V0 = 0, V1 = VB, K0 = 2 * VB, K1 = 2 * VB + KB;
  static constexpr int PEN = 2 * VB + 2 * KB;         // three 256-byte correction-offset tables
  static constexpr int SEL = PEN + 3 * 256;
  static constexpr int LDS = SEL + (kMaxBlocks / 32 + 8) * 4;
};

template <int DT>
struct Cfg {
  static constexpr int EB = Tr<DT>::EB;
  static constexpr int KPL = Tr<DT>::KPL;
  // bf16 / e4m3: K and V rows go HBM -> LDS by DMA, unpadded with XOR-swizzled
  // 16-byte chunks; V stays row-major and is read transposed.  fp32: rows are
  // staged through registers, V is written transposed, rows are padded.
  static constexpr bool DMA = DT != kF32;
  static constexpr int ROWB = kD * EB;                         // bytes of one K/V row
  static constexpr int KPITCH = DMA ? ROWB : ROWB + 16;        // bytes per staged K row
  static constexpr int VPITCH = DMA ? ROWB : kTile * EB + 16;  // V row (DMA) or V^T row (fp32)
  static constexpr int KBYTES = kTile * KPITCH;
  static constexpr int VBYTES = DMA ? kTile * VPITCH : kD * VPITCH;
  static constexpr int PENBYTES = 2 * 32 * 4;    // correction-step logit offsets, per lane half
  // e4m3: the lo part of the pooled keys of a correction step (k rows again)
  static constexpr int LOOFF = KBYTES + VBYTES + PENBYTES;
  static constexpr int STAGE = LOOFF + (DT == kE4M3 ? KBYTES : 0);
  // e4m3 pipelined loop: three rotating correction-offset tables after the stages
  static constexpr int PEN3 = 2 * STAGE;
  static constexpr int SELOFF = DT == kBF16 ? PipeL::SEL : DT == kE4M3 ? PEN3 + 3 * 256 : 2 * STAGE;  // selection bitmask
  static constexpr int LDS = DT == kBF16 ? PipeL::LDS : SELOFF + (kMaxBlocks / 32 + 8) * 4;
  static constexpr int NM0 = kD / (2 * KPL);     // MFMAs per 32x32 logit tile
  static constexpr int NM1 = kTile / (2 * KPL);  // MFMAs per 32-column output tile
  static constexpr int WGS = DT == kF32 ? 1 : 2; // workgroups per CU
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows written by one 1 KB DMA instruction
  static constexpr int NDMA = kTile / RPI / 4;   // DMA instructions per wave per K (or V) tile
};

// e4m3 staging: XOR swizzles of the 16-byte chunks of a 128-byte row, chosen
// so that the MFMA operand reads hit distinct LDS banks: K rows are read 16
// rows at a time at two chunks; V rows are read by the transpose loads 8 rows
// at a time at one or two chunks.
template <int DT>
__device__ __forceinline__ int swz_k(int r) {
  return (r >> 1) & 7;
}
template <int DT>
__device__ __forceinline__ int swz_v(int r) {
  return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from a buffer resource straight into LDS at lds + 16 * lane
// (lds is wave-uniform; it goes to M0).  Issued as inline assembly: for the
// load builtin the compiler cannot tell one LDS stage from the other, and it
// then waits for every DMA in flight before the next LDS read, which is the
// read of the stage being computed while the other one fills.  The DMA's
// completion is made explicit instead: every stage is published by wait_vmem()
// and a barrier before any wave reads it.
// The LDS address is a 32-bit integer: a generic pointer cast to LDS costs a
// 64-bit add and a null test per DMA.  The paged layouts keep the builtin: the
// compiler may hold their resources in vector registers, which the builtin
// turns into scalar operands and the assembly form cannot take.
template <bool ASM>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  if constexpr (ASM) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(uintptr_t)m0, 16, (int)voff, 0, 0, 0);
  }
}
// Transpose reads (see the operand builders below for the lane layout).
__device__ __forceinline__ i16x4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}
__device__ __forceinline__ i32x2 lds_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}
// A wave-uniform read of read-only data through the constant address space,
// so that it is a scalar load: a vector load would share the vector-memory
// counter with the LDS DMA in flight, and waiting for it would wait for them.
__device__ __forceinline__ int32_t scalar_read(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}
// Position of the r-th (from 0) set bit of m; r < popcount(m).
__device__ __forceinline__ int nth_set_bit(uint64_t m, int r) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __builtin_popcountll(m & ((1ull << w) - 1));
    if (r >= c) {
      r -= c;
      m >>= w;
      pos += w;
    }
  }
  return pos;
}
// Wait for this wave's outstanding vector-memory loads (including LDS DMA).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Instruction-group ordering hints for the scheduler (one ordered chain per
// block): a group of n instructions of the given class.
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgDsRead = 0x100;
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// x of this lane and of lane ^ 32 (the lane in the other half that holds
// the same query row), by one v_permlane32_swap instead of an LDS permute.
__device__ __forceinline__ float2 with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0]: lanes 0-31 keep their x, lanes 32-63 get x of lane - 32; r[1]: lanes
  // 0-31 get x of lane + 32, lanes 32-63 keep theirs
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_halves(float x) {
  const float2 p = with_other_half(x);
  return fmaxf(p.x, p.y);
}

// An MFMA accumulator held in place: the MFMA that produced it issues before
// this point and nothing moves it past (the asm reads and rewrites it).
__device__ __forceinline__ void hold(f32x16& x) { asm volatile("" : "+v"(x)); }

// An empty use of a register value: it must be computed before this point.
template <typename V>
__device__ __forceinline__ void pin(const V& x) {
  if constexpr (sizeof(V) == 4) {
    asm volatile("" ::"v"(x));
  } else if constexpr (sizeof(V) == 16) {
    const uint4 w = __builtin_bit_cast(uint4, x);
    asm volatile("" ::"v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w));
  }
}

// Position in a staged V^T row of key j (0..63) of the tile: keys are laid
// out in the order in which each lane half holds the probabilities of the
// two 32x32 logit tiles (key = 32 jt + 8 (r/4) + 4 half + r%4 for register r).
template <int KPL>
__device__ __forceinline__ int vt_pos(int j) {
  int jt = j >> 5, jj = j & 31;
  int half = (jj >> 2) & 1;
  int r = ((jj >> 3) << 2) | (jj & 3);
  int id = jt * 16 + r;
  return (id / KPL) * (2 * KPL) + half * KPL + (id % KPL);
}

// 8 consecutive elements (raw storage) of one K/V/mean row.
template <int DT>
struct Vec8 {
  static constexpr int W = 8 * Tr<DT>::EB / 4;  // dwords
  uint32_t w[W];
};

template <int DT>
__device__ __forceinline__ void ld8(Vec8<DT>& o, const char* p) {
  if constexpr (DT == kBF16) {
    uint4 a = *(const uint4*)p;
    o.w[0] = a.x; o.w[1] = a.y; o.w[2] = a.z; o.w[3] = a.w;
  } else if constexpr (DT == kE4M3) {
    uint2 a = *(const uint2*)p;
    o.w[0] = a.x; o.w[1] = a.y;
  } else {
    uint4 a = ((const uint4*)p)[0], b = ((const uint4*)p)[1];
    o.w[0] = a.x; o.w[1] = a.y; o.w[2] = a.z; o.w[3] = a.w;
    o.w[4] = b.x; o.w[5] = b.y; o.w[6] = b.z; o.w[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ void zero8(Vec8<DT>& o) {
#pragma unroll
  for (int i = 0; i < Vec8<DT>::W; ++i) o.w[i] = 0;
}

// element e (0..7) of a Vec8 as raw bits
template <int DT>
__device__ __forceinline__ uint32_t el(const Vec8<DT>& o, int e) {
  if constexpr (DT == kBF16)
    return (o.w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
  else if constexpr (DT == kE4M3)
    return (o.w[e >> 2] >> (8 * (e & 3))) & 0xffu;
  else
    return o.w[e];
}

struct Unit {
  int64_t s;
  int split, nsplit;
};

// K/V addressing modes of the attention kernel.
enum AddrMode : int {
  kContig = 0,    // K/V rows follow Q rows; one buffer resource per (request, kv head)
  kPagedTile = 1, // page size a multiple of 64: a 64-key tile lies inside one page
  kPagedAny = 2,  // any page size: one page-table lookup per key row ([V2] Eq. 22)
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufFlags = 0x00020000;  // raw dword buffer, range-checked

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0xffffffffull ? (int)0xffffffffu : (int)(uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufFlags);
}

// 8 consecutive elements of one K/V/mean row through a buffer resource
// (out-of-range offsets read as zero).
template <int DT>
__device__ __forceinline__ void bld8(Vec8<DT>& o, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (DT == kBF16) {
    u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    o.w[0] = a[0]; o.w[1] = a[1]; o.w[2] = a[2]; o.w[3] = a[3];
  } else if constexpr (DT == kE4M3) {
    u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    o.w[0] = a[0]; o.w[1] = a[1];
  } else {
    u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff + 16, (int)soff, 0);
    o.w[0] = a[0]; o.w[1] = a[1]; o.w[2] = a[2]; o.w[3] = a[3];
    o.w[4] = b[0]; o.w[5] = b[1]; o.w[6] = b[2]; o.w[7] = b[3];
  }
}

// Byte offset of token j's vector in the paged pool (one lookup, [V2] Eq. 22);
// an entry outside the pool sets kErrPage and reads slot 0.
__device__ __forceinline__ uint32_t paged_off(const Geo& g, const SegCoord& c, int j, uint32_t rowstride,
                                              uint32_t& err) {
  const int pg = j / g.page_size;
  const int64_t page = g.page_table[(int64_t)c.b * g.max_pages + pg];
  const int64_t slot = page * g.page_size + (j - pg * g.page_size);
  const bool ok = page >= 0 && slot < g.num_slots;
  err |= ok ? 0u : (uint32_t)kErrPage;
  return (uint32_t)(ok ? slot : 0) * rowstride;
}

constexpr uint32_t kNaN32 = 0x7fc00000u;
constexpr uint32_t kNaNbf16x2 = 0x7fc07fc0u;

template <int DT, bool DENSE, int AM, bool VC = false>
__global__ __launch_bounds__(256, Cfg<DT>::WGS) void attn_kernel(
    Geo g, WsLayout wl, char* __restrict__ ws, MeansLayout ml, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ idx, const char* __restrict__ means, int correction,
    void* __restrict__ out, float* __restrict__ lse, int nwg) {
  using C = Cfg<DT>;
  using Op = typename Tr<DT>::Op;
  constexpr int KPL = C::KPL;
  constexpr int EB = C::EB;
  extern __shared__ __align__(16) char smem[];
  // LDS address of smem, and the DMA of 16 bytes per lane to p + 16 * lane
  // for a pointer p into smem
  // (held opaque: otherwise the cast's null test is redone at every use)
  uint32_t sb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)smem);
  asm volatile("" : "+s"(sb));
  auto dma = [&](__amdgpu_buffer_rsrc_t r, const char* p, uint32_t voff) __attribute__((always_inline)) {
    dma16<AM == kContig>(r, sb + (uint32_t)(p - smem), voff);
  };
  uint32_t* selbits = (uint32_t*)(smem + C::SELOFF);

  // the wave index is uniform: in a scalar register, addresses derived from it
  // (LDS DMA destinations) need no per-instruction readfirstlane
  const int tid = thread_x(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // this wave's LDS base of the DMA destinations: the bf16 tiles' 1 KB pieces
  // wave + 4 i, the e4m3 tiles' rows 16 wave + ...; then a stage offset and an
  // immediate per DMA (held opaque, like sb)
  uint32_t sb_w1k = sb + (uint32_t)wave * 1024u, sb_wrow = sb + (uint32_t)(16 * wave * C::ROWB);
  asm volatile("" : "+s"(sb_w1k), "+s"(sb_wrow));
  const int half = lane >> 5, col = lane & 31;
  const UnitRec* units = (const UnitRec*)(ws + wl.units);
  // logits in log2 units: x = s * sl (+ 7 for a mean that stands for 128 keys)
  const float sl = g.scale * 1.4426950408889634f *
                   (DT == kE4M3 ? g.descale[0] * g.descale[1] : 1.f);
  const float cvs = DT == kE4M3 ? g.descale[2] : 1.f;
  constexpr float kOff = DT == kE4M3 ? 8.f : 0.f;  // e4m3: P scaled onto [0, 256] (Eq. 15)
  const uint32_t rowstride = (uint32_t)g.hkv * kD * EB;  // bytes from one token to the next

  // staging assignment: K rows kr + 16 i, columns kc..kc+7 (16 lanes per row);
  // V key quad vq (keys 4vq..4vq+3), columns vc..vc+7 (16 lanes per V^T row)
  const int kr = tid >> 4, kc = (tid & 15) * 8;
  const int vq = tid & 15, vc = (tid >> 4) * 8;
  const int vpos = vt_pos<KPL>(4 * vq);
  uint32_t voff_k[4], voff_v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    voff_k[i] = (uint32_t)(kr + 16 * i) * rowstride + kc * EB;
    voff_v[i] = (uint32_t)(4 * vq + i) * rowstride + vc * EB;
  }

  // bf16: per-lane byte offsets (within a 64-row tile of K or V rows) of the
  // DMA instructions q = wave + 4 i: lane L fills slot 64 q + L of the padded
  // tile, i.e. row (64 q + L) / slots-per-row, chunk (64 q + L) % slots-per-row
  // (a pad slot repeats chunk 15 of its row)
  uint32_t pdk[5], pdv[5];
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int sk = 64 * (wave + 4 * i) + lane, sv = sk;
      const int rk = sk / PipeL::KSL, ck = min(sk - rk * PipeL::KSL, 15);
      const int rv = sv / PipeL::VSL, cv = min(sv - rv * PipeL::VSL, 15);
      pdk[i] = (uint32_t)rk * rowstride + (uint32_t)ck * 16;
      pdv[i] = (uint32_t)rv * rowstride + (uint32_t)cv * 16;
    }
  }
  // bf16 operand addresses relative to a staged tile: K row jt*32 + col, chunk
  // 2 m + half; V^T rows for the transpose reads (see the operand builders)
  const int k16 = lane & 15, g16 = (lane >> 4) & 1;
  const int lane_k = col * PipeL::KP + half * 16;
  const int lane_v = (4 * half + (k16 >> 2)) * PipeL::VP + (16 * g16 + 4 * (k16 & 3)) * 2;

  // Units come from the own XCD's range (workgroups are dispatched to XCDs
  // round-robin by id), walked from its end through that range's counter;
  // once it is exhausted, from the other ranges.  The atomic for the next unit
  // is issued when a unit starts and its result is first needed when the
  // unit ends, so its latency hides behind the unit's loads.
  const int nx = nwg % kXcds == 0 ? kXcds : 1;  // nwg: the grid's workgroup count
  const int xcd = block_x() % nx;
  auto range_of = [&](int x, int& lo, int& hi) {
    lo = nx == kXcds ? g.hdr->xcd_start[x] : 0;
    hi = nx == kXcds && x + 1 < kXcds ? g.hdr->xcd_start[x + 1] : g.hdr->total_units;
  };
  // the next unit from ranges x0, x0 + 1, ... (mod nx), given the own range's ticket
  auto steal = [&](int x0) -> int {
    for (int a = 0; a < nx; ++a) {
      const int x = (x0 + a) % nx;
      int lo, hi;
      range_of(x, lo, hi);
      if (hi <= lo || atomicAdd(&g.hdr->xcd_counter[x][0], 0) >= hi - lo) continue;
      const int kk = atomicAdd(&g.hdr->xcd_counter[x][0], 1);
      if (kk < hi - lo) return hi - 1 - kk;
    }
    return -1;
  };
  int own_lo, own_hi;
  range_of(xcd, own_lo, own_hi);
  __shared__ int sh_unit;
  __shared__ int bad_w[4];  // per wave: some lane of the unit saw malformed input
  if (tid == 0) {
    const int kk = atomicAdd(&g.hdr->xcd_counter[xcd][0], 1);
    sh_unit = kk < own_hi - own_lo ? own_hi - 1 - kk : steal(xcd + 1);
  }
  __syncthreads();
  for (;;) {
    // the unit id is wave-uniform; saying so keeps every value derived from it
    // (segment geometry, base addresses, buffer resources) in scalar registers
    const int u = __builtin_amdgcn_readfirstlane(sh_unit);
    if (u < 0) break;
    int ticket = 0;
    if (tid == 0) ticket = atomicAdd(&g.hdr->xcd_counter[xcd][0], 1);
    const UnitRec ur = units[u];
    const Unit un{ur.s, ur.split_ns & 0xffff, ur.split_ns >> 16};
    SegCoord c;
    c.b = ur.b;
    c.h = ur.h;
    c.I = ur.I;
    c.L = ur.L;
    c.Lq = ur.Lq;
    c.off = ur.off;
    c.row0 = ur.row0;
    c.kv0 = ur.kv0;
    const TileGeo t = tile_geo(g, c);
    uint32_t err = 0;
    int T, seg0 = 0;
    if constexpr (DENSE) {
      T = t.t1 / kTile + 1;
    } else {
      seg0 = ur.seg0;
      T = ur.T;
      if (T < 0 || T > 2 * (t.beta1 + 1)) {
        err |= kErrIdx;
        T = 0;
      }
    }
    const int NC = (!DENSE && correction) ? (t.beta + kChunk - 1) / kChunk : 0;
    const int W = T + NC;
    const int per = (W + un.nsplit - 1) / un.nsplit;
    const int it0 = min(W, un.split * per), it1 = min(W, it0 + per);

    // K/V and pooled-means base addresses of this unit.  Each step builds its
    // buffer resources from base + step offset with the remaining bytes as the
    // range (the range check covers the per-lane offset only), so keys past the
    // end of the request read as zero in the contiguous layout.
    const char* kbase;
    const char* vbase;
    uint64_t kvbytes;
    if constexpr (AM == kContig) {
      const uint64_t base = ((uint64_t)c.kv0 * g.hkv + c.h) * kD * EB;
      kbase = (const char*)k + base;
      vbase = (const char*)v + base;
      kvbytes = c.L > 0 ? (uint64_t)(c.L - 1) * rowstride + kD * EB : 0;
    } else {
      const uint64_t base = (uint64_t)c.h * kD * EB;
      kbase = (const char*)k + base;
      vbase = (const char*)v + base;
      kvbytes = (uint64_t)(g.num_slots - 1) * rowstride + kD * EB;
    }
    const uint64_t mbase = ((uint64_t)ur.blk_base * g.hkv + c.h) * kD * EB;
    const char* kmbase = means + ml.kop + mbase;
    const char* vmbase = means + ml.vop + mbase;
    const char* klmbase = means + ml.klo8 + mbase;  // e4m3 only
    // transposed V (e4m3): this head's dim rows, and the transposed correction
    // operands ([chunk][head][dim][64 blocks]) of the request's first chunk
    const char* vtbase = (const char*)v + (AM == kContig ? (uint64_t)c.h * kD * g.vrow + c.kv0 : 0);
    const char* vtmbase = means + ml.vop + (uint64_t)((ur.blk_base >> 6) * g.hkv + c.h) * kD * kChunk;
    const uint64_t mbytes = (uint64_t)(((t.beta + kChunk - 1) / kChunk) * kChunk) * rowstride;
    // One buffer resource per operand for the whole unit: the request's K and V
    // rows of this head (contiguous layout) and its pooled means.  A step adds
    // its first row's offset to the per-lane offsets; rows of a tile past the
    // request's last row fall outside the range and read as zero.
    const __amdgpu_buffer_rsrc_t rk_t = make_rsrc(kbase, kvbytes), rv_t = make_rsrc(vbase, kvbytes);
    const __amdgpu_buffer_rsrc_t rk_m = make_rsrc(kmbase, mbytes), rv_m = make_rsrc(vmbase, mbytes);
    const __amdgpu_buffer_rsrc_t rl_m = make_rsrc(klmbase, mbytes);
    const uint32_t tile_bytes = (uint32_t)kTile * rowstride;  // kChunk == kTile rows

    if (NC > 0) {
      for (int w = tid; w <= (t.beta >> 5) + 2; w += 256) selbits[w] = 0;
      __syncthreads();
      for (int e = tid; e < T; e += 256) {
        const int J = idx[seg0 + e] >> 1;
        if (J >= 0 && J < t.beta) atomicOr(&selbits[J >> 5], 1u << (J & 31));
      }
    }
    __syncthreads();
    // correction chunks with work (a visible block that is not listed): one
    // bit per chunk, chunks 0-63 and 64-127 (beta <= 8192 blocks)
    uint64_t todo_lo = 0, todo_hi = 0;
    if (NC > 0) {
      auto chunk_has_work = [&](int ch) -> bool {
        if (ch >= NC) return false;
        const int n = min(kChunk, t.beta - ch * kChunk);
        const uint32_t m0 = n >= 32 ? 0xffffffffu : (1u << n) - 1u;
        const uint32_t m1 = n >= 64 ? 0xffffffffu : n <= 32 ? 0u : (1u << (n - 32)) - 1u;
        return ((~selbits[2 * ch] & m0) | (~selbits[2 * ch + 1] & m1)) != 0u;
      };
      todo_lo = __ballot(chunk_has_work(lane));
      todo_hi = __ballot(chunk_has_work(lane + 64));
    }

    // ---- the wave's 32 query rows: B operand of S^T = K Q^T, kept in registers
    const int row_in_tile = wave * 32 + col;
    const bool row_ok = row_in_tile < t.nrows;
    const int64_t prow = c.I * kRows + row_in_tile;
    const int qi = (int)(prow >> g.log2g);  // query index within the request
    const int pos = c.off + qi;             // its position (causal mask)
    const int head = c.h * g.g + (int)(prow & (g.g - 1));
    const int64_t qrow = (c.row0 + qi) * g.hq + head;
    Op qf[C::NM0];
#pragma unroll
    for (int m = 0; m < C::NM0; ++m) {
      const int d0 = m * 2 * KPL + half * KPL;
      const char* src = (const char*)q + (qrow * kD + d0) * EB;
      if constexpr (DT == kBF16) {
        uint4 w = row_ok ? *(const uint4*)src : make_uint4(0, 0, 0, 0);
        qf[m] = __builtin_bit_cast(bf16x8, w);
      } else if constexpr (DT == kE4M3) {
        i32x8 w = {};
        if (row_ok) {
          uint4 a = ((const uint4*)src)[0], b = ((const uint4*)src)[1];
          w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
          w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        }
        qf[m] = w;
      } else {
        qf[m] = row_ok ? *(const float*)src : 0.f;
      }
    }

    float m_i = -INFINITY, l_i = 0.f;
    f32x16 oacc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) oacc[nt] = f32x16{};

    // ---- steps: listed tiles backwards (Eq. 17), then the correction chunks
    // that have work.  The unit's steps are handed out in order from a window
    // of 64 held one per lane: lane j of w_it is the step index of the
    // (wb + j)-th step and lane j of w_p its listed tile (0 for a chunk); past
    // the unit's last step the index is it1.  Each wave fills its window
    // itself when the previous one is used up, and checks the listed tiles
    // there: descending (the list is strictly ascending) and inside the rows'
    // visible keys; a split also checks the entry its predecessor saw last.
    const int nt = max(0, min(it1, T) - it0);         // tile steps of the unit
    const int c_lo = max(it0, T) - T, c_hi = it1 - T;  // its chunk range
    uint64_t cm_lo = 0, cm_hi = 0;                     // chunks with work in it
    if (NC > 0) {
      cm_lo = __ballot(((todo_lo >> lane) & 1) && lane >= c_lo && lane < c_hi);
      cm_hi = __ballot(((todo_hi >> lane) & 1) && lane + 64 >= c_lo && lane + 64 < c_hi);
    }
    const int n1 = __builtin_popcountll(cm_lo);
    const int nsteps = nt + n1 + __builtin_popcountll(cm_hi);
    int prev_tile = 1 << 30;
    if constexpr (!DENSE) {
      if (it0 > 0 && it0 < T) prev_tile = idx[seg0 + T - it0];
    }
    int w_it = it1, w_p = 0, wb = -64, rd = 0;
    auto fill = [&]() {
      wb += 64;
      const int k = wb + lane;
      int e_it = it1, e_p = 0;
      if (k < nt) {
        e_it = it0 + k;
        if constexpr (DENSE) {
          e_p = T - 1 - e_it;
        } else {
          e_p = idx[seg0 + T - 1 - e_it];
        }
      } else if (k < nsteps) {
        // the chunk of rank r among those with work is step nt + r
        const int r = k - nt;
        e_it = T + (r < n1 ? nth_set_bit(cm_lo, r) : 64 + nth_set_bit(cm_hi, r - n1));
      }
      if constexpr (!DENSE) {
        const int before = __builtin_amdgcn_ds_bpermute(((lane + 63) & 63) * 4, e_p);
        const bool bad = k < nt && (e_p < 0 || (int64_t)e_p * kTile > t.t1 || e_p >= (lane == 0 ? prev_tile : before));
        if (__ballot(bad)) err |= kErrIdx;
        prev_tile = __builtin_amdgcn_readlane(e_p, 63);
        if (bad) e_p = 0;
      }
      w_it = e_it;
      w_p = e_p;
    };
    auto pop = [&](int& it, int& p) __attribute__((always_inline)) {
      if (rd - wb == 64) fill();
      it = __builtin_amdgcn_readlane(w_it, rd - wb);
      p = __builtin_amdgcn_readlane(w_p, rd - wb);
      ++rd;
    };

    // One-step paths (e4m3, fp32): output rescaling is deferred until a row's
    // max exceeds the max that its accumulators are scaled to by more than
    // 2^kTau (fp32: exact up to rounding, probabilities stay below 2^8).  e4m3
    // quantises P against the running max itself (Eq. 15), so there kTau is 0.
    // The bf16 pipeline below keeps its own reference maximum.
    constexpr float kTau = DT == kE4M3 ? 0.f : 8.f;
    bool fresh = true;  // nothing accumulated yet: the first max needs no rescale

    if constexpr (DT == kBF16) {
      // ---- bf16 mainloop, software-pipelined across steps.
      // MFMA groups of step n: A(n), B(n) = S^T of keys 0-31 / 32-63 (K(n)
      // operands), C(n), D(n) = O^T += V^T P^T for keys 0-31 / 32-63 (V(n)).
      // Iteration n issues D(n-1), B(n), C(n), A(n+1), 32 MFMA slots; the
      // softmax of keys 0-31 of step n runs in small pieces under D(n-1) and
      // B(n), that of keys 32-63 under C(n) and A(n+1), a few VALU
      // instructions per MFMA.  One barrier per iteration, between B(n) and
      // C(n): K(n+1) and V(n) (loaded one iteration earlier) become visible,
      // K(n+2) and V(n+1) are loaded.  K tiles alternate between two buffers
      // by step parity, V tiles likewise, correction offsets rotate through
      // three tables.  The first iteration's D(-1) multiplies V(0) by P = 0
      // (adding exact zeros); the last iteration's A(n+1) is computed
      // on stale data and not used.
      using PL = PipeL;
      auto kread = [&](const char* kb, int jt, int m) -> Op {
        return __builtin_bit_cast(bf16x8, *(const uint4*)(kb + jt * 32 * PL::KP + m * 32));
      };
      // keys 16 m1 + 4 half + 0..3 and +8 of V^T row nt*32 + lane%32
      auto vread = [&](const char* vb, int nt, int m1) -> Op {
        const i16x4 x = lds_tr16(vb + m1 * 16 * PL::VP + nt * 64);
        const i16x4 y = lds_tr16(vb + m1 * 16 * PL::VP + 8 * PL::VP + nt * 64);
        const i16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        return __builtin_bit_cast(bf16x8, z);
      };
      // DMA of the K (ISK) or V tile of step it into LDS at lds_off
      auto dma_bf16 = [&](auto isk_tag, int lds_off, int it, int p) {
        constexpr bool ISK = decltype(isk_tag)::value;
        constexpr int NQ = ISK ? PL::NK : PL::NV, SPR = ISK ? PL::KSL : PL::VSL;
        const char* base = ISK ? kbase : vbase;
        __amdgpu_buffer_rsrc_t r;
        uint32_t soff = 0;  // the step's first row within r
        bool rows = false;
        int j0 = 0;
        if (it < T) {
          j0 = p * kTile;
          if constexpr (AM == kContig) {
            r = ISK ? rk_t : rv_t;
            soff = (uint32_t)p * tile_bytes;
          } else if constexpr (AM == kPagedTile) {
            const int pg = j0 / g.page_size;
            const int64_t page = scalar_read(g.page_table + (int64_t)c.b * g.max_pages + pg);
            int64_t slot0 = page * g.page_size + (j0 - pg * g.page_size);
            if (page < 0 || slot0 + kTile > g.num_slots) {
              err |= kErrPage;
              slot0 = 0;
            }
            const uint64_t o = (uint64_t)slot0 * rowstride;
            const uint64_t tail = (uint64_t)max(0, c.L - 1 - j0) * rowstride + C::ROWB;
            r = make_rsrc(base + o, min(kvbytes > o ? kvbytes - o : (uint64_t)0, tail));
          } else {
            r = make_rsrc(base, kvbytes);
            rows = true;
          }
        } else {
          // a whole chunk of 64 means rows: the means are padded to full chunks
          // (the paged layouts build the resource per step: joined with their
          // tile resources, the per-unit one is taken for a divergent value and
          // every DMA becomes a loop over the lanes)
          if constexpr (AM == kContig) {
            r = ISK ? rk_m : rv_m;
            soff = (uint32_t)(it - T) * tile_bytes;
          } else {
            r = make_rsrc((ISK ? kmbase : vmbase) + (uint64_t)(it - T) * tile_bytes, mbytes);
          }
        }
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const int q = wave + 4 * i;
          if (i < 4 || q < NQ) {
            uint32_t voff = (ISK ? pdk[i] : pdv[i]) + soff;
            if constexpr (AM == kPagedAny) {
              if (rows) {
                // one page-table lookup per row; rows past the request read as zero
                const int sl = 64 * q + lane, row = sl / SPR, cc = min(sl - row * SPR, 15);
                const int j = j0 + row;
                voff = j < c.L ? paged_off(g, c, j, rowstride, err) + (uint32_t)cc * 16 : 0xfffffff0u;
              }
            }
            dma16<AM == kContig>(r, sb_w1k + (uint32_t)lds_off + 4096u * i, voff);
          }
        }
      };
      // correction offsets of step it (+7 where the block is corrected, -inf
      // where selected or not fully visible) into table ps, by wave 0
      auto pen_bf16 = [&](int ps, int it) {
        if (it >= T && tid < 64) {
          float* pen = (float*)(smem + PL::PEN + ps * 256);
          const int h = tid >> 5, kk = tid & 31;
          const int rho = 32 * (kk >> 4) + 8 * ((kk & 15) >> 2) + 4 * h + (kk & 3);
          const int J = (it - T) * kChunk + rho;
          const bool ok = J < t.beta && !((selbits[J >> 5] >> (J & 31)) & 1u);
          pen[tid] = ok ? 7.f : -INFINITY;
        }
      };

      int cur, cur_tile;
      pop(cur, cur_tile);
      if (cur < it1) {
        int nxt, nxt_tile;
        pop(nxt, nxt_tile);
        int bk = 0, ps = 0;  // parity of step n; its correction table n % 3
        // prologue: K(0), V(0), K(1) staged; A(0)
        dma_bf16(std::true_type{}, PL::K0, cur, cur_tile);
        pen_bf16(0, cur);
        dma_bf16(std::false_type{}, PL::V0, cur, cur_tile);
        if (nxt < it1) {
          dma_bf16(std::true_type{}, PL::K1, nxt, nxt_tile);
          pen_bf16(1, nxt);
        }
        wait_vmem();
        __syncthreads();

        f32x16 s0 = {}, s1 = {};
        Op p0[2], p1[2], ring[4];
        p1[0] = p1[1] = p0[0] = p0[1] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        {
          const char* kb = smem + PL::K0 + lane_k;
#pragma unroll
          for (int m = 0; m < 4; ++m) ring[m] = kread(kb, 0, m);
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const Op a = ring[m & 3];
            if (m + 4 < 8) ring[m & 3] = kread(kb, 0, m + 4);
            s0 = mma<DT>(a, qf[m], s0);
            __builtin_amdgcn_sched_barrier(0);
          }
          // operands of D(-1): V(0), times P = 0
          const char* vb = smem + PL::V0 + lane_v;
#pragma unroll
          for (int g2 = 0; g2 < 4; ++g2) ring[g2] = vread(vb, g2 >> 1, 2 + (g2 & 1));
        }

        // Softmax state.  The weights of a half step are first taken against
        // the reference mref = m_i, which sits kHead (log2 units) above the
        // row's running maximum, with no reduction at all; only when some
        // lane's 16 weights sum above 2^8 (a key more than about kHead + 4 above
        // the maximum, or the first visible key of a row, for which mref is
        // -1e30 so that every finite weight overflows) does the wave take the
        // exact maximum of the half, exchange it between the lane halves, and
        // compute the weights again against that maximum + kHead.  Exact up to
        // rounding: the weights stay within [2^-kHead, 2^8] times their true
        // scale, and the output and LSE use the same reference.  The headroom
        // makes the recomputation (and the rescale of the accumulators) rare
        // when a correction chunk's +7 raises the logits.
        constexpr float kHead = 8.f;
        float mref = -1e30f, resc = 1.f, psum = 0.f;
        bool need = false;
        uint32_t pw[8];  // the half's weights as bf16 pairs
        f32x4 pv[2];     // correction offsets of 8 registers, read one piece ahead
        auto weight = [&](auto kind_tag, float x, float m) -> float {
          constexpr int KIND = decltype(kind_tag)::value;
          return __builtin_amdgcn_exp2f(KIND == 2 ? x + (kOff - m) : fmaf(x, sl, kOff - m));
        };
        auto pack = [](float a, float b) -> uint32_t {
          const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
          return __builtin_bit_cast(uint32_t, v);
        };
        // piece k (0..15) of the softmax of a 32-key half sv (logit tile jt)
        auto sub = [&](auto kind_tag, f32x16& sv, int jt, int k, Op* ph, const f32x4* penp) {
          constexpr int KIND = decltype(kind_tag)::value;
          if (k == 0) {
            if constexpr (KIND == 2) {
              pv[0] = penp[0];
              pv[1] = penp[1];
            }
          } else if (k <= 2) {
            const int r0 = (k - 1) * 8;
            if constexpr (KIND == 0) {
              const int lim = pos - cur_tile * kTile - 4 * half;  // key j visible iff j <= pos - 64 p
#pragma unroll
              for (int r = r0; r < r0 + 8; ++r)
                if (32 * jt + 8 * (r >> 2) + (r & 3) > lim) sv[r] = -INFINITY;
            }
            if constexpr (KIND == 2) {
#pragma unroll
              for (int r = r0; r < r0 + 8; ++r) sv[r] = fmaf(sv[r], sl, pv[(r >> 2) & 1][r & 3]);
              if (k == 1) {
                pv[0] = penp[2];
                pv[1] = penp[3];
              }
            }
#pragma unroll
            for (int r = r0; r < r0 + 8; ++r) pin(sv[r]);
          } else if (k < 14 && k % 3 != 2) {
            // weights 2(k-3) and 2(k-3)+1: bf16 pair and the fp32 row sum
            // (plain adds: they issue beside the MFMAs, bf16 dot products would not)
            const int r = 2 * (k - 3 - (k - 3) / 3);
            const float e0 = weight(kind_tag, sv[r], mref), e1 = weight(kind_tag, sv[r + 1], mref);
            pw[r >> 1] = pack(e0, e1);
            psum = k == 3 ? e0 + e1 : psum + e0 + e1;
            pin(pw[r >> 1]);
            pin(psum);
          } else if (k == 14) {
            need = __any(!(psum <= 256.f));
            resc = 1.f;
            if (need) {
              float mh = sv[0];
#pragma unroll
              for (int r = 1; r < 16; ++r) mh = fmaxf(mh, sv[r]);
              mh = max_halves(mh);  // the other lane half holds the same query row
              const float m_half = KIND == 2 ? mh : mh * sl;  // tile steps hold raw dot products (sl > 0)
              // the new reference sits kHead above the maximum (m_i includes it)
              const float m_new = fmaxf(m_i, m_half + kHead);
              const float m_use = m_new == -INFINITY ? 0.f : m_new;
              resc = __builtin_amdgcn_exp2f(m_i - m_use);
              m_i = m_new;
              mref = m_new == -INFINITY ? -1e30f : m_new;
              psum = 0.f;
#pragma unroll
              for (int r = 0; r < 16; r += 2) {
                const float e0 = weight(kind_tag, sv[r], m_use), e1 = weight(kind_tag, sv[r + 1], m_use);
                pw[r >> 1] = pack(e0, e1);
                psum += e0 + e1;
              }
            }
            ph[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            ph[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
            pin(ph[0]);
            pin(ph[1]);
            pin(psum);
          }
        };
        auto commit = [&]() {
          l_i = fmaf(l_i, resc, psum);
          if (need && !fresh) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[nt][r] *= resc;
          }
          fresh = false;
        };

        int first = 1;
        auto iter = [&](auto kind_tag) {
          const char* kbc = smem + (bk ? PL::K1 : PL::K0) + lane_k;  // K(n)
          const char* kbn = smem + (bk ? PL::K0 : PL::K1) + lane_k;  // K(n+1)
          const char* vbc = smem + (bk ? PL::V1 : PL::V0) + lane_v;  // V(n)
          const char* vbp = smem + ((bk | first) ? PL::V0 : PL::V1) + lane_v;  // V(n-1); V(0) for D(-1)
          const f32x4* penp = (const f32x4*)(smem + PL::PEN + ps * 256) + half * 8;
          auto fetch = [&](int gs) -> Op {
            if (gs < 8) return vread(vbp, gs >> 1, 2 + (gs & 1));
            if (gs < 16) return kread(kbc, 1, gs - 8);
            if (gs < 24) return vread(vbc, (gs - 16) >> 1, (gs - 16) & 1);
            if (gs < 32) return kread(kbn, 0, gs - 24);
            return vread(vbc, (gs - 32) >> 1, 2 + (gs & 1));
          };
          auto mfma_slot = [&](int gs, const Op a) {
            if (gs < 8)
              oacc[gs >> 1] = mma<DT>(a, p1[gs & 1], oacc[gs >> 1]);
            else if (gs < 16)
              s1 = mma<DT>(a, qf[gs - 8], s1);
            else if (gs < 24)
              oacc[(gs - 16) >> 1] = mma<DT>(a, p0[(gs - 16) & 1], oacc[(gs - 16) >> 1]);
            else
              s0 = mma<DT>(a, qf[gs - 24], s0);
          };
          // slots 0-15: D(n-1), B(n); softmax of keys 0-31
          s1 = f32x16{};
#pragma unroll
          for (int gs = 0; gs < 16; ++gs) {
            const Op a = ring[gs & 3];
            if (gs + 4 < 16) ring[gs & 3] = fetch(gs + 4);
            sub(kind_tag, s0, 0, gs, p0, penp);
            mfma_slot(gs, a);
            __builtin_amdgcn_sched_barrier(0);
          }
          commit();
          // K(n+1), V(n) visible; K(n+2), V(n+1) loaded
          wait_vmem();
          __syncthreads();
          int nxt2 = nxt, nxt2_tile = 0;
          if (nxt < it1) pop(nxt2, nxt2_tile);
          if (nxt2 < it1) {
            dma_bf16(std::true_type{}, bk ? PL::K1 : PL::K0, nxt2, nxt2_tile);
            pen_bf16(ps == 0 ? 2 : ps - 1, nxt2);
          }
          if (nxt < it1) dma_bf16(std::false_type{}, bk ? PL::V0 : PL::V1, nxt, nxt_tile);
#pragma unroll
          for (int gs = 16; gs < 20; ++gs) ring[gs & 3] = fetch(gs);
          // slots 16-31: C(n), A(n+1); softmax of keys 32-63
          s0 = f32x16{};
#pragma unroll
          for (int gs = 16; gs < 32; ++gs) {
            const Op a = ring[gs & 3];
            ring[gs & 3] = fetch(gs + 4);
            sub(kind_tag, s1, 1, gs - 16, p1, penp + 4);
            mfma_slot(gs, a);
            __builtin_amdgcn_sched_barrier(0);
          }
          commit();
          bk ^= 1;
          ps = ps == 2 ? 0 : ps + 1;
          first = 0;
          cur = nxt;
          cur_tile = nxt_tile;
          nxt = nxt2;
          nxt_tile = nxt2_tile;
        };
        while (cur < it1 && cur < T && cur_tile * kTile + kTile - 1 > t.t0) iter(std::integral_constant<int, 0>{});
        while (cur < it1 && cur < T) iter(std::integral_constant<int, 1>{});
        if constexpr (!DENSE) {
          while (cur < it1) iter(std::integral_constant<int, 2>{});
        }
        // D of the last step (its V tile has the other parity)
        {
          const char* vb = smem + (bk ? PL::V0 : PL::V1) + lane_v;
#pragma unroll
          for (int gs = 0; gs < 8; ++gs) {
            const Op a = ring[gs & 3];
            if (gs + 4 < 8) ring[gs & 3] = vread(vb, (gs + 4) >> 1, 2 + (gs & 1));
            oacc[gs >> 1] = mma<DT>(a, p1[gs & 1], oacc[gs >> 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
    // e4m3: the denominator of Eq. 15 sums the rounded P; one more MFMA per
    // step with an all-ones A operand forms those sums (every row of the
    // product is the column sum of P^T), in place of decoding P back on the
    // VALU.  Only element 0 is read, so the rescale touches only it.
    f32x16 lacc = f32x16{};
    const Op ones = [] {
      Op o{};
      if constexpr (DT == kE4M3) {
#pragma unroll
        for (int w = 0; w < 8; ++w) o[w] = 0x38383838;  // e4m3 1.0
      }
      return o;
    }();
    // per-lane DMA offsets within a 64-row tile (bf16/e4m3): instruction q of
    // wave w fills rows 16w + RPI q + lane / CPR, chunk lane % CPR, which holds
    // the row's logical chunk (lane % CPR) ^ swizzle(row)
    uint32_t dk[C::NDMA > 0 ? C::NDMA : 1], dv[C::NDMA > 0 ? C::NDMA : 1];
    if constexpr (C::DMA) {
#pragma unroll
      for (int qq = 0; qq < C::NDMA; ++qq) {
        const int r = 16 * wave + C::RPI * qq + lane / C::CPR;
        const int cl = lane % C::CPR;
        dk[qq] = (uint32_t)r * rowstride + (uint32_t)((cl ^ swz_k<DT>(r)) * 16);
        dv[qq] = (uint32_t)r * rowstride + (uint32_t)((cl ^ swz_v<DT>(r)) * 16);
      }
    }
    // transposed V (VC): instruction qq of wave w fills dim rows 16 (2w + qq) ..
    // +15, four 16-byte pieces (keys 16 cs .. +15) per 64-byte row; the piece in
    // slot cl of row r holds logical piece cl ^ ((r >> 2) & 3), so that the
    // operand reads of 16 consecutive rows fall on distinct banks
    uint32_t dvt[2], dvm[2];
    int vt_cs[2];
    if constexpr (VC) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int r = 16 * (2 * wave + qq) + (lane >> 2);
        const int cs = (lane & 3) ^ ((r >> 2) & 3);
        vt_cs[qq] = cs;
        dvt[qq] = (uint32_t)(r * g.vrow + 16 * cs);
        dvm[qq] = (uint32_t)(r * kChunk + 16 * cs);
      }
    }
    // DMA of a transposed V tile (keys j0 .. j0 + 63 of every dim row; pieces
    // starting at or past the request's end read as zero)
    auto dma_vt = [&](int buf, __amdgpu_buffer_rsrc_t rv, int j0, bool means_tile) {
      char* vs = smem + buf * C::STAGE + C::KBYTES;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const uint32_t o = means_tile ? dvm[qq] : (j0 + 16 * vt_cs[qq] < c.L ? dvt[qq] : 0xfffffff0u);
        dma(rv, vs + 16 * (2 * wave + qq) * 64, o);
      }
    };
    Vec8<DT> kst[C::DMA ? 1 : 4], vst[C::DMA ? 1 : 4];

    // DMA of one 64-row K and V tile (rows past the range read as zero)
    auto dma_tile = [&](int buf, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv) {
      char* ks = smem + buf * C::STAGE;
      char* vs = ks + C::KBYTES;
#pragma unroll
      for (int qq = 0; qq < C::NDMA; ++qq) {
        const int r0 = 16 * wave + C::RPI * qq;
        dma(rk, ks + r0 * C::ROWB, dk[qq]);
        if constexpr (!VC) dma(rv, vs + r0 * C::ROWB, dv[qq]);
      }
    };
    // paged, any page size: one page-table lookup per row; rows past the request
    // get an offset outside the range and read as zero
    auto dma_tile_rows = [&](int buf, int j0, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv) {
      char* ks = smem + buf * C::STAGE;
      char* vs = ks + C::KBYTES;
#pragma unroll
      for (int qq = 0; qq < C::NDMA; ++qq) {
        const int r = 16 * wave + C::RPI * qq + lane / C::CPR;
        const int cl = lane % C::CPR;
        const int j = j0 + r;
        uint32_t base = 0xfffffff0u;
        if (j < c.L) base = paged_off(g, c, j, rowstride, err);
        const uint32_t ok = j < c.L ? 0u : 0xfffffff0u;
        const uint32_t ok_k = ok ? ok : base + (uint32_t)((cl ^ swz_k<DT>(r)) * 16);
        const uint32_t ok_v = ok ? ok : base + (uint32_t)((cl ^ swz_v<DT>(r)) * 16);
        const int r0 = 16 * wave + C::RPI * qq;
        dma(rk, ks + r0 * C::ROWB, ok_k);
        dma(rv, vs + r0 * C::ROWB, ok_v);
      }
    };

    auto write_pen = [&](int buf, int it) {
      if (it >= T && tid < 64) {
        // logit offset of each register of a correction step, per lane half:
        // + 7 (ln 128 in log2 units) where the block is corrected, -inf where it is
        // selected or not fully visible to the tile
        float* pen = (float*)(smem + buf * C::STAGE + C::KBYTES + C::VBYTES);
        const int h = tid >> 5, kk = tid & 31;
        const int rho = 32 * (kk >> 4) + 8 * ((kk & 15) >> 2) + 4 * h + (kk & 3);
        const int J = (it - T) * kChunk + rho;
        const bool ok = J < t.beta && !((selbits[J >> 5] >> (J & 31)) & 1u);
        pen[tid] = ok ? 7.f : -INFINITY;
      }
    };

    // issue the loads of step it into stage buf (DMA: straight to LDS)
    auto load_step = [&](int buf, int it, int p) {
      if (it < T) {
        const int j0 = p * kTile;
        if constexpr (AM == kContig) {
          const uint64_t o = (uint64_t)j0 * rowstride;
          const uint64_t left = kvbytes > o ? kvbytes - o : 0;
          const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + o, left), rv = make_rsrc(vbase + o, left);
          if constexpr (VC) {
            // this head's dim rows from key j0 on, up to the end of its last row
            const uint64_t vleft = (uint64_t)kD * g.vrow - (uint64_t)(c.kv0 + j0);
            dma_vt(buf, make_rsrc(vtbase + j0, vleft), j0, false);
          }
          if constexpr (C::DMA) {
            dma_tile(buf, rk, rv);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bld8<DT>(kst[i], rk, voff_k[i], 0);
              bld8<DT>(vst[i], rv, voff_v[i], 0);
            }
          }
        } else if constexpr (AM == kPagedTile) {
          const int pg = j0 / g.page_size;
          const int64_t page = scalar_read(g.page_table + (int64_t)c.b * g.max_pages + pg);
          int64_t slot0 = page * g.page_size + (j0 - pg * g.page_size);
          if (page < 0 || slot0 + kTile > g.num_slots) {
            err |= kErrPage;
            slot0 = 0;
          }
          const uint64_t o = (uint64_t)slot0 * rowstride;
          // rows past the end of the request read as zero: the range stops there
          const uint64_t tail = (uint64_t)max(0, c.L - 1 - j0) * rowstride + C::ROWB;
          const uint64_t left = min(kvbytes > o ? kvbytes - o : (uint64_t)0, tail);
          const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + o, left), rv = make_rsrc(vbase + o, left);
          if constexpr (VC) {
            // page [head][dim][p]: this head's dim rows of the page, from key j0 on
            const int64_t pg0 = slot0 / g.page_size, in_pg = slot0 - pg0 * g.page_size;
            const char* vb = (const char*)v + ((uint64_t)(pg0 * g.hkv + c.h) * kD) * g.page_size + in_pg;
            dma_vt(buf, make_rsrc(vb, (uint64_t)kD * g.page_size - in_pg), j0, false);
          }
          if constexpr (C::DMA) {
            dma_tile(buf, rk, rv);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bld8<DT>(kst[i], rk, voff_k[i], 0);
              bld8<DT>(vst[i], rv, voff_v[i], 0);
            }
          }
        } else {
          const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, kvbytes), rv = make_rsrc(vbase, kvbytes);
          if constexpr (C::DMA) {
            dma_tile_rows(buf, j0, rk, rv);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int jk = min(j0 + kr + 16 * i, c.L - 1);
              const int jv = min(j0 + 4 * vq + i, c.L - 1);
              bld8<DT>(kst[i], rk, paged_off(g, c, jk, rowstride, err) + kc * EB, 0);
              bld8<DT>(vst[i], rv, paged_off(g, c, jv, rowstride, err) + vc * EB, 0);
            }
          }
        }
      } else {
        // pooled means of blocks 64 ch .. 64 ch + 63 (past beta they are masked)
        const uint64_t o = (uint64_t)((it - T) * kChunk) * rowstride;
        const uint64_t left = mbytes > o ? mbytes - o : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kmbase + o, left), rv = make_rsrc(vmbase + o, left);
        if constexpr (VC) {
          const uint64_t mo = (uint64_t)(it - T) * g.hkv * kD * kChunk;
          dma_vt(buf, make_rsrc(vtmbase + mo, (uint64_t)kD * kChunk), 0, true);
        }
        if constexpr (C::DMA) {
          dma_tile(buf, rk, rv);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bld8<DT>(kst[i], rk, voff_k[i], 0);
            bld8<DT>(vst[i], rv, voff_v[i], 0);
          }
        }
        if constexpr (DT == kE4M3) {
          // the pooled keys' lo part, staged like the keys
          const __amdgpu_buffer_rsrc_t rl = make_rsrc(klmbase + o, left);
          char* ls = smem + buf * C::STAGE + C::LOOFF;
#pragma unroll
          for (int qq = 0; qq < C::NDMA; ++qq) dma(rl, ls + (16 * wave + C::RPI * qq) * C::ROWB, dk[qq]);
        }
      }
      if constexpr (C::DMA) write_pen(buf, it);
    };

    // fp32 only: registers -> LDS (K rows padded, V transposed)
    auto store_step = [&](int buf, int it) {
      if constexpr (!C::DMA) {
        char* ks = smem + buf * C::STAGE;
        char* vt = ks + C::KBYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          char* dst = ks + (kr + 16 * i) * C::KPITCH + kc * EB;
          ((uint4*)dst)[0] = make_uint4(kst[i].w[0], kst[i].w[1], kst[i].w[2], kst[i].w[3]);
          ((uint4*)dst)[1] = make_uint4(kst[i].w[4], kst[i].w[5], kst[i].w[6], kst[i].w[7]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          char* rowp = vt + (vc + e) * C::VPITCH;
#pragma unroll
          for (int i = 0; i < 4; ++i) *(uint32_t*)(rowp + vt_pos<KPL>(4 * vq + i) * 4) = el<DT>(vst[i], e);
        }
        write_pen(buf, it);
      }
    };

    // MFMA A operand m of logit tile jt (K rows) from stage buffer ks
    auto k_op = [&](const char* ks, int jt, int m) -> Op {
      const int rr = jt * 32 + col;
      if constexpr (DT == kE4M3) {
        const char* rp = ks + rr * C::ROWB;
        const int c0 = 4 * m + 2 * half, sw = swz_k<DT>(rr);
        const uint4 a = *(const uint4*)(rp + ((c0 ^ sw) << 4));
        const uint4 b = *(const uint4*)(rp + (((c0 + 1) ^ sw) << 4));
        i32x8 r;
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        return r;
      } else {
        return lds_op<DT>(ks + rr * C::KPITCH + half * KPL * EB + m * 2 * KPL * EB);
      }
    };
    // MFMA A operand m1 of output tile nt (V^T) from stage buffer
    auto v_op = [&](const char* vs, int nt, int m1) -> Op {
      if constexpr (VC) {
        // dim row nt*32 + col, keys 32 half .. +31 (logical pieces 2 half, 2 half + 1)
        const int d = nt * 32 + col, sw = (d >> 2) & 3;
        const char* rp = vs + d * 64;
        const uint4 a = *(const uint4*)(rp + (((2 * half) ^ sw) << 4));
        const uint4 b = *(const uint4*)(rp + (((2 * half + 1) ^ sw) << 4));
        i32x8 r;
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        return r;
      } else if constexpr (DT == kE4M3) {
        // 32 keys of column nt*32 + lane%32 in the register order of P: read t
        // (0..3) gives keys 16 t + 8 (i/4) + 4 half + i%4, i = 0..7
        const int k16 = lane & 15;
        const int colb = nt * 32 + 16 * ((lane >> 4) & 1) + 8 * (k16 & 1);
        const int i = k16 >> 1;
        i32x8 r;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int row = 16 * tt + 8 * (i >> 2) + 4 * half + (i & 3);
          const char* a = vs + row * C::ROWB + (((colb >> 4) ^ swz_v<DT>(row)) << 4) + (colb & 15);
          const i32x2 w = lds_tr8(a);
          r[2 * tt] = w[0];
          r[2 * tt + 1] = w[1];
        }
        return r;
      } else {
        return lds_op<DT>(vs + (nt * 32 + col) * C::VPITCH + half * KPL * EB + m1 * 2 * KPL * EB);
      }
    };

    if constexpr (DT == kE4M3 && !VC) {
      // ---- e4m3 mainloop, software-pipelined across steps.
      // Iteration k (step s_k) starts with s_k's logits in S, computed by the
      // previous iteration, and with P(s_{k-1}), the rounded weights of the step
      // before.  It issues the row-sum MFMA and PV(s_{k-1}) (4 MFMAs) with the
      // softmax of s_k in pieces between them, writes P(s_k) once PV(s_{k-1})
      // has read P, applies the (rare) rescale for a raised maximum, and ends
      // with QK(s_{k+1}) into S (4 MFMAs, 8 for a correction chunk: hi and the
      // 2^-4-scaled lo part).  One logit set and one weight set, so the loop
      // body fits the register budget of two waves per SIMD.  Stage par holds
      // K(s_{k+1}) and V(s_{k-1}); the iteration's DMA fills the other stage
      // with K(s_{k+2}) and V(s_k), whose previous contents were last read
      // before the previous barrier.  One barrier per iteration.  Correction
      // offsets rotate through three tables (those of s_k, s_{k+1} and s_{k+2}
      // are live at once).  Eq. 15: the weights of s_k are rounded against the
      // running maximum after s_k's own logits; the rescale follows PV(s_{k-1}),
      // so it covers every step before s_k.
      using OpE = i32x8;
      constexpr int PEN3 = C::PEN3;
      // per-lane LDS byte offsets (from smem) of the operand reads; stage, key
      // tile and key group are immediates on top
      uint32_t ka[4], va[4];
      {
        const int sw = swz_k<DT>(col);  // rows jt*32 + col share it: jt*32 >> 1 has no low 3 bits
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int part = 0; part < 2; ++part)
            ka[2 * m + part] = (uint32_t)(col * C::ROWB + (((4 * m + 2 * half + part) ^ sw) << 4));
        const int k16 = lane & 15;
        const int i = k16 >> 1;
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);  // + 16 tt (immediate)
        const int sv = swz_v<DT>(row);                      // the same for row + 16 tt
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int colb = nt * 32 + 16 * ((lane >> 4) & 1) + 8 * (k16 & 1);
          va[nt] = (uint32_t)(C::KBYTES + row * C::ROWB + (((colb >> 4) ^ sv) << 4) + (colb & 15));
        }
      }
      auto kread8 = [&](int st, int jt, int m, bool lo) __attribute__((always_inline)) -> OpE {
        const char* b = smem + st * C::STAGE + (lo ? C::LOOFF : 0) + jt * 32 * C::ROWB;  // st: 0 or 1
        const uint4 a0 = *(const uint4*)(b + ka[2 * m]);
        const uint4 a1 = *(const uint4*)(b + ka[2 * m + 1]);
        OpE r = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        return r;
      };
      auto vread8 = [&](int st, int nt) __attribute__((always_inline)) -> OpE {
        const char* b = smem + st * C::STAGE + va[nt];
        OpE r;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const i32x2 w = lds_tr8(b + tt * 16 * C::ROWB);
          r[2 * tt] = w[0];
          r[2 * tt + 1] = w[1];
        }
        return r;
      };
      // buffer resource, first-row offset and per-row mode of step it's K, V
      // or K-lo tile: rt for a listed tile (contiguous layout), rm for a chunk
      // of pooled means; the paged layouts build theirs from base
      auto step_src = [&](int it, int p, const char* base, const char* mb, __amdgpu_buffer_rsrc_t rt,
                          __amdgpu_buffer_rsrc_t rm, uint32_t& soff, bool& rows) __attribute__((always_inline))
          -> __amdgpu_buffer_rsrc_t {
        rows = false;
        soff = 0;
        if (it >= T) {
          if constexpr (AM == kContig) {
            soff = (uint32_t)(it - T) * tile_bytes;
            return rm;
          } else {
            // per step for the paged layouts (a join with their tile resources
            // would make the per-unit one divergent for the compiler)
            return make_rsrc(mb + (uint64_t)(it - T) * tile_bytes, mbytes);
          }
        }
        const int j0 = p * kTile;
        if constexpr (AM == kContig) {
          soff = (uint32_t)p * tile_bytes;
          return rt;
        } else if constexpr (AM == kPagedTile) {
          const int pg = j0 / g.page_size;
          const int64_t page = scalar_read(g.page_table + (int64_t)c.b * g.max_pages + pg);
          int64_t slot0 = page * g.page_size + (j0 - pg * g.page_size);
          if (page < 0 || slot0 + kTile > g.num_slots) {
            err |= kErrPage;
            slot0 = 0;
          }
          const uint64_t o = (uint64_t)slot0 * rowstride;
          const uint64_t tail = (uint64_t)max(0, c.L - 1 - j0) * rowstride + C::ROWB;
          return make_rsrc(base + o, min(kvbytes > o ? kvbytes - o : (uint64_t)0, tail));
        } else {
          rows = true;
          return make_rsrc(base, kvbytes);
        }
      };
      // DMA of one 64-row tile (K-side swizzle when isk) into LDS at dst
      auto dma_rows = [&](bool isk, char* dst, __amdgpu_buffer_rsrc_t r, uint32_t soff, bool rows, int j0)
                          __attribute__((always_inline)) {
#pragma unroll
        for (int qq = 0; qq < C::NDMA; ++qq) {
          uint32_t off = (isk ? dk[qq] : dv[qq]) + soff;
          if constexpr (AM == kPagedAny) {
            if (rows) {
              // one page-table lookup per row; rows past the request read as zero
              const int rr = 16 * wave + C::RPI * qq + lane / C::CPR;
              const int cl = lane % C::CPR;
              const int j = j0 + rr;
              off = 0xfffffff0u;
              if (j < c.L)
                off = paged_off(g, c, j, rowstride, err) + (uint32_t)((cl ^ (isk ? swz_k<DT>(rr) : swz_v<DT>(rr))) * 16);
            }
          }
          dma16<AM == kContig>(r, sb_wrow + (uint32_t)(dst - smem) + (uint32_t)(C::RPI * qq * C::ROWB), off);
        }
      };
      auto dma_k = [&](int st, int it, int p) __attribute__((always_inline)) {
        bool rows;
        uint32_t soff;
        const __amdgpu_buffer_rsrc_t r = step_src(it, p, kbase, kmbase, rk_t, rk_m, soff, rows);
        dma_rows(true, smem + st * C::STAGE, r, soff, rows, p * kTile);
        if (it >= T) {
          uint32_t soff2;
          bool rows2;
          const __amdgpu_buffer_rsrc_t rl = step_src(it, p, kbase, klmbase, rk_t, rl_m, soff2, rows2);
          dma_rows(true, smem + st * C::STAGE + C::LOOFF, rl, soff2, false, 0);
        }
      };
      auto dma_v = [&](int st, int it, int p) __attribute__((always_inline)) {
        bool rows;
        uint32_t soff;
        const __amdgpu_buffer_rsrc_t r = step_src(it, p, vbase, vmbase, rv_t, rv_m, soff, rows);
        dma_rows(false, smem + st * C::STAGE + C::KBYTES, r, soff, rows, p * kTile);
      };
      // correction offsets of step it into table ts (wave 0): +7 where the block
      // is corrected, -inf where it is selected or not fully visible
      auto pen3 = [&](int ts, int it) __attribute__((always_inline)) {
        if (it >= T && tid < 64) {
          float* pen = (float*)(smem + PEN3 + ts * 256);
          const int h = tid >> 5, kk = tid & 31;
          const int rho = 32 * (kk >> 4) + 8 * ((kk & 15) >> 2) + 4 * h + (kk & 3);
          const int J = (it - T) * kChunk + rho;
          const bool ok = J < t.beta && !((selbits[J >> 5] >> (J & 31)) & 1u);
          pen[tid] = ok ? 7.f : -INFINITY;
        }
      };

      f32x16 S[2];          // logits of the current step (keys 0-31, 32-63)
      OpE P = {};           // E4M3 probabilities of the previous step, then of the current one
      // QK of step it into S from stage st, in two parts: qk_read requests the
      // first two K operands into kr (early, so that their LDS latency passes
      // under other work), qk_mma issues the MFMAs and reads the other operands
      // two ahead: 4, or 8 for a correction chunk (hi, then the 2^-4-scaled lo
      // part).  Operand j: logit tile j % 2, key group (j / 2) % 2, lo if j >= 4,
      // so that consecutive MFMAs accumulate into different tiles.
      auto kop = [&](int st, int jj) __attribute__((always_inline)) -> OpE {
        return kread8(st, jj & 1, (jj >> 1) & 1, jj >= 4);
      };
      auto qk_read = [&](int st, OpE* kr) __attribute__((always_inline)) {
        kr[0] = kop(st, 0);
        kr[1] = kop(st, 1);
      };
      auto qk_mma = [&](int st, int it, OpE* kr) __attribute__((always_inline)) {
        const bool lo = it >= T;
        S[0] = f32x16{};
        S[1] = f32x16{};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const OpE a = kr[jj & 1];
          if (jj < 2 || lo) kr[jj & 1] = kop(st, jj + 2);
          S[jj & 1] = mma<DT>(a, qf[(jj >> 1) & 1], S[jj & 1]);
        }
        if (lo) {
#pragma unroll
          for (int jj = 4; jj < 8; ++jj) {
            const OpE a = kr[jj & 1];
            if (jj < 6) kr[jj & 1] = kop(st, jj + 2);
            S[jj & 1] = mma_lo8(a, qf[(jj >> 1) & 1], S[jj & 1]);
          }
        }
      };
      int cur, cur_tile;
      pop(cur, cur_tile);
      if (cur < it1) {
        int nxt, nxt_tile;
        pop(nxt, nxt_tile);
        int ts = 0;  // table of the current step
        // prologue: K(s0) -> stage 0, K(s1) -> stage 1, V(s0) -> stage 1 (PV of
        // iteration 0 multiplies it by P = 0: exact zeros); logits of s0
        dma_k(0, cur, cur_tile);
        pen3(0, cur);
        if (nxt < it1) {
          dma_k(1, nxt, nxt_tile);
          pen3(1, nxt);
        }
        dma_v(1, cur, cur_tile);
        wait_vmem();
        __syncthreads();
        {
          OpE kr[2];
          qk_read(0, kr);
          qk_mma(0, cur, kr);
        }
        __syncthreads();  // every wave has read stage 0's K before iteration 0 refills it

        int par = 1;       // stage the iteration reads: (k + 1) % 2
        bool first = true;
        float resc = 1.f;
        bool need = false;
        // one iteration, reading stage PAR and filling the other; P holds the
        // previous step's probabilities until the five MFMAs that read them have
        // issued, then the current step's
        // KIND: the step whose softmax the iteration takes (0 a listed tile that
        // reaches past the first row's position, 1 another listed tile, 2 a
        // correction chunk); the steps come in that order, one loop per kind
        auto iter = [&](auto kind_tag) __attribute__((always_inline)) {
          constexpr int KIND = decltype(kind_tag)::value;
          const int PAR = par;
          const int WR = 1 - PAR;  // stage the DMA fills
          // the step after next, and this iteration's DMA: K(s_{k+2}) and V(s_k)
          int nxt2 = nxt, nxt2_tile = 0;
          if (nxt < it1) pop(nxt2, nxt2_tile);
          const int ts2 = ts == 0 ? 2 : ts - 1;  // (ts + 2) % 3
          if (nxt2 < it1) {
            dma_k(WR, nxt2, nxt2_tile);
            pen3(ts2, nxt2);
          }
          dma_v(WR, cur, cur_tile);
          constexpr bool chunk = KIND == 2;
          // logits in log2 units are S * slk: a tile step holds raw dot products,
          // a correction step gets its scale and offset (+7, or -inf where masked)
          // applied here; keys past a row's position are masked here
          const float slk = chunk ? 1.f : sl;
          if constexpr (chunk) {
            const f32x4* penp = (const f32x4*)(smem + PEN3 + ts * 256) + half * 8;
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 pv = penp[jt * 4 + r4];
#pragma unroll
                for (int e = 0; e < 4; ++e) S[jt][4 * r4 + e] = fmaf(S[jt][4 * r4 + e], sl, pv[e]);
              }
          } else if constexpr (KIND == 0) {
            const int lim = pos - cur_tile * kTile - 4 * half;  // key j visible iff j <= pos - 64 p
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (32 * jt + 8 * (r >> 2) + (r & 3) > lim) S[jt][r] = -INFINITY;
          }
          float mrow = 0.f;  // the row maximum of the step's logits
          float m_use = 0.f;
          OpE Pn;  // the step's E4M3 probabilities, two words per exp piece
          auto piece = [&](int k) __attribute__((always_inline)) {
            if (k == 0) {
              float a = fmaxf(S[0][0], fmaxf(S[0][1], S[0][2]));
              float b = fmaxf(S[1][0], fmaxf(S[1][1], S[1][2]));
#pragma unroll
              for (int r = 3; r < 15; r += 2) {
                a = fmaxf(a, fmaxf(S[0][r], S[0][r + 1]));
                b = fmaxf(b, fmaxf(S[1][r], S[1][r + 1]));
              }
              a = fmaxf(a, fmaxf(S[0][15], b));
              mrow = fmaxf(S[1][15], a);
              pin(mrow);
            } else if (k == 1) {
              // Eq. 15: the running maximum after this step's logits (slk > 0)
              const float m_step = max_halves(mrow) * slk;
              const float m_new = first ? m_step : fmaxf(m_i, m_step);
              resc = first ? 1.f : __builtin_amdgcn_exp2f(m_i - (m_new == -INFINITY ? 0.f : m_new));
              need = !first && __any(m_new > m_i);
              m_i = m_new;
              m_use = m_i == -INFINITY ? 0.f : m_i;
              pin(m_use);
            } else {
              // weights of 8 logits, rounded to E4M3 at once (two words of Pn)
              const int jt = (k - 2) >> 1, r0 = ((k - 2) & 1) * 8;
              float e[8];
#pragma unroll
              for (int r = 0; r < 8; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(S[jt][r0 + r], slk, kOff - m_use));
              Pn[jt * 4 + r0 / 4] = (int)f32x4_to_e4m3x4(e[0], e[1], e[2], e[3]);
              Pn[jt * 4 + r0 / 4 + 1] = (int)f32x4_to_e4m3x4(e[4], e[5], e[6], e[7]);
              pin(Pn[jt * 4 + r0 / 4]);
              pin(Pn[jt * 4 + r0 / 4 + 1]);
            }
          };
          // MFMA slots: 0 the row sums and 1-4 PV(s_{k-1}) over the old weights
          // P, then 5-8 QK(s_{k+1}) into S (9-12: the lo part of a correction
          // chunk).  The softmax pieces of s_k run after slots 0-5; a logit
          // tile is consumed by two exp pieces before its first QK slot writes
          // it again.  Operands come through a two-deep ring: V tiles, then K,
          // read whether or not they are needed (a conditional read would make
          // the ring a join and its load a wait): after the unit's last step the
          // QK slots read a stale stage and their logits are never used; a
          // tile step's ring also brings the first two lo operands.
          const bool qlo = nxt < it1 && nxt >= T;
          auto fetch = [&](int sl2) __attribute__((always_inline)) -> OpE {
            return sl2 <= 4 ? vread8(PAR, sl2 - 1) : kop(PAR, sl2 - 5);
          };
          OpE ring[2];
          ring[1] = fetch(1);
          ring[0] = fetch(2);
          lacc = mma<DT>(ones, P, lacc);
          hold(lacc);
          piece(0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int sl2 = 1; sl2 <= 8; ++sl2) {
            const OpE a = ring[sl2 & 1];
            ring[sl2 & 1] = fetch(sl2 + 2);
            if (sl2 <= 4) {
              oacc[sl2 - 1] = mma<DT>(a, P, oacc[sl2 - 1]);
              hold(oacc[sl2 - 1]);
              piece(sl2);
            } else {
              const int jt = (sl2 - 5) & 1, m = (sl2 - 5) >> 1;
              S[jt] = mma<DT>(a, qf[m], m == 0 ? f32x16{} : S[jt]);
              hold(S[jt]);
              if (sl2 == 5) piece(5);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if (qlo) {
#pragma unroll
            for (int sl2 = 9; sl2 <= 12; ++sl2) {
              const OpE a = ring[sl2 & 1];
              if (sl2 + 2 <= 12) ring[sl2 & 1] = fetch(sl2 + 2);
              const int jt = (sl2 - 9) & 1, m = (sl2 - 9) >> 1;
              S[jt] = mma_lo8(a, qf[m], S[jt]);
              hold(S[jt]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          P = Pn;
          // the raised maximum rescales the sums of every earlier step
          if (need) {
            lacc[0] *= resc;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[nt][r] *= resc;
          }
          first = false;
          wait_vmem();
          __syncthreads();
          ts = ts == 2 ? 0 : ts + 1;
          cur = nxt;
          cur_tile = nxt_tile;
          nxt = nxt2;
          nxt_tile = nxt2_tile;
        };
        // steps in order (listed tiles, the masked ones first, then correction chunks)
        while (cur < it1 && cur < T && cur_tile * kTile + kTile - 1 > t.t0) {
          iter(std::integral_constant<int, 0>{});
          par ^= 1;
        }
        while (cur < it1 && cur < T) {
          iter(std::integral_constant<int, 1>{});
          par ^= 1;
        }
        if constexpr (!DENSE) {
          while (cur < it1) {
            iter(std::integral_constant<int, 2>{});
            par ^= 1;
          }
        }
        // PV of the last step: its V tile sits in the stage the last iteration
        // filled, which par now names
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) oacc[nt] = mma<DT>(vread8(par, nt), P, oacc[nt]);
        lacc = mma<DT>(ones, P, lacc);
      }
      l_i = half ? 0.f : lacc[0];
    } else {
    // ---- mainloop: loads for step n+1 are in flight while step n computes.
    // Three kinds of step, each run by a loop of its own so that no step pays
    // for another kind's work: listed tiles that reach past the first row's
    // position (causal mask), then the other listed tiles, then correction
    // chunks.  The listed tiles are visited in descending order, so the masked
    // ones come first.
    int cur, cur_tile;
    pop(cur, cur_tile);
    int buf = 0;
    if (cur < it1) {
      load_step(0, cur, cur_tile);
      store_step(0, cur);
    }
    if constexpr (C::DMA) wait_vmem();
    __syncthreads();

    auto run_step = [&](auto kind_tag) {
      constexpr int KIND = decltype(kind_tag)::value;  // 0 masked tile, 1 tile, 2 correction chunk
      int nxt, nxt_tile;
      pop(nxt, nxt_tile);
      if (nxt < it1) load_step(buf ^ 1, nxt, nxt_tile);
      const char* ks = smem + buf * C::STAGE;
      const char* vt = ks + C::KBYTES;

      f32x16 sacc[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        sacc[jt] = f32x16{};
#pragma unroll
        for (int m = 0; m < C::NM0; ++m) sacc[jt] = mma<DT>(k_op(ks, jt, m), qf[m], sacc[jt]);
        if constexpr (DT == kE4M3 && KIND == 2) {
          // pooled keys = hi + 2^-4 lo: the lo products accumulate into the same logits
#pragma unroll
          for (int m = 0; m < C::NM0; ++m) sacc[jt] = mma_lo8(k_op(ks + C::LOOFF, jt, m), qf[m], sacc[jt]);
        }
      }
      if constexpr (DT == kE4M3) {
        // key j of this lane's register r of logit tile jt: 32 jt + 8 (r/4) + 4 half + r%4
        float mx;
        if constexpr (KIND == 0) {
          const int lim = pos - cur_tile * kTile - 4 * half;  // key j visible iff j <= pos - 64 p
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * jt + 8 * (r >> 2) + (r & 3) > lim) sacc[jt][r] = -INFINITY;
        }
        if constexpr (KIND == 2) {
          // logit offsets of the step's pooled means (+7, or -inf where masked)
          const f32x4* pen = (const f32x4*)(vt + C::VBYTES) + half * 8;
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 pv = pen[jt * 4 + r4];
#pragma unroll
              for (int e = 0; e < 4; ++e) sacc[jt][4 * r4 + e] = fmaf(sacc[jt][4 * r4 + e], sl, pv[e]);
            }
        }
        {
          // two chains of three-input maxima over the 32 logits
          float a = fmaxf(sacc[0][0], fmaxf(sacc[0][1], sacc[0][2]));
          float b = fmaxf(sacc[1][0], fmaxf(sacc[1][1], sacc[1][2]));
#pragma unroll
          for (int r = 3; r < 15; r += 2) {
            a = fmaxf(a, fmaxf(sacc[0][r], sacc[0][r + 1]));
            b = fmaxf(b, fmaxf(sacc[1][r], sacc[1][r + 1]));
          }
          a = fmaxf(a, fmaxf(sacc[0][15], b));
          mx = fmaxf(sacc[1][15], a);
        }
        mx = max_halves(mx);
        // tile steps hold raw dot products (sl > 0); chunk steps are already scaled
        const float m_step = KIND == 2 ? mx : mx * sl;
        if (fresh) {
          m_i = m_step;
          fresh = false;
        } else if (__any(m_step > m_i + kTau)) {
          const float m_new = fmaxf(m_i, m_step);
          const float resc = __builtin_amdgcn_exp2f(m_i - (m_new == -INFINITY ? 0.f : m_new));
          lacc[0] *= resc;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[nt][r] *= resc;
          m_i = m_new;
        }
        const float m_use = m_i == -INFINITY ? 0.f : m_i;
        if constexpr (KIND != 2) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[jt][r] = __builtin_amdgcn_exp2f(fmaf(sacc[jt][r], sl, kOff - m_use));
        } else {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[jt][r] = __builtin_amdgcn_exp2f(sacc[jt][r] + (kOff - m_use));
        }

        // P^T as the B operands of O^T += V^T P^T
        Op pf[C::NM1];
        if constexpr (DT == kE4M3) {
          i32x8 b;
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int jt = w >> 2, r = (w & 3) * 4;
            const uint32_t word = f32x4_to_e4m3x4(sacc[jt][r], sacc[jt][r + 1], sacc[jt][r + 2], sacc[jt][r + 3]);
            b[w] = (int)word;
          }
          if constexpr (VC) {
            // word w of lane half h holds keys 4 gi .. 4 gi + 3, gi = 8 (w / 4) +
            // 2 (w % 4) + h; exchange halves so that half h holds keys 32 h .. 32 h
            // + 31 in order, matching the transposed V rows.  One lane-half swap
            // per pair (w, w + 4): the first result is [own w | half 0's w + 4],
            // the second [half 1's w | own w + 4], i.e. words 2j and 2j + 1 of
            // either half.
            i32x8 nb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)b[j], (uint32_t)b[4 + j], false, false);
              nb[2 * j] = (int)r[0];
              nb[2 * j + 1] = (int)r[1];
            }
            b = nb;
          }
          pf[0] = b;
        } else {
          float psum = 0.f;
#pragma unroll
          for (int m1 = 0; m1 < 32; ++m1) {
            const float pv = sacc[m1 >> 4][m1 & 15];
            psum += pv;
            pf[m1] = pv;
          }
          l_i += psum;
        }
        if constexpr (VC && KIND == 0) {
          // the tile holding the request's last key: bytes of keys past the end
          // (another request's values, or unused page slots) are cleared, so
          // that a zero weight never meets a NaN
          const int nvalid = c.L - cur_tile * kTile - 32 * half;
          if (__any(nvalid < 32)) {
            uint32_t bm[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const int nb = min(4, max(0, nvalid - 4 * w));
              bm[w] = nb == 4 ? 0xffffffffu : (1u << (8 * nb)) - 1u;
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              Op a = v_op(vt, nt, 0);
#pragma unroll
              for (int w = 0; w < 8; ++w) a[w] &= bm[w];
              oacc[nt] = mma<DT>(a, pf[0], oacc[nt]);
            }
          } else {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) oacc[nt] = mma<DT>(v_op(vt, nt, 0), pf[0], oacc[nt]);
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
            for (int m1 = 0; m1 < C::NM1; ++m1) oacc[nt] = mma<DT>(v_op(vt, nt, m1), pf[m1], oacc[nt]);
          }
        }
        lacc = mma<DT>(ones, pf[0], lacc);  // row sums of the rounded P
      } else {
        // Two halves of 32 keys (logit tile jt), each an online-softmax update
        // of its own.  The VALU work of half 0 overlaps the MFMAs of half 1's
        // logits, that of half 1 overlaps the P V MFMAs of half 0: the rescale
        // decision is taken without a branch, and only the (rare) rescale of
        // the accumulators is conditional.
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f32x16& sv = sacc[jt];
          if constexpr (KIND == 0) {
            const int lim = pos - cur_tile * kTile - 4 * half;  // key j visible iff j <= pos - 64 p
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * jt + 8 * (r >> 2) + (r & 3) > lim) sv[r] = -INFINITY;
          }
          if constexpr (KIND == 2) {
            const f32x4* pen = (const f32x4*)(vt + C::VBYTES) + half * 8 + jt * 4;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 pv = pen[r4];
#pragma unroll
              for (int e = 0; e < 4; ++e) sv[4 * r4 + e] = fmaf(sv[4 * r4 + e], sl, pv[e]);
            }
          }
          float a = fmaxf(sv[0], fmaxf(sv[1], sv[2]));
          float b = fmaxf(sv[8], fmaxf(sv[9], sv[10]));
          a = fmaxf(a, fmaxf(sv[3], sv[4]));
          b = fmaxf(b, fmaxf(sv[11], sv[12]));
          a = fmaxf(a, fmaxf(sv[5], sv[6]));
          b = fmaxf(b, fmaxf(sv[13], sv[14]));
          a = fmaxf(a, fmaxf(sv[7], b));
          float mh = fmaxf(a, sv[15]);
          {
            // the other lane half holds the same query row
            mh = max_halves(mh);
          }
          const float m_half = KIND == 2 ? mh : mh * sl;  // tile steps hold raw dot products (sl > 0)
          const bool need = __any(m_half > m_i + kTau);
          const float m_new = need ? fmaxf(m_i, m_half) : m_i;
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float resc = __builtin_amdgcn_exp2f(m_i - m_use);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sv[r] = __builtin_amdgcn_exp2f(KIND == 2 ? sv[r] + (kOff - m_use) : fmaf(sv[r], sl, kOff - m_use));
          Op ph[C::NM1 / 2];
          float psum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              psum += sv[r];
              ph[r] = sv[r];
            }
          l_i = fmaf(l_i, resc, psum);
          m_i = m_new;
          // P is complete here, before the rescale branch, so that its VALU
          // work shares a block with (and overlaps) the preceding MFMAs
#pragma unroll
          for (int q2 = 0; q2 < C::NM1 / 2; ++q2) pin(ph[q2]);
          if (need && !fresh) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[nt][r] *= resc;
          }
          fresh = false;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int q2 = 0; q2 < C::NM1 / 2; ++q2)
              oacc[nt] = mma<DT>(v_op(vt, nt, jt * (C::NM1 / 2) + q2), ph[q2], oacc[nt]);
        }
      }
      if (nxt < it1) store_step(buf ^ 1, nxt);
      if constexpr (C::DMA) wait_vmem();
      __syncthreads();
      buf ^= 1;
      cur = nxt;
      cur_tile = nxt_tile;
    };
    using KMasked = std::integral_constant<int, 0>;
    using KTile = std::integral_constant<int, 1>;
    using KChunk = std::integral_constant<int, 2>;
    while (cur < it1 && cur < T && cur_tile * kTile + kTile - 1 > t.t0) run_step(KMasked{});
    while (cur < it1 && cur < T) run_step(KTile{});
    if constexpr (!DENSE) {
      while (cur < it1) run_step(KChunk{});
    }
    // e4m3: the complete row sum sits in both lane halves; the epilogue adds halves
    if constexpr (DT == kE4M3) l_i = half ? 0.f : lacc[0];
    }

    }

    // ---- epilogue: results as floats; a unit that saw malformed input stores
    // NaN bit patterns instead (a separate branch, so no float select is involved)
    if (err) atomicOr(&g.hdr->err, (int)err);
    if (tid == 0) sh_unit = ticket < own_hi - own_lo ? own_hi - 1 - ticket : steal(xcd + 1);
    // each wave rewrites its own flag every unit, and a wave reaches this
    // write only after every wave has passed the unit's first barrier, that
    // is after every read of the previous unit's flags
    if (lane == 0) bad_w[wave] = __ballot(err != 0) != 0;
    __syncthreads();
    const bool bad = (bad_w[0] | bad_w[1] | bad_w[2] | bad_w[3]) != 0;
    const float2 lp = with_other_half(l_i);
    const float l_tot = lp.x + lp.y;
    if (DT == kBF16 && un.nsplit == 1 && !bad) {
      // bf16: the wave's 32 output rows pass through LDS (the K buffers, which
      // nothing reads after the unit's last barrier; rows padded to 272 bytes
      // so that the 32 rows' writes spread over the banks), and every store
      // then writes whole 16-byte pieces of 4 consecutive rows instead of
      // 8-byte pieces of 32.  Each wave reads back only its own rows, and a
      // wave's LDS accesses complete in order, so no barrier sits between.
      char* ob = smem + PipeL::K0 + wave * 32 * 272;
      const float inv = cvs / l_tot;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int n0 = nt * 32 + 8 * b4 + 4 * half;
          const uint32_t w0 = f32_to_bf16_bits(oacc[nt][4 * b4] * inv) |
                              ((uint32_t)f32_to_bf16_bits(oacc[nt][4 * b4 + 1] * inv) << 16);
          const uint32_t w1 = f32_to_bf16_bits(oacc[nt][4 * b4 + 2] * inv) |
                              ((uint32_t)f32_to_bf16_bits(oacc[nt][4 * b4 + 3] * inv) << 16);
          *(uint2*)(ob + col * 272 + n0 * 2) = make_uint2(w0, w1);
        }
      if (row_ok && lse && half == 0)
        lse[(c.row0 + qi) * g.hq + head] = (m_i + __builtin_amdgcn_logf(l_tot) - kOff) * 0.6931471805599453f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4), c16 = lane & 15;
        if (wave * 32 + r < t.nrows) {
          const int64_t pr = c.I * kRows + wave * 32 + r;
          const int64_t orow = (c.row0 + (pr >> g.log2g)) * g.hq + c.h * g.g + (int)(pr & (g.g - 1));
          *(uint4*)((char*)out + orow * kD * 2 + c16 * 16) = *(const uint4*)(ob + r * 272 + c16 * 16);
        }
      }
    } else if (un.nsplit == 1) {
      if (row_ok) {
        if (!bad) {
          const float inv = cvs / l_tot;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
              const int n0 = nt * 32 + 8 * b4 + 4 * half;
              const float o0 = oacc[nt][4 * b4] * inv, o1 = oacc[nt][4 * b4 + 1] * inv;
              const float o2 = oacc[nt][4 * b4 + 2] * inv, o3 = oacc[nt][4 * b4 + 3] * inv;
              if constexpr (DT == kF32) {
                *(float4*)((float*)out + qrow * kD + n0) = make_float4(o0, o1, o2, o3);
              } else {
                const uint32_t w0 = f32_to_bf16_bits(o0) | ((uint32_t)f32_to_bf16_bits(o1) << 16);
                const uint32_t w1 = f32_to_bf16_bits(o2) | ((uint32_t)f32_to_bf16_bits(o3) << 16);
                *(uint2*)((uint16_t*)out + qrow * kD + n0) = make_uint2(w0, w1);
              }
            }
          if (lse && half == 0)
            lse[(c.row0 + qi) * g.hq + head] =
                (m_i + __builtin_amdgcn_logf(l_tot) - kOff) * 0.6931471805599453f;
        } else {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
              const int n0 = nt * 32 + 8 * b4 + 4 * half;
              if constexpr (DT == kF32)
                *(uint4*)((float*)out + qrow * kD + n0) = make_uint4(kNaN32, kNaN32, kNaN32, kNaN32);
              else
                *(uint2*)((uint16_t*)out + qrow * kD + n0) = make_uint2(kNaNbf16x2, kNaNbf16x2);
            }
          if (lse && half == 0) ((uint32_t*)lse)[(c.row0 + qi) * g.hq + head] = kNaN32;
        }
      }
    } else {
      // partial result of one split: O (unnormalised), m (log2), l
      const int64_t slot = un.s * wl.umax + un.split;
      float* po = (float*)(ws + wl.part_o) + slot * kRows * kD;
      float* pml = (float*)(ws + wl.part_ml) + slot * 2 * kRows;
      if (!bad) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const int n0 = nt * 32 + 8 * b4 + 4 * half;
            *(float4*)(po + row_in_tile * kD + n0) =
                make_float4(oacc[nt][4 * b4], oacc[nt][4 * b4 + 1], oacc[nt][4 * b4 + 2], oacc[nt][4 * b4 + 3]);
          }
        if (half == 0) {
          pml[row_in_tile] = m_i;
          pml[kRows + row_in_tile] = l_tot;
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4)
            *(uint4*)(po + row_in_tile * kD + nt * 32 + 8 * b4 + 4 * half) =
                make_uint4(kNaN32, kNaN32, kNaN32, kNaN32);
        if (half == 0) {
          pml[row_in_tile] = m_i;
          ((uint32_t*)pml)[kRows + row_in_tile] = kNaN32;
        }
      }
    }
  }
}

// Merge the splits of every split segment in split order (deterministic).
template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(Geo g, WsLayout wl, const char* __restrict__ ws,
                                                      void* __restrict__ out, float* __restrict__ lse) {
  const int64_t s = block_x();
  const int32_t* nsplit = (const int32_t*)(ws + wl.counts);
  const int U = nsplit[s];
  if (U <= 1) return;
  const SegCoord c = seg_coord(g, s);
  const TileGeo t = tile_geo(g, c);
  const int r = thread_x() >> 1, n0 = (thread_x() & 1) * 64;
  if (r >= t.nrows) return;
  const float* po = (const float*)(ws + wl.part_o);
  const float* pml = (const float*)(ws + wl.part_ml);
  float M = -INFINITY;
  for (int u = 0; u < U; ++u) M = fmaxf(M, pml[(s * wl.umax + u) * 2 * kRows + r]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float wgt[16];
  float L = 0.f;
  for (int u = 0; u < U; ++u) {
    const float* ml = pml + (s * wl.umax + u) * 2 * kRows;
    wgt[u] = __builtin_amdgcn_exp2f(ml[r] - Mu);
    L += wgt[u] * ml[kRows + r];
  }
  const float cvs = DT == kE4M3 ? g.descale[2] : 1.f;
  const float inv = cvs / L;
  const int64_t prow = c.I * kRows + r;
  const int qi = (int)(prow >> g.log2g);  // query index within the request
  const int head = c.h * g.g + (int)(prow & (g.g - 1));
  const int64_t qrow = (c.row0 + qi) * g.hq + head;
  for (int n = n0; n < n0 + 64; n += 4) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int u = 0; u < U; ++u) {
      const float4 o = *(const float4*)(po + ((s * wl.umax + u) * kRows + r) * kD + n);
      a[0] += wgt[u] * o.x;
      a[1] += wgt[u] * o.y;
      a[2] += wgt[u] * o.z;
      a[3] += wgt[u] * o.w;
    }
    if constexpr (DT == kF32) {
      *(float4*)((float*)out + qrow * kD + n) = make_float4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
    } else {
      uint32_t w0 = f32_to_bf16_bits(a[0] * inv) | ((uint32_t)f32_to_bf16_bits(a[1] * inv) << 16);
      uint32_t w1 = f32_to_bf16_bits(a[2] * inv) | ((uint32_t)f32_to_bf16_bits(a[3] * inv) << 16);
      *(uint2*)((uint16_t*)out + qrow * kD + n) = make_uint2(w0, w1);
    }
  }
  if (lse && n0 == 0) {
    constexpr float kOffL = DT == kE4M3 ? 8.f : 0.f;
    lse[(c.row0 + qi) * g.hq + head] = (Mu + __builtin_amdgcn_logf(L) - kOffL) * 0.6931471805599453f;
  }
}

int attn_wgs_per_cu(int dtype) { return dtype == kF32 ? Cfg<kF32>::WGS : Cfg<kBF16>::WGS; }

template <int DT, bool DENSE, int AM, bool VC = false>
static hipError_t launch_attn_t(const Geo& g, const WsLayout& wl, char* ws, const MeansLayout& ml,
                                const void* q, const void* k, const void* v, const int32_t* cu,
                                const int32_t* idx, const char* means, int correction, void* out,
                                float* lse, int grid, hipStream_t st) {
  hipError_t e = set_lds_limit((const void*)attn_kernel<DT, DENSE, AM, VC>, Cfg<DT>::LDS);
  if (e != hipSuccess) return e;
  attn_kernel<DT, DENSE, AM, VC><<<grid, 256, Cfg<DT>::LDS, st>>>(g, wl, ws, ml, q, k, v, cu, idx, means,
                                                                      correction, out, lse, grid);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_attn_dt(const Geo& g, const WsLayout& wl, char* ws, const MeansLayout& ml,
                                 const void* q, const void* k, const void* v, const int32_t* cu,
                                 const int32_t* idx, const char* means, int dense, int correction,
                                 void* out, float* lse, int grid, hipStream_t st) {
  const int am = !g.page_table ? kContig : (g.page_size % kTile == 0 ? kPagedTile : kPagedAny);
  if constexpr (DT == kE4M3) {
    if (g.vcols) {  // transposed V: contiguous or 64-multiple pages (checked on the host)
#define FP_VC(DENSE, AMV) \
  launch_attn_t<DT, DENSE, AMV, true>(g, wl, ws, ml, q, k, v, cu, idx, means, DENSE ? 0 : correction, out, lse, grid, st)
      if (dense) return am == kContig ? FP_VC(true, kContig) : FP_VC(true, kPagedTile);
      return am == kContig ? FP_VC(false, kContig) : FP_VC(false, kPagedTile);
#undef FP_VC
    }
  }
#define FP_AM(DENSE, AMV) \
  launch_attn_t<DT, DENSE, AMV>(g, wl, ws, ml, q, k, v, cu, idx, means, DENSE ? 0 : correction, out, lse, grid, st)
  if (dense) return am == kContig ? FP_AM(true, kContig) : am == kPagedTile ? FP_AM(true, kPagedTile) : FP_AM(true, kPagedAny);
  return am == kContig ? FP_AM(false, kContig) : am == kPagedTile ? FP_AM(false, kPagedTile) : FP_AM(false, kPagedAny);
#undef FP_AM
}

hipError_t launch_attn(const Geo& g, const WsLayout& wl, char* ws, const MeansLayout& ml, const void* q,
                       const void* k, const void* v, const int32_t* cu, const int32_t* idx,
                       const char* means, int dense, int correction, void* out, float* lse, int grid,
                       hipStream_t st) {
  switch (g.dtype) {
    case kBF16:
      return launch_attn_dt<kBF16>(g, wl, ws, ml, q, k, v, cu, idx, means, dense, correction, out, lse, grid, st);
    case kF32:
      return launch_attn_dt<kF32>(g, wl, ws, ml, q, k, v, cu, idx, means, dense, correction, out, lse, grid, st);
    default:
      return launch_attn_dt<kE4M3>(g, wl, ws, ml, q, k, v, cu, idx, means, dense, correction, out, lse, grid, st);
  }
}

hipError_t launch_combine(const Geo& g, const WsLayout& wl, char* ws, void* out, float* lse, hipStream_t st) {
  dim3 grid((unsigned)g.n_seg);
  switch (g.dtype) {
    case kBF16: combine_kernel<kBF16><<<grid, 256, 0, st>>>(g, wl, ws, out, lse); break;
    case kF32: combine_kernel<kF32><<<grid, 256, 0, st>>>(g, wl, ws, out, lse); break;
    default: combine_kernel<kE4M3><<<grid, 256, 0, st>>>(g, wl, ws, out, lse); break;
  }
  return hipGetLastError();
}

}  // namespace fp
