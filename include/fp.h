/*
 * fp.h -- C ABI of libfp.so: FlashPrefill V2 block-sparse causal prefill
 * attention on AMD Instinct MI355X (gfx950).
 *
 * Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context
 * LLM Serving" (arXiv 2608.19758), cited below as [V2] with its section and
 * equation numbers.
 *
 * Two stages per attention layer ([V2] §3.4):
 *   fp_select       index stage: pool K/V per 128-token block, score the
 *                   PackGQA query tiles against the pooled keys, keep the
 *                   blocks at or above alpha * max plus the sink, window and
 *                   diagonal blocks, and write the CSR index of selected
 *                   64-token tiles.
 *   fp_sparse_attn  attention stage: exact online-softmax attention over the
 *                   listed tiles, plus one mean-correction term per pruned
 *                   block that every row of the tile can see.
 *   fp_dense_attn   dense causal attention on the same kernel (the baseline).
 * and one diagnostic:
 *   fp_block_mass   exact per-block attention mass of every query tile, and
 *                   the mean surrogate of the blocks the correction replaces
 *                   (how much attention the selection keeps).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *     every buffer; the library allocates no device memory.  Its only device
 *     state is the static scratch of fp_sparse_attn_static (a file-scope
 *     array each GPU holds from library load to process end).
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     is the default stream).  Only fp_read_device_error synchronises.
 *   - Host-visible arguments are validated before anything is launched; a bad
 *     call returns a negative fp_status, launches nothing, and leaves a
 *     description in fp_last_error().
 *   - Malformed device data that only the GPU can see (a page id outside the
 *     pool, an idx entry that is out of range or not ascending) sets a flag in
 *     the workspace header and writes NaN into the affected output rows;
 *     fp_read_device_error reports it.
 *   - Layouts (row-major, element = head_dim-vector):
 *       Q, O     [total_q][num_heads_q][head_dim], rows ragged by cu_seqlens_q
 *       K, V     contiguous: [total_kv][num_heads_kv][head_dim], rows ragged by
 *                cu_seqlens_kv (by cu_seqlens_q when that is NULL)
 *                paged:      [num_pool_slots][num_heads_kv][head_dim]; token j of
 *                request b lives in slot page_table[b][j/p]*p + j%p ([V2] Eq. 22)
 *       V (E4M3 only, v_layout = FP_V_COLS) stored transposed, each value
 *                vector a column ([V2] §3.3 Eq. 16, first case):
 *                contiguous: [num_heads_kv][head_dim][total_kv], element
 *                (row t, head h, dim c) at (h*head_dim + c)*total_kv + t, every
 *                K/V offset (and so total_kv) a multiple of 16;
 *                paged: [num_pool_slots/p][num_heads_kv][head_dim][p] (p a
 *                multiple of 64), token j of request b at
 *                ((page*num_heads_kv + h)*head_dim + c)*p + j%p, page =
 *                page_table[b][j/p]
 *       LSE      [total_q][num_heads_q] float, natural log
 *   - Element types: FP_F32 (float), FP_BF16 (bfloat16), FP_E4M3 (OCP E4M3FN
 *     with per-tensor descales c_q, c_k, c_v, [V2] §3.3 Eq. 15).  O is bf16
 *     for FP_BF16 and FP_E4M3 inputs, float for FP_F32.
 *   - Query packing ([V2] §3.3 Eq. 12-13): packed row r of KV head h is
 *     position r/g of query head h*g + r%g, g = num_heads_q/num_heads_kv.  A
 *     query tile is 128 packed rows; one CSR segment per (request, KV head,
 *     tile), segments ordered by request, then KV head, then tile.
 *   - CSR ([V2] §3.3 Eq. 17): cu[n_segments+1] is the exclusive prefix sum of
 *     the per-segment counts; idx[cu[s] .. cu[s+1]) lists the ascending ids of
 *     the segment's selected 64-token key tiles, relative to the request
 *     (tile p covers tokens 64p .. 64p+63).
 *   - Not thread-safe per workspace: calls that share a workspace must be
 *     ordered on one stream.
 */
#ifndef FP_H
#define FP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP_OK = 0,
  FP_ERR_INVALID_ARG = -1,        /* a NULL pointer, a negative size, inconsistent lengths */
  FP_ERR_UNSUPPORTED = -2,        /* a valid but unsupported shape (head_dim != 128, ...) */
  FP_ERR_WORKSPACE_TOO_SMALL = -3,
  FP_ERR_CAPACITY_TOO_SMALL = -4, /* idx buffer smaller than fp_sizes.idx_capacity */
  FP_ERR_LAUNCH = -5,             /* the HIP runtime refused a launch */
  FP_ERR_DEVICE = -6              /* fp_read_device_error: the device flagged bad data */
} fp_status;

typedef enum { FP_F32 = 0, FP_BF16 = 1, FP_E4M3 = 2 } fp_dtype;

/* Storage of V: rows (each token's vector contiguous, like K) or columns
 * (each head's values transposed, [V2] §3.3 Eq. 16's column-major FP8 V,
 * consumed without a copy; FP_E4M3 only). */
typedef enum { FP_V_ROWS = 0, FP_V_COLS = 1 } fp_v_layout;

/* One batch of prefill requests.  Built once per forward step and shared by
 * every layer ([V2] §3.4, serving integration).  A request has L_kv keys and
 * L_q <= L_kv queries; the queries are its last L_q positions, i.e. query i
 * sits at position L_kv - L_q + i: a prefill chunk over a cached prefix, with
 * the index re-run for every chunk ([V2] §4.3 "Compatibility with Chunked
 * Prefill").  Leaving both cu_seqlens_kv pointers NULL means L_kv = L_q
 * (fresh prefill). */
typedef struct {
  int32_t num_reqs;              /* >= 1 */
  int32_t num_heads_q;           /* multiple of num_heads_kv */
  int32_t num_heads_kv;          /* >= 1; g = num_heads_q/num_heads_kv is a power of 2 <= 128 */
  int32_t head_dim;              /* must be 128 */
  const int32_t* cu_seqlens_q;   /* [num_reqs+1] row offsets of Q/O (and of contiguous K/V when
                                    cu_seqlens_kv is NULL) */
  const int32_t* cu_seqlens_q_host; /* (host) the same values; sizes grids, checked for order */
  const int32_t* page_table;     /* [num_reqs][max_pages_per_req] page ids, or NULL = contiguous */
  int32_t page_size;             /* p >= 1, any value ([V2] Eq. 22); ignored when contiguous */
  int32_t max_pages_per_req;     /* row stride of page_table; >= ceil(max L_kv / p) */
  int64_t num_pool_slots;        /* rows of the paged K/V pool; ignored when contiguous */
  int32_t dtype;                 /* fp_dtype of Q, K and V */
  const float* descale;          /* [3] = {c_q, c_k, c_v} for FP_E4M3, else NULL */
  float softmax_scale;           /* sigma; 0 means 1/sqrt(head_dim) */
  const int32_t* cu_seqlens_kv;  /* [num_reqs+1] K/V lengths as offsets (rows of contiguous K/V),
                                    or NULL: the same as cu_seqlens_q */
  const int32_t* cu_seqlens_kv_host; /* (host) the same values, or NULL; given together with
                                        cu_seqlens_kv; every L_kv >= its L_q */
  int32_t v_layout;              /* fp_v_layout; FP_V_COLS needs FP_E4M3, and when paged a page
                                    size that is a multiple of 64 and num_pool_slots a multiple of
                                    it */
} fp_problem;

/* Block selection settings ([V2] §3.1 Eq. 3, §3.3 Eq. 20, defaults in §4.1:
 * B = 128, 256 sink tokens = 2 blocks, 512-token window = 4 blocks, alpha = 0.1). */
typedef struct {
  float alpha;            /* threshold factor, finite and >= 0 (0 keeps every causal block) */
  int32_t block_size;     /* must be 128 */
  int32_t sink_blocks;    /* blocks J < sink_blocks are always kept */
  int32_t window_blocks;  /* the window_blocks blocks just before a tile's own block are kept */
} fp_select_params;

typedef struct {
  int64_t n_segments;     /* CSR segments; cu has n_segments+1 entries */
  int64_t idx_capacity;   /* int32 entries idx must hold (every causal tile of every segment) */
  size_t means_bytes;     /* bytes of the pooled-statistics buffer */
  size_t workspace_bytes; /* bytes of the workspace every call below takes */
  int64_t max_blocks;     /* largest number of candidate blocks of a segment (energies stride) */
} fp_sizes;

/* Sizes of every caller-owned buffer for this problem.  Needs the device that
 * will run the calls to be current (the split policy depends on its CU count). */
fp_status fp_query_sizes(const fp_problem* prob, const fp_select_params* params,
                         fp_sizes* out /* (host) */);

/* Block means of K and V ([V2] §3.2 Eq. 5): kbar_J = mean of the keys of
 * block J, over the block's actual token count; likewise vbar.  E4M3 inputs
 * are descaled first.  Writes `means` (means_bytes).  Its first two arrays are
 * float kbar and vbar, [NB][num_heads_kv][head_dim] each, where request b's
 * blocks start at block fp_block_base(b) = sum over earlier requests of
 * ceil(ceil(L_kv/128)/64)*64; the rest of the buffer holds derived operand
 * copies private to the library.  fp_select calls this itself. */
fp_status fp_pool(const fp_problem* prob, const void* k, const void* v, void* means, void* ws,
                  size_t ws_bytes, void* stream);

/* Index stage ([V2] §3.1, §3.3 "Single-Pass Score and Selection"): pooling,
 * scoring of every (query tile, causal block J <= beta) pair with
 * E_J = sum over the tile's rows of exp(sigma q.kbar_J - M), selection
 * E_J >= alpha * max E or J forced (J < sink_blocks, beta - window_blocks <= J
 * < beta, J == beta), and CSR expansion of each kept block J into tiles 2J and
 * 2J+1 (a tile starting after the tile's last query position is dropped).
 * energies (optional, may be NULL): [n_segments][max_blocks] floats receive
 * E_J / max E for the candidate blocks J <= beta1 (the block of the segment's
 * last position) and -1 beyond.  With energies requested every block is
 * scored at full precision; without, most blocks are scored at reduced
 * precision under an error bound and only those the bound leaves undecided are
 * scored again, which yields the same cu/idx.  idx_capacity is the int32 size of
 * idx and must be >= fp_sizes.idx_capacity. */
fp_status fp_select(const fp_problem* prob, const fp_select_params* params, const void* q,
                    const void* k, const void* v, int32_t* cu, int32_t* idx,
                    int64_t idx_capacity, void* means, float* energies, void* ws,
                    size_t ws_bytes, void* stream);

/* Attention stage ([V2] §3.2 Eq. 6, §3.3): for each row of each segment,
 * online softmax over the tokens i <= position of the listed tiles, plus, when
 * mean_correction != 0, one term per block J < beta that no listed tile
 * covers, with logit sigma q.kbar_J + ln 128 and value vbar_J.  cu/idx/means
 * are fp_select's outputs for the same problem (idx may be any valid CSR:
 * ascending tile ids p with 64p <= the segment's last position).  out is O;
 * lse (optional) receives the natural-log log-sum-exp of each row. */
fp_status fp_sparse_attn(const fp_problem* prob, const fp_select_params* params, const void* q,
                         const void* k, const void* v, const int32_t* cu, const int32_t* idx,
                         const void* means, int32_t mean_correction, void* out, float* lse,
                         void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation as fp_sparse_attn (every argument means what it means there),
 * with the library's own static device scratch in place of a caller
 * workspace.  Each GPU the library runs on holds FP_STATIC_SCRATCH_BYTES of
 * it until the process ends; the scratch's address on the current device is
 * looked up on the first call there.  KV splitting is off (a work unit is a
 * whole query tile), so outputs equal fp_sparse_attn's run with
 * FP_MAX_SPLITS=1 bit for bit.  A problem whose workspace exceeds the scratch
 * (about 80 bytes per CSR segment plus a few KB) returns
 * FP_ERR_WORKSPACE_TOO_SMALL with nothing launched; no device memory is
 * allocated on any path.  Every call on a GPU uses that GPU's one scratch:
 * calls that overlap on one GPU (two streams, two host threads) race and
 * must be ordered by the caller.  The device error flag of these calls lives
 * in the scratch and is not readable through fp_read_device_error; malformed
 * device data still turns the affected rows into NaN. */
#define FP_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
fp_status fp_sparse_attn_static(const fp_problem* prob, const fp_select_params* params, const void* q,
                                const void* k, const void* v, const int32_t* cu, const int32_t* idx,
                                const void* means, int32_t mean_correction, void* out, float* lse,
                                void* stream);

/* Dense causal attention of the same problem through the same kernel
 * ([V2] §4.1: the dense reference that shares the sparse operator's
 * pipeline).  lse is optional. */
fp_status fp_dense_attn(const fp_problem* prob, const void* q, const void* k, const void* v,
                        void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Exact block attention mass, the selection-recall diagnostic ("FlashPrefill:
 * Instantaneous Pattern Discovery and Thresholding for Ultra-Fast Long-Context
 * Prefilling", §3.1: exact identification scores every query against every
 * key and averages the per-block attention over the tile's queries; its
 * AM-GM argument pairs the pooled surrogate with the true block sum).  For
 * each segment s and candidate block J <= beta1 (n = the segment's valid rows,
 * t_r a row's position, LSE_r its dense log-sum-exp):
 *   mass[s][J]      = (1/n) sum_r sum_{i in block J, i <= t_r} exp(sigma q_r.k_i - LSE_r)
 *   surrogate[s][J] = (1/n) sum_r 128 exp(sigma q_r.kbar_J - LSE_r)  for J < beta,
 *                     0 for beta <= J <= beta1
 * and -1 for J > beta1.  Both are [n_segments][max_blocks] floats; a
 * segment's masses sum to 1.  lse: [total_q][num_heads_q] natural-log dense
 * LSE of the same rows (required): fp_dense_attn's for fp32 and bf16 inputs;
 * for E4M3 inputs that of the descaled values (fp_dense_attn on their fp32
 * decoding), since the E4M3 path's LSE carries Eq. 15's rounding.  surrogate may be NULL; when
 * given, means must hold fp_pool's (or fp_select's) output for this problem.
 * Costs about half a dense attention call (Q K^T of every visible pair). */
fp_status fp_block_mass(const fp_problem* prob, const void* q, const void* k, const float* lse,
                        const void* means, float* mass, float* surrogate, void* ws, size_t ws_bytes,
                        void* stream);

/* Synchronises `stream`, then reads and clears the device error flag of the
 * workspace.  *flag (host) receives the flag bits (0 = no error; bit 0: page
 * id outside the pool; bit 1: idx entry out of range or not ascending).
 * Returns FP_ERR_DEVICE when a flag was set. */
fp_status fp_read_device_error(void* ws, void* stream, int32_t* flag /* (host) */);

/* First block of request b in the pooled-statistics arrays (host arithmetic
 * on the K/V lengths); -1 if b is out of range. */
int64_t fp_block_base(const fp_problem* prob, int32_t b);

const char* fp_status_string(fp_status s);
const char* fp_last_error(void); /* thread-local detail of the last failing call */

#ifdef __cplusplus
}
#endif
#endif /* FP_H */
