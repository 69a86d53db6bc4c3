/*
 * csa.h - C ABI of the CSA sparse-attention decode step on MI355X (gfx950).
 *
 * One decode step of compressed sparse attention, in three calls issued in
 * order on one HIP stream:
 *
 *   csa_indexer_score      score every causally visible compressed row
 *                          (csa_indexer_score_fp8: from an FP8 key cache)
 *   csa_topk               pick the Top-K rows per query token (or bypass)
 *   csa_sparse_attn_decode attend the raw window plus the picked rows, merge
 *                          the two softmax streams, undo RoPE, pack heads
 *
 * and, before them, csa_swa_writeback, which commits the step's new window
 * entries to the window cache.
 *
 * The step is the one described on the pages "Perf: skip redundant CSA
 * scoring and fuse gather unpack" (description and changes table: scoring and
 * sorting skipped when the ratio-4 cache fits IDX_TOPK, causal visibility
 * kept, bounded Top-K indices emitted) and "Perf: fuse HCA merge, inverse
 * RoPE, and packing" (description and changes table: the raw and compressed
 * softmax merge, inverse RoPE and grouped packing in one pass, written into a
 * preallocated grouped output).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is a DEVICE pointer to a contiguous, row-major,
 *   16-byte aligned buffer owned by the caller.  The shape pointer is HOST
 *   memory.  The library allocates nothing and keeps no pointer after a call
 *   returns; its only state is the static device array behind
 *   csa_sparse_attn_decode_noalloc.  Calls are reentrant (calls that share a
 *   workspace, or that array, must not overlap in time).
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   Calls only enqueue work; ordering is the stream order.
 * - Element type of q, k_win, v_win, k_cmp, v_cmp, q_idx, k_idx and out is
 *   shape->dtype (CSA_DTYPE_BF16 or CSA_DTYPE_F32).  w, scores, rope tables
 *   and workspace are float32; start_pos and topk_idx are int32.
 * - Errors are returned as status codes, never by aborting or printing.  All
 *   argument checks run on the host before anything is enqueued, so on any
 *   error other than CSA_ERR_LAUNCH no output has been touched.
 * - An empty problem (batch == 0 or q_per_req == 0) is valid and does nothing.
 *
 * Positions and visibility
 * ------------------------
 * Query token s of request b sits at position p = start_pos[b] + s.  A
 * compressed row j summarises raw tokens R*j .. R*j+R-1 and is visible to p
 * once all of them are at or before p: n_vis(p) = floor((p+1)/R).  A token
 * "fits" when n_vis(p) <= K; then it is not scored and its Top-K list is
 * simply every visible row.  The device trusts start_pos but clamps p to
 * [0, max_len-1], so a start_pos outside the contract cannot make it read out
 * of bounds.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                       */
  CSA_ERR_BAD_SHAPE = 2,   /* a size is negative, zero where it must not be,
                              or inconsistent (H % G, odd Dr, Dr > D, ...)     */
  CSA_ERR_BAD_DTYPE = 3,   /* dtype is not CSA_DTYPE_F32 / CSA_DTYPE_BF16      */
  CSA_ERR_CAPACITY = 4,    /* n_cap, w_cap or rope_rows too small for max_len  */
  CSA_ERR_ALIGNMENT = 5,   /* a tensor pointer is not 16-byte aligned          */
  CSA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the query says    */
  CSA_ERR_LAUNCH = 7,      /* the HIP runtime refused a launch                 */
  CSA_ERR_UNSUPPORTED = 8  /* valid but outside what the kernels are built for
                              (see csa_shape_t for the supported ranges)       */
} csa_status_t;

typedef enum { CSA_DTYPE_F32 = 0, CSA_DTYPE_BF16 = 1 } csa_dtype_t;

/* Sizes of one decode step.  Supported ranges (CSA_ERR_UNSUPPORTED outside):
 *   head_dim, idx_dim in {64, 128}; 1 <= heads <= 64; 1 <= idx_heads <= 64;
 *   1 <= topk <= 4096; win >= 1.  Scoring and Top-K take any q_per_req: a
 *   prefill chunk of T tokens per request is q_per_req = T (the prefill
 *   indexer of "Fix: port the DeepSeek-V4 MoE, hc_pre and prefill fixes to
 *   DSpark", description), each token with its own causal visibility. */
typedef struct {
  int32_t batch;      /* B: requests                                          */
  int32_t q_per_req;  /* S: query tokens per request (p = start_pos[b] + s)    */
  int32_t ratio;      /* R: raw tokens per compressed row (the pages use 4)    */
  int32_t n_cap;      /* compressed rows allocated per request                 */
  int32_t topk;       /* K: IDX_TOPK                                           */
  int32_t win;        /* WIN: raw sliding-window length (includes token p)     */
  int32_t w_cap;      /* ring capacity of the window cache, >= win + S - 1     */
  int32_t heads;      /* H: query heads; one KV head shared by all of them     */
  int32_t head_dim;   /* D                                                     */
  int32_t rope_dim;   /* Dr: even, <= D; the last Dr dims hold RoPE pairs      */
  int32_t idx_heads;  /* Hi: indexer heads                                     */
  int32_t idx_dim;    /* Di: indexer head dim                                  */
  int32_t out_groups; /* G: output head groups, H % G == 0                     */
  int32_t max_len;    /* host bound: max over b of start_pos[b] + S            */
  int32_t dtype;      /* csa_dtype_t                                           */
} csa_shape_t;

/* Paged compressed caches.
 *
 * Instead of a dense [B][n_cap][...] buffer per request, a compressed cache
 * may live in a pool of fixed-size blocks shared by all requests, located
 * through a per-request block table (the cache pools with allocator slot
 * mappings of "Fix: complete DeepSeek V4 TP CSA decode", description; the
 * block-table form is this library's reading).  Logical row j of request b is
 * pool row  block_table[b * blocks_per_req + j / block_size] * block_size
 * + j % block_size.
 *   block_table    [B][blocks_per_req] int32, device memory, 16-byte aligned
 *                  (CSA_ERR_ALIGNMENT otherwise); entries that logical rows
 *                  j < n_vis use must lie in [0, n_blocks)
 *   blocks_per_req >= ceil(n_cap / block_size) (CSA_ERR_CAPACITY otherwise)
 *   block_size     rows per block: a power of two, 16 .. 4096
 *                  (CSA_ERR_BAD_SHAPE otherwise)
 *   n_blocks       blocks in the pool, >= 1; n_blocks * block_size must fit
 *                  int32, and a pool of attention K or V rows must stay below
 *                  2^31 - 4096 bytes (CSA_ERR_UNSUPPORTED otherwise)
 * The struct itself is host memory, read during the call only; a NULL
 * struct or table is CSA_ERR_NULL_PTR. */
typedef struct {
  const int32_t* block_table;
  int32_t blocks_per_req;
  int32_t block_size;
  int64_t n_blocks;
} csa_pages_t;

/* Indexer scores of every visible compressed row.
 *
 * For each query token (b,s) that does not fit (n_vis(p) > K) and each
 * visible row j < n_vis(p):
 *   scores[b][s][j] = sum_{h < Hi} w[b][s][h] * relu(q_idx[b][s][h] . k_idx[b][j])
 * The indexer and its skipping for cache-fitting requests are described on
 * "Perf: skip redundant CSA scoring and fuse gather unpack" (description); the
 * weighted-relu form is the indexer formula of the decode workloads.
 * Products use the input type, sums are float32 (bf16 MFMA, fp32 accumulate).
 *
 *   q_idx  [B][S][Hi][Di]  dtype
 *   w      [B][S][Hi]      float32
 *   k_idx  [B][n_cap][Di]  dtype  (rows >= n_vis are never read)
 *   start_pos [B]          int32
 *   scores [B][S][n_cap]   float32, written only at (non-fitting token, j < n_vis);
 *                          every other entry is left as the caller had it.
 * Requires n_cap >= floor(max_len / R) (else CSA_ERR_CAPACITY).
 */
csa_status_t csa_indexer_score(const csa_shape_t* shape, const void* q_idx, const float* w,
                               const void* k_idx, const int32_t* start_pos, float* scores,
                               void* stream);

/* Indexer scores from an FP8 indexer key cache.
 *
 * Same result contract as csa_indexer_score, with key row j of request b
 * given as OCP FP8 E4M3 codes ("e4m3fn": bias 7, largest finite 448, code
 * S.1111.111 is NaN) and one fp32 scale:
 *   k_idx[b][j][c] = k_scale[b][j] * e4m3(k_idx8[b][j][c])
 * The pages pass the indexer key cache together with its scale ("Fix:
 * complete DeepSeek V4 TP CSA decode", description); the encoding and the
 * per-row granularity are this library's reading.  The codes are widened to
 * bf16 exactly, so products stay exact and sums are float32 as in
 * csa_indexer_score; the scale multiplies each row's head sum.
 *
 *   q_idx   [B][S][Hi][Di]  bf16 (shape->dtype must be CSA_DTYPE_BF16, else
 *                           CSA_ERR_BAD_DTYPE)
 *   w       [B][S][Hi]      float32
 *   k_idx8  [B][n_cap][Di]  uint8 E4M3 codes (NaN codes are outside the contract)
 *   k_scale [B][n_cap]      float32, >= 0 and finite
 *   start_pos, scores       as csa_indexer_score
 */
csa_status_t csa_indexer_score_fp8(const csa_shape_t* shape, const void* q_idx, const float* w,
                                   const uint8_t* k_idx8, const float* k_scale,
                                   const int32_t* start_pos, float* scores, void* stream);

/* csa_indexer_score / csa_indexer_score_fp8 over a paged indexer key cache.
 *
 *   k_pool   [n_blocks][block_size][Di]: keys in shape->dtype, or E4M3 codes
 *            when k_scale is non-NULL
 *   k_scale  NULL, or [n_blocks][block_size] float32 per-row scales (FP8 keys;
 *            then shape->dtype must be CSA_DTYPE_BF16)
 *   pages    the block table of the indexer key cache (see csa_pages_t)
 * Every other argument, and the result, as csa_indexer_score.  Unmapped or
 * out-of-range table entries for visible rows are outside the contract; the
 * device clamps them into the pool so that no access leaves it.
 */
csa_status_t csa_indexer_score_paged(const csa_shape_t* shape, const void* q_idx, const float* w,
                                     const void* k_pool, const float* k_scale,
                                     const csa_pages_t* pages, const int32_t* start_pos,
                                     float* scores, void* stream);

/* Workspace bytes csa_topk needs for this shape (0 means none).  Launches of
 * fewer than 2048 query tokens whose rows can exceed 32768 visible entries
 * (K <= 1024, at most a quarter of the row) split each row over several
 * workgroups and merge their candidates; their candidates and counts live in
 * the workspace (contents need no initialisation). */
size_t csa_topk_workspace_bytes(const csa_shape_t* shape);

/* Causal Top-K selection, with the fits-in-Top-K bypass.
 *
 * For a token with n_vis(p) <= K (it fits): topk_idx = 0, 1, ..., n_vis-1,
 * then -1 up to K; scores are not read.  Otherwise: the K rows j < n_vis with
 * the largest scores, where equal scores (compared as values, so -0 == +0)
 * go to the lower index; the chosen indices are written in ascending order.
 * The bypass is the one on "Perf: skip redundant CSA scoring and fuse gather
 * unpack" (description: bounded indices instead of scoring and sorting); the
 * need to hold for widths past 256 is stated on "Fix: port the DeepSeek-V4
 * MoE, hc_pre and prefill fixes to DSpark" (description, indexer top-k item).
 * The result is bit-exact: it depends on the score values only.
 * NaN scores are outside the contract.
 *
 *   scores   [B][S][n_cap] float32 (read only at j < n_vis of non-fitting tokens)
 *   topk_idx [B][S][K]     int32 output
 * ws: at least csa_topk_workspace_bytes() bytes, 16-byte aligned (may be NULL
 * when that is 0; CSA_ERR_WORKSPACE when missing or smaller).
 * Requires n_cap >= floor(max_len / R).
 */
csa_status_t csa_topk(const csa_shape_t* shape, const float* scores, const int32_t* start_pos,
                      int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes csa_sparse_attn_decode needs for this shape (split
 * partials).  0 for shapes that a single workgroup per token finishes by
 * itself: window and Top-K rows within 12 waves of at most 64 rows each
 * (fp32 rows of 128 dims: 16 rows), at most 4096 tokens, and at least 384
 * such waves in all.  Its contents need no initialisation; calls that overlap
 * in time must not share a workspace. */
size_t csa_sparse_attn_workspace_bytes(const csa_shape_t* shape);

/* Two-stream sparse attention of every query token, merged, RoPE undone, packed.
 *
 * For token (b,s) at position p and each head h (one KV head shared by all):
 *   window stream:     raw positions max(0, p-WIN+1) .. p, read from the ring
 *                      slot pos mod w_cap of k_win / v_win;
 *   compressed stream: every entry j of topk_idx[b][s][:] with 0 <= j < n_cap
 *                      (other entries are padding), rows of k_cmp / v_cmp;
 *   each stream: logits l = softmax_scale * (q[b][s][h] . k), its own max and
 *   sum; the two are merged by their maxima and sums (an empty stream weighs
 *   nothing); the output o = merged sum / merged denominator.
 * Then the last Dr dims, taken as pairs (D-Dr+2i, D-Dr+2i+1), are turned back
 * by the position's angle: x' = x*cos + y*sin, y' = -x*sin + y*cos with
 * cos = rope_cos[p][i], sin = rope_sin[p][i]; the value is rounded once to
 * dtype and head h is written to group g = h / (H/G) at slot h mod (H/G).
 * The merge, inverse RoPE and grouped packing follow "Perf: fuse HCA merge,
 * inverse RoPE, and packing" (description, changes table); the window and the
 * bounded row count WIN + min(n_vis, K) follow "Fix: port the DeepSeek-V4 MoE,
 * hc_pre and prefill fixes to DSpark" (description, last item).
 * Every reduction is in a fixed order (no floating-point atomics), so two
 * calls on the same inputs give bitwise identical outputs.
 *
 *   q        [B][S][H][D]        dtype (RoPE already applied upstream)
 *   k_win, v_win [B][w_cap][D]   dtype
 *   k_cmp, v_cmp [B][n_cap][D]   dtype
 *   topk_idx [B][S][K]           int32 (ascending or not; duplicates count twice)
 *   rope_cos, rope_sin [rope_rows][Dr/2] float32, rope_rows >= max_len
 *   out      [G][B*S][(H/G)*D]   dtype output
 *   ws       at least csa_sparse_attn_workspace_bytes(shape) bytes, 16-byte
 *            aligned (may be NULL when that is 0)
 * Requires w_cap >= win + S - 1.  One request's slice of a K or V cache
 * (n_cap or w_cap rows) must stay below 2^31 - 4096 bytes, else
 * CSA_ERR_UNSUPPORTED.
 */
csa_status_t csa_sparse_attn_decode(const csa_shape_t* shape, const void* q, const void* k_win,
                                    const void* v_win, const void* k_cmp, const void* v_cmp,
                                    const int32_t* topk_idx, const int32_t* start_pos,
                                    const float* rope_cos, const float* rope_sin,
                                    int32_t rope_rows, float softmax_scale, void* out, void* ws,
                                    size_t ws_bytes, void* stream);

/* csa_sparse_attn_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, checks and result as csa_sparse_attn_decode,
 * without the workspace: the split partials live in a static device array of
 * the library (csa_sparse_attn_noalloc_max_workspace_bytes() bytes, 32 MiB;
 * each GPU the library runs on holds its own copy until the process ends).
 * The call allocates nothing and frees nothing.
 *   - A shape whose workspace (csa_sparse_attn_workspace_bytes) exceeds that
 *     size is refused with CSA_ERR_WORKSPACE before anything is enqueued.
 *     A shape whose workspace is 0 does not touch the array.
 *   - The first call on a GPU looks up that GPU's copy of the array (the
 *     GPU that runs `stream`); CSA_ERR_LAUNCH if the lookup fails.
 *   - Every call on one GPU shares that GPU's array and leaves the last
 *     call's partials in it: calls that overlap in time on one GPU (other
 *     streams, other threads) race and give undefined results.  Calls
 *     ordered on one stream are safe.
 */
csa_status_t csa_sparse_attn_decode_noalloc(const csa_shape_t* shape, const void* q,
                                            const void* k_win, const void* v_win,
                                            const void* k_cmp, const void* v_cmp,
                                            const int32_t* topk_idx, const int32_t* start_pos,
                                            const float* rope_cos, const float* rope_sin,
                                            int32_t rope_rows, float softmax_scale, void* out,
                                            void* stream);

/* Size of the static array behind csa_sparse_attn_decode_noalloc (bytes). */
size_t csa_sparse_attn_noalloc_max_workspace_bytes(void);

/* Window-cache writeback of the step's new tokens, by slot mapping.
 *
 * Copies the K and V rows of every new token t = b*S + s to row
 * slot_mapping[t] of the caches, bit for bit; every entry is committed for any
 * token count (the writeback of "Perf: parallelize the DSpark TP-4 SWA decode
 * hot tasks", description, and its review: the tail of a partial tile must not
 * be dropped).  A slot outside [0, n_slots) is padding and writes nothing.
 * Two entries naming the same slot leave that row with either one.
 * With the per-request rings of csa_sparse_attn_decode seen as one flat cache
 * [B*w_cap][D], token (b, s) at position p belongs in row b*w_cap + p mod w_cap;
 * writing it there before the attention call makes it part of its own window.
 * Uses shape->batch, q_per_req, head_dim and dtype only.
 *
 *   k_new, v_new     [B*S][D]     dtype
 *   slot_mapping     [B*S]        int32
 *   k_cache, v_cache [n_slots][D] dtype, updated in place
 * Requires D * element size to be a multiple of 16 bytes (else
 * CSA_ERR_UNSUPPORTED).
 */
csa_status_t csa_swa_writeback(const csa_shape_t* shape, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                               int64_t n_slots, void* stream);

/* csa_sparse_attn_decode with the compressed K and V caches paged, and
 * optionally the window rings too.  The pages keep their caches in
 * allocator-mapped pools ("Fix: complete DeepSeek V4 TP CSA decode",
 * description) and commit window rows through a slot mapping into one flat
 * cache ("Perf: parallelize the DSpark TP-4 SWA decode hot tasks", review);
 * reading the window through a block table is this library's reading.
 *
 *   k_pool, v_pool [n_blocks][block_size][D] dtype
 *   pages          the block table of the compressed K/V cache (see
 *                  csa_pages_t); entries reached by valid Top-K indices must
 *                  lie in [0, n_blocks) (outside the contract otherwise; the
 *                  device clamps them into the pool)
 *   win_pages      NULL: k_win / v_win are the per-request rings
 *                  [B][w_cap][D].  Otherwise the block table of the window
 *                  rings and k_win / v_win are pools
 *                  [win n_blocks][win block_size][D]: ring slot r (position
 *                  pos, r = pos mod w_cap) of request b is pool row
 *                  block_table[b * blocks_per_req + r / block_size]
 *                  * block_size + r % block_size, and blocks_per_req *
 *                  block_size >= w_cap (CSA_ERR_CAPACITY otherwise).  The
 *                  other csa_pages_t rules apply as for `pages`.
 * csa_swa_writeback places a step's new rows in either layout: its slot
 * mapping names the pool row of each token's ring slot.  Every other
 * argument, the workspace query and the result as csa_sparse_attn_decode.
 */
csa_status_t csa_sparse_attn_decode_paged(const csa_shape_t* shape, const void* q,
                                          const void* k_win, const void* v_win, const void* k_pool,
                                          const void* v_pool, const csa_pages_t* pages,
                                          const int32_t* topk_idx, const int32_t* start_pos,
                                          const float* rope_cos, const float* rope_sin,
                                          int32_t rope_rows, float softmax_scale, void* out,
                                          void* ws, size_t ws_bytes, void* stream,
                                          const csa_pages_t* win_pages);

/* Static text for a status code (never NULL). */
const char* csa_status_string(csa_status_t status);

/* ABI version of this header (bumped on any incompatible change). */
int32_t csa_abi_version(void);

#define CSA_ABI_VERSION 2

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
