// extern "C" surface of libcsa: host-side argument checks, workspace sizing
// and dispatch to the kernels.  Every check runs before anything is enqueued,
// so a refused call leaves every output untouched; none of them touches the
// GPU, so they behave the same on a machine without one.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/csa.h"
#include "kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks every call shares.  Sets *empty when there is no query token.
csa_status_t check_common(const csa_shape_t* sh, bool* empty) {
  if (!sh) return CSA_ERR_NULL_PTR;
  if (sh->dtype != CSA_DTYPE_F32 && sh->dtype != CSA_DTYPE_BF16) return CSA_ERR_BAD_DTYPE;
  if (sh->batch < 0 || sh->q_per_req < 0) return CSA_ERR_BAD_SHAPE;
  *empty = sh->batch == 0 || sh->q_per_req == 0;
  if (*empty) return CSA_OK;
  if (sh->ratio < 1 || sh->n_cap < 1 || sh->topk < 1 || sh->win < 1 || sh->w_cap < 1 ||
      sh->heads < 1 || sh->head_dim < 1 || sh->rope_dim < 0 || sh->idx_heads < 1 ||
      sh->idx_dim < 1 || sh->out_groups < 1 || sh->max_len < sh->q_per_req)
    return CSA_ERR_BAD_SHAPE;
  if (sh->topk > 4096) return CSA_ERR_UNSUPPORTED;
  // int32 index arithmetic inside the kernels
  if ((int64_t)sh->batch * sh->q_per_req * sh->topk > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

csa_status_t check_selection(const csa_shape_t* sh) {
  if (sh->n_cap < sh->max_len / sh->ratio) return CSA_ERR_CAPACITY;
  return CSA_OK;
}

csa_status_t to_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH; }

// A block table and its pool: block size a power of two in [16, 4096], enough
// blocks per request for `rows` logical rows (n_cap, or w_cap for a window
// ring), a pool whose row count fits int32 and whose rows of row_bytes stay
// below max_pool_bytes.
csa_status_t check_pages(const csa_shape_t* sh, const csa_pages_t* pg, int64_t rows, int64_t row_bytes,
                         int64_t max_pool_bytes, int* shift) {
  if (!pg || !pg->block_table) return CSA_ERR_NULL_PTR;
  const int32_t bs = pg->block_size;
  if (bs < 16 || bs > 4096 || (bs & (bs - 1))) return CSA_ERR_BAD_SHAPE;
  if (pg->n_blocks < 1 || pg->blocks_per_req < 1) return CSA_ERR_BAD_SHAPE;
  if ((int64_t)pg->blocks_per_req * bs < rows) return CSA_ERR_CAPACITY;
  // (divisions, so that no product of caller sizes can overflow)
  if (pg->n_blocks > INT32_MAX / bs || pg->n_blocks * bs > max_pool_bytes / row_bytes)
    return CSA_ERR_UNSUPPORTED;
  if ((int64_t)sh->batch * pg->blocks_per_req > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(pg->block_table) & 15u) != 0) return CSA_ERR_ALIGNMENT;
  *shift = __builtin_ctz((unsigned)bs);
  return CSA_OK;
}

// Split partials of csa_sparse_attn_decode_noalloc: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in for the
// symbol): the device address of each GPU's copy is looked up once with
// hipGetSymbolAddress, with that GPU current, and kept per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU that runs `stream` (NULL on failure).
void* scratch_address(hipStream_t stream) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

csa_status_t csa_indexer_score(const csa_shape_t* sh, const void* q_idx, const float* w,
                               const void* k_idx, const int32_t* start_pos, float* scores,
                               void* stream) {
  bool empty = false;
  csa_status_t st = check_common(sh, &empty);
  if (st != CSA_OK || empty) return st;
  if (!q_idx || !w || !k_idx || !start_pos || !scores) return CSA_ERR_NULL_PTR;
  if (sh->idx_dim != 64 && sh->idx_dim != 128) return CSA_ERR_UNSUPPORTED;
  if (sh->idx_heads > 64 || (sh->q_per_req + 63) / 64 > 65535) return CSA_ERR_UNSUPPORTED;
  if ((st = check_selection(sh)) != CSA_OK) return st;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(start_pos) ||
      !aligned16(scores))
    return CSA_ERR_ALIGNMENT;
  csa::ScoreArgs a{q_idx, w, k_idx, start_pos, scores, sh->batch, sh->q_per_req, sh->idx_heads,
                   sh->idx_dim, sh->n_cap, sh->topk, sh->ratio, sh->max_len, sh->dtype, nullptr, 0,
                   nullptr, 0, 0, 0};
  (void)hipGetLastError();  // report only what these launches cause
  return to_status(csa::launch_indexer_score(a, static_cast<hipStream_t>(stream)));
}

csa_status_t csa_indexer_score_fp8(const csa_shape_t* sh, const void* q_idx, const float* w,
                                   const uint8_t* k_idx8, const float* k_scale,
                                   const int32_t* start_pos, float* scores, void* stream) {
  bool empty = false;
  csa_status_t st = check_common(sh, &empty);
  if (st != CSA_OK || empty) return st;
  if (!q_idx || !w || !k_idx8 || !k_scale || !start_pos || !scores) return CSA_ERR_NULL_PTR;
  if (sh->dtype != CSA_DTYPE_BF16) return CSA_ERR_BAD_DTYPE;  // bf16 queries only
  if (sh->idx_dim != 64 && sh->idx_dim != 128) return CSA_ERR_UNSUPPORTED;
  if (sh->idx_heads > 64 || (sh->q_per_req + 63) / 64 > 65535) return CSA_ERR_UNSUPPORTED;
  if ((st = check_selection(sh)) != CSA_OK) return st;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx8) || !aligned16(k_scale) ||
      !aligned16(start_pos) || !aligned16(scores))
    return CSA_ERR_ALIGNMENT;
  csa::ScoreArgs a{q_idx, w, k_idx8, start_pos, scores, sh->batch, sh->q_per_req, sh->idx_heads,
                   sh->idx_dim, sh->n_cap, sh->topk, sh->ratio, sh->max_len, sh->dtype, k_scale, 0,
                   nullptr, 0, 0, 0};
  (void)hipGetLastError();  // report only what these launches cause
  return to_status(csa::launch_indexer_score(a, static_cast<hipStream_t>(stream)));
}

size_t csa_topk_workspace_bytes(const csa_shape_t* sh) {
  bool empty = false;
  if (check_common(sh, &empty) != CSA_OK || empty || check_selection(sh) != CSA_OK) return 0;
  return csa::topk_plan(sh->batch, sh->q_per_req, sh->n_cap, sh->topk, sh->ratio, sh->max_len).ws_bytes;
}

csa_status_t csa_topk(const csa_shape_t* sh, const float* scores, const int32_t* start_pos,
                      int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  csa_status_t st = check_common(sh, &empty);
  if (st != CSA_OK || empty) return st;
  if (!scores || !start_pos || !topk_idx) return CSA_ERR_NULL_PTR;
  if ((st = check_selection(sh)) != CSA_OK) return st;
  const csa::TopkPlan pl =
      csa::topk_plan(sh->batch, sh->q_per_req, sh->n_cap, sh->topk, sh->ratio, sh->max_len);
  if (pl.ws_bytes && (!ws || ws_bytes < pl.ws_bytes)) return CSA_ERR_WORKSPACE;
  if (!aligned16(scores) || !aligned16(start_pos) || !aligned16(topk_idx) || (pl.ws_bytes && !aligned16(ws)))
    return CSA_ERR_ALIGNMENT;
  csa::TopkArgs a{scores, start_pos, topk_idx, sh->batch, sh->q_per_req, sh->n_cap, sh->topk,
                  sh->ratio, sh->max_len, nullptr, nullptr, 0, 0, 0};
  if (pl.two_pass) {
    char* w = static_cast<char*>(ws);
    a.cand = reinterpret_cast<uint2*>(w);
    a.cand_count = reinterpret_cast<int32_t*>(w + pl.cand_bytes);
    a.chunk_keys = pl.chunk_keys;
    a.n_chunks = pl.n_chunks;
    a.chunk_cap = pl.chunk_cap;
  }
  (void)hipGetLastError();
  return to_status(csa::launch_topk(a, static_cast<hipStream_t>(stream)));
}

size_t csa_sparse_attn_workspace_bytes(const csa_shape_t* sh) {
  bool empty = false;
  if (check_common(sh, &empty) != CSA_OK || empty) return 0;
  return csa::attn_plan(sh->batch, sh->q_per_req, sh->heads, sh->head_dim, sh->win, sh->topk, sh->dtype).ws_bytes;
}

static csa_status_t attn_decode(const csa_shape_t* sh, const void* q, const void* k_win,
                                const void* v_win, const void* k_cmp, const void* v_cmp,
                                const int32_t* topk_idx, const int32_t* start_pos,
                                const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                                float softmax_scale, void* out, void* ws, size_t ws_bytes,
                                void* stream, const csa_pages_t* pages, int block_shift,
                                const csa_pages_t* win_pages, int win_shift,
                                bool use_scratch = false) {
  bool empty = false;
  csa_status_t st = check_common(sh, &empty);
  if (st != CSA_OK || empty) return st;
  if (!q || !k_win || !v_win || !k_cmp || !v_cmp || !topk_idx || !start_pos || !out)
    return CSA_ERR_NULL_PTR;
  if (sh->rope_dim > 0 && (!rope_cos || !rope_sin)) return CSA_ERR_NULL_PTR;
  if ((sh->rope_dim & 1) || sh->rope_dim > sh->head_dim || sh->heads % sh->out_groups != 0)
    return CSA_ERR_BAD_SHAPE;
  if (!std::isfinite(softmax_scale)) return CSA_ERR_BAD_SHAPE;
  if (sh->head_dim != 64 && sh->head_dim != 128) return CSA_ERR_UNSUPPORTED;
  if (sh->heads > 64) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)sh->w_cap < (int64_t)sh->win + sh->q_per_req - 1) return CSA_ERR_CAPACITY;
  if (sh->rope_dim > 0 && rope_rows < sh->max_len) return CSA_ERR_CAPACITY;
  {  // one request's cache slice is addressed with 32-bit byte offsets
    const int64_t row = (int64_t)sh->head_dim * (sh->dtype == CSA_DTYPE_BF16 ? 2 : 4);
    if ((int64_t)sh->n_cap * row > csa::kMaxSliceBytes || (int64_t)sh->w_cap * row > csa::kMaxSliceBytes)
      return CSA_ERR_UNSUPPORTED;
  }
  const csa::AttnPlan pl =
      csa::attn_plan(sh->batch, sh->q_per_req, sh->heads, sh->head_dim, sh->win, sh->topk, sh->dtype);
  if (use_scratch ? pl.ws_bytes > kScratchBytes : (pl.ws_bytes && (!ws || ws_bytes < pl.ws_bytes)))
    return CSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_win) || !aligned16(v_win) || !aligned16(k_cmp) ||
      !aligned16(v_cmp) || !aligned16(topk_idx) || !aligned16(start_pos) || !aligned16(out) ||
      (!use_scratch && pl.ws_bytes && !aligned16(ws)) || (rope_cos && !aligned16(rope_cos)) ||
      (rope_sin && !aligned16(rope_sin)))
    return CSA_ERR_ALIGNMENT;
  if (use_scratch && pl.ws_bytes) {  // every check has passed: only now touch the device
    ws = scratch_address(static_cast<hipStream_t>(stream));
    if (!ws) return CSA_ERR_LAUNCH;
  }
  char* wsb = static_cast<char*>(ws);
  csa::AttnArgs a{};
  a.q = q;
  a.k_win = k_win;
  a.v_win = v_win;
  a.k_cmp = k_cmp;
  a.v_cmp = v_cmp;
  a.topk_idx = topk_idx;
  a.start_pos = start_pos;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.out = out;
  a.ws_o = reinterpret_cast<float*>(wsb);
  a.ws_ml = reinterpret_cast<float*>(wsb + pl.ws_o_bytes);
  a.batch = sh->batch;
  a.q_per_req = sh->q_per_req;
  a.n_cap = sh->n_cap;
  a.topk = sh->topk;
  a.win = sh->win;
  a.w_cap = sh->w_cap;
  a.heads = sh->heads;
  a.head_dim = sh->head_dim;
  a.rope_dim = sh->rope_dim;
  a.out_groups = sh->out_groups;
  a.max_len = sh->max_len;
  a.dtype = sh->dtype;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.chunks_per_wave = pl.chunks_per_wave;
  a.n_split_win = pl.n_split_win;
  a.n_split_cmp = pl.n_split_cmp;
  a.waves_win = pl.waves_win;
  a.waves_cmp = pl.waves_cmp;
  if (pages) {
    a.block_table = pages->block_table;
    a.blocks_per_req = pages->blocks_per_req;
    a.block_shift = block_shift;
    a.n_blocks = pages->n_blocks;
  }
  if (win_pages) {
    a.win_table = win_pages->block_table;
    a.win_blocks_per_req = win_pages->blocks_per_req;
    a.win_shift = win_shift;
    a.win_n_blocks = win_pages->n_blocks;
  }
  (void)hipGetLastError();
  return to_status(csa::launch_sparse_attn(a, static_cast<hipStream_t>(stream)));
}

csa_status_t csa_sparse_attn_decode(const csa_shape_t* sh, const void* q, const void* k_win,
                                    const void* v_win, const void* k_cmp, const void* v_cmp,
                                    const int32_t* topk_idx, const int32_t* start_pos,
                                    const float* rope_cos, const float* rope_sin,
                                    int32_t rope_rows, float softmax_scale, void* out, void* ws,
                                    size_t ws_bytes, void* stream) {
  return attn_decode(sh, q, k_win, v_win, k_cmp, v_cmp, topk_idx, start_pos, rope_cos, rope_sin,
                     rope_rows, softmax_scale, out, ws, ws_bytes, stream, nullptr, 0, nullptr, 0);
}

csa_status_t csa_sparse_attn_decode_noalloc(const csa_shape_t* sh, const void* q,
                                            const void* k_win, const void* v_win,
                                            const void* k_cmp, const void* v_cmp,
                                            const int32_t* topk_idx, const int32_t* start_pos,
                                            const float* rope_cos, const float* rope_sin,
                                            int32_t rope_rows, float softmax_scale, void* out,
                                            void* stream) {
  return attn_decode(sh, q, k_win, v_win, k_cmp, v_cmp, topk_idx, start_pos, rope_cos, rope_sin,
                     rope_rows, softmax_scale, out, nullptr, 0, stream, nullptr, 0, nullptr, 0,
                     /*use_scratch=*/true);
}

size_t csa_sparse_attn_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

csa_status_t csa_swa_writeback(const csa_shape_t* sh, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                               int64_t n_slots, void* stream) {
  if (!sh) return CSA_ERR_NULL_PTR;
  if (sh->dtype != CSA_DTYPE_F32 && sh->dtype != CSA_DTYPE_BF16) return CSA_ERR_BAD_DTYPE;
  if (sh->batch < 0 || sh->q_per_req < 0 || sh->head_dim < 1 || n_slots < 0) return CSA_ERR_BAD_SHAPE;
  if (sh->batch == 0 || sh->q_per_req == 0) return CSA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return CSA_ERR_NULL_PTR;
  const int64_t row = (int64_t)sh->head_dim * (sh->dtype == CSA_DTYPE_BF16 ? 2 : 4);
  const int64_t tokens = (int64_t)sh->batch * sh->q_per_req;
  if (row % 16 != 0 || tokens * (row / 16) > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(slot_mapping) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return CSA_ERR_ALIGNMENT;
  const csa::WritebackArgs a{k_new, v_new, slot_mapping, k_cache, v_cache, n_slots, (int)tokens, (int)row};
  (void)hipGetLastError();
  return to_status(csa::launch_swa_writeback(a, static_cast<hipStream_t>(stream)));
}

csa_status_t csa_indexer_score_paged(const csa_shape_t* sh, const void* q_idx, const float* w,
                                     const void* k_pool, const float* k_scale,
                                     const csa_pages_t* pages, const int32_t* start_pos,
                                     float* scores, void* stream) {
  bool empty = false;
  csa_status_t st = check_common(sh, &empty);
  if (st != CSA_OK || empty) return st;
  if (!q_idx || !w || !k_pool || !start_pos || !scores) return CSA_ERR_NULL_PTR;
  if (k_scale && sh->dtype != CSA_DTYPE_BF16) return CSA_ERR_BAD_DTYPE;  // FP8 keys: bf16 queries
  if (sh->idx_dim != 64 && sh->idx_dim != 128) return CSA_ERR_UNSUPPORTED;
  if (sh->idx_heads > 64 || (sh->q_per_req + 63) / 64 > 65535) return CSA_ERR_UNSUPPORTED;
  if ((st = check_selection(sh)) != CSA_OK) return st;
  int shift = 0;
  const int64_t row = k_scale ? sh->idx_dim : (int64_t)sh->idx_dim * (sh->dtype == CSA_DTYPE_BF16 ? 2 : 4);
  if ((st = check_pages(sh, pages, sh->n_cap, row, INT64_MAX, &shift)) != CSA_OK) return st;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_pool) || !aligned16(start_pos) ||
      !aligned16(scores) || (k_scale && !aligned16(k_scale)))
    return CSA_ERR_ALIGNMENT;
  csa::ScoreArgs a{q_idx, w, k_pool, start_pos, scores, sh->batch, sh->q_per_req, sh->idx_heads,
                   sh->idx_dim, sh->n_cap, sh->topk, sh->ratio, sh->max_len, sh->dtype, k_scale, 0,
                   pages->block_table, pages->blocks_per_req, shift, pages->n_blocks};
  (void)hipGetLastError();
  return to_status(csa::launch_indexer_score(a, static_cast<hipStream_t>(stream)));
}

csa_status_t csa_sparse_attn_decode_paged(const csa_shape_t* sh, const void* q,
                                          const void* k_win, const void* v_win, const void* k_pool,
                                          const void* v_pool, const csa_pages_t* pages,
                                          const int32_t* topk_idx, const int32_t* start_pos,
                                          const float* rope_cos, const float* rope_sin,
                                          int32_t rope_rows, float softmax_scale, void* out,
                                          void* ws, size_t ws_bytes, void* stream,
                                          const csa_pages_t* win_pages) {
  bool empty = false;
  csa_status_t st = check_common(sh, &empty);
  if (st != CSA_OK || empty) return st;
  if (!pages) return CSA_ERR_NULL_PTR;
  int shift = 0, win_shift = 0;
  const int64_t row = (int64_t)sh->head_dim * (sh->dtype == CSA_DTYPE_BF16 ? 2 : 4);
  if ((st = check_pages(sh, pages, sh->n_cap, row, csa::kMaxSliceBytes, &shift)) != CSA_OK) return st;
  if (win_pages &&
      (st = check_pages(sh, win_pages, sh->w_cap, row, csa::kMaxSliceBytes, &win_shift)) != CSA_OK)
    return st;
  return attn_decode(sh, q, k_win, v_win, k_pool, v_pool, topk_idx, start_pos, rope_cos, rope_sin,
                     rope_rows, softmax_scale, out, ws, ws_bytes, stream, pages, shift, win_pages,
                     win_shift);
}

const char* csa_status_string(csa_status_t s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL_PTR: return "a required pointer is NULL";
    case CSA_ERR_BAD_SHAPE: return "invalid or inconsistent sizes";
    case CSA_ERR_BAD_DTYPE: return "unknown dtype";
    case CSA_ERR_CAPACITY: return "cache, ring or RoPE table capacity too small for max_len";
    case CSA_ERR_ALIGNMENT: return "a tensor pointer is not 16-byte aligned";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_LAUNCH: return "HIP kernel launch failed";
    case CSA_ERR_UNSUPPORTED: return "sizes outside the range the kernels are built for";
  }
  return "unknown status";
}

int32_t csa_abi_version(void) { return CSA_ABI_VERSION; }

}  // extern "C"
