// Launch entry points of the CSA decode kernels (internal to libcsa).
// Host-side argument checking happens in api.hip before any of these run;
// each launcher only picks a kernel instantiation and enqueues it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

struct ScoreArgs {
  const void* q_idx;        // [B][S][Hi][Di]
  const float* w;           // [B][S][Hi]
  const void* k_idx;        // [B][n_cap][Di] in dtype, or E4M3 codes when k_scale is set
  const int32_t* start_pos; // [B]
  float* scores;            // [B][S][n_cap]
  int batch, q_per_req, idx_heads, idx_dim, n_cap, topk, ratio, max_len, dtype;
  const float* k_scale;     // [B][n_cap] per-row scale of an FP8 key cache, else null
  int tok_per_block;        // query tokens per workgroup (set by the launcher)
  // paged key cache (block_table non-null): k_idx / k_scale are pools of
  // (1 << block_shift)-row blocks; logical row j of request b is pool row
  // block_table[b * blocks_per_req + (j >> block_shift)] << block_shift | (j & mask)
  const int32_t* block_table;
  int blocks_per_req, block_shift;
  int64_t n_blocks;
  int gemm_key_blocks, gemm_row_blocks;  // GEMM-shaped prefill grid (set by the launcher)
  int stream_scores;        // decode-shaped kernel's score stores (set by the launcher): 0 buffer
                            // stores, 1 non-temporal buffer stores, 2 non-temporal global stores
                            // (rows past 32-bit offsets)
};

struct TopkArgs {
  const float* scores;      // [B][S][n_cap]
  const int32_t* start_pos; // [B]
  int32_t* topk_idx;        // [B][S][K]
  int batch, q_per_req, n_cap, topk, ratio, max_len;
  // two-pass selection (workspace): candidates of chunk c of token t at
  // cand[(t * n_chunks + c) * chunk_cap ..], their count at
  // cand_count[t * n_chunks + c] (-1: more than chunk_cap)
  uint2* cand;
  int32_t* cand_count;
  int chunk_keys, n_chunks, chunk_cap;
};

// Plan of the Top-K launch; a function of the shape only, so the workspace
// query and the launch always agree.
struct TopkPlan {
  bool two_pass;        // rows split over several workgroups, then merged
  int chunk_keys;       // keys per chunk workgroup (256 threads x keys per thread)
  int n_chunks, chunk_cap;
  size_t cand_bytes, count_bytes, ws_bytes;
};

TopkPlan topk_plan(int batch, int q_per_req, int n_cap, int topk, int ratio, int max_len);

struct AttnArgs {
  const void* q;            // [B][S][H][D]
  const void* k_win;        // [B][w_cap][D]
  const void* v_win;
  const void* k_cmp;        // [B][n_cap][D]
  const void* v_cmp;
  const int32_t* topk_idx;  // [B][S][K]
  const int32_t* start_pos; // [B]
  const float* rope_cos;    // [rope_rows][Dr/2]
  const float* rope_sin;
  void* out;                // [G][B*S][(H/G)*D]
  float* ws_o;              // [B*S][n_split][H][D]   split partial sums
  float* ws_ml;             // [B*S][n_split][H][2]   split (max, sum), base-2 logits
  int batch, q_per_req, n_cap, topk, win, w_cap, heads, head_dim, rope_dim, out_groups,
      max_len, dtype;
  float scale_log2;         // softmax_scale * log2(e)
  int chunks_per_wave, n_split_win, n_split_cmp;
  // one workgroup per token (waves_win + waves_cmp > 0): that many waves walk
  // the window and the Top-K list; no split partials
  int waves_win, waves_cmp;
  // paged compressed K/V (block_table non-null): k_cmp / v_cmp are pools, as
  // for ScoreArgs
  const int32_t* block_table;
  int blocks_per_req, block_shift;
  int64_t n_blocks;
  // paged window (win_table non-null): k_win / v_win are pools and ring slot
  // r of request b is pool row
  // win_table[b * win_blocks_per_req + (r >> win_shift)] << win_shift | (r & mask)
  const int32_t* win_table;
  int win_blocks_per_req, win_shift;
  int64_t win_n_blocks;
};

struct WritebackArgs {
  const void* k_new;           // [T][D] new rows (T = B*S)
  const void* v_new;
  const int32_t* slot_mapping; // [T] destination row, padding outside [0, n_slots)
  void* k_cache;               // [n_slots][D]
  void* v_cache;
  int64_t n_slots;
  int n_tokens, row_bytes;     // row_bytes: a multiple of 16
};

// Split plan of the attention kernel; a function of the shape only, so the
// workspace query and the launch always agree.
struct AttnPlan {
  int chunks_per_wave;  // 16-row chunks per wave
  // one workgroup per token: waves per stream (0, 0 for the split kernels)
  int waves_win, waves_cmp;
  // split kernels: 4 waves per workgroup
  int rows_per_split;   // 64 * chunks_per_wave
  int n_split_win, n_split_cmp;
  size_t ws_o_floats, ws_ml_floats;
  size_t ws_o_bytes, ws_ml_bytes, ws_bytes;
};

AttnPlan attn_plan(int batch, int q_per_req, int heads, int head_dim, int win, int topk, int dtype);

// Largest per-request K or V cache slice (bytes) the attention kernel
// addresses: offsets are 32-bit and out-of-range rows use offsets >= 2^31.
constexpr int64_t kMaxSliceBytes = 0x7FFFF000LL;

hipError_t launch_indexer_score(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);
hipError_t launch_swa_writeback(const WritebackArgs& a, hipStream_t stream);

}  // namespace csa
