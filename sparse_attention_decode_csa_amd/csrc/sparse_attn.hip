// Two-stream sparse attention for one decode step, with the stream merge,
// inverse RoPE and grouped packing fused into one epilogue pass.
//
// Streams per query token (one KV head shared by all H query heads):
//   window     raw positions max(0, p-WIN+1) .. p from the ring k_win/v_win
//              (slot = pos mod w_cap);
//   compressed the rows named by the token's Top-K list (entries outside
//              [0, n_cap) are padding).
// Each stream keeps its own softmax max and sum; the two are then merged, the
// RoPE half of the output is turned back by the query position's angle, and
// heads are packed into G groups ("Perf: fuse HCA merge, inverse RoPE, and
// packing", description and changes table).  The row bound per token is
// WIN + min(n_vis, K) ("Fix: port the DeepSeek-V4 MoE, hc_pre and prefill
// fixes to DSpark", description, last item).
//
// Design on gfx950:
//   attn_split_kernel: a workgroup of 4 waves owns one (token, split), i.e.
//   up to 4 * 16 * CPW consecutive entries of ONE stream; each wave owns a
//   contiguous run of 16 * CPW of them and walks it in 16-row chunks.
//   - Latency first: the wave fetches the row numbers of its whole run with a
//     single load (one Top-K entry, or one ring slot, per lane) and hands them
//     to the lanes that need them with cross-lane moves, so no chunk waits on
//     an index load; the next chunk's K/V loads are issued before the current
//     chunk is computed (one chunk of prefetch, all in registers).
//   - K and V are read with buffer loads against a per-request range; a row
//     that is padding or past the end gets an out-of-range offset, which the
//     hardware answers with zeros without touching memory.
//   - logits^T = K q^T (16x16x32 bf16 MFMA, or 16x16x4 fp32) leaves lane
//     (head n, group g) with rows 4g..4g+3 of the chunk, which is exactly the
//     B operand of the 16x16x16 PV product O^T += V^T P^T.  Its A operand
//     takes V straight from registers: lane (m, g) loads rows 4g..4g+3 at
//     dims [m*D/16, (m+1)*D/16) and output row m of d-tile t stands for dim
//     m*D/16 + t.  No LDS round trip and no transpose for V.
//   - The 4 waves' (max, sum, O) are merged through LDS in fixed wave order
//     into one split partial in the workspace.
//   attn_finish_kernel: one thread per (token, head, dim pair) merges the
//   window splits in ascending order, the compressed splits in ascending
//   order, then the two streams, normalises, applies the inverse RoPE rotation
//   in fp32, rounds once and writes the packed group layout.
// No floating-point atomics anywhere: every reduction has a fixed order, so
// results are bitwise reproducible.  Logits are kept in base 2 (scale * log2 e
// folded into the scale) so every exponential is one v_exp_f32.
#include "device_common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kChunk = 16;  // rows per MFMA chunk
constexpr int kWaves = 4;
constexpr int kTokenMaxWaves = 12;  // waves of the one-workgroup-per-token kernel
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any valid range

template <typename T, int D>
struct AttnGeo {
  static constexpr int ES = sizeof(T);
  static constexpr int ROW = D * ES;            // bytes per K or V row
  static constexpr int CH = ROW / 64;           // K: 16-byte loads per lane per chunk
  static constexpr int VB = ROW / 16;           // V: bytes per lane per row (D/16 elements)
  static constexpr int VW = VB / 4;             // V: dwords per lane per row
  static constexpr int DT = D / 16;             // output d tiles
  static constexpr int MO_STRIDE = D + 4;       // floats per (wave, head) row of the merge area
  static_assert(CH >= 1 && VW >= 2, "unsupported head_dim");
};

// One chunk in flight: K as the A operand of logits^T, V as the A operand of
// O^T, and which of the lane's four V rows (4g + i) carry a row.
template <typename T, int D>
struct Chunk {
  using G = AttnGeo<T, D>;
  u32x4_t kf[G::CH];
  uint32_t vr[4][G::VW];
  uint32_t valid;  // bit i: row 4g + i exists
};

__device__ __forceinline__ uint32_t row_offset_from(uint32_t rowoff, int src_lane) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)rowoff);
}

template <typename T, int D>
__device__ __forceinline__ void load_chunk(Chunk<T, D>& ch, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                           uint32_t rowoff, int c, int n16, int g) {
  using G = AttnGeo<T, D>;
  const uint32_t ko = row_offset_from(rowoff, kChunk * c + n16);
#pragma unroll
  for (int cc = 0; cc < G::CH; ++cc)
    ch.kf[cc] = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(ko + 64 * cc + 16 * g), 0, 0);
  ch.valid = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t vo = row_offset_from(rowoff, kChunk * c + 4 * g + i);
    ch.valid |= (vo < kOutOfRange ? 1u : 0u) << i;
    const int off = (int)(vo + G::VB * n16);
    if constexpr (G::VW == 2) {
      const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, 0);
      ch.vr[i][0] = x[0];
      ch.vr[i][1] = x[1];
    } else {
#pragma unroll
      for (int w4 = 0; w4 < G::VW / 4; ++w4) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(vrs, off + 16 * w4, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) ch.vr[i][4 * w4 + e] = x[e];
      }
    }
  }
}

// One chunk of the online softmax: logits, rescale of the running state and
// O^T += V^T P^T.
template <typename T, int D>
__device__ __forceinline__ void compute_chunk(const Chunk<T, D>& ch, const u32x4_t (&qf)[AttnGeo<T, D>::CH],
                                              f32x4_t (&acc)[AttnGeo<T, D>::DT], float& m_run, float& l_run,
                                              float scale_log2) {
  using G = AttnGeo<T, D>;
  f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cc = 0; cc < G::CH; ++cc) sc = mma_chunk<T>(ch.kf[cc], qf[cc], sc);
  float lg[4];
  float cmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lg[i] = (ch.valid >> i) & 1u ? sc[i] * scale_log2 : -INFINITY;
    cmax = fmaxf(cmax, lg[i]);
  }
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
  const float m_new = fmaxf(m_run, cmax);
  if (m_new == -INFINITY) return;  // wave-uniform: no row seen yet
  const float alpha = exp2f(m_run - m_new);  // 0 while nothing was seen
  float pr[4];
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[i] = lg[i] == -INFINITY ? 0.0f : exp2f(lg[i] - m_new);
    psum += pr[i];
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int t = 0; t < G::DT; ++t) acc[t] *= alpha;
  if constexpr (G::ES == 2) {
    const u32x2_t pw = {float_to_bf16_bits(pr[0]) | (float_to_bf16_bits(pr[1]) << 16),
                        float_to_bf16_bits(pr[2]) | (float_to_bf16_bits(pr[3]) << 16)};
    const bf16x4_t pb = __builtin_bit_cast(bf16x4_t, pw);
#pragma unroll
    for (int t = 0; t < G::DT; ++t) {
      const int w = t >> 1;
      // element t of rows 4g..4g+3: low or high half of dword w
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      const u32x2_t av = {__builtin_amdgcn_perm(ch.vr[1][w], ch.vr[0][w], sel),
                          __builtin_amdgcn_perm(ch.vr[3][w], ch.vr[2][w], sel)};
      acc[t] = mfma_bf16_k16(__builtin_bit_cast(bf16x4_t, av), pb, acc[t]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < G::DT; ++t) acc[t] = mfma_f32(u32_as_float(ch.vr[i][t]), pr[i], acc[t]);
  }
}

// Output dims (d, d+1) of head h of token tok, already normalised: the
// inverse RoPE rotation of the pair by the position's angle (cs, sn) when it
// lies in the rotary dims, one rounding, the packed group layout.
template <typename T, int D>
__device__ __forceinline__ void store_pair(const AttnArgs& a, int tok, int h, int d, float x, float y, float cs,
                                           float sn) {
  const int Hg = a.heads / a.out_groups;
  if (d >= D - a.rope_dim) {  // inverse RoPE: turn the pair back by the position's angle
    const float xr = x * cs + y * sn;
    const float yr = y * cs - x * sn;
    x = xr;
    y = yr;
  }
  const int grp = h / Hg, hl = h - grp * Hg;
  const size_t o = ((size_t)grp * a.batch * a.q_per_req + tok) * Hg * D + (size_t)hl * D + d;
  if constexpr (sizeof(T) == 2) {
    const uint32_t packed = float_to_bf16_bits(x) | (float_to_bf16_bits(y) << 16);
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + o) = packed;
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + o) = make_float2(x, y);
  }
}

// B operand of logits^T: q^T of token tok, column n16 = head h0 + n16 (zero
// for padded heads).  Depends on nothing else, so it is issued first.
template <typename T, int D>
__device__ __forceinline__ void load_query(const AttnArgs& a, int tok, int h0, int n16, int g,
                                           u32x4_t (&qf)[AttnGeo<T, D>::CH]) {
  using G = AttnGeo<T, D>;
  const int h = h0 + n16;  // this lane's head of the group of 16 starting at h0
  const char* qp = static_cast<const char*>(a.q) + ((size_t)tok * a.heads + min(h, a.heads - 1)) * G::ROW + g * 16;
#pragma unroll
  for (int c = 0; c < G::CH; ++c) {
    const u32x4_t v = ld16(qp + c * 64);
    qf[c] = h < a.heads ? v : u32x4_t{0, 0, 0, 0};
  }
}

// One wave's pass over entries [e_lo, e_lo + 16 * CPW) of one stream of token
// (b, s): its online-softmax state, with lane (n16, g) holding O[head n16][d]
// for d = g*D/4 + (D/16)*i + t in acc[t][i], the head's running max in m_run
// and the head's sum over the wave's rows in l_tot (same in the 4 lanes of a
// head).
template <typename T, int D, int CPW>
__device__ __forceinline__ void wave_pass(const AttnArgs& a, bool win, int b, int s, int e_lo, int lane,
                                          const u32x4_t (&qf)[AttnGeo<T, D>::CH], f32x4_t (&acc)[AttnGeo<T, D>::DT],
                                          float& m_run, float& l_tot) {
  using G = AttnGeo<T, D>;
  constexpr int RPW = kChunk * CPW;  // rows per wave
  static_assert(RPW <= 64, "one row number per lane");
  const int n16 = lane & 15, g = lane >> 4;
  const int tok = b * a.q_per_req + s;

  // The byte offset of the row behind entry e_lo + lane (kOutOfRange for
  // padding or past the end).
  int e_hi;
  uint32_t rowoff;
  if (win) {
    const int p = clamp_pos(a.start_pos[b] + s, a.max_len);
    const int nrows = min(a.win, p + 1);
    const int first_pos = p - nrows + 1;
    e_hi = min(nrows, e_lo + RPW);
    const int e = e_lo + lane;
    const int slot = (first_pos + e) % a.w_cap;
    const bool ok = lane < RPW && e < e_hi;
    if (a.win_table) {  // paged ring: pool row through the window's table (clamped into the pool)
      const int blk = a.win_table[(size_t)b * a.win_blocks_per_req + (ok ? (slot >> a.win_shift) : 0)];
      const int64_t pb = min((int64_t)max(blk, 0), a.win_n_blocks - 1);
      const int64_t prow = (pb << a.win_shift) + (slot & ((1 << a.win_shift) - 1));
      rowoff = ok ? (uint32_t)(prow * G::ROW) : kOutOfRange;
    } else {
      rowoff = ok ? (uint32_t)slot * G::ROW : kOutOfRange;
    }
  } else {
    e_hi = min(a.topk, e_lo + RPW);
    const int e = e_lo + lane;
    const int j = (lane < RPW && e < e_hi) ? a.topk_idx[(size_t)tok * a.topk + e] : -1;
    const bool ok = j >= 0 && j < a.n_cap;
    if (a.block_table) {  // paged: pool row through the block table (clamped into the pool)
      const int blk = a.block_table[(size_t)b * a.blocks_per_req + (ok ? (j >> a.block_shift) : 0)];
      const int64_t pb = min((int64_t)max(blk, 0), a.n_blocks - 1);
      const int64_t prow = (pb << a.block_shift) + (j & ((1 << a.block_shift) - 1));
      rowoff = ok ? (uint32_t)(prow * G::ROW) : kOutOfRange;
    } else {
      rowoff = ok ? (uint32_t)j * G::ROW : kOutOfRange;
    }
  }
  const int nrows_wave = e_hi - e_lo;  // may be <= 0

  // the request's slice of its cache, or for a paged cache the whole pool;
  // the host keeps either below 2^31 bytes
  const bool pooled = win ? a.win_table != nullptr : a.block_table != nullptr;
  const size_t rows_req = win ? (size_t)a.w_cap : (size_t)a.n_cap;
  const size_t base_row = pooled ? 0 : (size_t)b * rows_req;
  const size_t pool_rows = win ? (size_t)(a.win_n_blocks << a.win_shift) : (size_t)(a.n_blocks << a.block_shift);
  const size_t range_rows = pooled ? pool_rows : rows_req;
  const char* kreq = static_cast<const char*>(win ? a.k_win : a.k_cmp) + base_row * G::ROW;
  const char* vreq = static_cast<const char*>(win ? a.v_win : a.v_cmp) + base_row * G::ROW;
  const int range = (int)(range_rows * G::ROW);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kreq, range);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vreq, range);

#pragma unroll
  for (int t = 0; t < G::DT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  m_run = -INFINITY;
  float l_run = 0.0f;

  // Chunks, one ahead: chunk c + 1 is in flight while chunk c is computed.
  // The loads are issued unconditionally (rows past the end cost no memory
  // traffic), so the compiler can count them exactly and wait for chunk c
  // alone; a load under a runtime branch would make it wait for everything.
  // A scheduling barrier after each chunk keeps later loads from being
  // hoisted above it, which would only raise register pressure.  A chunk
  // whose rows are all padding is skipped (it would leave the state as is).
  Chunk<T, D> buf[2];
  load_chunk<T, D>(buf[0], krs, vrs, rowoff, 0, n16, g);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    if (c + 1 < CPW) load_chunk<T, D>(buf[(c + 1) & 1], krs, vrs, rowoff, c + 1, n16, g);
    __builtin_amdgcn_sched_barrier(0);
    if (kChunk * c < nrows_wave && __builtin_amdgcn_ballot_w64(buf[c & 1].valid != 0) != 0)  // wave-uniform
      compute_chunk<T, D>(buf[c & 1], qf, acc, m_run, l_run, a.scale_log2);
    __builtin_amdgcn_sched_barrier(0);
  }

  // per-head sum over the 4 lanes that share a head column
  l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
}

// Split partials of a token, merged in ascending split order into the state
// of their stream (window splits first, then compressed).  Loads of up to MB
// splits (one batch) are issued before any of them is used, so a token with
// at most MB splits costs one round trip.  The launch takes MB = 8 when every
// token has at most 8 splits and MB = 16 otherwise.

struct StreamState {
  float m, l, o0, o1;
};

__device__ __forceinline__ void merge_into(StreamState& st, float m, float l, float2 o) {
  if (!(l > 0.0f)) return;  // empty split: its partial sum was never written
  const float mn = fmaxf(st.m, m);
  const float fo = exp2f(st.m - mn), fn = exp2f(m - mn);
  st.l = st.l * fo + l * fn;
  st.o0 = st.o0 * fo + o.x * fn;
  st.o1 = st.o1 * fo + o.y * fn;
  st.m = mn;
}

// (max, sum, dim pair of the partial sum) of splits b0 .. b0+MB-1
// for one (token, head, dim pair); splits past the last read as empty.
template <int MB>
struct SplitBatch {
  float m[MB], l[MB];
  float2 o[MB];
};

template <int MB>
__device__ __forceinline__ void load_splits(const AttnArgs& a, int tok, int h, int d, int D, int b0,
                                            SplitBatch<MB>& sb) {
  const int NS = a.n_split_win + a.n_split_cmp;
#pragma unroll
  for (int k = 0; k < MB; ++k) {
    const int sp = min(b0 + k, NS - 1);
    const size_t r = ((size_t)tok * NS + sp) * a.heads + h;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + 2 * r);
    sb.m[k] = ml.x;
    sb.l[k] = b0 + k < NS ? ml.y : 0.0f;
    sb.o[k] = *reinterpret_cast<const float2*>(a.ws_o + r * D + d);
  }
}

template <int MB>
__device__ __forceinline__ void merge_splits(const AttnArgs& a, int b0, const SplitBatch<MB>& sb, StreamState& w,
                                             StreamState& c) {
#pragma unroll
  for (int k = 0; k < MB; ++k) {
    if (b0 + k < a.n_split_win) merge_into(w, sb.m[k], sb.l[k], sb.o[k]);
    else merge_into(c, sb.m[k], sb.l[k], sb.o[k]);
  }
}

// Final output of one (token, head, dim pair) from all of the token's split
// partials: stream merges, normalisation, inverse RoPE, one rounding, packed
// group layout.  The first batch of partials does not depend on the token's
// position, so it is read before the position and the RoPE table row that
// depends on it: the two reads overlap instead of adding up.
template <typename T, int D, int MB>
__device__ __forceinline__ void finish_item(const AttnArgs& a, int tok, int item) {
  const int r0 = D - a.rope_dim;
  const int h = item / (D / 2), d = 2 * (item - h * (D / 2));
  const int NS = a.n_split_win + a.n_split_cmp;
  SplitBatch<MB> sb;
  load_splits<MB>(a, tok, h, d, D, 0, sb);
  const int S = a.q_per_req;
  const int p = clamp_pos(a.start_pos[tok / S] + tok % S, a.max_len);
  float cs = 1.0f, sn = 0.0f;
  if (d >= r0) {
    const int i = (d - r0) >> 1;
    cs = a.rope_cos[(size_t)p * (a.rope_dim >> 1) + i];
    sn = a.rope_sin[(size_t)p * (a.rope_dim >> 1) + i];
  }
  StreamState w{-INFINITY, 0.0f, 0.0f, 0.0f}, c = w;
  merge_splits(a, 0, sb, w, c);
  for (int b0 = MB; b0 < NS; b0 += MB) {
    load_splits<MB>(a, tok, h, d, D, b0, sb);
    merge_splits(a, b0, sb, w, c);
  }
  // stream merge: an empty stream (sum 0) carries no weight
  const float M = fmaxf(w.m, c.m);
  const float fw = w.l > 0.0f ? exp2f(w.m - M) : 0.0f;
  const float fc = c.l > 0.0f ? exp2f(c.m - M) : 0.0f;
  const float inv = 1.0f / (fw * w.l + fc * c.l);
  store_pair<T, D>(a, tok, h, d, (fw * w.o0 + fc * c.o0) * inv, (fw * w.o1 + fc * c.o1) * inv, cs, sn);
}

constexpr int kFinishThreads = 256;

template <typename T, int D, int CPW>
__global__ __launch_bounds__(kWaves * 64, 3) void attn_split_kernel(AttnArgs a) {
  using G = AttnGeo<T, D>;
  constexpr int RPW = kChunk * CPW;  // rows per wave
  constexpr int RPS = kWaves * RPW;  // rows per split
  static_assert(RPW <= 64, "one row number per lane");
  __shared__ __attribute__((aligned(16))) float mo[kWaves * 16 * G::MO_STRIDE];  // [wave][head][d]
  __shared__ float wml[kWaves][16][2];  // per-wave (max, sum) per head
  __shared__ float wfac[kWaves][16];    // per-wave rescale factor per head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int S = a.q_per_req, H = a.heads;
  const int NSW = a.n_split_win, NS = a.n_split_win + a.n_split_cmp;
  const int NHG = (H + 15) >> 4;  // groups of 16 heads

  // logical block order (b, split, s, head group): the head groups of one
  // (token, split) read the same rows and the S tokens of a request the same
  // window rows; neighbours share an XCD and its L2.
  const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int hg = logical % NHG;
  const int s = (logical / NHG) % S;
  const int split = (logical / (NHG * S)) % NS;
  const int b = logical / (NHG * S * NS);
  const int tok = b * S + s;
  const bool win = split < NSW;
  const int h0 = hg * 16, HL = min(16, H - h0);  // this group's heads
  float* ml_out = a.ws_ml + (((size_t)tok * NS + split) * H + h0) * 2;
  float* o_out = a.ws_o + (((size_t)tok * NS + split) * H + h0) * D;

  u32x4_t qf[G::CH];
  load_query<T, D>(a, tok, h0, n16, g, qf);
  f32x4_t acc[G::DT];
  float m_run, l_tot;
  const int e_lo = (win ? split : split - NSW) * RPS + wave * RPW;
  wave_pass<T, D, CPW>(a, win, b, s, e_lo, lane, qf, acc, m_run, l_tot);

  // ---- the 4 waves' partials, merged in fixed wave order.  Lane (n16, g)
  // holds O[head n16][d] for d = g*D/4 + (D/16)*i + t in acc[t][i].
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < G::DT; ++t)
      mo[(wave * 16 + n16) * G::MO_STRIDE + g * (D / 4) + (D / 16) * i + t] = acc[t][i];
  if (g == 0) {
    wml[wave][n16][0] = m_run;
    wml[wave][n16][1] = l_tot;
  }
  __syncthreads();
  if (tid < kWaves * 16) {  // rescale factor of wave w for head h
    const int w = tid >> 4, h = tid & 15;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, wml[v][h][0]);
    wfac[w][h] = wml[w][h][1] > 0.0f ? exp2f(wml[w][h][0] - M) : 0.0f;
    if (w == 0 && h < HL) {
      float Lsum = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float f = wml[v][h][1] > 0.0f ? exp2f(wml[v][h][0] - M) : 0.0f;
        Lsum += f * wml[v][h][1];
      }
      ml_out[2 * h] = M;
      ml_out[2 * h + 1] = Lsum;
    }
  }
  __syncthreads();
  for (int item = tid; item < HL * D; item += kWaves * 64) {
    const int h = item / D, d = item - h * D;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += wfac[w][h] * mo[(w * 16 + h) * G::MO_STRIDE + d];
    o_out[(size_t)h * D + d] = o;
  }
}

// The epilogue: one thread per (token, head, dim pair), after every split
// partial of the step has been written (stream order).
template <typename T, int D, int MB>
__global__ __launch_bounds__(kFinishThreads) void attn_finish_kernel(AttnArgs a) {
  const int tok = blockIdx.x;
  const int item = blockIdx.y * kFinishThreads + threadIdx.x;
  if (item >= a.heads * (D / 2)) return;
  finish_item<T, D, MB>(a, tok, item);
}

// Maximum and sum over each 16-lane row of the wave with DPP moves (quad
// swaps, then half-row and row mirrors); every lane of the row ends with the
// same bits.
__device__ __forceinline__ float dpp_f(float x, int ctrl) {
  switch (ctrl) {  // the control must be a constant
    case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
    case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
    case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xf, 0xf, false));
  }
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f(x, 0xB1));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f(x, 0x4E));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f(x, 0x141));  // row_half_mirror
  return fmaxf(x, dpp_f(x, 0x140));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f(x, 0xB1);
  x += dpp_f(x, 0x4E);
  x += dpp_f(x, 0x141);
  return x + dpp_f(x, 0x140);
}

// LDS DMA of 4 bytes per lane to lds + 4 * lane (wave 0 of the workgroup).
__device__ __forceinline__ void dma4_global(const float* src, float* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// The whole step of one token in one workgroup, for shapes whose window and
// Top-K rows fit 12 waves of at most 4 chunks: waves [0, WW) walk the window,
// waves [WW, WW + WC) the Top-K list, each as one split wave does.  Their
// states meet in LDS and the workgroup finishes the token itself: per head,
// each stream's max and sum over its waves (register reductions of a fixed
// pattern), the stream merge and each wave's output factor; then per 4 output
// dims the factor-weighted sum over the waves in fixed order, the inverse
// RoPE, one rounding and the packed store.  No partials leave the workgroup
// and there is no second launch.
template <typename T, int D, int CPW>
__global__ __launch_bounds__(kTokenMaxWaves * 64) void attn_token_kernel(AttnArgs a) {
  using G = AttnGeo<T, D>;
  constexpr int RPW = kChunk * CPW;
  __shared__ __attribute__((aligned(16))) float mo[kTokenMaxWaves * 16 * G::MO_STRIDE];  // [wave][head][d]
  __shared__ float wml[kTokenMaxWaves][16][2];  // per-wave (max, sum) per head
  __shared__ float wfac[kTokenMaxWaves][16];    // per-wave output factor per head
  __shared__ float rope_cs[D / 2], rope_sn[D / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = a.waves_win + a.waves_cmp;
  const int n16 = lane & 15, g = lane >> 4;
  const int S = a.q_per_req, H = a.heads, WW = a.waves_win;
  // neighbouring tokens (the S tokens of a request read the same window rows)
  // land on the same XCD
  const int tok = xcd_contiguous(blockIdx.x, gridDim.x);
  const int b = tok / S, s = tok - b * S;
  const bool win = wave < WW;

  u32x4_t qf[G::CH];
  load_query<T, D>(a, tok, 0, n16, g, qf);  // at most 16 heads
  // the position's RoPE row, copied straight into LDS (no registers held
  // across the gather); the barrier before the merge waits for it
  const int half = a.rope_dim >> 1;
  if (tid < half) {
    const int p = clamp_pos(a.start_pos[b] + s, a.max_len);
    dma4_global(a.rope_cos + (size_t)p * half + tid, rope_cs);
    dma4_global(a.rope_sin + (size_t)p * half + tid, rope_sn);
  }
  f32x4_t acc[G::DT];
  float m_run, l_tot;
  wave_pass<T, D, CPW>(a, win, b, s, (win ? wave : wave - WW) * RPW, lane, qf, acc, m_run, l_tot);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < G::DT; ++t)
      mo[(wave * 16 + n16) * G::MO_STRIDE + g * (D / 4) + (D / 16) * i + t] = acc[t][i];
  if (g == 0) {
    wml[wave][n16][0] = m_run;
    wml[wave][n16][1] = l_tot;
  }
  __syncthreads();  // also waits for every wave's outstanding loads, the RoPE copy included
  // Output factor of wave u for head h.  Lanes 16j .. 16j+15 of a wave hold
  // waves 0 .. 15 of head 4*hg + j, so each stream's max and sum over its
  // waves are 16-lane reductions in registers (fixed pattern: every lane of
  // the row gets the same bits).
  for (int hg = wave; hg < 4; hg += nw) {  // wave-uniform
    const int h = 4 * hg + (lane >> 4), u = lane & 15;
    const bool live = u < nw, uw = u < WW;
    const float m = live ? wml[u][h][0] : -INFINITY;
    const float l = live ? wml[u][h][1] : 0.0f;
    const float Mw = row16_max(uw ? m : -INFINITY);
    const float Mc = row16_max(uw ? -INFINITY : m);
    const float f = l > 0.0f ? exp2f(m - (uw ? Mw : Mc)) : 0.0f;  // a wave that saw no row weighs nothing
    const float Lw = row16_sum(uw ? f * l : 0.0f);
    const float Lc = row16_sum(uw ? 0.0f : f * l);
    // stream merge: an empty stream (sum 0) carries no weight
    const float M = fmaxf(Mw, Mc);
    const float fw = Lw > 0.0f ? exp2f(Mw - M) : 0.0f;
    const float fc = Lc > 0.0f ? exp2f(Mc - M) : 0.0f;
    const float inv = 1.0f / (fw * Lw + fc * Lc);
    if (live) wfac[u][h] = f * (uw ? fw : fc) * inv;
  }
  __syncthreads();
  const int r0 = D - a.rope_dim;
  for (int item = tid; item < H * (D / 4); item += nw * 64) {  // 4 dims per item
    const int h = item / (D / 4), d = 4 * (item - h * (D / 4));
    f32x4_t o4 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // every slot read at once (slots past nw hold no wave and are skipped)
#pragma unroll
    for (int v = 0; v < kTokenMaxWaves; ++v) {
      const float f = wfac[v][h];
      const f32x4_t o = *reinterpret_cast<const f32x4_t*>(&mo[(v * 16 + h) * G::MO_STRIDE + d]);
      if (v < nw) o4 += f * o;
    }
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const bool rot = d + e >= r0;
      const int i = rot ? (d + e - r0) >> 1 : 0;
      store_pair<T, D>(a, tok, h, d + e, o4[e], o4[e + 1], rot ? rope_cs[i] : 1.0f, rot ? rope_sn[i] : 0.0f);
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  const int tokens = a.batch * a.q_per_req;
  constexpr bool kWideRows = sizeof(T) == 4 && D == 128;  // one chunk per wave only
  if (a.waves_win + a.waves_cmp > 0) {  // one workgroup per token
    const dim3 tgrid(tokens), tblock(64 * (a.waves_win + a.waves_cmp));
    switch (a.chunks_per_wave) {
      case 1: hipLaunchKernelGGL((attn_token_kernel<T, D, 1>), tgrid, tblock, 0, st, a); break;
      case 2:
        if constexpr (kWideRows) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((attn_token_kernel<T, D, 2>), tgrid, tblock, 0, st, a);
        break;
      case 4:
        if constexpr (kWideRows) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((attn_token_kernel<T, D, 4>), tgrid, tblock, 0, st, a);
        break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int NS = a.n_split_win + a.n_split_cmp;
  const dim3 grid(tokens * NS * ((a.heads + 15) / 16));
  switch (a.chunks_per_wave) {
    case 1: hipLaunchKernelGGL((attn_split_kernel<T, D, 1>), grid, dim3(kWaves * 64), 0, st, a); break;
    case 2:
      if constexpr (kWideRows) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((attn_split_kernel<T, D, 2>), grid, dim3(kWaves * 64), 0, st, a);
      break;
    case 4:
      if constexpr (kWideRows) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((attn_split_kernel<T, D, 4>), grid, dim3(kWaves * 64), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid(tokens, (a.heads * (D / 2) + kFinishThreads - 1) / kFinishThreads);
  if (NS <= 8)
    hipLaunchKernelGGL((attn_finish_kernel<T, D, 8>), fgrid, dim3(kFinishThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_finish_kernel<T, D, 16>), fgrid, dim3(kFinishThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int batch, int q_per_req, int heads, int head_dim, int win, int topk, int dtype) {
  AttnPlan pl{};
  // The most rows per wave (4, 2 or 1 chunks of 16) that still gives at least
  // CSA_ATTN_MIN_SPLITS workgroups, so that a small batch spreads over more
  // CUs while a large one keeps its partials few.  A wave loads its first two
  // chunks together, so 2 chunks cost no more round trips than 1 and halve
  // the partials the finish merges (measured, 16 tokens of 640 rows: 12.2 us
  // against 12.8 with 1 chunk and 13.4 with 4; 16 tokens of 1280 rows: 13.8 us
  // with 4 chunks against 16.5 with 1).  fp32 rows of 128 dims take one chunk
  // per wave: two in flight would not fit the register budget.
#ifndef CSA_ATTN_MIN_SPLITS
#define CSA_ATTN_MIN_SPLITS 64
#endif
  const long long tokens = (long long)batch * q_per_req;
  const bool wide_rows = dtype != 1 && head_dim == 128;
  int cpw = 1;
  for (int c : {4, 2}) {
    if (wide_rows) break;
    const int rps = kWaves * kChunk * c;
    const long long n = tokens * ((win + rps - 1) / rps + (topk + rps - 1) / rps);
    if (n >= CSA_ATTN_MIN_SPLITS) {
      cpw = c;
      break;
    }
  }
  // One workgroup per token (no split partials, no second launch) when the
  // window and Top-K rows fit kTokenMaxWaves waves with the fewest chunks per
  // wave (4 at most), the step has at most CSA_ATTN_TOKEN_MAX_TOKENS tokens,
  // and its waves number at least CSA_ATTN_TOKEN_MIN_WAVES (1.5 per CU).  On a
  // smaller step the split kernels, with a single chunk per wave and many
  // more workgroups, have more loads in flight and finish sooner from cold
  // caches, the second launch included.
#ifndef CSA_ATTN_TOKEN_MAX_TOKENS
#define CSA_ATTN_TOKEN_MAX_TOKENS 4096
#endif
#ifndef CSA_ATTN_TOKEN_MIN_WAVES
#define CSA_ATTN_TOKEN_MIN_WAVES 384
#endif
  if (tokens <= CSA_ATTN_TOKEN_MAX_TOKENS && heads <= 16) {
    for (int c : {1, 2, 4}) {
      if (wide_rows && c > 1) break;
      const int ww = (win + kChunk * c - 1) / (kChunk * c), wc = (topk + kChunk * c - 1) / (kChunk * c);
      if (ww + wc > kTokenMaxWaves) continue;
      if (tokens * (ww + wc) >= CSA_ATTN_TOKEN_MIN_WAVES) {
        pl.chunks_per_wave = c;
        pl.waves_win = ww;
        pl.waves_cmp = wc;
        return pl;  // no workspace
      }
      break;
    }
  }
  pl.chunks_per_wave = cpw;
  pl.rows_per_split = kWaves * kChunk * cpw;
  pl.n_split_win = (win + pl.rows_per_split - 1) / pl.rows_per_split;
  pl.n_split_cmp = (topk + pl.rows_per_split - 1) / pl.rows_per_split;
  const size_t parts = (size_t)tokens * (pl.n_split_win + pl.n_split_cmp) * heads;
  pl.ws_o_floats = parts * head_dim;
  pl.ws_ml_floats = parts * 2;
  pl.ws_o_bytes = (pl.ws_o_floats * 4 + 255) / 256 * 256;
  pl.ws_ml_bytes = (pl.ws_ml_floats * 4 + 255) / 256 * 256;
  pl.ws_bytes = pl.ws_o_bytes + pl.ws_ml_bytes;
  return pl;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
  if (a.dtype == 1) return a.head_dim == 128 ? launch_typed<__bf16, 128>(a, st) : launch_typed<__bf16, 64>(a, st);
  return a.head_dim == 128 ? launch_typed<float, 128>(a, st) : launch_typed<float, 64>(a, st);
}

}  // namespace csa
