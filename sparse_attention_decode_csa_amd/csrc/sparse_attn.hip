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
//   attn_split_kernel:
//   A workgroup of 4 waves owns one (token, split): up to 128 * TPW rows of
//   ONE stream.  Each wave takes TPW 32-row tiles (the 4 waves cover 128
//   consecutive rows per step) and keeps an online softmax across them.
//   - K rows go straight from HBM into the MFMA A operand (16-byte contiguous
//     loads per lane); logits^T = K q^T puts heads on the lane axis, so the
//     softmax statistics of a head live in the 4 lanes sharing its column.
//   - V needs tile rows on the k axis of the PV MFMA, so each wave stages its
//     32 x D V tile in LDS transposed (4 rows x 8 dims per lane, 64-bit LDS
//     writes, 16-byte chunks XOR-swizzled by d / 8) and reads it back as
//     16-byte operand fragments.
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

constexpr int kTileRows = 32;
constexpr int kWaves = 4;

template <typename T, int D>
struct AttnLayout {
  static constexpr int ES = sizeof(T);
  static constexpr int CH = D * ES / 64;   // 64-byte chunks per row (K fragments)
  static constexpr int NP = D * ES / 16;   // 16-byte pieces per row
  static constexpr int EP = 16 / ES;       // elements per piece
  static constexpr int DT = D / 16;        // output d tiles
  static constexpr int UPL = NP / 8;       // V staging units (4 rows x 1 piece) per lane
  static constexpr int RS = 32 * ES;       // LDS bytes per transposed V d-row (32 tile rows)
  static constexpr int NCH = RS / 16;      // 16-byte chunks per d-row
  static constexpr int VT_BYTES = D * RS;
  static constexpr int MO_STRIDE = D + 1;  // floats per (wave, head) row in the merge area
  static constexpr int MERGE_BYTES = kWaves * 16 * MO_STRIDE * 4;
  static constexpr int SMEM = (kWaves * VT_BYTES > MERGE_BYTES) ? kWaves * VT_BYTES : MERGE_BYTES;
  static_assert(UPL >= 1 && NP % 8 == 0, "head_dim too small for the V staging layout");
};

// Position of tile row r (0..31) inside a transposed V d-row.  Rows are
// permuted so that the 8 rows a lane needs for one PV operand, rows
// {4g..4g+3, 16+4g..16+4g+3}, sit contiguously at 8g .. 8g+7.
__device__ __forceinline__ int vt_pos_of_quad(int quad) { return 8 * (quad & 3) + 4 * (quad >> 2); }

// Byte address of position `pos` of d-row `d` in a wave's transposed V tile.
// The 16-byte chunk index is XOR-swizzled by d / 8, so the staging writes of
// lanes that differ in d by multiples of 8 fall in different banks; a lane's
// operand read stays one contiguous 16-byte chunk.
template <int RS, int NCH, int ES>
__device__ __forceinline__ int vt_off(int d, int pos) {
  const int byte = pos * ES;
  return d * RS + (((byte >> 4) ^ ((d >> 3) & (NCH - 1))) << 4) + (byte & 15);
}

// Split partials of one stream, merged in ascending split order.  Loads of
// up to kMergeBatch splits are issued before any of them is used.
constexpr int kMergeBatch = 8;

struct StreamState {
  float m, l, o0, o1;
};

__device__ __forceinline__ StreamState merge_splits(const AttnArgs& a, int tok, int NS, int h, int d,
                                                    int D, int lo, int hi) {
  StreamState st{-INFINITY, 0.0f, 0.0f, 0.0f};
  for (int b0 = lo; b0 < hi; b0 += kMergeBatch) {
    float m[kMergeBatch], l[kMergeBatch];
    float2 ov[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int sp = min(b0 + k, hi - 1);
      const size_t r = ((size_t)tok * NS + sp) * a.heads + h;
      const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + 2 * r);
      m[k] = ml.x;
      l[k] = b0 + k < hi ? ml.y : 0.0f;
      ov[k] = *reinterpret_cast<const float2*>(a.ws_o + r * D + d);
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (!(l[k] > 0.0f)) continue;  // empty split: its partial sum was never written
      const float mn = fmaxf(st.m, m[k]);
      const float fo = exp2f(st.m - mn), fn = exp2f(m[k] - mn);
      st.l = st.l * fo + l[k] * fn;
      st.o0 = st.o0 * fo + ov[k].x * fn;
      st.o1 = st.o1 * fo + ov[k].y * fn;
      st.m = mn;
    }
  }
  return st;
}

// Final output of one (token, head, dim pair) from all of the token's split
// partials: stream merges, normalisation, inverse RoPE, one rounding, packed
// group layout.
template <typename T, int D>
__device__ __forceinline__ void finish_item(const AttnArgs& a, int tok, int p, int item) {
  const int H = a.heads, G = a.out_groups, Hg = H / G;
  const int NSW = a.n_split_win, NS = a.n_split_win + a.n_split_cmp;
  const int T_ = a.batch * a.q_per_req;
  const int r0 = D - a.rope_dim;
  const int h = item / (D / 2), d = 2 * (item - h * (D / 2));
  float cs = 1.0f, sn = 0.0f;
  if (d >= r0) {  // issue the table loads early
    const int i = (d - r0) >> 1;
    cs = a.rope_cos[(size_t)p * (a.rope_dim >> 1) + i];
    sn = a.rope_sin[(size_t)p * (a.rope_dim >> 1) + i];
  }
  const StreamState w = merge_splits(a, tok, NS, h, d, D, 0, NSW);
  const StreamState c = merge_splits(a, tok, NS, h, d, D, NSW, NS);
  // stream merge: an empty stream (sum 0) carries no weight
  const float M = fmaxf(w.m, c.m);
  const float fw = w.l > 0.0f ? exp2f(w.m - M) : 0.0f;
  const float fc = c.l > 0.0f ? exp2f(c.m - M) : 0.0f;
  const float inv = 1.0f / (fw * w.l + fc * c.l);
  float x = (fw * w.o0 + fc * c.o0) * inv;
  float y = (fw * w.o1 + fc * c.o1) * inv;
  if (d >= r0) {  // inverse RoPE: turn the pair back by the position's angle
    const float xr = x * cs + y * sn;
    const float yr = y * cs - x * sn;
    x = xr;
    y = yr;
  }
  const int grp = h / Hg, hl = h - grp * Hg;
  const size_t o = ((size_t)grp * T_ + tok) * Hg * D + (size_t)hl * D + d;
  if constexpr (sizeof(T) == 2) {
    const uint32_t packed = float_to_bf16_bits(x) | (float_to_bf16_bits(y) << 16);
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + o) = packed;
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + o) = make_float2(x, y);
  }
}

constexpr int kFinishThreads = 256;

template <typename T, int D, int TPW>
__global__ __launch_bounds__(kWaves * 64, 4) void attn_split_kernel(AttnArgs a) {
  using L = AttnLayout<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[L::SMEM];
  __shared__ float wml[kWaves][16][2];   // per-wave (max, sum) per head
  __shared__ float wfac[kWaves][16];     // per-wave rescale factor per head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int S = a.q_per_req, H = a.heads;
  const int NSW = a.n_split_win, NS = a.n_split_win + a.n_split_cmp;

  // logical block order (b, split, s): the S tokens of a request that read the
  // same window rows are neighbours, hence on the same XCD and its L2.
  const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int s = logical % S;
  const int split = (logical / S) % NS;
  const int b = logical / (S * NS);
  const int tok = b * S + s;
  const int p = clamp_pos(a.start_pos[b] + s, a.max_len);
  constexpr int RPS = kWaves * kTileRows * TPW;

  const bool win = split < NSW;
  int e_begin, e_end, first_pos = 0;
  if (win) {
    const int nrows = min(a.win, p + 1);
    first_pos = p - nrows + 1;
    e_begin = split * RPS;
    e_end = min(nrows, e_begin + RPS);
  } else {
    e_begin = (split - NSW) * RPS;
    e_end = min(a.topk, e_begin + RPS);
  }
  float* ml_out = a.ws_ml + ((size_t)tok * NS + split) * H * 2;
  float* o_out = a.ws_o + ((size_t)tok * NS + split) * H * D;

  if (e_begin < e_end) {  // block-uniform: this split has rows
    const char* kbase = static_cast<const char*>(win ? a.k_win : a.k_cmp);
    const char* vbase = static_cast<const char*>(win ? a.v_win : a.v_cmp);
    const int32_t* list = a.topk_idx + (size_t)tok * a.topk;
    const size_t rbase = win ? (size_t)b * a.w_cap : (size_t)b * a.n_cap;
    const size_t row_bytes = (size_t)D * L::ES;
    // Row of list entry e: its byte offset and whether it carries a row.
    auto lookup = [&](int e, bool& valid) -> size_t {
      if (e >= e_end) {
        valid = false;
        return rbase * row_bytes;
      }
      if (win) {
        valid = true;
        return (rbase + (size_t)((first_pos + e) % a.w_cap)) * row_bytes;
      }
      const int j = list[e];
      valid = (j >= 0) & (j < a.n_cap);
      return (rbase + (size_t)(valid ? j : 0)) * row_bytes;
    };

    // B operand of logits^T: q^T, column = head n16 (zero for padded heads).
    u32x4_t qf[L::CH];
    {
      const char* qp = static_cast<const char*>(a.q) + ((size_t)tok * H + min(n16, H - 1)) * row_bytes + g * 16;
#pragma unroll
      for (int c = 0; c < L::CH; ++c) {
        const u32x4_t v = ld16(qp + c * 64);
        qf[c] = n16 < H ? v : u32x4_t{0, 0, 0, 0};
      }
    }

    f32x4_t acc[L::DT];
#pragma unroll
    for (int dt = 0; dt < L::DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    char* vt = smem + wave * L::VT_BYTES;

    // Tiles run one after the other: a scheduling barrier at the end of each
    // tile keeps the next tile's loads out of the current tile's registers,
    // which holds occupancy at 4 workgroups per CU, so every split of a large
    // batch can be resident at once.
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      const int e0 = e_begin + (it * kWaves + wave) * kTileRows;
      if (e0 >= e_end) break;  // wave-uniform

      // K rows e0 + 16t + n16 as the A operand (16 bytes of each 64-byte chunk)
      u32x4_t kf[2][L::CH];
      bool kval[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const char* rp = kbase + lookup(e0 + 16 * t + n16, kval[t]) + g * 16;
#pragma unroll
        for (int c = 0; c < L::CH; ++c) kf[t][c] = ld16(rp + c * 64);
      }
      // V: unit u = (quad q of 4 rows, 16-byte piece pc); masked rows read as zero
      u32x4_t vpc[L::UPL][4];
#pragma unroll
      for (int k = 0; k < L::UPL; ++k) {
        const int u = lane + kWave * k, q = u & 7, pc = u >> 3;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bool v;
          const size_t off = lookup(e0 + 4 * q + jj, v);
          const u32x4_t x = ld16(vbase + off + pc * 16);
          vpc[k][jj] = v ? x : u32x4_t{0, 0, 0, 0};
        }
      }

      // logits^T tile: lane (head n16, g) holds rows 16t + 4g + i
      f32x4_t sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < L::CH; ++c) sc[t] = mma_chunk<T>(kf[t][c], qf[c], sc[t]);
      }

      // stage V transposed: d-row d holds the 32 tile rows at permuted positions
      wave_lds_fence();  // the previous tile's operand reads precede these writes
#pragma unroll
      for (int k = 0; k < L::UPL; ++k) {
        const int u = lane + kWave * k, q = u & 7, pc = u >> 3;
        const int pos = vt_pos_of_quad(q);
#pragma unroll
        for (int x = 0; x < L::EP; ++x) {
          const int d = pc * L::EP + x;
          char* dst = vt + vt_off<L::RS, L::NCH, L::ES>(d, pos);
          if constexpr (L::ES == 2) {
            const int w = x >> 1;
            uint32_t lo, hi;
            if (x & 1) {
              lo = (vpc[k][0][w] >> 16) | (vpc[k][1][w] & 0xFFFF0000u);
              hi = (vpc[k][2][w] >> 16) | (vpc[k][3][w] & 0xFFFF0000u);
            } else {
              lo = (vpc[k][0][w] & 0xFFFFu) | (vpc[k][1][w] << 16);
              hi = (vpc[k][2][w] & 0xFFFFu) | (vpc[k][3][w] << 16);
            }
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{lo, hi};
          } else {
            *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{vpc[k][0][x], vpc[k][1][x], vpc[k][2][x], vpc[k][3][x]};
          }
        }
      }
      wave_lds_fence();

      // base-2 logits; rows past the stream or without a row are masked
      const uint32_t vm0 = (uint32_t)__ballot(kval[0]) & 0xFFFFu;  // lanes 0..15: rows 0..15
      const uint32_t vm1 = (uint32_t)__ballot(kval[1]) & 0xFFFFu;  // rows 16..31
      float lg[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = ((t ? vm1 : vm0) >> (4 * g + i)) & 1u;
          lg[t][i] = ok ? sc[t][i] * a.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, lg[t][i]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      if (m_new != -INFINITY) {  // wave-uniform: masks are per row
        const float alpha = exp2f(m_run - m_new);  // 0 while nothing was seen
        float pr[2][4];
        float psum = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pr[t][i] = lg[t][i] == -INFINITY ? 0.0f : exp2f(lg[t][i] - m_new);
            psum += pr[t][i];
          }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < L::DT; ++dt) acc[dt] *= alpha;

        // O^T += V^T P^T: A = V^T (row d, tile rows on k), B = P^T (column = head)
        if constexpr (L::ES == 2) {
          u32x4_t pw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int t = w >> 1, i0 = 2 * (w & 1);
            pw[w] = float_to_bf16_bits(pr[t][i0]) | (float_to_bf16_bits(pr[t][i0 + 1]) << 16);
          }
          const bf16x8_t pf = as_bf16x8(pw);
#pragma unroll
          for (int dt = 0; dt < L::DT; ++dt) {
            const u32x4_t vf =
                *reinterpret_cast<const u32x4_t*>(vt + vt_off<L::RS, L::NCH, L::ES>(16 * dt + n16, 8 * g));
            acc[dt] = mfma_bf16(as_bf16x8(vf), pf, acc[dt]);
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < L::DT; ++dt) {
            const int d = 16 * dt + n16;
            const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(vt + vt_off<L::RS, L::NCH, L::ES>(d, 8 * g));
            const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(vt + vt_off<L::RS, L::NCH, L::ES>(d, 8 * g + 4));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              acc[dt] = mfma_f32(u32_as_float(v0[j]), pr[0][j], acc[dt]);
              acc[dt] = mfma_f32(u32_as_float(v1[j]), pr[1][j], acc[dt]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // per-head sum over the 4 lanes that share a head column
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);

    // ---- the 4 waves' partials, merged in fixed wave order
    __syncthreads();  // every wave is done with its V tile; reuse LDS
    float* mo = reinterpret_cast<float*>(smem);  // [wave][head][MO_STRIDE]
#pragma unroll
    for (int dt = 0; dt < L::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mo[(wave * 16 + n16) * L::MO_STRIDE + 16 * dt + 4 * g + i] = acc[dt][i];
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
      if (w == 0 && h < H) {
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
    for (int item = tid; item < H * D; item += kWaves * 64) {
      const int h = item / D, d = item - h * D;
      float part[kWaves], f[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        part[w] = mo[(w * 16 + h) * L::MO_STRIDE + d];
        f[w] = wfac[w][h];
      }
      float o = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += f[w] * part[w];
      o_out[(size_t)h * D + d] = o;
    }
  } else if (tid < H) {  // nothing in this split (short window)
    ml_out[2 * tid] = -INFINITY;
    ml_out[2 * tid + 1] = 0.0f;
  }
}

// The epilogue: one thread per (token, head, dim pair), after every split
// partial of the step has been written (stream order).
template <typename T, int D>
__global__ __launch_bounds__(kFinishThreads) void attn_finish_kernel(AttnArgs a) {
  const int tok = blockIdx.x;
  const int item = blockIdx.y * kFinishThreads + threadIdx.x;
  if (item >= a.heads * (D / 2)) return;
  const int S = a.q_per_req;
  const int p = clamp_pos(a.start_pos[tok / S] + tok % S, a.max_len);
  finish_item<T, D>(a, tok, p, item);
}

template <typename T, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  const int tokens = a.batch * a.q_per_req;
  const int NS = a.n_split_win + a.n_split_cmp;
  const dim3 grid(tokens * NS);
  switch (a.tiles_per_wave) {
    case 1: hipLaunchKernelGGL((attn_split_kernel<T, D, 1>), grid, dim3(kWaves * 64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_split_kernel<T, D, 2>), grid, dim3(kWaves * 64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid(tokens, (a.heads * (D / 2) + kFinishThreads - 1) / kFinishThreads);
  hipLaunchKernelGGL((attn_finish_kernel<T, D>), fgrid, dim3(kFinishThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int batch, int q_per_req, int heads, int head_dim, int win, int topk) {
  AttnPlan pl{};
  // Two tiles per wave (256 rows per split) once there are enough rows for
  // every split workgroup to stay resident in one round; one tile (128 rows)
  // below that, so small batches still spread over many CUs.
#ifndef CSA_ATTN_TPW2_ROWS
#define CSA_ATTN_TPW2_ROWS 65536
#endif
  const long long rows = (long long)batch * q_per_req * (win + topk);
  pl.tiles_per_wave = rows >= CSA_ATTN_TPW2_ROWS ? 2 : 1;
  pl.rows_per_split = kWaves * kTileRows * pl.tiles_per_wave;
  pl.n_split_win = (win + pl.rows_per_split - 1) / pl.rows_per_split;
  pl.n_split_cmp = (topk + pl.rows_per_split - 1) / pl.rows_per_split;
  const size_t tokens = (size_t)batch * q_per_req;
  const size_t parts = tokens * (pl.n_split_win + pl.n_split_cmp) * heads;
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
