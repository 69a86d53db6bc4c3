// Indexer scoring over the ratio-4 compressed cache.
//
//   score[b][s][j] = sum_h w[b][s][h] * relu(q_idx[b][s][h] . k_idx[b][j])
//
// for every causally visible row j of every token that does not fit Top-K
// (the indexer of "Perf: skip redundant CSA scoring and fuse gather unpack",
// description; its scoring is skipped for tokens whose visible cache fits).
//
// Design: the step streams k_idx once per request (every token of a request
// shares it), so it is HBM-bound; the contraction runs on MFMA with the
// request's S*Hi query rows as the M dimension (zero-padded to 16) and 16 keys
// as N.  A prefill chunk (many query tokens per request, the prefill indexer
// of "Fix: port the DeepSeek-V4 MoE, hc_pre and prefill fixes to DSpark",
// description) is cut into blocks of at most 64 query rows, a third grid
// dimension; each block reads the keys its own tokens see, mostly from L2.
// Key tiles stream HBM -> LDS by DMA in whole rows, several tiles in flight
// per wave, and each lane reads its 16-byte MFMA operand pieces back from LDS.
// The per-head relu and weighted sum runs in registers when the head count is
// 4, 8 or 16 (each lane's four result rows are heads of one token), else
// through a small per-wave LDS tile; either way in a fixed head order.  On the
// register path the block's scores are written after its key stream, through
// LDS, as contiguous streaming stores.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace csa {
namespace {

#ifndef CSA_SCORE_TILES_PER_WAVE
#define CSA_SCORE_TILES_PER_WAVE 8
#endif
#ifndef CSA_SCORE_TILE_BUFFERS
#define CSA_SCORE_TILE_BUFFERS 4
#endif
constexpr int kScoreWaves = 4;
constexpr int kScoreTilesPerWave = CSA_SCORE_TILES_PER_WAVE;               // 16-key tiles
constexpr int kScoreBufs = CSA_SCORE_TILE_BUFFERS;                         // tiles in flight per wave
constexpr int kScoreKeysPerBlock = kScoreWaves * kScoreTilesPerWave * 16;  // 512

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Key rows travel HBM -> LDS by DMA (global_load_lds_dwordx4): one instruction
// moves 1 KiB, i.e. whole rows, so every 128-byte line is consumed by a single
// request and the non-temporal hint can keep the stream from displacing the
// rest of the cache.  In LDS the 16-byte piece p of tile row r sits at slot
// p ^ (r % pieces-per-row); the MFMA operand reads (16 rows, one piece each)
// then spread over the banks.  The DMA fixes the LDS slot of each lane, so the
// swizzle is applied on the global side: the lane that fills slot s fetches
// piece s ^ (r % pieces-per-row).
template <int ROW>
struct ScoreTile {
  static constexpr int NPR = ROW / 16;      // 16-byte pieces per row
  static constexpr int RPI = 1024 / ROW;    // rows per DMA instruction
  static constexpr int NPT = 16 * ROW / 1024;  // DMA instructions per 16-row tile
  static constexpr int BYTES = 16 * ROW;
  static_assert(NPR >= 4 && RPI >= 1 && NPT >= 1, "unsupported row size");
};

// Eight OCP E4M3 codes (two dwords, lowest byte first) as eight bf16 values
// in the MFMA operand order.  Every E4M3 value has at most 4 significant bits,
// so the high half of its fp32 decoding is the exact bf16 value.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  auto pk = [](float lo, float hi) {  // high halves of two fp32 values
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                                 0x07060302u);
  };
  return u32x4_t{pk(a.x, a.y), pk(b.x, b.y), pk(c.x, c.y), pk(d.x, d.y)};
}

// HI > 0: the indexer head count, a power of two in 4 .. 16, so that the four
// result rows a lane holds (4g .. 4g+3 of a 16-row tile) belong to one token
// and the head sum finishes with at most two cross-lane adds.  HI == 0: any
// head count, summed through a small per-wave LDS tile.
// KF8: the keys are an FP8 cache (E4M3 codes plus one fp32 scale per row,
// the indexer key cache and its scale of "Fix: complete DeepSeek V4 TP CSA
// decode", description).  Rows are half as long, the codes are widened to
// bf16 exactly in registers, the bf16 query is unchanged, and the row's scale
// multiplies its head sum (relu is positively homogeneous, so
// scale * sum_h w_h relu(q_h . c) = sum_h w_h relu(q_h . (scale * c))).
// PG: the key cache (and the FP8 scales) are pools of blocks located through
// a per-request block table; the workgroup loads the table entries of its
// 512 keys once, one per lane, and each tile takes its block from one lane
// (blocks are at least 16 rows, so a 16-row tile never straddles two).
template <typename T, int DI, int MT, int HI, bool KF8, bool PG>
__global__ __launch_bounds__(256) void indexer_score_kernel(ScoreArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int QROW = DI * ES;              // bytes per query row
  constexpr int ROW = KF8 ? DI : DI * ES;    // bytes per key row
  constexpr int CH = QROW / 64;              // 32-dim MFMA k-steps per row; 16 B of each per lane
  static_assert(CH >= 1 && QROW % 64 == 0, "row must be a whole number of 64-byte chunks");
  static_assert(!KF8 || (ES == 2 && CH % 2 == 0), "FP8 keys pair with bf16 queries");
  using TL = ScoreTile<ROW>;
  constexpr int ROWS = MT * 16;      // padded query rows
  constexpr int RP = 17;             // padded LDS row length (floats)

  // tiles in flight per wave, as many as asked for within 128 KiB of tile buffers
  constexpr int NB = kScoreBufs * kScoreWaves * TL::BYTES <= 128 * 1024 ? kScoreBufs
                                                                         : 128 * 1024 / (kScoreWaves * TL::BYTES);
  __shared__ __attribute__((aligned(1024))) char tiles[kScoreWaves][NB][TL::BYTES];
  __shared__ float red[HI ? 1 : kScoreWaves][HI ? 1 : ROWS][RP];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  // This workgroup's tokens: s0 .. s0+S-1 of request b (one block of at most
  // 64 query rows; a decode step is one block, a prefill chunk several).
  const int s0 = blockIdx.z * a.tok_per_block;
  const int S = min(a.q_per_req - s0, a.tok_per_block), Hi = a.idx_heads, SH = S * Hi;
  const int sp = a.start_pos[b] + s0;      // position of the block's first token
  const size_t tok0 = (size_t)b * a.q_per_req + s0;

  // Rows scored for this block: the largest visible count among its tokens
  // that do not fit Top-K.
  int nmax = 0;
  for (int s = 0; s < S; ++s) {
    const int nv = min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap);
    if (nv > a.topk) nmax = max(nmax, nv);
  }
  const int key0 = blockIdx.x * kScoreKeysPerBlock;
  if (key0 >= nmax) return;  // whole workgroup: nothing visible in this chunk

  // Row of the key cache (or scale array) holding logical row j of request b,
  // where jt = min(first row of j's 16-row tile, nmax - 1) is wave-uniform.
  // Dense: b * n_cap + j.  Paged: the workgroup's slice of the block table is
  // held one entry per lane (logical block (key0 >> shift) + lane, clamped
  // into the pool); blocks are at least 16 rows, so every row a tile loads
  // (rows past nmax are clamped to nmax - 1 = jt) lies in jt's block, which
  // one lane read gives.
  int pblk = 0;
  if constexpr (PG) {
    const int lb = min((key0 >> a.block_shift) + lane, a.blocks_per_req - 1);
    const int e = a.block_table[(size_t)b * a.blocks_per_req + lb];
    pblk = (int)min((int64_t)max(e, 0), a.n_blocks - 1);
  }
  auto key_row = [&](int jt, int j) -> size_t {
    if constexpr (PG) {
      const int blk = __builtin_amdgcn_readlane(pblk, (jt >> a.block_shift) - (key0 >> a.block_shift));
      return ((size_t)blk << a.block_shift) + (size_t)(j & ((1 << a.block_shift) - 1));
    } else {
      (void)jt;
      return (size_t)b * a.n_cap + j;
    }
  };
  // wave-uniform first row of tile t of this wave (clamped to a real row)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto tile_key0 = [&](int t) { return key0 + (t * kScoreWaves + wave_u) * 16; };

  // per-row scales of this lane's key in each tile (FP8 keys), loaded first:
  // every load issued before the tile DMAs is older than them, so the tile
  // waits below can count DMA instructions only
  float ks[KF8 ? kScoreTilesPerWave : 1];
  if constexpr (KF8) {
#pragma unroll
    for (int t = 0; t < kScoreTilesPerWave; ++t)
      ks[t] = a.k_scale[key_row(min(tile_key0(t), nmax - 1), min(tile_key0(t) + n16, nmax - 1))];
  }

  // A operand: query row qr = mt*16 + n16 (token qr / Hi, head qr % Hi).
  // Rows past S*Hi (padding to 16) load a copy of the last real row and are
  // never used: on the register path they belong to token indices >= S, whose
  // sums are not stored; on the LDS path the head sum reads real rows only.
  // Nothing consumes these loads before the MFMAs, so no wait delays the DMAs.
  u32x4_t qa[MT][CH];
  float wv[MT][4];
  const char* qbase = static_cast<const char*>(a.q_idx) + tok0 * Hi * QROW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int qr = mt * 16 + n16;
    const char* qp = qbase + (size_t)min(qr, SH - 1) * QROW;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // k-step c, group g: dims [32c + 8g, +8); with FP8 keys, whose lane reads
      // 16 contiguous codes per two steps, dims [64(c/2) + 16g + 8(c%2), +8)
      const int qoff = KF8 ? 128 * (c >> 1) + 32 * g + 16 * (c & 1) : 64 * c + 16 * g;
      qa[mt][c] = ld16(qp + qoff);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * g + i;   // result rows this lane holds
      wv[mt][i] = a.w[tok0 * Hi + min(row, SH - 1)];
    }
  }
  // Fast path: the token of tile mt's rows 4g..4g+3 and its visible count.
  int tok_of[MT], nv_of[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int s = HI ? (mt * 16 + 4 * g) / (HI ? HI : 1) : 0;
    tok_of[mt] = s;
    nv_of[mt] = s < S ? min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap) : 0;
  }
  const char* kbase = static_cast<const char*>(a.k_idx);   // rows addressed by key_row()
  // Tiles are interleaved over the 4 waves (tile_key0) so that at each step
  // the block reads 4 consecutive 16-row tiles.
  auto issue_tile = [&](int t) {
    const int k0 = tile_key0(t), jt = min(k0, nmax - 1);
    char* dst = tiles[wave][t % NB];
#pragma unroll
    for (int k = 0; k < TL::NPT; ++k) {
      const int r = k * TL::RPI + lane / TL::NPR;            // tile row this lane fetches
      const int piece = (lane % TL::NPR) ^ (r % TL::NPR);
      const int j = min(k0 + r, nmax - 1);                   // clamp: a real row
      // (the address is formed outside the builtin's argument list: a lambda
      // call inside it keeps the host pass from emitting the kernel's stub)
      const char* src = kbase + key_row(jt, j) * ROW + 16 * piece;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + 1024 * k),
                                       16, 0, kNonTemporal);
    }
  };
  // the query loads above are older than every tile DMA, so waiting for them
  // does not wait for the tiles
#pragma unroll
  for (int t = 0; t < NB && t < kScoreTilesPerWave; ++t) issue_tile(t);

  float* srow = a.scores + tok0 * a.n_cap;
  // register path: each tile's head sums, written after the tile loop
  float outv[kScoreTilesPerWave][HI > 0 ? MT : 1];

#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    // Tile t has landed once at most the DMA instructions of the younger tiles
    // in flight are outstanding (other memory operations only make this wait
    // longer, never shorter).
    constexpr int kAhead = NB - 1;
    const int younger = (t + kAhead < kScoreTilesPerWave ? kAhead : kScoreTilesPerWave - 1 - t);
    static_assert(kAhead <= 7 && 7 * TL::NPT <= 63, "tile waits cover at most 7 younger tiles");
    switch (younger) {  // t is a compile-time constant after unrolling
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<1 * TL::NPT>(); break;
      case 2: wait_vmcnt<2 * TL::NPT>(); break;
      case 3: wait_vmcnt<3 * TL::NPT>(); break;
      case 4: wait_vmcnt<4 * TL::NPT>(); break;
      case 5: wait_vmcnt<5 * TL::NPT>(); break;
      case 6: wait_vmcnt<6 * TL::NPT>(); break;
      default: wait_vmcnt<7 * TL::NPT>(); break;
    }
    const char* src = tiles[wave][t % NB];
    u32x4_t kb[CH];
    if constexpr (KF8) {
#pragma unroll
      for (int c2 = 0; c2 < CH / 2; ++c2) {
        const int slot = (4 * c2 + g) ^ (n16 % TL::NPR);
        const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + n16 * ROW + 16 * slot);
        kb[2 * c2] = e4m3x8_to_bf16(raw[0], raw[1]);
        kb[2 * c2 + 1] = e4m3x8_to_bf16(raw[2], raw[3]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int slot = (4 * c + g) ^ (n16 % TL::NPR);
        kb[c] = *reinterpret_cast<const u32x4_t*>(src + n16 * ROW + 16 * slot);
      }
    }
    if (t + NB < kScoreTilesPerWave) {
      wait_lgkmcnt0();  // the operand reads of this buffer are done: refill it
      issue_tile(t + NB);
    }
    const int tkey0 = tile_key0(t);
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[mt] = mma_chunk<T>(qa[mt][c], kb[c], acc[mt]);
    }
    // lane holds dot(query row mt*16+4g+i, key tkey0+n16)
    if constexpr (HI > 0) {
      // heads in ascending order: the lane's four, then pairs of lanes
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = acc[mt][i];
          sum += wv[mt][i] * (d > 0.0f ? d : 0.0f);
        }
        if constexpr (HI >= 8) sum += __shfl_xor(sum, 16);
        if constexpr (HI >= 16) sum += __shfl_xor(sum, 32);
        if constexpr (KF8) sum *= ks[t];
        outv[t][mt] = sum;
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = acc[mt][i];
          red[wave][mt * 16 + 4 * g + i][n16] = wv[mt][i] * (d > 0.0f ? d : 0.0f);
        }
      wave_lds_fence();
      for (int e = lane; e < S * 16; e += kWave) {
        const int s = e >> 4, n = e & 15;
        const int nv = min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap);
        float sum = 0.0f;
        for (int h = 0; h < Hi; ++h) sum += red[wave][s * Hi + h][n];
        if constexpr (KF8) sum *= ks[t];  // n == n16: this lane's key
        const int j = tkey0 + n;
        if (nv > a.topk && j < nv) srow[(size_t)s * a.n_cap + j] = sum;
      }
      wave_lds_fence();
    }
  }

  if constexpr (HI > 0) {
    // The block's scores of each token are staged through the tile buffers
    // (idle once every wave has left the tile loop) and written as contiguous
    // 16-byte pieces, with the streaming hint when the step's scores are many
    // (stream_scores).  One scattered 64-byte write per tile and token,
    // interleaved with the key stream, cost more than their share of the
    // traffic.
    constexpr int kStageTok = (int)sizeof(tiles) / (kScoreKeysPerBlock * 4);  // tokens per pass
    // the block's score rows, S tokens (the launcher takes the global-store
    // form, stream_scores == 2, when they could reach 2^31 bytes)
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(srow, a.stream_scores == 2 ? 0 : (int)((size_t)S * a.n_cap * 4));
    static_assert(kStageTok >= 1, "the tile buffers hold at least one token's scores");
    float* stage = reinterpret_cast<float*>(&tiles[0][0][0]);
    const bool writer = (g & (HI / 4 - 1)) == 0;  // lanes holding a finished head sum
    for (int s0p = 0; s0p < S; s0p += kStageTok) {
      __syncthreads();  // the tile buffers (or the previous pass) are free
#pragma unroll
      for (int t = 0; t < kScoreTilesPerWave; ++t) {
        const int kl = (t * kScoreWaves + wave) * 16 + n16;  // key - key0
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int ts = tok_of[mt] - s0p;
          if (writer && ts >= 0 && ts < kStageTok) stage[ts * kScoreKeysPerBlock + kl] = outv[t][mt];
        }
      }
      __syncthreads();
      const int np = min(kStageTok, S - s0p);
      for (int e = threadIdx.x; e < np * (kScoreKeysPerBlock / 4); e += kScoreWaves * kWave) {
        const int ts = e / (kScoreKeysPerBlock / 4), q4 = e - ts * (kScoreKeysPerBlock / 4);
        const int s = s0p + ts;
        const int nv = min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap);
        const int j0 = key0 + 4 * q4;
        if (nv <= a.topk || j0 >= nv) continue;  // Top-K bypass, or past the visible rows
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + ts * kScoreKeysPerBlock + 4 * q4);
        if (a.stream_scores == 2) {  // rows past 32-bit offsets: 64-bit addresses, streaming
          float* dst = srow + (size_t)s * a.n_cap + j0;
          const uint32_t m = (uint32_t)min(4, nv - j0);
          if (m == 4 && (a.n_cap & 3) == 0) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
          } else {
            const uint32_t e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3];  // constant indices
            __builtin_nontemporal_store(e0, reinterpret_cast<uint32_t*>(dst));
            if (m > 1) __builtin_nontemporal_store(e1, reinterpret_cast<uint32_t*>(dst + 1));
            if (m > 2) __builtin_nontemporal_store(e2, reinterpret_cast<uint32_t*>(dst + 2));
            if (m > 3) __builtin_nontemporal_store(e3, reinterpret_cast<uint32_t*>(dst + 3));
          }
          continue;
        }
        const int off = (int)(((size_t)s * a.n_cap + j0) * 4);  // in the block's rows (srs)
        // Buffer stores whose cache policy is an immediate: two stores that
        // differ only in a hint would be merged into one without it.
        if (j0 + 4 <= nv && (a.n_cap & 3) == 0) {  // whole piece, 16-byte aligned row
          if (a.stream_scores)
            __builtin_amdgcn_raw_buffer_store_b128(v, srs, off, 0, kNonTemporal);
          else
            __builtin_amdgcn_raw_buffer_store_b128(v, srs, off, 0, 0);
        } else {
          const uint32_t e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3];  // constant indices
          const int m = nv - j0;  // 1 .. 3
          if (a.stream_scores) {
            __builtin_amdgcn_raw_buffer_store_b32(e0, srs, off, 0, kNonTemporal);
            if (m > 1) __builtin_amdgcn_raw_buffer_store_b32(e1, srs, off + 4, 0, kNonTemporal);
            if (m > 2) __builtin_amdgcn_raw_buffer_store_b32(e2, srs, off + 8, 0, kNonTemporal);
            if (m > 3) __builtin_amdgcn_raw_buffer_store_b32(e3, srs, off + 12, 0, kNonTemporal);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(e0, srs, off, 0, 0);
            if (m > 1) __builtin_amdgcn_raw_buffer_store_b32(e1, srs, off + 4, 0, 0);
            if (m > 2) __builtin_amdgcn_raw_buffer_store_b32(e2, srs, off + 8, 0, 0);
            if (m > 3) __builtin_amdgcn_raw_buffer_store_b32(e3, srs, off + 12, 0, 0);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill shape: many query rows per request (a chunk of tokens).  The
// decode-shaped kernel above gives each wave its own key tiles against at
// most 64 query rows.  Here a block of 4 waves takes 256 query rows (64 per
// wave) and the waves read one shared ring of key steps (32 keys, >= 4 KiB),
// so a key row leaves L2 once per 256 query rows.  Each wave issues its share
// of every step's DMA and one LDS barrier per step publishes the step.
//
// The contraction is v_mfma_f32_32x32x16_bf16 with the query rows permuted so
// that the 16 result rows a lane holds are whole tokens (Hi = 4, 8 or 16):
// the head sum needs no cross-lane exchange, and each score store writes two
// contiguous 128-byte runs (32 keys of two tokens).  The stores are buffer
// stores issued unconditionally (masked lanes get an offset past the buffer),
// so every step issues the same number of vector memory instructions and the
// DMA waits can count them exactly: vector memory operations retire in order,
// so a wait for a step also waits for whatever was issued before it.
constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = kGemmWaves * kWave;
constexpr int kGemmRows = kGemmWaves * 64;        // query rows per block
constexpr int kGemmKeys = 1024;                   // keys per block
#ifndef CSA_GEMM_BUFS
#define CSA_GEMM_BUFS 8
#endif
#ifndef CSA_GEMM_BLOCKS_PER_CU
#define CSA_GEMM_BLOCKS_PER_CU 2
#endif
#ifndef CSA_GEMM_OVERLAP
#define CSA_GEMM_OVERLAP 1
#endif
constexpr int kGemmBufs = CSA_GEMM_BUFS;          // key steps in the ring
// Cache policy of the key DMA.  Every row block of a request reads the same
// key rows (128 row blocks of a 4096-token chunk), so the keys are loaded
// with the default policy and stay in L2 for the other row blocks; the
// non-temporal hint of the decode-shaped kernel, whose keys are read once,
// made each row block fetch them again from the fabric (measured on 2 x 4096
// tokens of 7168-8192 rows: 192 -> 142 MB fetched per launch, 141 -> 135 us).
// (Streaming the query rows past L2 as well measured slower: 164 us.)
constexpr int kGemmKeyPolicy = 0;
constexpr int kGemmStepKeys = 32;                 // one 32-key MFMA N tile

// wait_vmcnt for counts above the counter's range: waiting for more is safe
template <int N>
__device__ __forceinline__ void wait_vmcnt_sat() {
  wait_vmcnt<(N < 63 ? N : 63)>();
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// KF8: FP8 key cache (E4M3 codes, one fp32 scale per row).  The ring holds
// the codes; each lane widens its 8 codes per k-step to bf16 (exact: every
// E4M3 value is a bf16 value) and the row's scale multiplies the head sum, as
// in the kernel above.
template <int DI, int HI, bool PG, bool KF8>
__global__ __launch_bounds__(kGemmThreads, CSA_GEMM_BLOCKS_PER_CU) void indexer_score_gemm_kernel(ScoreArgs a) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  constexpr int QROW = DI * 2;                         // bytes per query row
  constexpr int ROW = KF8 ? DI : DI * 2;               // bytes per key row
  constexpr int KS = DI / 16;                          // 16-dim MFMA k-steps
  constexpr int MT = 2;                                // 32-row M tiles per wave
  constexpr int TPL = 16 / HI;                         // tokens per lane per M tile
  using TL = ScoreTile<ROW>;                           // 16-row tile layout (piece swizzle)
  constexpr int NB = kGemmBufs;
  constexpr int STEP_BYTES = 2 * TL::BYTES;            // 32 keys
  constexpr int NSTEPS = kGemmKeys / kGemmStepKeys;
  constexpr int DPW = 2 * TL::NPT / kGemmWaves;        // DMA instructions per wave per step
  constexpr int NST = MT * TPL;                        // score stores per wave per step
  static_assert(DPW >= 1 && DPW * kGemmWaves == 2 * TL::NPT, "a step splits evenly over the waves");
  static_assert(HI == 4 || HI == 8 || HI == 16, "whole tokens per lane");
  static_assert(NSTEPS >= 2 * NB, "a block spans at least two ring rounds");

  __shared__ __attribute__((aligned(1024))) char ring[NB][STEP_BYTES];
  __shared__ float kscale[KF8 ? kGemmKeys : 1];        // scales of the block's key rows

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  // Block order: a 1-D grid over (key block, request, row block) with the
  // row block varying fastest, dealt out so that each XCD takes a contiguous
  // range: the row blocks that read one key block run on one XCD, together,
  // and share its L2, whatever the number of key blocks (in natural order,
  // consecutive row blocks land on different XCDs: measured 161 against
  // 137 us).
  const int n_kb = a.gemm_key_blocks, n_rb = a.gemm_row_blocks;
  const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int rb = logical % n_rb, b = (logical / n_rb) % a.batch, kb = logical / (n_rb * a.batch);
  constexpr int TOK = kGemmRows / HI;                  // tokens per block
  const int s0 = rb * TOK;
  const int S = min(a.q_per_req - s0, TOK), SH = S * HI;
  const int sp = a.start_pos[b] + s0;
  const size_t tok0 = (size_t)b * a.q_per_req + s0;

  int nmax = 0;  // rows scored for this block: the largest visible count among non-fitting tokens
  for (int s = 0; s < S; ++s) {
    const int nv = min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap);
    if (nv > a.topk) nmax = max(nmax, nv);
  }
  const int key0 = kb * kGemmKeys;
  if (key0 >= nmax) return;  // whole block
  const int nsteps = min(NSTEPS, (nmax - key0 + kGemmStepKeys - 1) / kGemmStepKeys);

  // block table slice, one entry per lane (see the kernel above)
  int pblk = 0;
  if constexpr (PG) {
    const int lb = min((key0 >> a.block_shift) + lane, a.blocks_per_req - 1);
    const int e = a.block_table[(size_t)b * a.blocks_per_req + lb];
    pblk = (int)min((int64_t)max(e, 0), a.n_blocks - 1);
  }

  // A operand.  M tile mt of this wave holds block rows wave*64 + mt*32 ...;
  // MFMA row m (lane l32 supplies row l32) carries token
  // (m % 8 / 4) * TPL + i / HI and head i % HI of the tile, i = m / 8 * 4 + m % 4,
  // so that result slot v of lane (l32, half) is token half*TPL + v/HI, head
  // v % HI.  Rows past the block's tokens copy the last real row.
  u32x4_t qa[MT][KS];
  float wv[MT][16];
  uint32_t sbase[MT][TPL];   // byte offset of (token, key l32) in the block's score rows
  int slim[MT][TPL];         // store while key0 + st*32 < slim (visible count - l32; 0: never)
  const char* qbase = static_cast<const char*>(a.q_idx) + tok0 * HI * QROW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int tile_row0 = wave * 64 + mt * 32;
    {
      const int m = l32, i = (m >> 3) * 4 + (m & 3);
      const int row = tile_row0 + ((m >> 2) & 1) * TPL * HI + i;  // token*HI + head, in block rows
      const char* qp = qbase + (size_t)min(row, SH - 1) * QROW + 16 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qa[mt][ks] = ld16(qp + 32 * ks);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v)
      wv[mt][v] = a.w[tok0 * HI + min(tile_row0 + half * TPL * HI + v, SH - 1)];
#pragma unroll
    for (int tt = 0; tt < TPL; ++tt) {
      const int s = tile_row0 / HI + half * TPL + tt;
      const int nv = s < S ? min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap) : 0;
      sbase[mt][tt] = (uint32_t)(min(s, S - 1) * a.n_cap + l32) * 4u;
      slim[mt][tt] = nv > a.topk ? nv - l32 : INT32_MIN;   // past the block, or fits Top-K: never
    }
  }
  // FP8: the scales of keys key0 + 4*tid .. +3 (rows past nmax repeat the
  // last one), loaded before any DMA and published by the first step's barrier
  float ksv[KF8 ? 4 : 1];
  if constexpr (KF8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = min(key0 + 4 * (int)threadIdx.x + i, nmax - 1);
      size_t row = (size_t)b * a.n_cap + j;
      if constexpr (PG) {
        const int blk = __shfl(pblk, (j >> a.block_shift) - (key0 >> a.block_shift));
        row = ((size_t)blk << a.block_shift) + (size_t)(j & ((1 << a.block_shift) - 1));
      }
      ksv[i] = a.k_scale[row];
    }
  }
  // scores of this block's tokens, addressed by buffer stores (32-bit offsets)
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.scores + tok0 * a.n_cap, (int)((size_t)S * a.n_cap * 4));

  // DMA of step st: instruction i = wave*DPW + d fills tile u = i / NPT, rows
  // k*RPI + lane/NPR (k = i % NPT) with the piece swizzle of the kernel above.
  // Dense keys: buffer loads against the request's key rows.  The whole byte
  // offset, step included, goes in the per-lane offset: the range check of a
  // raw buffer access covers that offset only (the scalar offset is added
  // unchecked), so rows at or past n_cap read as zero without touching
  // memory, even for the steps the prologue issues past the last one.  Rows
  // past nmax but below n_cap are read and never used.  Paged keys: rows
  // clamped to nmax - 1 and mapped through the block table.
  int lrow[DPW];
  uint32_t loff[DPW];
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int i = wave * DPW + d, u = i / TL::NPT, k = i % TL::NPT;
    const int r = k * TL::RPI + lane / TL::NPR;
    const int piece = (lane % TL::NPR) ^ (r % TL::NPR);
    lrow[d] = u * 16 + r;
    loff[d] = (uint32_t)(lrow[d] * ROW + 16 * piece);
  }
  const char* kreq = static_cast<const char*>(a.k_idx) + (PG ? 0 : (size_t)b * a.n_cap * ROW);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kreq, PG ? 0 : a.n_cap * ROW);
  auto issue_step = [&](int st, int slot) {
    char* dst = ring[slot];
    const int step0 = key0 + st * kGemmStepKeys;
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int i = wave * DPW + d, u = i / TL::NPT, k = i % TL::NPT;
      char* lds = dst + u * TL::BYTES + 1024 * k;
      if constexpr (PG) {
        const int jt = min(step0 + u * 16, nmax - 1), j = min(step0 + lrow[d], nmax - 1);
        const int blk = __builtin_amdgcn_readlane(pblk, (jt >> a.block_shift) - (key0 >> a.block_shift));
        const size_t row = ((size_t)blk << a.block_shift) + (size_t)(j & ((1 << a.block_shift) - 1));
        dma16_global<kGemmKeyPolicy>(kreq + row * ROW + (loff[d] - (uint32_t)(lrow[d] * ROW)), lds);
      } else {
        // < 2^32: n_cap * ROW < 2^31 and step0 < n_cap + kGemmKeys
        dma16_buffer<kGemmKeyPolicy>(krs, lds, loff[d] + (uint32_t)step0 * (uint32_t)ROW, 0u);
      }
    }
  };

  // One step: publish it, refill the buffer freed by the previous step, run
  // its 16 MFMAs, and meanwhile finish the previous step: head sums and NST
  // unconditional score stores (the first step's are dummies past the buffer,
  // so every step issues the same count).  The two are independent, so the
  // matrix core and the vector ALU overlap within the wave.
  f32x16_t acc_prev[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_prev[mt] = f32x16_t{};
  auto finish = [&](const f32x16_t (&acc)[MT], int st_done) {
    const int jb = key0 + st_done * kGemmStepKeys;  // key of lane l32 = jb + l32; st_done < 0: dummy
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) {
        // heads in ascending order; relu as one integer max on the bits
        float sum = 0.0f;
#pragma unroll
        for (int h = 0; h < HI; ++h) {
          const float x = acc[mt][tt * HI + h];
          sum += wv[mt][tt * HI + h] * relu_bits(x);
        }
        if constexpr (KF8) sum *= kscale[max(st_done, 0) * kGemmStepKeys + l32];
        const uint32_t off = st_done >= 0 && jb < slim[mt][tt] ? sbase[mt][tt] + (uint32_t)jb * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sum), srs, off, 0, kNonTemporal);
      }
    }
  };
  auto run_step = [&](int st, int slot, int issue_slot, bool issue) {
    block_lds_barrier();  // every wave's share of step st is in; step st - 1 is read by all
    if (issue) issue_step(st + NB - 1, issue_slot);
    const char* src = ring[slot];
    const int u = l32 >> 4, r = l32 & 15;  // B operand: key l32, dims 16*ks + 8*half .. +8
    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t kb;
      if constexpr (KF8) {  // dims 16*ks + 8*half .. +8: half of piece ks
        const int sl = ks ^ (r % TL::NPR);
        const uint2 w = *reinterpret_cast<const uint2*>(src + u * TL::BYTES + r * ROW + 16 * sl + 8 * half);
        kb = u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true))};
      } else {
        const int sl = (2 * ks + half) ^ (r % TL::NPR);
        kb = *reinterpret_cast<const u32x4_t*>(src + u * TL::BYTES + r * ROW + 16 * sl);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qa[mt][ks]),
                                                          __builtin_bit_cast(bf16x8_t, kb), acc[mt], 0, 0, 0);
    }
#if CSA_GEMM_OVERLAP
    finish(acc_prev, st - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc_prev[mt] = acc[mt];
#else
    finish(acc, st);
#endif
  };

  // A fixed number of steps in flight (steps past nsteps load rows that are
  // never consumed; the last wait covers them), then one wait that covers the
  // query and weight loads, which are older than every DMA.
#pragma unroll
  for (int st = 0; st < NB - 1; ++st) issue_step(st, st);
  wait_vmcnt<(NB - 1) * DPW>();
  if constexpr (KF8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kscale[4 * threadIdx.x + i] = ksv[i];
  }

  // Step st is in once at most the younger operations are outstanding: the
  // DMA of up to NB - 2 younger steps and the stores of the up to NB - 1
  // steps computed since its DMA was issued (vector memory operations retire
  // in order).  Full rounds of NB steps run unrolled with constant waits and
  // buffers; the tail counts at run time (fewer stores counted: a longer,
  // still correct wait).
  int st = 0;
  if (nsteps >= 2 * NB - 1) {  // first round: all NB - 2 younger steps issued, st stores since
    static_for<0, NB>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      wait_vmcnt_sat<DPW * (NB - 2) + NST * u>();
      run_step(u, u, (u + NB - 1) % NB, true);
    });
    st = NB;
    for (; st + 2 * NB - 1 <= nsteps; st += NB) {  // steady rounds
      static_for<0, NB>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        wait_vmcnt_sat<DPW * (NB - 2) + NST * (NB - 1)>();
        run_step(st + u, u, (u + NB - 1) % NB, true);
      });
    }
  }
  for (; st < nsteps; ++st) {  // tail
    const int younger = min(NB - 2, nsteps - 1 - st);
    if (st >= NB - 1) {
      switch (younger) {
        case 0: wait_vmcnt_sat<NST * (NB - 1)>(); break;
        case 1: wait_vmcnt_sat<DPW * 1 + NST * (NB - 1)>(); break;
        case 2: wait_vmcnt_sat<DPW * 2 + NST * (NB - 1)>(); break;
        case 3: wait_vmcnt_sat<DPW * 3 + NST * (NB - 1)>(); break;
        case 4: wait_vmcnt_sat<DPW * 4 + NST * (NB - 1)>(); break;
        case 5: wait_vmcnt_sat<DPW * 5 + NST * (NB - 1)>(); break;
        default: wait_vmcnt_sat<DPW * 6 + NST * (NB - 1)>(); break;
      }
    } else {
      switch (younger) {
        case 0: wait_vmcnt_sat<0>(); break;
        case 1: wait_vmcnt_sat<DPW * 1>(); break;
        case 2: wait_vmcnt_sat<DPW * 2>(); break;
        case 3: wait_vmcnt_sat<DPW * 3>(); break;
        case 4: wait_vmcnt_sat<DPW * 4>(); break;
        case 5: wait_vmcnt_sat<DPW * 5>(); break;
        default: wait_vmcnt_sat<DPW * 6>(); break;
      }
    }
    run_step(st, st % NB, (st + NB - 1) % NB, st + NB - 1 < nsteps);
  }
#if CSA_GEMM_OVERLAP
  finish(acc_prev, nsteps - 1);
#endif
  wait_vmcnt<0>();  // no DMA may still be writing this block's LDS when it exits
}

template <int DI, bool PG, bool KF8>
hipError_t launch_gemm(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  switch (a.idx_heads) {
    case 4: hipLaunchKernelGGL((indexer_score_gemm_kernel<DI, 4, PG, KF8>), grid, dim3(kGemmThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((indexer_score_gemm_kernel<DI, 8, PG, KF8>), grid, dim3(kGemmThreads), 0, st, a); break;
    case 16: hipLaunchKernelGGL((indexer_score_gemm_kernel<DI, 16, PG, KF8>), grid, dim3(kGemmThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int DI, int HI, bool KF8, bool PG>
hipError_t launch_mt(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  const int mt = (a.tok_per_block * a.idx_heads + 15) / 16;
  switch (mt) {
    case 1: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 1, HI, KF8, PG>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 2, HI, KF8, PG>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 3, HI, KF8, PG>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 4, HI, KF8, PG>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int DI, bool KF8, bool PG>
hipError_t launch_hi(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  switch (a.idx_heads) {
    case 4: return launch_mt<T, DI, 4, KF8, PG>(a, grid, st);
    case 8: return launch_mt<T, DI, 8, KF8, PG>(a, grid, st);
    case 16: return launch_mt<T, DI, 16, KF8, PG>(a, grid, st);
    default: return launch_mt<T, DI, 0, KF8, PG>(a, grid, st);
  }
}

template <bool PG>
hipError_t launch_layout(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  if (a.k_scale) {  // FP8 key cache, bf16 queries (checked by the caller)
    return a.idx_dim == 128 ? launch_hi<__bf16, 128, true, PG>(a, grid, st)
                            : launch_hi<__bf16, 64, true, PG>(a, grid, st);
  }
  if (a.dtype == 1) {
    return a.idx_dim == 128 ? launch_hi<__bf16, 128, false, PG>(a, grid, st)
                            : launch_hi<__bf16, 64, false, PG>(a, grid, st);
  }
  return a.idx_dim == 128 ? launch_hi<float, 128, false, PG>(a, grid, st)
                          : launch_hi<float, 64, false, PG>(a, grid, st);
}

}  // namespace

hipError_t launch_indexer_score(const ScoreArgs& in, hipStream_t st) {
  const int n_bound = std::min(in.n_cap, in.max_len / in.ratio);
  if (n_bound <= in.topk) return hipSuccess;  // every token fits Top-K: nothing to score
  // Prefill chunks with bf16 queries, bf16 keys or 128-dim FP8 keys, and 4, 8
  // or 16 heads: the shared-key-step kernel, from the query-row count per
  // request at which it overtakes the kernel above (measured: about 2048 rows
  // with bf16 keys, 4096 with FP8 keys, whose widening costs it VALU issue;
  // below that its few 256-row blocks leave most CUs idle).
#ifndef CSA_SCORE_GEMM_MIN_ROWS
#define CSA_SCORE_GEMM_MIN_ROWS 2048
#endif
#ifndef CSA_SCORE_GEMM_MIN_ROWS_FP8
#define CSA_SCORE_GEMM_MIN_ROWS_FP8 4096
#endif
  const long long rows_req = (long long)in.q_per_req * in.idx_heads;
  const long long min_rows = in.k_scale ? CSA_SCORE_GEMM_MIN_ROWS_FP8 : CSA_SCORE_GEMM_MIN_ROWS;
  if (in.dtype == 1 && (!in.k_scale || in.idx_dim == 128) && rows_req >= min_rows &&
      (in.idx_heads == 4 || in.idx_heads == 8 || in.idx_heads == 16)) {
    const int tok_per_block = kGemmRows / in.idx_heads;
    const int row_blocks = (in.q_per_req + tok_per_block - 1) / tok_per_block;
    // a block's score rows and a request's key rows are addressed with 32-bit byte offsets
    if (row_blocks <= 65535 && (long long)tok_per_block * in.n_cap * 4 < 0x7FFFF000LL &&
        (long long)in.n_cap * in.idx_dim * 2 < 0x7FFFF000LL) {
      ScoreArgs g = in;
      g.gemm_key_blocks = (n_bound + kGemmKeys - 1) / kGemmKeys;
      g.gemm_row_blocks = row_blocks;
      const long long blocks = (long long)g.gemm_key_blocks * in.batch * row_blocks;
      if (blocks > INT32_MAX) return hipErrorInvalidValue;
      const dim3 grid((unsigned)blocks);
      if (g.k_scale)
        return g.block_table ? launch_gemm<128, true, true>(g, grid, st) : launch_gemm<128, false, true>(g, grid, st);
      if (g.block_table)
        return g.idx_dim == 128 ? launch_gemm<128, true, false>(g, grid, st) : launch_gemm<64, true, false>(g, grid, st);
      return g.idx_dim == 128 ? launch_gemm<128, false, false>(g, grid, st) : launch_gemm<64, false, false>(g, grid, st);
    }
  }
  // Query rows per workgroup: all of a request's when they fit in 64 (decode),
  // else blocks of floor(64 / Hi) tokens (prefill chunks).
  ScoreArgs a = in;
  a.tok_per_block = a.q_per_req * a.idx_heads <= 64 ? a.q_per_req : 64 / a.idx_heads;
  // Streaming (non-temporal) score stores when the step writes many scores:
  // they then keep the key stream's traffic in order (wide Top-K step, 16 MiB
  // of scores: score kernel 91.9 -> 88.3 us, Top-K after it 17.1 -> 17.7 us);
  // a few scores are better kept in the caches the Top-K reads them from
  // (long-context step, 1 MiB: score kernel 12.9 -> 12.5 us, Top-K 12.3 ->
  // 11.9 us with ordinary stores).
#ifndef CSA_SCORE_STREAM_MIN_BYTES
#define CSA_SCORE_STREAM_MIN_BYTES (4ll << 20)
#endif
  a.stream_scores = (long long)a.batch * a.q_per_req * n_bound * 4 >= CSA_SCORE_STREAM_MIN_BYTES;
  // a workgroup's score rows are reached by 32-bit buffer offsets below 2^31
  // bytes; past that (n_cap in the millions) by 64-bit streaming stores
  if ((long long)a.tok_per_block * a.n_cap * 4 > 0x7FFFF000LL) a.stream_scores = 2;
  const int row_blocks = (a.q_per_req + a.tok_per_block - 1) / a.tok_per_block;
  if (row_blocks > 65535) return hipErrorInvalidValue;
  dim3 grid((n_bound + kScoreKeysPerBlock - 1) / kScoreKeysPerBlock, a.batch, row_blocks);
  return a.block_table ? launch_layout<true>(a, grid, st) : launch_layout<false>(a, grid, st);
}

}  // namespace csa
