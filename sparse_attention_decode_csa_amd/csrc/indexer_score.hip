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
// as N.  Each lane loads 16 contiguous bytes of one key row per 64-byte chunk
// straight into the MFMA B operand, so a wave reads whole 256-byte rows with
// no LDS staging and no reuse to exploit.  The per-head relu and weighted sum
// runs in registers when the head count is 4, 8 or 16 (each lane's four
// result rows are heads of one token), else through a small per-wave LDS
// tile; either way in a fixed head order.
#include "device_common.h"
#include "kernels.h"

namespace csa {
namespace {

#ifndef CSA_SCORE_TILES_PER_WAVE
#define CSA_SCORE_TILES_PER_WAVE 8
#endif
#ifndef CSA_SCORE_UNROLL
#define CSA_SCORE_UNROLL 4
#endif
constexpr int kScoreWaves = 4;
constexpr int kScoreTilesPerWave = CSA_SCORE_TILES_PER_WAVE;               // 16-key tiles
constexpr int kScoreUnroll = CSA_SCORE_UNROLL;                             // tiles per load group
constexpr int kScoreGroups = kScoreTilesPerWave / kScoreUnroll;
constexpr int kScoreKeysPerBlock = kScoreWaves * kScoreTilesPerWave * 16;  // 512

// HI > 0: the indexer head count, a power of two in 4 .. 16, so that the four
// result rows a lane holds (4g .. 4g+3 of a 16-row tile) belong to one token
// and the head sum finishes with at most two cross-lane adds.  HI == 0: any
// head count, summed through a small per-wave LDS tile.
template <typename T, int DI, int MT, int HI>
__global__ __launch_bounds__(256) void indexer_score_kernel(ScoreArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int CH = DI * ES / 64;   // 64-byte chunks per row; a lane holds 16 B of each
  static_assert(CH >= 1 && DI * ES % 64 == 0, "row must be a whole number of 64-byte chunks");
  constexpr int ROWS = MT * 16;      // padded query rows
  constexpr int RP = 17;             // padded LDS row length (floats)

  __shared__ float red[HI ? 1 : kScoreWaves][HI ? 1 : ROWS][RP];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  const int S = a.q_per_req, Hi = a.idx_heads, SH = S * Hi;
  const int sp = a.start_pos[b];

  // Rows scored for this request: the largest visible count among its tokens
  // that do not fit Top-K.
  int nmax = 0;
  for (int s = 0; s < S; ++s) {
    const int nv = min(n_visible(clamp_pos(sp + s, a.max_len), a.ratio), a.n_cap);
    if (nv > a.topk) nmax = max(nmax, nv);
  }
  const int key0 = blockIdx.x * kScoreKeysPerBlock;
  if (key0 >= nmax) return;  // whole workgroup: nothing visible in this chunk

  // A operand: query row qr = mt*16 + n16 (token qr / Hi, head qr % Hi);
  // padded rows load a real row and are zeroed, so the loads stay unconditional.
  u32x4_t qa[MT][CH];
  float wv[MT][4];
  const char* qbase = static_cast<const char*>(a.q_idx) + (size_t)b * SH * DI * ES;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int qr = mt * 16 + n16;
    const char* qp = qbase + (size_t)min(qr, SH - 1) * DI * ES + g * 16;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const u32x4_t v = ld16(qp + c * 64);
      qa[mt][c] = qr < SH ? v : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * g + i;   // result rows this lane holds
      const float wr = a.w[(size_t)b * SH + min(row, SH - 1)];
      wv[mt][i] = row < SH ? wr : 0.0f;
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

  const char* kbase = static_cast<const char*>(a.k_idx) + (size_t)b * a.n_cap * DI * ES;
  float* srow = a.scores + (size_t)b * S * a.n_cap;

  // Tiles are interleaved over the 4 waves so that at each step the block
  // reads 4 consecutive 16-row tiles (16 KiB contiguous for Di = 128 bf16).
  auto tile_key0 = [&](int t) { return key0 + (t * kScoreWaves + wave) * 16; };
  auto load_group = [&](int grp, u32x4_t (&dst)[kScoreUnroll][CH]) {
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int j = min(tile_key0(grp * kScoreUnroll + u) + n16, nmax - 1);  // clamp: a real row
      const char* rp = kbase + (size_t)j * DI * ES + g * 16;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
#if CSA_SCORE_STREAMING_LOADS
        dst[u][c] = ld16_stream(rp + c * 64);
#else
        dst[u][c] = ld16(rp + c * 64);  // plain loads measured faster than the non-temporal hint
#endif
      }
    }
  };

  u32x4_t kb[2][kScoreUnroll][CH];
  load_group(0, kb[0]);
#pragma unroll
  for (int grp = 0; grp < kScoreGroups; ++grp) {
    if (grp + 1 < kScoreGroups) load_group(grp + 1, kb[(grp + 1) & 1]);  // prefetch
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int tkey0 = tile_key0(grp * kScoreUnroll + u);
      f32x4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[mt] = mma_chunk<T>(qa[mt][c], kb[grp & 1][u][c], acc[mt]);
      }
      // lane holds dot(query row mt*16+4g+i, key tkey0+n16)
      if constexpr (HI > 0) {
        // heads in ascending order: the lane's four, then pairs of lanes
        const int j = tkey0 + n16;
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
          const bool writer = (g & (HI / 4 - 1)) == 0;
          if (writer && tok_of[mt] < S && nv_of[mt] > a.topk && j < nv_of[mt])
            srow[(size_t)tok_of[mt] * a.n_cap + j] = sum;
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
          const int j = tkey0 + n;
          if (nv > a.topk && j < nv) srow[(size_t)s * a.n_cap + j] = sum;
        }
        wave_lds_fence();
      }
    }
  }
}

template <typename T, int DI, int HI>
hipError_t launch_mt(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  const int mt = (a.q_per_req * a.idx_heads + 15) / 16;
  switch (mt) {
    case 1: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 1, HI>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 2, HI>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 3, HI>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((indexer_score_kernel<T, DI, 4, HI>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int DI>
hipError_t launch_hi(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  switch (a.idx_heads) {
    case 4: return launch_mt<T, DI, 4>(a, grid, st);
    case 8: return launch_mt<T, DI, 8>(a, grid, st);
    case 16: return launch_mt<T, DI, 16>(a, grid, st);
    default: return launch_mt<T, DI, 0>(a, grid, st);
  }
}

}  // namespace

hipError_t launch_indexer_score(const ScoreArgs& a, hipStream_t st) {
  const int n_bound = std::min(a.n_cap, a.max_len / a.ratio);
  if (n_bound <= a.topk) return hipSuccess;  // every token fits Top-K: nothing to score
  dim3 grid((n_bound + kScoreKeysPerBlock - 1) / kScoreKeysPerBlock, a.batch);
  if (a.dtype == 1) {
    return a.idx_dim == 128 ? launch_hi<__bf16, 128>(a, grid, st) : launch_hi<__bf16, 64>(a, grid, st);
  }
  return a.idx_dim == 128 ? launch_hi<float, 128>(a, grid, st) : launch_hi<float, 64>(a, grid, st);
}

}  // namespace csa
