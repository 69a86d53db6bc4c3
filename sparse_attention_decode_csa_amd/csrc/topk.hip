// Causal Top-K selection with the fits-in-Top-K bypass.
//
// Tokens whose visible compressed cache fits within K are not sorted at all:
// their list is every visible row, 0 .. n_vis-1, then -1 ("Perf: skip
// redundant CSA scoring and fuse gather unpack", description and changes
// table: bounded indices instead of scoring and sorting).  Other tokens keep
// the K rows with the largest scores, lower index first among equal scores,
// written in ascending row order.  That order makes the general path and the
// bypass agree whenever every visible row fits.
//
// Design (one 1024-thread workgroup per query token):
//   1. Map each score to an unsigned key whose integer order is the float
//      order (-0 folded onto +0), and keep the whole row in LDS (up to 32768
//      rows = 128 KiB of the 160 KiB a gfx950 workgroup may hold).
//   2. Find the exact K-th largest key with four 8-bit MSB-first radix
//      passes: per-wave 256-bin LDS histograms of the keys that still match
//      the decided prefix, a suffix scan, and the bin where the running count
//      crosses the remaining rank.  This yields the threshold key T and how
//      many keys equal to T are taken (the lowest-indexed ones).
//   3. Emit in ascending index order: each wave owns a contiguous segment of
//      the row, counts its "above T" and "equal to T" keys with ballots, a
//      block-wide prefix over the 16 waves gives each wave its output offset
//      and its share of the tied keys, and a second ballot walk writes the
//      indices.
// The selection never depends on a floating-point operation, so it is exact
// and identical from run to run.  The pages' own design is a blocked sort with
// merge stages that quadruple the block length and must reach 1024 past width
// 256 ("Fix: port the DeepSeek-V4 MoE, hc_pre and prefill fixes to DSpark",
// description); with ascending-index output no sorted order is needed at all,
// so selection replaces the sort and has no width-dependent stage to miss.
#include "device_common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkLdsRows = 32768;
constexpr int kHistWords = kTopkWaves * 256;
constexpr int kMiscWords = 64;

// Unsigned key with the same order as the float value; -0 and +0 map to the
// same key, so they tie and the index decides.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                      // [16 waves][256 bins]
  uint32_t* cnt = smem + kHistWords;          // [256]
  int* misc = reinterpret_cast<int*>(cnt + 256);
  uint32_t* keys = smem + kHistWords + 256 + kMiscWords;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = blockIdx.x;
  const int S = a.q_per_req, b = tok / S, s = tok % S;
  const int p = clamp_pos(a.start_pos[b] + s, a.max_len);
  const int n = min(n_visible(p, a.ratio), a.n_cap);
  const int K = a.topk;
  int32_t* out = a.topk_idx + (size_t)tok * K;

  if (n <= K) {  // fits: every visible row, no scoring needed
    for (int i = tid; i < K; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }

  const float* row = a.scores + (size_t)tok * a.n_cap;
  if (IN_LDS)
    for (int i = tid; i < n; i += kTopkThreads) keys[i] = order_key(row[i]);
  auto key_at = [&](int i) -> uint32_t { return IN_LDS ? keys[i] : order_key(row[i]); };

  // ---- exact K-th largest key by MSB-first radix select
  if (tid == 0) {
    misc[0] = 0;
    misc[1] = 0;
  }
  uint32_t prefix = 0u, pmask = 0u;
  int krem = K;  // rank still to place among keys matching the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kHistWords; i += kTopkThreads) hist[i] = 0u;
    __syncthreads();
    uint32_t* wh = hist + wave * 256;
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t k = key_at(i);
      if ((k & pmask) == prefix) atomicAdd(&wh[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t t = 0u;
      for (int w = 0; w < kTopkWaves; ++w) t += hist[w * 256 + tid];
      cnt[tid] = t;
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 4*lane .. 4*lane+3; count of bins above them by a
      // suffix scan over lanes
      const uint32_t c0 = cnt[4 * lane], c1 = cnt[4 * lane + 1], c2 = cnt[4 * lane + 2],
                     c3 = cnt[4 * lane + 3];
      const uint32_t local = c0 + c1 + c2 + c3;
      uint32_t suf = local;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_down(suf, off);
        if (lane + off < kWave) suf += t;
      }
      uint32_t run = suf - local;  // keys in higher bins
      const uint32_t cs[4] = {c3, c2, c1, c0};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (run < (uint32_t)krem && (uint32_t)krem <= run + cs[d]) {
          misc[0] = 4 * lane + 3 - d;
          misc[1] = (int)run;
        }
        run += cs[d];
      }
    }
    __syncthreads();
    const int bin = misc[0], above = misc[1];
    prefix |= (uint32_t)bin << shift;
    pmask |= 0xFFu << shift;
    krem -= above;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the K-th largest key
  const int keq = krem;       // how many keys equal to T are taken

  // ---- ascending-index emission
  int* wgt = misc;                   // [16] keys above T per wave segment
  int* weq = misc + kTopkWaves;      // [16] keys equal to T per wave segment
  const int seg = ((n + kTopkThreads - 1) / kTopkThreads) * kWave;
  const int beg = min(n, wave * seg), end = min(n, beg + seg);
  int cgt = 0, ceq = 0;
  for (int base = beg; base < end; base += kWave) {
    const int i = base + lane;
    const uint32_t k = i < end ? key_at(i) : 0u;
    cgt += __popcll(__ballot(i < end && k > T));
    ceq += __popcll(__ballot(i < end && k == T));
  }
  if (lane == 0) {
    wgt[wave] = cgt;
    weq[wave] = ceq;
  }
  __syncthreads();
  int eq_before = 0, out_pos = 0;
  for (int w = 0; w < wave; ++w) {
    const int take = min(weq[w], max(0, keq - eq_before));
    out_pos += wgt[w] + take;
    eq_before += weq[w];
  }
  for (int base = beg; base < end; base += kWave) {
    const int i = base + lane;
    const uint32_t k = i < end ? key_at(i) : 0u;
    const bool gt = i < end && k > T;
    const bool eq = i < end && k == T;
    const uint64_t meq = __ballot(eq);
    const bool sel = gt || (eq && eq_before + popc_below(meq) < keq);
    const uint64_t msel = __ballot(sel);
    const int dst = out_pos + popc_below(msel);
    if (sel && dst < K) out[dst] = i;  // exactly K are selected; the bound is a safeguard
    out_pos += __popcll(msel);
    eq_before += __popcll(meq);
  }
}

constexpr size_t kTopkSmemBase = (size_t)(kHistWords + 256 + kMiscWords) * 4;

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int n_bound = std::min(a.n_cap, a.max_len / a.ratio);
  const int tokens = a.batch * a.q_per_req;
  if (n_bound <= kTopkLdsRows) {
    const size_t smem = kTopkSmemBase + (size_t)std::max(n_bound, 1) * 4;
    static bool attr_set = false;  // idempotent; racing first calls set the same value
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)(kTopkSmemBase + (size_t)kTopkLdsRows * 4));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    hipLaunchKernelGGL(topk_kernel<true>, dim3(tokens), dim3(kTopkThreads), smem, st, a);
  } else {
    hipLaunchKernelGGL(topk_kernel<false>, dim3(tokens), dim3(kTopkThreads), kTopkSmemBase, st, a);
  }
  return hipGetLastError();
}

}  // namespace csa
