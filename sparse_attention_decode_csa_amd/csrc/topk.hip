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
//      order (-0 folded onto +0).  Rows of up to 32768 candidates are held in
//      registers: thread t keeps keys t, t+1024, t+2048, ..., all loads issued
//      before any use, so the row is fetched in one memory round trip.
//   2. Find the exact K-th largest key with four 8-bit MSB-first radix
//      passes: per-wave 256-bin LDS histograms of the keys that still match
//      the decided prefix, a suffix scan, and the bin where the running count
//      crosses the remaining rank.  This yields the threshold key T and how
//      many keys equal to T are taken (the lowest-indexed ones).
//   3. Emit in ascending index order: slice r (keys 1024r .. 1024r+1023) is
//      spread over the 16 waves in index order, so ballots give each (slice,
//      wave) its count of keys above T and equal to T; one wave scans those
//      counts in index order into output offsets and tie ranks, and a second
//      ballot walk writes the indices.
//   Longer rows (more than 32768 candidates) use the same selection with the
//   keys re-read from global memory in every pass.
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
constexpr int kHistWords = kTopkWaves * 256;
constexpr int kMiscWords = 64;

// Unsigned key with the same order as the float value; -0 and +0 map to the
// same key, so they tie and the index decides.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rows longer than the register-resident kernel holds: same selection, keys
// re-read from global memory (L2) in every pass.
__global__ __launch_bounds__(kTopkThreads) void topk_global_kernel(TopkArgs a) {
  __shared__ uint32_t smem[kHistWords + 256 + kMiscWords];
  uint32_t* hist = smem;                      // [16 waves][256 bins]
  uint32_t* cnt = smem + kHistWords;          // [256]
  int* misc = reinterpret_cast<int*>(cnt + 256);

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
  auto key_at = [&](int i) -> uint32_t { return order_key(row[i]); };

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

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_reg_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kHistWords];        // [16 waves][256 bins]
  __shared__ uint32_t cnt[256];
  __shared__ int misc[2];
  __shared__ int seg_gt[KPT * kTopkWaves], seg_eq[KPT * kTopkWaves];     // [slice][wave]
  __shared__ int seg_off[KPT * kTopkWaves], seg_eqoff[KPT * kTopkWaves];

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

  // ---- the row, in registers (invalid slots read a real entry and are masked)
  const float* row = a.scores + (size_t)tok * a.n_cap;
  uint32_t key[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) key[r] = order_key(row[min(r * kTopkThreads + tid, n - 1)]);
  auto valid = [&](int r) { return r * kTopkThreads + tid < n; };

  // ---- exact K-th largest key by MSB-first radix select
  uint32_t prefix = 0u, pmask = 0u;
  int krem = K;
  uint32_t* wh = hist + wave * 256;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kHistWords; i += kTopkThreads) hist[i] = 0u;
    if (tid == 0) misc[0] = misc[1] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      if (valid(r) && (key[r] & pmask) == prefix) atomicAdd(&wh[(key[r] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 256) {
      uint32_t t = 0u;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) t += hist[w * 256 + tid];
      cnt[tid] = t;
    }
    __syncthreads();
    if (wave == 0) {
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
    prefix |= (uint32_t)misc[0] << shift;
    pmask |= 0xFFu << shift;
    krem -= misc[1];
  }
  const uint32_t T = prefix;  // the K-th largest key
  const int keq = krem;       // keys equal to T that are taken

  // ---- counts per (slice, wave), in index order
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int cg = __popcll(__ballot(valid(r) && key[r] > T));
    const int ce = __popcll(__ballot(valid(r) && key[r] == T));
    if (lane == 0) {
      seg_gt[r * kTopkWaves + wave] = cg;
      seg_eq[r * kTopkWaves + wave] = ce;
    }
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int PL = KPT * kTopkWaves / kWave;  // entries per lane, contiguous
    const int e0 = lane * PL;
    int le = 0;
#pragma unroll
    for (int k = 0; k < PL; ++k) le += seg_eq[e0 + k];
    int E = wave_inclusive_scan(le) - le;
    int sel[PL], ls = 0;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int eq = seg_eq[e0 + k];
      seg_eqoff[e0 + k] = E;
      sel[k] = seg_gt[e0 + k] + min(eq, max(0, keq - E));
      E += eq;
      ls += sel[k];
    }
    int O = wave_inclusive_scan(ls) - ls;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      seg_off[e0 + k] = O;
      O += sel[k];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool gt = valid(r) && key[r] > T;
    const bool eq = valid(r) && key[r] == T;
    const uint64_t meq = __ballot(eq);
    const bool take = gt || (eq && seg_eqoff[r * kTopkWaves + wave] + popc_below(meq) < keq);
    const uint64_t msel = __ballot(take);
    const int dst = seg_off[r * kTopkWaves + wave] + popc_below(msel);
    if (take && dst < K) out[dst] = r * kTopkThreads + tid;  // exactly K are taken; bound is a safeguard
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int n_bound = std::min(a.n_cap, a.max_len / a.ratio);
  const dim3 grid(a.batch * a.q_per_req), block(kTopkThreads);
  if (n_bound <= 4 * kTopkThreads) {
    hipLaunchKernelGGL(topk_reg_kernel<4>, grid, block, 0, st, a);
  } else if (n_bound <= 8 * kTopkThreads) {
    hipLaunchKernelGGL(topk_reg_kernel<8>, grid, block, 0, st, a);
  } else if (n_bound <= 16 * kTopkThreads) {
    hipLaunchKernelGGL(topk_reg_kernel<16>, grid, block, 0, st, a);
  } else if (n_bound <= 32 * kTopkThreads) {
    hipLaunchKernelGGL(topk_reg_kernel<32>, grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL(topk_global_kernel, grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace csa
