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
//      registers, thread t owning a contiguous slice, all loads issued at once.
//   2. Exact K-th largest key by MSB-first 8-bit radix select over LDS
//      histograms.  For long rows the select first runs on a strided sample
//      (one or two keys per thread), to a sample rank that keeps somewhat
//      more than K rows;
//      the rows at or above that threshold are compacted, and the exact
//      select runs on those candidates only.  When the sample misleads (fewer
//      than K rows kept, or more than the candidate buffer holds) the exact
//      select runs on the whole row instead, so only the speed depends on the
//      data.  The result is the threshold key T and how many keys equal to T
//      are taken (the lowest-indexed ones).
//   3. Emit in ascending index order: each thread counts its keys above and
//      equal to T, one block scan turns the counts into output offsets and
//      tie ranks, and each thread writes its slice.
//   Longer rows (more than 32768 candidates) are split over several
//   workgroups in a decode-sized launch (two passes: per-chunk candidates
//   above a sampled threshold, then an exact merge, below), and otherwise use
//   the same selection with the keys re-read from global memory in every
//   pass.
// The selection never depends on a floating-point operation, so it is exact
// and identical from run to run.  The pages' own design is a blocked sort with
// merge stages that quadruple the block length and must reach 1024 past width
// 256 ("Fix: port the DeepSeek-V4 MoE, hc_pre and prefill fixes to DSpark",
// description); with ascending-index output no sorted order is needed at all,
// so selection replaces the sort and has no width-dependent stage to miss.
// (A bitonic sort of the sampled candidates in registers and LDS, 2048 wide,
// in place of their radix select, was measured slower: decode Top-K 30.1
// against 18.8 us on 128 rows of 32768, 24.6 against 13.9 us on 16 rows of
// 8-16k, its 66 dependent exchange stages each a cross-lane or LDS round
// trip.)
#include "device_common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kTopkThreads = 1024;
// launches of at least this many tokens (prefill chunks) select in 4-wave
// blocks, several per CU; fewer tokens (decode) take 16-wave blocks, or the
// two-pass selection for rows past 32768 keys
#define CSA_TOPK_SMALL_BLOCK_TOKENS_DEFAULT 2048
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

constexpr int kGlobalSmemWords = kHistWords + 256 + kMiscWords;

// Exact selection of the K largest of row[0 .. n) (n > K) by one workgroup of
// kTopkThreads, with the keys re-read from global memory (L2) in every pass,
// written to out[0 .. K) in ascending index order.  smem: kGlobalSmemWords.
__device__ void select_row_global(const float* row, int n, int K, int32_t* out, uint32_t* smem) {
  uint32_t* hist = smem;                      // [16 waves][256 bins]
  uint32_t* cnt = smem + kHistWords;          // [256]
  int* misc = reinterpret_cast<int*>(cnt + 256);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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

// Rows longer than the register-resident kernel holds: the same selection,
// keys re-read from global memory (L2) in every pass.
__global__ __launch_bounds__(kTopkThreads) void topk_global_kernel(TopkArgs a) {
  __shared__ uint32_t smem[kGlobalSmemWords];
  const int tid = threadIdx.x;
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
  select_row_global(a.scores + (size_t)tok * a.n_cap, n, K, out, smem);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: four
// row_shr steps scan each 16-lane row (lanes shifted in from outside the row
// read 0), then each row adds the totals of the rows below it, read with
// readlane.  No LDS round trip.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Exclusive prefix sum of one int per thread over a block of NW waves, in
// thread order; also returns the block total.  `red` holds one int per wave.
template <int NW, bool TAIL = true>
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) red[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = red[w];
    before += w < wave ? t : 0;
    total += t;
  }
  if (TAIL) __syncthreads();  // red may be written again (callers that never do pass false)
  return before + inc - v;
}

// Maximum over the 64 lanes of a wave with DPP moves (row_shr within each
// 16-lane row, then readlane of the four row maxima).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(r0, r1), max(r2, r3));
}

// block_exclusive_scan that also reduces a maximum over the block through
// the same barriers.  `red` holds two ints per wave.
template <int NW, bool TAIL = true>
__device__ __forceinline__ int block_exclusive_scan_max(int v, uint32_t mx, int* red, int& total,
                                                        uint32_t& block_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  const uint32_t wm = wave_max(mx);
  if (lane == kWave - 1) {
    red[2 * wave] = inc;
    red[2 * wave + 1] = (int)wm;
  }
  __syncthreads();
  int before = 0;
  total = 0;
  block_max = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = red[2 * w];
    before += w < wave ? t : 0;
    total += t;
    block_max = max(block_max, (uint32_t)red[2 * w + 1]);
  }
  if (TAIL) __syncthreads();  // red may be written again (callers that never do pass false)
  return before + inc - v;
}

// Histograms of the block-wide selections, double buffered by pass parity so
// that zeroing the next pass's histogram needs no barrier of its own.
constexpr int kHistStride = 257;   // per-wave copies sit off the bank period
template <int NW>
struct alignas(16) SelectSmem {  // 16-byte aligned: the bin scan reads uint4
  uint32_t hist[2][NW * kHistStride];
  uint32_t cnt[2][256];
  int res[2][3];   // per pass parity: (bin, keys above the bin, keys in the bin)
  int red[2 * NW];
  uint32_t list[kWave];  // the few keys left in the chosen bin, ranked directly
  int nlist;
  int fin[2];            // (T, keq) of that ranking
};

// Block-wide minimum and maximum of one key per thread (invalid threads pass
// UINT32_MAX / 0).  `red` holds two ints per wave.
template <int NW, bool TAIL = true>
__device__ __forceinline__ void block_min_max(uint32_t lo, uint32_t hi, int* red, uint32_t& mn,
                                              uint32_t& mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
  }
  if (lane == 0) {
    red[2 * wave] = (int)lo;
    red[2 * wave + 1] = (int)hi;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, (uint32_t)red[2 * w]);
    mx = max(mx, (uint32_t)red[2 * w + 1]);
  }
  if (TAIL) __syncthreads();  // red may be written again (callers that never do pass false)
}

// Exact selection over keys spread across the block: thread t holds NK keys,
// read through key(r) with validity valid(r).  Every valid key lies in
// [lo, hi].  Finds the k-th largest key T, how many keys equal to T belong to
// the top k (keq; the rest of the top k is strictly above T).  MSB-first
// radix passes of up to 8 bits over only the bits below the common prefix of
// lo and hi (keys in a narrow range share their leading bits, and those are
// exactly the digits on which histogram atomics would pile up on one bin).
// PER_WAVE selects one histogram per wave (many keys) or one shared
// histogram (few keys).  With max_passes < 4 the select stops early and T is
// the lower edge of the bin holding the k-th key (at least k keys are >= T).
// With FINISH_SMALL, once the chosen bin holds at most 64 keys and digits are
// still to resolve, one wave ranks those keys directly (each against all of
// them) instead: the same T and keq for one pass's cost, where each further
// radix pass costs about as much (measured: decode Top-K 16.3 -> 15.7 us,
// prefill chunk 102 -> 97 us).  (12-bit digits were measured too: the
// single-wave scan of 4096 bins cost more than the pass they save.)  No
// floating point anywhere.
template <int NW, bool PER_WAVE, int NK, bool FINISH_SMALL, bool CLEARED = false, typename Key, typename Valid>
__device__ void block_radix_select(Key key, Valid valid, int k, uint32_t lo, uint32_t hi,
                                   SelectSmem<NW>& sm, uint32_t& T, int& keq, int max_passes = 4) {
  constexpr int DB = 8, kBins = 1 << DB, NT = NW * kWave;
  static_assert(NT >= kBins, "one thread per bin sums the per-wave histograms");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWords = PER_WAVE ? NW * kHistStride : kBins;
  const int nb = lo == hi ? 0 : 32 - __clz(lo ^ hi);   // bits still to decide
  uint32_t pmask = nb == 32 ? 0u : ~((1u << nb) - 1u);
  uint32_t prefix = lo & pmask;
  int krem = k;
  // CLEARED: the caller guarantees hist[0] is zero and nlist is 0, both
  // behind a barrier already
  if (!CLEARED) {
    for (int i = tid; i < kWords; i += NT) sm.hist[0][i] = 0u;
    if (FINISH_SMALL && tid == 0) sm.nlist = 0;
    __syncthreads();
  }
  int pass = 0;
  for (int top = nb; top > 0; top -= DB, ++pass) {
    const int shift = top > DB ? top - DB : 0;
    const uint32_t dmask = (1u << (top - shift)) - 1u;
    const int par = pass & 1;
    uint32_t* h = sm.hist[par];
    uint32_t* wh = PER_WAVE ? h + wave * kHistStride : h;
#pragma unroll
    for (int r = 0; r < NK; ++r) {
      const uint32_t kv = key(r);
      if (valid(r) && (kv & pmask) == prefix) atomicAdd(&wh[(kv >> shift) & dmask], 1u);
    }
    // the other buffer was last read before the previous pass's final barrier
    for (int i = tid; i < kWords; i += NT) sm.hist[par ^ 1][i] = 0u;
    __syncthreads();
    const uint32_t* c = h;
    if (PER_WAVE) {
      if (tid < 256) {
        uint32_t t = 0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += h[w * kHistStride + tid];
        sm.cnt[par][tid] = t;
      }
      __syncthreads();
      c = sm.cnt[par];
    }
    if (wave == 0) {
      // lane owns bins 4*lane .. 4*lane+3 (one 16-byte read), the higher lanes
      // the higher bins, so an exclusive prefix over lanes in reverse order
      // counts the keys in all higher bins
      const uint4 v = *reinterpret_cast<const uint4*>(c + kBins - 4 * (lane + 1));
      const int e[4] = {(int)v.w, (int)v.z, (int)v.y, (int)v.x};  // bins downward
      const int local = e[0] + e[1] + e[2] + e[3];
      int run = wave_inclusive_scan(local) - local;
      const int b0 = kBins - 1 - 4 * lane;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (run < krem && krem <= run + e[d]) {
          sm.res[par][0] = b0 - d;
          sm.res[par][1] = run;
          sm.res[par][2] = e[d];
        }
        run += e[d];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sm.res[par][0] << shift;
    pmask |= dmask << shift;
    krem -= sm.res[par][1];
    if (pass + 1 == max_passes) break;
    if constexpr (FINISH_SMALL) {
      if (shift > 0 && sm.res[par][2] <= kWave) {  // block-uniform
        // the keys of the chosen bin: exactly the valid keys with the prefix
#pragma unroll
        for (int r = 0; r < NK; ++r) {
          const uint32_t kv = key(r);
          if (valid(r) && (kv & pmask) == prefix) sm.list[atomicAdd(&sm.nlist, 1)] = kv;
        }
        __syncthreads();
        if (wave == 0) {
          // the krem-th largest of them is T; lanes holding a key equal to
          // T all find the same (T, keq)
          const int n = sm.nlist;
          const uint32_t mine = lane < n ? sm.list[lane] : 0u;
          int gt = 0, eq = 0;
          for (int j = 0; j < n; ++j) {
            const uint32_t o = sm.list[j];
            gt += o > mine ? 1 : 0;
            eq += o == mine ? 1 : 0;
          }
          if (lane < n && gt < krem && krem <= gt + eq) {
            sm.fin[0] = (int)mine;
            sm.fin[1] = krem - gt;
          }
        }
        __syncthreads();
        T = (uint32_t)sm.fin[0];
        keq = sm.fin[1];
        return;
      }
    }
  }
  T = prefix;
  keq = krem;
}

// Candidate buffer: rows whose key clears the sampled threshold, kept as
// (key, row index) pairs in ascending row order.
// Candidate capacity of a block of NW waves: 16-wave blocks (decode) keep
// up to 8192 candidates; 4-wave blocks (launches of many tokens) 2048, so
// that their LDS stays small and several share a CU (4096 measured slower on
// prefill chunks: 141 us against 110 us for 8192 rows of 7168-8192 keys).
#ifndef CSA_TOPK_SMALL_CAND_CAP
#define CSA_TOPK_SMALL_CAND_CAP 2048
#endif
constexpr int cand_cap(int nw) { return nw >= 16 ? 8192 : CSA_TOPK_SMALL_CAND_CAP; }


// Ascending-index emission of the selection {key > T} plus the keq
// lowest-indexed keys equal to T, over items that thread t holds as a
// contiguous run in index order: item(j) for j < cnt gives (key, row index).
template <int NW, int NJ, typename Item>
__device__ __forceinline__ void emit_selection(Item item, int cnt, uint32_t T, int keq,
                                               int32_t* out, int K, int* red) {
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j < cnt) {
      const uint32_t kv = item(j).x;
      gt += kv > T ? 1 : 0;
      eq += kv == T ? 1 : 0;
    }
  }
  int tot;
  // both counts packed in one int: each block total is at most 32768 < 2^16
  // every caller ends its kernel after the emission: red is not written again
  const int before = block_exclusive_scan<NW, false>(gt | (eq << 16), red, tot);
  int eq_rank = before >> 16;
  int dst = (before & 0xFFFF) + min(eq_rank, keq);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j < cnt) {
      const uint2 it = item(j);
      const bool is_eq = it.x == T;
      const bool take = it.x > T || (is_eq && eq_rank < keq);
      eq_rank += is_eq ? 1 : 0;
      if (take && dst < K) out[dst] = (int32_t)it.y;  // exactly K are taken; bound is a safeguard
      dst += take ? 1 : 0;
    }
  }
}

// A block of NW waves per token.  Thread t owns the contiguous slice
// [t*KPT, t*KPT + KPT) of the row; with VEC4 the slice is read with 16-byte
// loads (rows 16-byte aligned).  Blocks whose rows can exceed the candidate
// buffer carry it (and the sampled-threshold path); smaller ones go straight
// to the whole-row selection and keep their LDS small, so that many of them
// share a CU when a launch holds many tokens (prefill chunks).
template <int NW, int KPT, bool VEC4>
__global__ __launch_bounds__(NW * kWave) void topk_reg_kernel(TopkArgs a) {
  constexpr int NT = NW * kWave;
  constexpr int kCandCap = cand_cap(NW);
  constexpr bool kCandPath = NT * KPT > kCandCap;
  __shared__ SelectSmem<NW> sm;

  const int tid = threadIdx.x;
  const int tok = blockIdx.x;
  const int S = a.q_per_req, b = tok / S, s = tok % S;
  const float* row = a.scores + (size_t)tok * a.n_cap;
  const int i0 = tid * KPT;
  // The 16-byte loads of the thread's slice do not depend on the position,
  // so they are issued before it arrives (a token that fits Top-K discards
  // them); nothing past n_cap is read.
  const bool vec_slice = VEC4 && i0 + KPT <= a.n_cap;
  float4 raw[VEC4 ? KPT / 4 : 1];
  if (vec_slice) {
#pragma unroll
    for (int j = 0; j < KPT; j += 4) raw[j / 4] = *reinterpret_cast<const float4*>(row + i0 + j);
  }
  const int p = clamp_pos(a.start_pos[b] + s, a.max_len);
  const int n = min(n_visible(p, a.ratio), a.n_cap);
  const int K = a.topk;
  int32_t* out = a.topk_idx + (size_t)tok * K;

  if (n <= K) {  // fits: every visible row, no scoring needed
    for (int i = tid; i < K; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  // (a sampled threshold keeps somewhat more than K rows: only tried while
  // K leaves room for that in the buffer)
  const bool cand_path = kCandPath && n > kCandCap && 2 * K <= kCandCap;  // block-uniform
  if (cand_path) {
    // the sample select's first histogram, cleared while the row is still
    // arriving, behind a barrier that does not wait for the row's loads
    if (tid < 256) sm.hist[0][tid] = 0u;
    block_lds_barrier();
  }

  // ---- the row, in registers.  Slots past n hold a copy of a valid key of
  // the same thread (or of row n-1), so they never widen the key range.
  uint32_t key[KPT];
  if (vec_slice) {
#pragma unroll
    for (int j = 0; j < KPT; j += 4) {
      const float4 v = raw[j / 4];
      key[j] = order_key(v.x);
      key[j + 1] = order_key(v.y);
      key[j + 2] = order_key(v.z);
      key[j + 3] = order_key(v.w);
    }
    if (i0 + KPT > n) {  // the one thread straddling n
#pragma unroll
      for (int j = 0; j < KPT; ++j) key[j] = i0 + j < n ? key[j] : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = i0 + j < n ? order_key(row[i0 + j]) : 0u;
  }
  auto valid = [&](int j) { return i0 + j < n; };
  uint32_t kmax = key[0];  // slots past n hold key 0, below every float's key: they never raise it
#pragma unroll
  for (int j = 1; j < KPT; ++j) kmax = max(kmax, key[j]);

  if constexpr (kCandPath) if (cand_path) {
    __shared__ uint2 cand[kCandCap];  // (key, row index)
    constexpr int kCandPerThread = kCandCap / NT;
    // ---- threshold from a strided sample.  Thread t offers NS rows, one from
    // each sub-slice of SUB = KPT/NS registers: row t*KPT + i*SUB + t%SUB of
    // sub-slice i.  How many of them exist has a closed form (no scan): all
    // NS for threads whose slice lies below n, those with i*SUB + t%SUB < n%KPT
    // for the thread straddling n, none past it.  16-wave blocks offer one row
    // per thread (1024 samples); 4-wave blocks two (512), which measured
    // 98 against 108 us on 8192 rows of 7168-8192 keys (four: 103 us, the
    // sample's own histogram passes cost more).
    // Two 8-bit passes over the full key range fix the top 16 key bits: the
    // threshold is the lower edge of the 16-bit bin holding the sample rank,
    // which keeps somewhat more rows than the sample rank alone.
    constexpr int NS = NW >= 16 ? 1 : 2;
    constexpr int SUB = KPT / NS;
    static_assert(KPT % NS == 0, "whole sub-slices");
    const int jo = tid % SUB;
    uint32_t sk[NS];  // key[i*SUB + jo] without a dynamic register index
    bool sv[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sk[i] = 0u;
#pragma unroll
      for (int jj = 0; jj < SUB; ++jj) sk[i] = jj == jo ? key[i * SUB + jj] : sk[i];
      sv[i] = valid(i * SUB + jo);
    }
    const int q = n / KPT, rr = n % KPT;
    int m = NS * min(q, NT);
    if (q < NT) {
#pragma unroll
      for (int i = 0; i < NS; ++i) m += (i * SUB + q % SUB < rr) ? 1 : 0;
    }
    // sample rank expected at row rank K, plus three standard deviations, so
    // that the threshold keeps at least K rows
    const int ks0 = (int)(((long long)K * m + n - 1) / n);
    const int ks = min(m, ks0 + 3 * (int)sqrtf((float)ks0) + 4);
    uint32_t tau;
    int unused;
    block_radix_select<NW, false, NS, false, /*CLEARED=*/true>(
        [&](int r) { return sk[r]; }, [&](int r) { return sv[r]; }, ks, 0u, 0xFFFFFFFFu, sm, tau, unused, 2);
    // ---- rows at or above the threshold, compacted in row order; the same
    // barriers give the row maximum
    // slots past n hold key 0, and no float has key 0: against a threshold of
    // at least 1 they need no separate test
    tau = max(tau, 1u);
    int mine = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) mine += key[j] >= tau ? 1 : 0;
    int c;
    uint32_t row_max;
    // (no barrier after the scan: the candidate path passes two before
    // sm.red is written again, the fallback one of its own)
    int pos = block_exclusive_scan_max<NW, false>(mine, kmax, sm.red, c, row_max);
    if (c >= K && c <= kCandCap) {  // block-uniform
      // the sample select's second (last) pass cleared hist[0], so the exact
      // select below starts without clearing it; the barrier after the
      // candidates makes nlist's reset visible too
      if (tid == 0) sm.nlist = 0;
      // only candidates are written (measured a little faster than writing
      // every slot with the misses sent to a spare slot)
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool hit = key[j] >= tau;
        if (hit) cand[pos] = make_uint2(key[j], (uint32_t)(i0 + j));
        pos += hit ? 1 : 0;
      }
      __syncthreads();
      // thread t takes a contiguous run of the candidates (so the emission
      // stays in row order) into registers, all its LDS reads in flight at
      // once: the radix passes and the small-bin list then read no LDS
      const int cpt = (c + NT - 1) / NT;
      const int c0 = min(c, tid * cpt), cnt = min(c, c0 + cpt) - c0;
      uint2 cv[kCandPerThread];
#pragma unroll
      for (int j = 0; j < kCandPerThread; ++j) cv[j] = j < cnt ? cand[c0 + j] : make_uint2(0u, 0u);
      // every candidate lies in [tau, row max]; few keys per thread, so one
      // shared histogram
      uint32_t T;
      int keq;
      block_radix_select<NW, false, kCandPerThread, true, /*CLEARED=*/true>(
          [&](int r) { return cv[r].x; }, [&](int r) { return r < cnt; }, K, tau, row_max, sm, T, keq);
      // emission over the candidates only
      emit_selection<NW, kCandPerThread>([&](int j) { return cv[j]; }, cnt, T, keq, out, K, sm.red);
      return;
    }
    __syncthreads();  // every thread has read the scan's sm.red before the fallback writes it
  }
  // ---- whole-row selection and emission
  uint32_t kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < KPT; ++j) kmin = min(kmin, valid(j) ? key[j] : 0xFFFFFFFFu);
  uint32_t row_min, row_max;
  // the select's first histogram and list, cleared behind the reduction's
  // barrier (nothing reads them before); the reduction's sm.red is written
  // again only by the emission, behind the select's barriers
  for (int i = tid; i < NW * kHistStride; i += NT) sm.hist[0][i] = 0u;
  if (tid == 0) sm.nlist = 0;
  block_min_max<NW, false>(kmin, kmax, sm.red, row_min, row_max);
  uint32_t T;
  int keq;
  block_radix_select<NW, true, KPT, true, /*CLEARED=*/true>([&](int j) { return key[j]; }, valid, K, row_min,
                                                            row_max, sm, T, keq);
  const int cnt = max(0, min(KPT, n - i0));
  emit_selection<NW, KPT>([&](int j) { return make_uint2(key[j], (uint32_t)(i0 + j)); }, cnt, T,
                          keq, out, K, sm.red);
}

template <int NW, int KPT>
void launch_reg(const TopkArgs& a, bool vec4, hipStream_t st) {
  const dim3 grid(a.batch * a.q_per_req), block(NW * kWave);
  if (vec4)
    hipLaunchKernelGGL((topk_reg_kernel<NW, KPT, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_reg_kernel<NW, KPT, false>), grid, block, 0, st, a);
}

// Rows of up to 32 keys per thread: the smallest slice that holds n_bound.
template <int NW>
bool launch_reg_sized(const TopkArgs& a, int n_bound, bool vec4, hipStream_t st) {
  constexpr int NT = NW * kWave;
  if (n_bound <= 4 * NT) launch_reg<NW, 4>(a, vec4, st);
  else if (n_bound <= 8 * NT) launch_reg<NW, 8>(a, vec4, st);
  else if (n_bound <= 16 * NT) launch_reg<NW, 16>(a, vec4, st);
  else if (n_bound <= 32 * NT) launch_reg<NW, 32>(a, vec4, st);
  else return false;
  return true;
}

// ---------------------------------------------------------------------------
// Decode-sized launches: a few hundred long rows or fewer.  One workgroup per
// row would leave most CUs idle while it reads its row and runs its chain of
// barriers, so each row is split over several workgroups and merged:
//   pass 1 (topk_chunk_kernel), one 256-thread workgroup per (token, chunk of
//     256 * KPT keys): the chunk's keys in registers; a sample of the whole
//     row (256 groups of 4 consecutive keys, at positions that depend on the
//     row length only, so every chunk of the row draws the same 1024 keys)
//     gives the same threshold tau in every chunk's workgroup: the sample key
//     of the rank expected at row rank K plus four standard deviations, so
//     that at least K keys of the row clear it with near certainty.  The
//     chunk's keys >= tau are compacted, in row order, into the chunk's slot
//     of the workspace (with their count; a slot holds a whole chunk, -1
//     marks a chunk past its slot's capacity should a plan ever make slots
//     smaller).
//   pass 2 (topk_merge_kernel), one 1024-thread workgroup per token: the
//     token's candidates, chunk by chunk (so in row order), at most 4 per
//     thread; the exact selection over them (every key >= the K-th largest
//     candidate is a candidate, since all keys >= tau are), then the
//     ascending-index emission of the candidate path above.  When the sample
//     misleads (fewer than K candidates, a chunk past its capacity, or more
//     candidates than the merge holds) the merge selects over the whole row
//     from global memory instead: only the speed depends on the data.
constexpr int kChunkThreads = 256;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kSampleGroups = kChunkThreads;           // one group of 4 keys per thread
constexpr int kSamples = 4 * kSampleGroups;
constexpr int kMergePerThread = 8;
constexpr int kMergeCap = kTopkThreads * kMergePerThread;

// First key of sample group g in a row of n >= 4 keys: spread over the row,
// a multiple of 4, and g's group ends inside the row.
__device__ __forceinline__ int sample_group_start(int g, int n) {
  return (int)(((long long)g * (n - 4)) / (kSampleGroups - 1)) & ~3;
}

template <int KPT, bool VEC4>
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(TopkArgs a) {
  __shared__ SelectSmem<kChunkWaves> sm;
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, tok = blockIdx.y;
  const int S = a.q_per_req, b = tok / S, s = tok % S;
  const float* row = a.scores + (size_t)tok * a.n_cap;
  const int i0 = chunk * (kChunkThreads * KPT) + tid * KPT;
  // the chunk's loads first: they do not depend on the position (a token
  // that fits Top-K discards them); nothing past n_cap is read
  const bool vec_slice = VEC4 && i0 + KPT <= a.n_cap;
  float4 raw[VEC4 ? KPT / 4 : 1];
  if (vec_slice) {
#pragma unroll
    for (int j = 0; j < KPT; j += 4) raw[j / 4] = *reinterpret_cast<const float4*>(row + i0 + j);
  }
  const int p = clamp_pos(a.start_pos[b] + s, a.max_len);
  const int n = min(n_visible(p, a.ratio), a.n_cap);
  const int K = a.topk;
  int32_t* cnt_out = a.cand_count + (size_t)tok * a.n_chunks + chunk;
  if (n <= K) return;  // fits: the merge emits every visible row and reads nothing here
  if (chunk * (kChunkThreads * KPT) >= n) {
    if (tid == 0) *cnt_out = 0;
    return;
  }
  // sample group of this thread: 4 keys inside the row (a row shorter than 4
  // keys repeats its last one)
  uint32_t sk[4];
  {
    const int q = n >= 4 ? sample_group_start(tid, n) : 0;
    if (VEC4 && n >= 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + q);
      sk[0] = order_key(v.x);
      sk[1] = order_key(v.y);
      sk[2] = order_key(v.z);
      sk[3] = order_key(v.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sk[e] = order_key(row[min(q + e, n - 1)]);
    }
  }
  uint32_t key[KPT];
  if (vec_slice) {
#pragma unroll
    for (int j = 0; j < KPT; j += 4) {
      const float4 v = raw[j / 4];
      key[j] = order_key(v.x);
      key[j + 1] = order_key(v.y);
      key[j + 2] = order_key(v.z);
      key[j + 3] = order_key(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = order_key(row[min(i0 + j, n - 1)]);
  }
  auto valid = [&](int j) { return i0 + j < n; };

  // tau: the sample key of rank ks (exact: the select runs to the end)
  const int ks0 = (int)(((long long)K * kSamples + n - 1) / n);
  const int ks = min(kSamples, ks0 + 4 * (int)sqrtf((float)ks0) + 4);
  uint32_t tau;
  int unused;
  block_radix_select<kChunkWaves, false, 4, true>([&](int r) { return sk[r]; }, [&](int) { return true; }, ks,
                                                  0u, 0xFFFFFFFFu, sm, tau, unused);
  // the chunk's keys >= tau, compacted in row order
  int mine = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) mine += (valid(j) && key[j] >= tau) ? 1 : 0;
  int total;
  int pos = block_exclusive_scan<kChunkWaves>(mine, sm.red, total);
  if (total > a.chunk_cap) {  // block-uniform
    if (tid == 0) *cnt_out = -1;
    return;
  }
  uint2* cand = a.cand + ((size_t)tok * a.n_chunks + chunk) * a.chunk_cap;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool hit = valid(j) && key[j] >= tau;
    if (hit) cand[pos] = make_uint2(key[j], (uint32_t)(i0 + j));
    pos += hit ? 1 : 0;
  }
  if (tid == 0) *cnt_out = total;
}

__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(TopkArgs a) {
  __shared__ SelectSmem<kTopkWaves> sm;
  __shared__ uint32_t gsm[kGlobalSmemWords];   // the whole-row fallback
  __shared__ int first[65];                    // first candidate of each chunk
  __shared__ int status[2];                    // (total candidates, any chunk past its capacity)
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
  // candidates per chunk (the chunks holding visible keys: at most 64)
  const int nch = (n + a.chunk_keys - 1) / a.chunk_keys;
  if (wave == 0) {
    const int c = lane < nch ? a.cand_count[(size_t)tok * a.n_chunks + lane] : 0;
    const uint64_t over = __ballot(c < 0);
    const int inc = wave_inclusive_scan(max(c, 0));
    first[lane + 1] = inc;
    if (lane == 0) first[0] = 0;
    if (lane == kWave - 1) {
      status[0] = inc;
      status[1] = over != 0 ? 1 : 0;
    }
  }
  __syncthreads();
  const int total = status[0];
  if (status[1] || total < K || total > kMergeCap) {  // block-uniform
    select_row_global(a.scores + (size_t)tok * a.n_cap, n, K, out, gsm);
    return;
  }
  // thread t holds candidates [4t, 4t + 4): row order
  uint2 cv[kMergePerThread];
  const int c0 = tid * kMergePerThread;
  const int cnt = max(0, min(kMergePerThread, total - c0));
  uint32_t kmax = 0u;
#pragma unroll
  for (int j = 0; j < kMergePerThread; ++j) {
    const int i = min(c0 + j, total - 1);
    int c = 0;  // chunk of candidate i: first[c] <= i < first[c + 1]
    for (int step = 32; step > 0; step >>= 1)
      if (c + step <= nch - 1 && first[c + step] <= i) c += step;
    cv[j] = a.cand[((size_t)tok * a.n_chunks + c) * a.chunk_cap + (i - first[c])];
    kmax = max(kmax, cv[j].x);
  }
  // every candidate lies in [smallest candidate, row max] (the range only
  // decides how many radix passes run)
  uint32_t cmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < kMergePerThread; ++j) cmin = j < cnt ? min(cmin, cv[j].x) : cmin;
  uint32_t lo, row_max;
  block_min_max<kTopkWaves>(cmin, kmax, sm.red, lo, row_max);
  uint32_t T;
  int keq;
  block_radix_select<kTopkWaves, false, kMergePerThread, true>(
      [&](int r) { return cv[r].x; }, [&](int r) { return r < cnt; }, K, lo, row_max, sm, T, keq);
  emit_selection<kTopkWaves, kMergePerThread>([&](int j) { return cv[j]; }, cnt, T, keq, out, K, sm.red);
}

template <int KPT>
void launch_two_pass(const TopkArgs& a, bool vec4, hipStream_t st) {
  const dim3 grid(a.n_chunks, a.batch * a.q_per_req);
  if (vec4)
    hipLaunchKernelGGL((topk_chunk_kernel<KPT, true>), grid, dim3(kChunkThreads), 0, st, a);
  else
    hipLaunchKernelGGL((topk_chunk_kernel<KPT, false>), grid, dim3(kChunkThreads), 0, st, a);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(a.batch * a.q_per_req), dim3(kTopkThreads), 0, st, a);
}

}  // namespace

TopkPlan topk_plan(int batch, int q_per_req, int n_cap, int topk, int ratio, int max_len) {
  TopkPlan pl{};
  const long long tokens = (long long)batch * q_per_req;
  const int n_bound = std::min(n_cap, max_len / ratio);
  // Two passes for decode-sized launches of rows longer than one workgroup's
  // registers hold (32768 keys; there the one-workgroup selection re-reads
  // the row from L2 in every pass), with K small enough that the merge's
  // 8192 candidates hold the sampled threshold's expected count (about 2.9 K
  // at K = 1024 of 131072) with a wide margin.
#ifndef CSA_TOPK_TWO_PASS_MIN_ROW
#define CSA_TOPK_TWO_PASS_MIN_ROW 32769
#endif
#ifndef CSA_TOPK_TWO_PASS
#define CSA_TOPK_TWO_PASS 1
#endif
  if (CSA_TOPK_TWO_PASS && tokens < CSA_TOPK_SMALL_BLOCK_TOKENS_DEFAULT && n_bound >= CSA_TOPK_TWO_PASS_MIN_ROW &&
      topk <= 1024 && n_bound >= 4 * topk) {
    // the largest chunk (1024 .. 8192 keys) that still gives every CU a
    // workgroup, within the 64 chunks per row the merge reads
    int kpt = 0;
    for (int k : {32, 16, 8, 4}) {
      const long long chunks = (n_bound + kChunkThreads * k - 1) / (kChunkThreads * k);
      if (chunks > 64) break;
      kpt = k;
      if (tokens * chunks >= 256) break;
    }
    const int chunks = kpt ? (n_bound + kChunkThreads * kpt - 1) / (kChunkThreads * kpt) : 0;
    if (chunks < 2) return pl;  // rows too long for 64 chunks, or too short to split
    pl.two_pass = true;
    pl.chunk_keys = kChunkThreads * kpt;
    pl.n_chunks = (n_bound + pl.chunk_keys - 1) / pl.chunk_keys;
    // a slot holds a whole chunk: however the winners cluster in the row, no
    // chunk overflows (the number of candidates is a property of the row)
    pl.chunk_cap = pl.chunk_keys;
    pl.cand_bytes = ((size_t)tokens * pl.n_chunks * pl.chunk_cap * 8 + 255) / 256 * 256;
    pl.count_bytes = ((size_t)tokens * pl.n_chunks * 4 + 255) / 256 * 256;
    pl.ws_bytes = pl.cand_bytes + pl.count_bytes;
  }
  return pl;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int n_bound = std::min(a.n_cap, a.max_len / a.ratio);
  const long long tokens = (long long)a.batch * a.q_per_req;
  // rows start 16-byte aligned when n_cap is a multiple of 4 floats
  const bool vec4 = (a.n_cap & 3) == 0;
  if (a.cand) {  // the two-pass plan (the caller sized the workspace by topk_plan)
    switch (a.chunk_keys / kChunkThreads) {
      case 4: launch_two_pass<4>(a, vec4, st); break;
      case 8: launch_two_pass<8>(a, vec4, st); break;
      case 16: launch_two_pass<16>(a, vec4, st); break;
      case 32: launch_two_pass<32>(a, vec4, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // A decode step has few tokens: one 16-wave block per token, for latency.
  // A prefill chunk has thousands: 4-wave blocks (several per CU) when every
  // row fits in their registers.
#ifndef CSA_TOPK_SMALL_BLOCK_TOKENS
#define CSA_TOPK_SMALL_BLOCK_TOKENS CSA_TOPK_SMALL_BLOCK_TOKENS_DEFAULT
#endif
#ifndef CSA_TOPK_SMALL_BLOCK_WAVES
#define CSA_TOPK_SMALL_BLOCK_WAVES 4
#endif
  if (tokens >= CSA_TOPK_SMALL_BLOCK_TOKENS && launch_reg_sized<CSA_TOPK_SMALL_BLOCK_WAVES>(a, n_bound, vec4, st))
    return hipGetLastError();
  if (!launch_reg_sized<kTopkWaves>(a, n_bound, vec4, st))
    hipLaunchKernelGGL(topk_global_kernel, dim3(a.batch * a.q_per_req), dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
