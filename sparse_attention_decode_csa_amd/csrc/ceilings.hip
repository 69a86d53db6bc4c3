// Memory-system ceiling probes: kernels that move the bytes of one kernel of
// the decode step in that kernel's access pattern and compute nothing, so the
// kernel's duration can be set against what the memory system gives that
// pattern.  Built into a library of its own; nothing on the decode path calls
// them.  Each probe XORs what it loads into one register and writes it only
// if it equals a fixed constant (practically never), so the loads stay.
#include "device_common.h"
#include "csa_ceilings.h"

namespace csa {
namespace {

constexpr uint32_t kSinkMagic = 0x5A17C0DEu;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any range below 2^31

// ---- LDS-DMA stream (the score kernel's key stream) --------------------------
constexpr int kDmaWaves = 4;
constexpr int kDmaTile = 4096;         // bytes per wave per tile: 4 DMA instructions of 1 KiB
constexpr int kDmaTilesPerWave = 8;
constexpr int kDmaRing = 4;            // tiles in flight per wave
constexpr int kDmaWgBytes = kDmaWaves * kDmaTilesPerWave * kDmaTile;
constexpr int kDmaPage = CSA_CEILING_DMA_PAGE_BYTES;
static_assert(kDmaWgBytes == CSA_CEILING_DMA_WG_BYTES, "workgroup bytes");
static_assert(kDmaPage % kDmaTile == 0, "a tile never straddles a page");

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Tiles are interleaved over the waves, so at each step the workgroup reads
// kDmaWaves consecutive tiles (16 KiB), as the score kernel does.
__global__ __launch_bounds__(kDmaWaves * 64) void stream_dma_kernel(const char* src, const int32_t* page_order,
                                                                     int n_pages, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char ring[kDmaWaves][kDmaRing][kDmaTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t wg0 = (size_t)blockIdx.x * kDmaWgBytes;
  auto tile_offset = [&](int t) { return wg0 + (size_t)(t * kDmaWaves + wave) * kDmaTile; };
  // Paged: lane t holds the pool page of the wave's tile t, loaded before any
  // DMA is issued (so waiting for it never waits for tiles).
  int my_page = 0;
  if (page_order && lane < kDmaTilesPerWave)
    my_page = (int)((uint32_t)page_order[tile_offset(lane) / kDmaPage] % (uint32_t)n_pages);
  auto issue = [&](int t) {
    const size_t logical = tile_offset(t);
    size_t phys = logical;
    if (page_order) phys = (size_t)__builtin_amdgcn_readlane(my_page, t) * kDmaPage + logical % kDmaPage;
    char* dst = ring[wave][t % kDmaRing];
#pragma unroll
    for (int k = 0; k < kDmaTile / 1024; ++k) {
      const char* p = src + phys + 1024 * k + 16 * lane;
      dma16_global<kNonTemporal>(p, dst + 1024 * k);
    }
  };
#pragma unroll
  for (int t = 0; t < kDmaRing; ++t) issue(t);
  u32x4_t acc = u32x4_t{0, 0, 0, 0};
  constexpr int kPerTile = kDmaTile / 1024;
#pragma unroll
  for (int t = 0; t < kDmaTilesPerWave; ++t) {
    // tile t has landed once only the younger tiles' DMAs are outstanding
    const int younger = t + kDmaRing - 1 < kDmaTilesPerWave ? kDmaRing - 1 : kDmaTilesPerWave - 1 - t;
    switch (younger) {  // a compile-time constant after unrolling
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<1 * kPerTile>(); break;
      case 2: wait_vm<2 * kPerTile>(); break;
      default: wait_vm<3 * kPerTile>(); break;
    }
    const char* tile = ring[wave][t % kDmaRing];
#pragma unroll
    for (int k = 0; k < kPerTile; ++k) acc ^= *reinterpret_cast<const u32x4_t*>(tile + 1024 * k + 16 * lane);
    wait_lgkm0();  // the slot is read before the next DMA overwrites it
    if (t + kDmaRing < kDmaTilesPerWave) issue(t + kDmaRing);
  }
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == kSinkMagic) sink[0] = v;
}

// ---- plain vector-load stream ---------------------------------------------
constexpr int kVecInFlight = 8;

template <int NT>
__global__ __launch_bounds__(NT) void stream_vec_kernel(const char* src, int per_wg, uint32_t* sink) {
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(src + (size_t)blockIdx.x * per_wg);
  const int n = per_wg / 16;
  u32x4_t acc = u32x4_t{0, 0, 0, 0};
  for (int i = threadIdx.x; i < n; i += NT * kVecInFlight) {
    u32x4_t v[kVecInFlight];
#pragma unroll
    for (int u = 0; u < kVecInFlight; ++u) {
      const int j = i + u * NT;
      v[u] = j < n ? p[j] : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kVecInFlight; ++u) acc ^= v[u];
  }
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == kSinkMagic) sink[0] = v;
}

// ---- row gather (the attention's K/V rows) ----------------------------------
constexpr int kRowBytes = 256;
constexpr int kGatherRowsPerWave = 4;
constexpr int kGatherWaves = 4;

__global__ __launch_bounds__(kGatherWaves * 64) void gather_kernel(const char* k, const char* v, int range,
                                                                   const int32_t* rows, int n_rows, uint32_t* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = (blockIdx.x * kGatherWaves + wave) * kGatherRowsPerWave + lane / 16;  // 16 lanes per row
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k, range);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v, range);
  const int j = r < n_rows ? rows[r] : -1;
  const bool ok = j >= 0 && (int64_t)j * kRowBytes < (int64_t)range;
  const uint32_t off = ok ? (uint32_t)j * kRowBytes + 16u * (lane % 16) : kOutOfRange;
  const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0);
  const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0);
  const u32x4_t acc = a ^ b;
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kSinkMagic) sink[0] = x;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -2; }

}  // namespace
}  // namespace csa

extern "C" {

int csa_ceiling_stream_dma(const void* src, int64_t bytes, const int32_t* page_order, int32_t n_pages,
                           uint32_t* sink, void* stream) {
  using namespace csa;
  if (!src || !sink || bytes <= 0 || bytes % kDmaWgBytes != 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return -1;
  if (bytes / kDmaWgBytes > INT32_MAX) return -1;
  if (page_order && n_pages <= 0) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_dma_kernel, dim3((unsigned)(bytes / kDmaWgBytes)), dim3(kDmaWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(src), page_order, n_pages, sink);
  return launched();
}

int csa_ceiling_stream_vec(const void* src, int64_t bytes, int32_t bytes_per_wg, int32_t threads, uint32_t* sink,
                           void* stream) {
  using namespace csa;
  if (!src || !sink || bytes <= 0 || bytes_per_wg <= 0 || bytes_per_wg % 16 != 0 || bytes % bytes_per_wg != 0 ||
      (threads != 256 && threads != 1024) || (reinterpret_cast<uintptr_t>(src) & 15))
    return -1;
  if (bytes / bytes_per_wg > INT32_MAX) return -1;
  (void)hipGetLastError();
  const dim3 grid((unsigned)(bytes / bytes_per_wg));
  if (threads == 256)
    hipLaunchKernelGGL(stream_vec_kernel<256>, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(src), bytes_per_wg, sink);
  else
    hipLaunchKernelGGL(stream_vec_kernel<1024>, grid, dim3(1024), 0, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(src), bytes_per_wg, sink);
  return launched();
}

int csa_ceiling_gather(const void* k, const void* v, int64_t cache_bytes, const int32_t* rows, int32_t n_rows,
                       uint32_t* sink, void* stream) {
  using namespace csa;
  if (!k || !v || !rows || !sink || n_rows <= 0 || cache_bytes <= 0 || cache_bytes % kRowBytes != 0 ||
      cache_bytes >= (int64_t)kOutOfRange || (reinterpret_cast<uintptr_t>(k) & 15) ||
      (reinterpret_cast<uintptr_t>(v) & 15))
    return -1;
  constexpr int per_wg = kGatherWaves * kGatherRowsPerWave;
  (void)hipGetLastError();
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((n_rows + per_wg - 1) / per_wg)), dim3(kGatherWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(k), static_cast<const char*>(v),
                     (int)cache_bytes, rows, n_rows, sink);
  return launched();
}

}  // extern "C"
