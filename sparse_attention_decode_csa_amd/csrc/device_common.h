// Device helpers shared by the CSA decode kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand convention used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32): lane l supplies row (l % 16) of A and column
// (l % 16) of B; its k-slots are chosen by g = l / 16.  The result tile
// D[16][16] lands with lane l holding column (l % 16), rows 4g .. 4g+3.
// Because the contraction is a plain sum, any assignment of real k indices to
// (g, element) slots works as long as A and B use the same one; the kernels
// pick assignments that make each lane's global loads 16-byte contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// 16-byte global load / store (one dwordx4 per lane).
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Streaming load for data read exactly once (hint: do not keep in cache).
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Reinterpret 32 bits as a float.  Takes a scalar on purpose: applying
// __builtin_bit_cast directly to an ext-vector element (v[e]) was compiled as
// a cast of element 0 for every e, so vector elements must be extracted to a
// scalar first.
__device__ __forceinline__ float u32_as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
// relu(x) = x > 0 ? x : +0 as one integer max on the bits (negative floats,
// -0 included, are negative integers).  Takes a scalar: pass vector elements
// through a float variable (a bit cast written on an ext-vector element has
// compiled to element 0 for every index).
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x16 bf16: lane l supplies 4 elements of A row (l % 16) and of B
// column (l % 16), k-slots 4g .. 4g+3.
__device__ __forceinline__ f32x4_t mfma_bf16_k16(bf16x4_t a, bf16x4_t b, f32x4_t c) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                    c, 0, 0, 0);
}

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle).  Loads through such a resource whose offset falls outside its
// byte range return zero and do not access memory.
constexpr int kBufferConfig = 0x00020000;

// Cache-policy operand of the LDS DMA builtin: non-temporal (streamed data).
constexpr int kNonTemporal = 2;

// Buffer resource over [base, base + bytes).  base and bytes must be the same
// in every lane; they are moved to scalar registers explicitly, since a
// resource the compiler cannot prove uniform turns each load into a loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* up = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufferConfig);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 64-byte k-chunk of a row, i.e. each lane's 16 bytes: the bf16 form is a
// single 16x16x32 MFMA; the fp32 form is four 16x16x4 MFMAs, one per element.
template <typename T>
__device__ __forceinline__ f32x4_t mma_chunk(u32x4_t a, u32x4_t b, f32x4_t c);

template <>
__device__ __forceinline__ f32x4_t mma_chunk<__bf16>(u32x4_t a, u32x4_t b, f32x4_t c) {
  return mfma_bf16(as_bf16x8(a), as_bf16x8(b), c);
}

template <>
__device__ __forceinline__ f32x4_t mma_chunk<float>(u32x4_t a, u32x4_t b, f32x4_t c) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c = mfma_f32(u32_as_float(a[e]), u32_as_float(b[e]), c);
  return c;
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int popc_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Keeps the compiler from moving LDS accesses of one wave across this point.
// LDS serves one wave's requests in issue order, so a wave that writes LDS and
// then reads what other lanes of the same wave wrote needs no s_barrier.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS DMA: 16 bytes per lane from global memory (or a buffer) to LDS at
// lds + 16 * lane.  Kept in device functions: a call of these builtins
// written directly in a kernel body can keep the host compilation pass from
// emitting the kernel's launch stub.
template <int AUX>
__device__ __forceinline__ void dma16_global(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ void dma16_buffer(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voffset,
                                             uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                           soffset, 0, AUX);
}

// Workgroup barrier for LDS only: this wave's LDS operations complete, then
// s_barrier.  __syncthreads() also fences global memory, which on this target
// waits for every outstanding vector memory operation (vmcnt(0)), including
// LDS DMA prefetches still in flight; callers of this barrier wait for the DMA
// they need themselves.  The memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void block_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroups are dealt to the 8 XCDs round-robin by dispatch order.  This maps
// a dispatch index to a logical index such that each XCD receives one
// contiguous run of logical indices, so neighbouring logical work items share
// an XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, slot = bid / kXcd;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Causally visible compressed rows at position p (rows summarise R raw
// tokens each; a row is visible once its whole block is at or before p).
__device__ __forceinline__ int n_visible(int p, int ratio) { return (p + 1) / ratio; }

__device__ __forceinline__ int clamp_pos(int p, int max_len) {
  return p < 0 ? 0 : (p >= max_len ? max_len - 1 : p);
}

}  // namespace csa
