/* Memory-system ceiling probes for the CSA decode step (libcsa_ceilings.so).
 *
 * These are not part of the decode path and compute nothing the method
 * defines.  Each probe moves the bytes of one kernel of libcsa.so in that
 * kernel's access pattern and does nothing else with them, so that the
 * kernel's duration can be set against what the memory system delivers for
 * the same pattern:
 *
 *   csa_ceiling_stream_dma  the indexer key stream as the score kernel reads
 *                           it: 128 KiB per workgroup of 4 waves, each wave
 *                           keeping 4 tiles of 4 KiB in flight, HBM -> LDS by
 *                           DMA (1 KiB per instruction, non-temporal), either
 *                           in address order or with 16 KiB pages taken in
 *                           the order of a page table (a paged key pool);
 *   csa_ceiling_stream_vec  bytes read with plain 16-byte vector loads, one
 *                           contiguous range per workgroup (the key stream
 *                           without LDS DMA; the Top-K's score rows);
 *   csa_ceiling_gather      the attention's row gather: 256-byte K and V rows
 *                           named by a list of row numbers, 4 rows per wave
 *                           (16 lanes per row, one 16-byte piece per lane).
 *
 * The cost model they pin is the pages' own concern with moving gathered rows
 * and streamed keys straight into their consumers ("Perf: skip redundant CSA
 * scoring and fuse gather unpack", description).
 *
 * Conventions: every pointer is a device pointer owned by the caller; `stream`
 * is a hipStream_t (NULL = the null stream); calls are asynchronous.  `sink`
 * points to at least 4 writable device bytes: a probe writes sink[0] only in
 * the practically impossible case that its running XOR of the loaded data
 * equals a fixed constant, which keeps the loads from being optimised away;
 * its content carries no result.  Return value: 0 when the kernel was
 * launched, -1 when an argument is refused (nothing was launched), -2 when
 * the launch failed.
 */
#ifndef CSA_CEILINGS_H
#define CSA_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes per workgroup of csa_ceiling_stream_dma (the score kernel's block of
 * 512 rows of 256 bytes) and its page size when a page order is given. */
#define CSA_CEILING_DMA_WG_BYTES 131072
#define CSA_CEILING_DMA_PAGE_BYTES 16384

/* Reads `bytes` bytes by LDS DMA.  `bytes` must be a positive multiple of
 * CSA_CEILING_DMA_WG_BYTES and `src` 16-byte aligned.  With `page_order` NULL
 * the workgroups read `bytes` bytes of `src` in consecutive 128 KiB ranges.
 * Otherwise `src` is a pool of n_pages >= 1 pages of
 * CSA_CEILING_DMA_PAGE_BYTES bytes, `page_order` holds
 * bytes / CSA_CEILING_DMA_PAGE_BYTES entries, and logical page i is read from
 * pool page page_order[i] mod n_pages (as a block table maps a request's
 * logical blocks into a pool). */
int csa_ceiling_stream_dma(const void* src, int64_t bytes, const int32_t* page_order, int32_t n_pages,
                           uint32_t* sink, void* stream);

/* Reads `bytes` bytes from `src` with 16-byte vector loads, 8 per thread in
 * flight, one contiguous range of `bytes_per_wg` bytes per workgroup of
 * `threads` threads (256 or 1024; a 1024-thread workgroup over 128 KiB loads
 * its whole range at once, as the decode Top-K loads a row of 32768 scores).
 * `bytes_per_wg` must be a positive multiple of 16 that divides `bytes`;
 * `src` 16-byte aligned. */
int csa_ceiling_stream_vec(const void* src, int64_t bytes, int32_t bytes_per_wg, int32_t threads, uint32_t* sink,
                           void* stream);

/* Reads row rows[i] (i < n_rows) of both `k` and `v`, each a cache of
 * 256-byte rows of `cache_bytes` bytes (a multiple of 256, below 2^31).  A
 * row number outside [0, cache_bytes / 256) reads as zeros without touching
 * memory (buffer range check).  `rows` holds n_rows int32 entries. */
int csa_ceiling_gather(const void* k, const void* v, int64_t cache_bytes, const int32_t* rows, int32_t n_rows,
                       uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_CEILINGS_H */
