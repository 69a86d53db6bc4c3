// Window-cache writeback: the step's new K and V rows, scattered to the cache
// rows named by a slot mapping ("Perf: parallelize the DSpark TP-4 SWA decode
// hot tasks", description, writeback item; its review asks that every slot
// mapping entry be committed even when the row count is not a multiple of the
// tile).
//
// Design: one thread per 16-byte piece of a row, K and V both; the grid is
// rounded up and the last block is masked by the piece count, so no entry is
// dropped for any token count.  A slot outside [0, n_slots) is padding.  The
// copy is bit for bit.  HBM-bound and tiny (the step's tokens only).
#include "device_common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kWbThreads = 256;

__global__ __launch_bounds__(kWbThreads) void swa_writeback_kernel(WritebackArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kWbThreads + threadIdx.x;
  const int ppr = a.row_bytes / 16;  // 16-byte pieces per row
  if (i >= (int64_t)a.n_tokens * ppr) return;
  const int t = (int)(i / ppr), piece = (int)(i - (int64_t)t * ppr);
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.n_slots) return;
  const size_t src = (size_t)t * a.row_bytes + 16 * piece;
  const size_t dst = (size_t)slot * a.row_bytes + 16 * piece;
  const u32x4_t k = ld16(static_cast<const char*>(a.k_new) + src);
  const u32x4_t v = ld16(static_cast<const char*>(a.v_new) + src);
  *reinterpret_cast<u32x4_t*>(static_cast<char*>(a.k_cache) + dst) = k;
  *reinterpret_cast<u32x4_t*>(static_cast<char*>(a.v_cache) + dst) = v;
}

}  // namespace

hipError_t launch_swa_writeback(const WritebackArgs& a, hipStream_t st) {
  const int64_t pieces = (int64_t)a.n_tokens * (a.row_bytes / 16);
  if (pieces == 0) return hipSuccess;
  const dim3 grid((unsigned)((pieces + kWbThreads - 1) / kWbThreads));  // ceil: the tail block is masked
  hipLaunchKernelGGL(swa_writeback_kernel, grid, dim3(kWbThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
