// The allocation-free backward entry point (fa_bwd_noalloc, include/fa.h).
//
// Callers that cannot allocate device memory -- code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc -- get the
// backward pass without a workspace argument.  Its workspace (two floats per
// query row: -rowsum(dO * O) and the saved LSE in base 2) lives in the file-
// scope device array below, of fixed size, which every GPU the library runs
// on holds from the first call until the process ends.  The kernels are
// those of fa_bwd / fa_bwd_blocksparse; only where the workspace comes from
// differs.
//
// Host code never uses the array's name as a device address (on the host
// that name is a stand-in, not the allocation): on the first call on a
// device, with that device current, its address is looked up once with
// hipGetSymbolAddress and kept per device; the kernels receive that pointer.
// Nothing in the workspace has to start at zero: the first backward kernel
// writes every element the others read.  All calls on one GPU share the
// array, so calls that overlap in time on one GPU (other streams, other
// threads) race on it.
#include <mutex>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

// FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES (16 MiB): two floats per query row, so
// B * H * N_q up to 2,097,152 rows (e.g. 16 heads x 128K queries); larger
// problems are refused.
constexpr size_t kScratchBytes = FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device, guarded by g_mu

// The workspace for a call on the current device: the size check first (no
// HIP call), then the device's address of the array, looked up on the first
// call on that device.
fa_status_t static_workspace(size_t need, void **ws, size_t *bytes) {
  if (need > kScratchBytes)
    return fa::set_error(FA_ERR_UNSUPPORTED,
                         "fa_bwd_noalloc: workspace of %zu bytes exceeds the %zu-byte static array "
                         "(B*H*N_q too large; use fa_bwd with a caller workspace)",
                         need, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa::set_error(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fa::set_error(FA_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fa::set_error(FA_ERR_HIP, "hipGetSymbolAddress of the static workspace failed: %s",
                           hipGetErrorString(e));
    g_ptr[dev] = ptr;
  }
  *ws = g_ptr[dev];
  *bytes = kScratchBytes;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status_t fa_bwd_noalloc(const fa_problem_t *p, const uint8_t *block_mask, int32_t mask_block,
                           int64_t mask_head_stride, const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *dout, void *dq, void *dk,
                           void *dv, void *stream) {
  return fa::bwd_impl(p, block_mask, mask_block, mask_head_stride, block_mask != nullptr, q, k, v, o,
                      lse, dout, dq, dk, dv, nullptr, 0, FA_BWD_ALL, stream, static_workspace);
}

}  // extern "C"
