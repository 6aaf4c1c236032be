// Decode attention without a caller workspace, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation). The split-K partials live in one
// library-held device array per GPU instead of a workspace argument.
//
// The array is a file-scope __device__ variable, so the runtime places one
// copy on every GPU that loads the library, at its own address, held until
// the process ends. Host code never passes the array's name to a kernel (in
// host code that name is a stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "pagedkv.h"

namespace {

static_assert(PKV_SCRATCH_BYTES % 256 == 0, "scratch is whole 256-byte lines");
__device__ __align__(256) unsigned char scratch[PKV_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current device's scratch array (looked up on
// the first call on each device).
int scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return pkv::set_error(PKV_ELAUNCH, "paged_decode_attn_noalloc: no current device");
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return pkv::set_error(PKV_ELAUNCH,
                              "paged_decode_attn_noalloc: hipGetSymbolAddress of the scratch "
                              "array failed");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

}  // namespace

extern "C" int paged_decode_attn_noalloc(const pkv_pool *pool, int32_t plane_id,
                                         int32_t layer_id, const void *q, int32_t num_q_heads,
                                         const int32_t *page_table, int32_t page_table_stride,
                                         const int32_t *seq_lens, int32_t batch,
                                         int32_t max_seq_len, float scale, int32_t partition,
                                         void *out, float *lse, void *stream) {
  return pkv::decode_scratch(pool, plane_id, layer_id, q, num_q_heads, page_table,
                             page_table_stride, seq_lens, batch, max_seq_len, scale, partition,
                             out, lse, scratch_ptr, (size_t)PKV_SCRATCH_BYTES, stream);
}
