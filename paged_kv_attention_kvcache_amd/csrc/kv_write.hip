// store_kv for gfx950: scatter each token's K/V rows to the slots the
// scheduler hands out ("Faster fuzzy minds", section "LOTUS": handing the
// same slots again overwrites in place).
//
// One thread moves one 16-byte chunk of one (token, kv head) row of K and the
// same chunk of V. Consecutive threads cover consecutive chunks of a row, so
// both the reads of the dense [T][Hkv][D] input and the writes into the
// (page, kv head) tile row are 16-byte vectors, coalesced per row.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, const int32_t *__restrict__ slots,
    int32_t num_tokens, int32_t hkv, int32_t chunks_per_row, int32_t num_pages,
    uint4 *__restrict__ kb, uint4 *__restrict__ vb) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t per_token = (size_t)hkv * chunks_per_row;
  if (idx >= (size_t)num_tokens * per_token) return;
  const int t = (int)(idx / per_token);
  const int rem = (int)(idx % per_token);
  const int h = rem / chunks_per_row, c = rem % chunks_per_row;
  const int s = slots[t];
  if (s < 0 || s / kPage >= num_pages) return;
  const int page = s / kPage, off = s % kPage;
  const size_t dst = (((size_t)page * hkv + h) * kPage + off) * chunks_per_row + c;
  kb[dst] = k[idx];
  vb[dst] = v[idx];
}

hipError_t launch_kv_write(const Bank &b, const void *k, const void *v, const int32_t *slots,
                           int32_t num_tokens, hipStream_t stream) {
  const int bytes = b.dtype == 1 ? 2 : 4;
  const int cpr = b.head_dim * bytes / 16;
  const size_t n = (size_t)num_tokens * b.num_kv_heads * cpr;
  const int block = 256;
  const dim3 grid((unsigned)((n + block - 1) / block));
  hipLaunchKernelGGL(kv_write_kernel, grid, dim3(block), 0, stream,
                     static_cast<const uint4 *>(k), static_cast<const uint4 *>(v), slots,
                     num_tokens, b.num_kv_heads, cpr, b.num_pages, static_cast<uint4 *>(b.k),
                     static_cast<uint4 *>(b.v));
  return hipGetLastError();
}

}  // namespace pkv
