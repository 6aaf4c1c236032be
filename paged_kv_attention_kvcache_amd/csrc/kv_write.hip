// store_kv for gfx950: scatter each token's K/V rows to the slots the
// scheduler hands out ("Faster fuzzy minds", section "LOTUS": handing the
// same slots again overwrites in place).
//
// Consecutive threads cover consecutive 16-byte chunks of a (token, kv head)
// row of K (and the same chunks of V), so both the reads of the dense
// [T][Hkv][D] input and the writes into the (page, kv head) tile row are
// 16-byte vectors, coalesced per row.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

constexpr int kWriteUnroll = 4;  // chunks per thread, all loaded before any store

// Chunk i of the dense input is chunk c of kv head h of token t, with
// i = (t * hkv + h) * cpr + c. A workgroup moves kWriteUnroll * 256
// consecutive chunks; each thread issues its kWriteUnroll K and V loads
// (16 bytes each, streamed: the input is read once) before its stores, so a
// thread keeps eight loads in flight. 32-bit index arithmetic: the host
// splits a write into launches of fewer than 2^31 chunks.
__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, const int32_t *__restrict__ slots,
    uint32_t n, uint32_t per_token, uint32_t cpr, int32_t hkv, int32_t num_pages,
    uint4 *__restrict__ kb, uint4 *__restrict__ vb) {
  const uint32_t base = blockIdx.x * (256u * kWriteUnroll) + threadIdx.x;
  uint4 kr[kWriteUnroll], vr[kWriteUnroll];
  size_t dst[kWriteUnroll];
  bool ok[kWriteUnroll];
#pragma unroll
  for (int j = 0; j < kWriteUnroll; ++j) {
    const uint32_t i = base + (uint32_t)j * 256u;
    const uint32_t ii = i < n ? i : 0u;
    const uint32_t t = ii / per_token, rem = ii - t * per_token;
    const uint32_t h = rem / cpr, c = rem - h * cpr;
    const int s = slots[t];
    ok[j] = i < n && s >= 0 && s / kPage < num_pages;
    const int sc = ok[j] ? s : 0;
    dst[j] = (((size_t)(sc / kPage) * hkv + h) * kPage + sc % kPage) * cpr + c;
    kr[j] = load_stream(k + ii);
    vr[j] = load_stream(v + ii);
  }
#pragma unroll
  for (int j = 0; j < kWriteUnroll; ++j)
    if (ok[j]) {
      kb[dst[j]] = kr[j];
      vb[dst[j]] = vr[j];
    }
}

hipError_t launch_kv_write(const Bank &b, const void *k, const void *v, const int32_t *slots,
                           int32_t num_tokens, hipStream_t stream) {
  const int bytes = b.dtype == 1 ? 2 : 4;
  const uint32_t cpr = (uint32_t)(b.head_dim * bytes / 16);
  const uint32_t per_token = (uint32_t)b.num_kv_heads * cpr;
  // tokens per launch: fewer than 2^31 chunks
  const int32_t max_tokens = (int32_t)(0x7fffffffu / per_token);
  for (int32_t t0 = 0; t0 < num_tokens; t0 += max_tokens) {
    const int32_t nt = num_tokens - t0 < max_tokens ? num_tokens - t0 : max_tokens;
    const uint32_t n = (uint32_t)nt * per_token;
    const uint32_t per_block = 256u * kWriteUnroll;
    const dim3 grid((n + per_block - 1) / per_block);
    const size_t in0 = (size_t)t0 * per_token;
    hipLaunchKernelGGL(kv_write_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint4 *>(k) + in0, static_cast<const uint4 *>(v) + in0,
                       slots + t0, n, per_token, cpr, b.num_kv_heads, b.num_pages,
                       static_cast<uint4 *>(b.k), static_cast<uint4 *>(b.v));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
