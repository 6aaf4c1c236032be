// Chunked causal prefill over paged context for gfx950, vector-ALU path
// (fp32 data and head_dim 64; bf16 at head_dim 128 runs on matrix cores).
//
// An extend-prefill of a span ("Faster fuzzy minds", section "LOTUS"; a
// prefix-cache hit prefills only the suffix, section "When scheduler does
// the work"): the chunk's K/V are already in the pool, and packed query row j
// of request r sits at position seq_len - q_len + j and sees keys 0..that
// position. One workgroup takes one (query row, kv head) and the whole GQA
// group of query heads, streaming its visible pages with the same span code
// as decode.
#include "fold_valu.hpp"
#include "launch.hpp"

namespace pkv {

template <typename E, int D, int G>
__global__ __launch_bounds__(kBlock) void prefill_valu(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const typename E::storage *__restrict__ q, int32_t hq, const int32_t *__restrict__ cu_q_lens,
    int32_t batch, const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t max_seq_len, float qscale,
    typename E::storage *__restrict__ out, float *__restrict__ lse) {
  __shared__ float2 lds_ml[kWaves * G];
  __shared__ float lds_acc[kWaves * G * D];

  const int row = blockIdx.x, kvh = blockIdx.y;
  // Request owning this packed row: the last r with cu_q_lens[r] <= row.
  int a = 0, b = batch;  // invariant: cu[a] <= row < cu[b]
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (cu_q_lens[mid] <= row) a = mid; else b = mid;
  }
  const int r = a;
  const int qlen = cu_q_lens[r + 1] - cu_q_lens[r];
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  const int pos = min(n - qlen + (row - cu_q_lens[r]), n - 1);
  const int hi = max(pos + 1, 0);

  ValuFold<E, D, G> f(q + ((size_t)row * hq + (size_t)kvh * G) * D, qscale);
  typename ValuFold<E, D, G>::State st;
  f.reset(st);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_pages = hi > 0 ? (hi - 1) / kPage + 1 : 0;
  const int npw = n_pages > w ? (n_pages - w + kWaves - 1) / kWaves : 0;
  if (npw > 0)
    stream_pages(f, st, kb, vb, page_table + (size_t)r * pt_stride, num_pages, hkv, kvh, w, npw,
                 kWaves, 0, hi);
  f.finish_wave(st);
  emit_to_lds(f, st, w, lds_ml, lds_acc);
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
    const int g = idx / D, d = idx % D;
    float M, L, A;
    combine_waves<G, D>(lds_ml, lds_acc, g, d, M, L, A);
    finish<E>(out, lse, (size_t)row * hq + (size_t)kvh * G + g, D, d, M, L, A);
  }
}

template <typename E, int D, int G>
static hipError_t prefill_valu_launch(const PrefillArgs &a, hipStream_t stream) {
  const dim3 grid(a.total_q, a.bank.num_kv_heads);
  hipLaunchKernelGGL((prefill_valu<E, D, G>), grid, dim3(kBlock), 0, stream,
                     static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                     a.bank.num_pages, a.bank.num_kv_heads,
                     static_cast<const typename E::storage *>(a.q), a.num_q_heads, a.cu_q_lens,
                     a.batch, a.page_table, a.pt_stride, a.seq_lens, a.max_seq_len,
                     a.scale * kLog2e, static_cast<typename E::storage *>(a.out), a.lse);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t prefill_by_group(const PrefillArgs &a, hipStream_t stream) {
  switch (a.num_q_heads / a.bank.num_kv_heads) {
    case 1: return prefill_valu_launch<E, D, 1>(a, stream);
    case 2: return prefill_valu_launch<E, D, 2>(a, stream);
    case 4: return prefill_valu_launch<E, D, 4>(a, stream);
    case 8: return prefill_valu_launch<E, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  if (a.total_q == 0) return hipSuccess;
  if (prefill_cols_supported(a)) return launch_prefill_cols(a, stream);
  if (prefill_mfma_supported(a)) return launch_prefill_mfma(a, stream);
  if (a.bank.dtype == 1)
    return a.bank.head_dim == 128 ? prefill_by_group<BF16, 128>(a, stream)
                                  : prefill_by_group<BF16, 64>(a, stream);
  return a.bank.head_dim == 128 ? prefill_by_group<F32, 128>(a, stream)
                                : prefill_by_group<F32, 64>(a, stream);
}

}  // namespace pkv
