// Short prefill chunks (bf16, head_dim 128) on the decode matrix-core fold.
//
// A prefix-cache hit prefills only the few suffix tokens after the shared
// prefix ("Faster fuzzy minds", section "When scheduler does the work"), so a
// chunk can hold as few query rows per request as a GQA group holds heads.
// When every request's rows times the group fit 16 columns, the request's
// rows of one kv head are a single 16-column operand of the decode fold: the
// work is one pass over the (request, kv head) context, HBM-bound like a
// decode step, instead of a 32-row query tile per head that is mostly empty.
// Column c is query row c / gh (gh query heads per kv head) of head
// kvh * gh + c % gh; packed row j of a request with q_len rows and seq_len n
// sees keys 0 .. n - q_len + j (the causal rule of the extend-prefill). One
// workgroup per (request, kv head); its waves interleave the pages and merge
// in wave order through LDS, as a whole-context decode workgroup does.
#include <algorithm>

#include "fold_mfma.hpp"
#include "launch.hpp"

namespace pkv {

namespace {

constexpr int kColWaves = 4;  // the fold needs more than an 8-wave workgroup's registers
constexpr int kCols = 16;
using ColFold = MfmaFold<kCols, true>;

}  // namespace

__global__ __launch_bounds__(64 * kColWaves) void prefill_cols(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const uint16_t *__restrict__ q, int32_t hq, const int32_t *__restrict__ cu_q_lens,
    int32_t total_q, int32_t max_rows, const int32_t *__restrict__ page_table,
    int32_t pt_stride, const int32_t *__restrict__ seq_lens, int32_t max_seq_len, float qscale,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  constexpr int W = kColWaves, D = 128;
  __shared__ float2 lds_ml[W * kCols];
  __shared__ float lds_acc[W * kCols * D];

  const int kvh = blockIdx.x % hkv, r = blockIdx.x / hkv;
  const int gh = hq / hkv;
  // Tables are clamped so that every access stays inside the buffers.
  const int q0 = min(max(cu_q_lens[r], 0), total_q);
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  const int q_len = min(min(max(cu_q_lens[r + 1] - q0, 0), n), min(total_q - q0, max_rows));
  if (q_len == 0) return;
  const int cols = q_len * gh;

  ColFold f(q, q0, hq, kvh, gh, cols, n - q_len, qscale);
  ColFold::State st;
  f.reset(st);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_pages = (n + kPage - 1) / kPage;
  const int npw = n_pages > w ? (n_pages - w + W - 1) / W : 0;
  if (npw > 0)
    stream_pages(f, st, kb, vb, page_table + (size_t)r * pt_stride, num_pages, hkv, kvh, w, npw,
                 W, 0, n);
  f.finish_wave(st);
  emit_to_lds(f, st, w, lds_ml, lds_acc);
  __syncthreads();

  for (int idx = threadIdx.x; idx < cols * D; idx += 64 * W) {
    const int c = idx / D, d = idx % D;
    float M, L, A;
    combine_waves<kCols, D, W>(lds_ml, lds_acc, c, d, M, L, A);
    finish<BF16>(out, lse, (size_t)(q0 + c / gh) * hq + (size_t)kvh * gh + c % gh, D, d, M, L,
                 A);
  }
}

bool prefill_cols_supported(const PrefillArgs &a) {
  const int gh = a.num_q_heads / a.bank.num_kv_heads;
  return a.bank.dtype == 1 && a.bank.head_dim == 128 && a.max_q_len >= 1 &&
         (long long)a.max_q_len * gh <= kCols;
}

hipError_t launch_prefill_cols(const PrefillArgs &a, hipStream_t stream) {
  const long long blocks = (long long)a.batch * a.bank.num_kv_heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int max_rows = kCols / (a.num_q_heads / a.bank.num_kv_heads);
  hipLaunchKernelGGL(prefill_cols, dim3((unsigned)blocks), dim3(64 * kColWaves), 0, stream,
                     static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                     a.bank.num_pages, a.bank.num_kv_heads, static_cast<const uint16_t *>(a.q),
                     a.num_q_heads, a.cu_q_lens, a.total_q, std::min(a.max_q_len, max_rows),
                     a.page_table, a.pt_stride, a.seq_lens, a.max_seq_len, a.scale * kLog2e,
                     static_cast<uint16_t *>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace pkv
