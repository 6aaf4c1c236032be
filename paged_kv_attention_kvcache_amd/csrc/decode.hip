// Split-K paged decode attention for gfx950 with fixed partitions: partial
// kernel + fixed-order combine kernel.
//
// One query per request sits at position seq_len - 1 and reads the whole
// context through the page table ("Faster fuzzy minds", sections "When
// scheduler does the work" and "So why is this hard for latent / looped
// models?"). The context is cut into partitions of `partition` tokens; one
// workgroup handles one (partition, kv head, request) and all query heads of
// that kv head's GQA group, so every K/V byte is read from HBM once per call.
// Partials (m, l, acc) are fp32 in base-2 units; the combine kernel folds
// them in partition order (deterministic). Rows whose context fits one
// partition are finished directly by the partial kernel, and the combine
// kernel is launched only when some row can span several partitions.
#include <algorithm>
#include <atomic>

#include "folds.hpp"
#include "launch.hpp"

namespace pkv {

// Waves per decode workgroup. A workgroup streams one (request, kv head)
// context and a wave's page loads in flight are bounded by its registers, so
// a context's streaming rate grows with its waves: for GQA groups of 2, 8
// waves let the longest contexts (which set the call's duration) finish
// sooner (measured +6% over 4 on 64 requests of 512-2048 tokens). Such
// workgroups fill a CU one at a time, so small batches run as persistent
// workgroups that each take a balanced list of contexts (decode_whole). A group of 1 has
// half the arithmetic per page and measured faster with 4 (+7% on 16
// requests of 200-2000 tokens, 32 heads); larger groups need more than the
// 256 registers a wave of an 8-wave workgroup may hold, so they use 4 too.
template <class F>
constexpr int decode_waves() {
  return F::kGroup == 2 ? 8 : 4;
}
constexpr int kWholeMaxBatch = 64;  // requests decode_whole ranks (one per lane)

// Combines partitions 0 .. np-1 of row `rowh` (in order) for output dim d.
__device__ __forceinline__ void combine_row(const float *__restrict__ part_m,
                                            const float *__restrict__ part_l,
                                            const float *__restrict__ part_acc, size_t rowh,
                                            int max_parts, int np, int D, int d, float &M,
                                            float &L, float &A) {
  const float *pm = part_m + rowh * max_parts;
  const float *pl = part_l + rowh * max_parts;
  // Unrolled so that several partitions' loads are in flight at once (the
  // fold order, and so the result, is unchanged).
  M = -INFINITY;
#pragma unroll 8
  for (int j = 0; j < np; ++j) M = fmaxf(M, pm[j]);
  const float ms = (M == -INFINITY) ? 0.f : M;
  L = 0.f;
  A = 0.f;
#pragma unroll 8
  for (int j = 0; j < np; ++j) {
    const float f = fast_exp2(pm[j] - ms);
    L = fmaf(pl[j], f, L);
    A = fmaf(part_acc[(rowh * max_parts + j) * D + d], f, A);
  }
}

// One workgroup per (partition j, kv head, request): its W waves take pages
// w, w+W, ... of the partition, their states meet in LDS.
template <typename E, class F, int W>
__global__ __launch_bounds__(64 * W) void decode_block(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const typename E::storage *__restrict__ q, int32_t hq,
    const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t max_seq_len, float qscale, int32_t partition,
    int32_t max_parts, typename E::storage *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_acc,
    const typename E::storage *__restrict__ k_new, const typename E::storage *__restrict__ v_new,
    uint4 *kb_w, uint4 *vb_w, LatestArgs la) {
  constexpr int G = F::kGroup, D = F::kHeadDim;
  constexpr int kThreads = 64 * W;
  __shared__ float2 lds_ml[W * G];
  __shared__ float lds_acc[W * G * D];

  const int j = blockIdx.x, kvh = blockIdx.y, r = blockIdx.z;
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  const int np = min((n + partition - 1) / partition, max_parts);
  const int lo = j * partition;
  if (j > 0 && j >= np) return;  // partition past the context (whole block exits)
  const int hi = min(lo + partition, n);

  F f(q + ((size_t)r * hq + (size_t)kvh * G) * D, qscale);
  if constexpr (F::kLatest) f.la = la;
  typename F::State st;
  f.reset(st);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p_first = lo / kPage;
  const int n_pages = hi > lo ? (hi - 1) / kPage - p_first + 1 : 0;
  const int npw = n_pages > w ? (n_pages - w + W - 1) / W : 0;
  const int32_t *pt_row = page_table + (size_t)r * pt_stride;
  if (k_new && n > 0 && n - 1 >= lo && n - 1 < hi) {
    const int pa = (n - 1) / kPage;  // page of the newest token
    if ((pa - p_first) % W == w)
      f.set_append(k_new + ((size_t)r * hkv + kvh) * D, v_new + ((size_t)r * hkv + kvh) * D,
                   n - 1, kb_w, vb_w, min(max(pt_row[pa], 0), num_pages - 1), hkv, kvh);
  }
  if (npw > 0)
    stream_pages(f, st, kb, vb, pt_row, num_pages, hkv, kvh, p_first + w, npw, W, lo, hi,
                 F::kLatest ? la.depth + (size_t)r * la.stride : nullptr);
  f.finish_wave(st);
  emit_to_lds(f, st, w, lds_ml, lds_acc);
  __syncthreads();

  const size_t row0 = (size_t)r * hq + (size_t)kvh * G;
  if (np <= 1) {  // the whole context in one partition: finish here
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int g = idx / D, d = idx % D;
      float M, L, A;
      combine_waves<G, D, W>(lds_ml, lds_acc, g, d, M, L, A);
      finish<E>(out, lse, row0 + g, D, d, M, L, A);
    }
    return;
  }
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    float M, L, A;
    combine_waves<G, D, W>(lds_ml, lds_acc, g, d, M, L, A);
    const size_t pj = (row0 + g) * max_parts + j;
    part_acc[pj * D + d] = A;
    if (d == 0) {
      part_m[pj] = M;
      part_l[pj] = L;
    }
  }
}

// Whole contexts with persistent workgroups (batch <= 64, one request per
// lane for the ranking). The (request, kv head) units are ranked longest
// context first; workgroup k of M takes ranks k, 2M-1-k, 2M+k, 4M-1-k, ...
// (a "snake" over the ranking), so each workgroup pairs a long context with
// a short one and all carry nearly the same number of pages. A workgroup
// starts its next unit as soon as the current one is written, instead of
// leaving the compute unit to a new workgroup that must first fetch its
// lengths, query and page ids. Each unit is folded exactly as decode_block
// folds a whole context (same page interleave over the waves, same
// wave-order merge), so the results are bitwise identical to it.
template <typename E, class F, int W>
__global__ __launch_bounds__(64 * W) void decode_whole(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const typename E::storage *__restrict__ q, int32_t hq,
    const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t batch, int32_t max_seq_len, float qscale,
    typename E::storage *__restrict__ out, float *__restrict__ lse,
    const typename E::storage *__restrict__ k_new, const typename E::storage *__restrict__ v_new,
    uint4 *kb_w, uint4 *vb_w, LatestArgs la, int32_t pair) {
  constexpr int G = F::kGroup, D = F::kHeadDim;
  constexpr int kThreads = 64 * W;
  __shared__ float2 lds_ml[W * G];
  __shared__ float lds_acc[W * G * D];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Lane i < batch: the clamped length of request i and its rank in
  // longest-first order (ties by index); and whether its first page is also
  // another request's first page (a shared prefix: its pages are then read
  // with cached loads, so that the other requests find them in L2).
  // (The first page id is loaded together with the length: one round trip
  // to memory instead of two before the ranking.)
  const int first0 = lane < batch ? page_table[(size_t)lane * pt_stride] : 0;
  const int mine = lane < batch ? min(max(seq_lens[lane], 0), max_seq_len) : -1;
  const int first = mine > 0 ? first0 : -1 - lane;
  int rank = 0;
  bool shared = false;
  for (int j = 0; j < batch; ++j) {
    const int o = __builtin_amdgcn_readlane(mine, j);
    rank += (o > mine) || (o == mine && j < lane);
    shared |= j != lane && __builtin_amdgcn_readlane(first, j) == first;
  }
  const int units = batch * hkv, M = gridDim.x, k = blockIdx.x;
  for (int it = 0;; ++it) {
    const int base = 2 * M * (it >> 1);
    int u = (it & 1) ? base + 2 * M - 1 - k : base + k;
    // With two workgroups per compute unit (pair: M = 2 x CUs), workgroups
    // k and k + M/2 share one; the second half takes its first units in
    // reverse order (in steps of 8, keeping u % 8 = k % 8, the die of
    // workgroup k), so a long context shares its compute unit with a short
    // one and soon has it alone.
    if (pair && it == 0 && k >= M / 2) {
      const int j = k - M / 2;
      u = M / 2 + (M / 2 - 8 - (j & ~7)) + (j & 7);
    }
    if (u >= units) {
      if (it == 0) continue;  // a permuted first unit may be past the end
      break;  // ranks grow with it
    }
    const int kvh = u % hkv;
    const unsigned long long hit = __ballot(lane < batch && rank == u / hkv);
    const int r = hit ? __ffsll(hit) - 1 : 0;
    const int n = __builtin_amdgcn_readlane(mine, r);

    F f(q + ((size_t)r * hq + (size_t)kvh * G) * D, qscale);
    if constexpr (F::kLatest) f.la = la;
    typename F::State st;
    f.reset(st);
    const int n_pages = (n + kPage - 1) / kPage;
    const int npw = n_pages > w ? (n_pages - w + W - 1) / W : 0;
    const int32_t *pt_row = page_table + (size_t)r * pt_stride;
    if (k_new && n > 0) {
      const int pa = (n - 1) / kPage;  // page of the newest token
      if (pa % W == w)
        f.set_append(k_new + ((size_t)r * hkv + kvh) * D, v_new + ((size_t)r * hkv + kvh) * D,
                     n - 1, kb_w, vb_w, min(max(pt_row[pa], 0), num_pages - 1), hkv, kvh);
    }
    if (npw > 0) {
      const uint8_t *ex_row = F::kLatest ? la.depth + (size_t)r * la.stride : nullptr;
      bool done = false;
      if constexpr (!F::kLatest && F::kGroup == 1) {
        if (__builtin_amdgcn_readlane((int)shared, r)) {
          stream_pages<F, NoStepHook, true>(f, st, kb, vb, pt_row, num_pages, hkv, kvh, w, npw,
                                            W, 0, n, ex_row);
          done = true;
        }
      }
      if (!done)
        stream_pages(f, st, kb, vb, pt_row, num_pages, hkv, kvh, w, npw, W, 0, n, ex_row);
    }
    f.finish_wave(st);
    emit_to_lds(f, st, w, lds_ml, lds_acc);
    __syncthreads();
    const size_t row0 = (size_t)r * hq + (size_t)kvh * G;
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int g = idx / D, d = idx % D;
      float Mx, L, A;
      combine_waves<G, D, W>(lds_ml, lds_acc, g, d, Mx, L, A);
      finish<E>(out, lse, row0 + g, D, d, Mx, L, A);
    }
    __syncthreads();  // the next unit reuses the LDS
  }
}

// Combine partitions 0 .. ceil(n / partition) - 1 of one (request, head)
// row, in order. One thread per output dim.
template <typename E>
__global__ __launch_bounds__(128) void decode_reduce(
    int32_t hq, int32_t D, const int32_t *__restrict__ seq_lens, int32_t max_seq_len,
    int32_t partition, int32_t max_parts, const float *__restrict__ part_m,
    const float *__restrict__ part_l, const float *__restrict__ part_acc,
    typename E::storage *__restrict__ out, float *__restrict__ lse, int skip_single) {
  const int row = blockIdx.x, r = row / hq;
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  const int np = min((n + partition - 1) / partition, max_parts);
  if (skip_single && np <= 1) return;  // finished by the partial kernel
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float M, L, A;
    combine_row(part_m, part_l, part_acc, row, max_parts, np, D, d, M, L, A);
    finish<E>(out, lse, row, D, d, M, L, A);
  }
}

template <typename E, class F>
static hipError_t decode_fold(const DecodeArgs &a, hipStream_t stream) {
  constexpr int D = F::kHeadDim;
  const dim3 grid(a.max_parts, a.bank.num_kv_heads, a.batch);
  constexpr int W = decode_waves<F>();
  if (a.max_parts == 1 && a.batch <= kWholeMaxBatch) {
    // As many persistent workgroups as are resident at once. The occupancy
    // is a property of the kernel binary, which is built for gfx950 alone,
    // so one cached value serves every device; host threads that race to
    // fill it store the same value.
    static std::atomic<int> cached{0};
    int per_cu = cached.load(std::memory_order_relaxed);
    if (per_cu == 0) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_whole<E, F, W>, 64 * W, 0) !=
              hipSuccess ||
          nb < 1)
        nb = 1;
      per_cu = nb;
      cached.store(nb, std::memory_order_relaxed);
    }
    const int units = a.batch * a.bank.num_kv_heads;
    const int blocks = std::min(units, a.num_cus * per_cu);
    const int pair = blocks == 2 * a.num_cus && a.num_cus % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((decode_whole<E, F, W>), dim3(blocks), dim3(64 * W), 0, stream,
                       static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                       a.bank.num_pages, a.bank.num_kv_heads,
                       static_cast<const typename E::storage *>(a.q), a.num_q_heads,
                       a.page_table, a.pt_stride, a.seq_lens, a.batch, a.max_seq_len,
                       a.scale * kLog2e, static_cast<typename E::storage *>(a.out), a.lse,
                       static_cast<const typename E::storage *>(a.k_new),
                       static_cast<const typename E::storage *>(a.v_new),
                       static_cast<uint4 *>(a.bank.k), static_cast<uint4 *>(a.bank.v),
                       a.latest, pair);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_block<E, F, W>), grid, dim3(64 * W), 0, stream,
                     static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                     a.bank.num_pages, a.bank.num_kv_heads,
                     static_cast<const typename E::storage *>(a.q), a.num_q_heads, a.page_table,
                     a.pt_stride, a.seq_lens, a.max_seq_len, a.scale * kLog2e, a.partition,
                     a.max_parts, static_cast<typename E::storage *>(a.out), a.lse, a.part_m,
                     a.part_l, a.part_acc, static_cast<const typename E::storage *>(a.k_new),
                     static_cast<const typename E::storage *>(a.v_new),
                     static_cast<uint4 *>(a.bank.k), static_cast<uint4 *>(a.bank.v), a.latest);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return launch_reduce(a.bank.dtype, a.batch, a.num_q_heads, D, a.seq_lens, a.max_seq_len,
                       a.partition, a.max_parts, a.part_m, a.part_l, a.part_acc, a.out, a.lse,
                       true, stream);
}

template <typename E, int D>
static hipError_t decode_by_group(const DecodeArgs &a, hipStream_t stream) {
  if (a.latest.depth) {  // early exit
    switch (a.num_q_heads / a.bank.num_kv_heads) {
      case 1: return decode_fold<E, typename FoldFor<E, D, 1, true>::type>(a, stream);
      case 2: return decode_fold<E, typename FoldFor<E, D, 2, true>::type>(a, stream);
      case 4: return decode_fold<E, typename FoldFor<E, D, 4, true>::type>(a, stream);
      case 8: return decode_fold<E, typename FoldFor<E, D, 8, true>::type>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (a.num_q_heads / a.bank.num_kv_heads) {
    case 1: return decode_fold<E, typename FoldFor<E, D, 1>::type>(a, stream);
    case 2: return decode_fold<E, typename FoldFor<E, D, 2>::type>(a, stream);
    case 4: return decode_fold<E, typename FoldFor<E, D, 4>::type>(a, stream);
    case 8: return decode_fold<E, typename FoldFor<E, D, 8>::type>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (decode_parts_supported(a)) return launch_decode_parts(a, stream);
  if (a.bank.dtype == 1)
    return a.bank.head_dim == 128 ? decode_by_group<BF16, 128>(a, stream)
                                  : decode_by_group<BF16, 64>(a, stream);
  return a.bank.head_dim == 128 ? decode_by_group<F32, 128>(a, stream)
                                : decode_by_group<F32, 64>(a, stream);
}

hipError_t launch_reduce(int32_t dtype, int32_t batch, int32_t hq, int32_t D,
                         const int32_t *seq_lens, int32_t max_seq_len, int32_t partition,
                         int32_t max_parts, const float *part_m, const float *part_l,
                         const float *part_acc, void *out, float *lse, bool skip_single,
                         hipStream_t stream) {
  const dim3 grid(batch * hq), block(D < 128 ? D : 128);
  if (dtype == 1)
    hipLaunchKernelGGL(decode_reduce<BF16>, grid, block, 0, stream, hq, D, seq_lens,
                       max_seq_len, partition, max_parts, part_m, part_l, part_acc,
                       static_cast<uint16_t *>(out), lse, skip_single ? 1 : 0);
  else
    hipLaunchKernelGGL(decode_reduce<F32>, grid, block, 0, stream, hq, D, seq_lens,
                       max_seq_len, partition, max_parts, part_m, part_l, part_acc,
                       static_cast<float *>(out), lse, skip_single ? 1 : 0);
  return hipGetLastError();
}

}  // namespace pkv
