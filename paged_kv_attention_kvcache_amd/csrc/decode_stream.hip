// Balanced split-K ("stream-K") paged decode attention for gfx950.
//
// The work of one decode call is the sequence of (request, kv head, page)
// triples in request-major order; unit u = (request r, kv head h) owns
// pages(r) = ceil(seq_len / 16) consecutive entries. Every wave of the grid
// takes one contiguous, equal-sized range of that sequence, so all waves
// stream the same number of pages (+-1) and stay busy until the end, whatever
// the spread of sequence lengths. A wave folds the pages of a unit in order;
// a unit that lies wholly inside one wave's range is finished by that wave,
// otherwise each wave writes its segment as fp32 partials (at most two per
// wave: the unit its range starts in, slot 0, and the unit it ends in, slot
// 1) and the combine kernel folds a unit's segments in wave order, which is
// position order. The split depends only on the sequence lengths and the
// grid size, so results are bitwise repeatable and independent of where the
// pages live.
#include <algorithm>
#include <atomic>

#include "folds.hpp"
#include "launch.hpp"

namespace pkv {

__device__ __forceinline__ int pages_of(const int32_t *seq_lens, int r, int max_seq_len) {
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  return (n + kPage - 1) / kPage;
}

// Partitions of request r (an empty context owns one).
__device__ __forceinline__ int parts_of(const int32_t *seq_lens, int r, int max_seq_len, int pp,
                                        int max_parts) {
  return min(max(1, (pages_of(seq_lens, r, max_seq_len) + pp - 1) / pp), max_parts);
}

// First entry of the range of wave w, for `total` entries over `nw` waves.
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t total, int64_t nw) {
  return w * total / nw;
}

// Block-wide exclusive prefix over rows of hkv * count(r): cum[r] for r <= B
// (cum[B] = total), in LDS. Every thread of the block must call it.
template <class Count>
__device__ void row_prefix_of(Count count, int batch, int hkv, int *cum) {
  __shared__ int wave_tot[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (batch + kBlock - 1) / kBlock;
  const int r0 = tid * per;
  int sum = 0;
  for (int i = 0; i < per; ++i)
    if (r0 + i < batch) sum += hkv * count(r0 + i);
  int x = sum;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[w] = x;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wave_tot[i];
  int run = before + x - sum;  // exclusive prefix of this thread's first row
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < batch) {
      cum[r] = run;
      run += hkv * count(r);
    }
  }
  if (tid == kBlock - 1) cum[batch] = run;
  __syncthreads();
}

// The prefix over rows of hkv * pages(r).
__device__ __forceinline__ void row_prefix(const int32_t *__restrict__ seq_lens, int batch,
                                           int max_seq_len, int hkv, int *cum) {
  row_prefix_of([&](int r) { return pages_of(seq_lens, r, max_seq_len); }, batch, hkv, cum);
}

// Partial slot (wave, slot) of head g: (m, l) and acc[D].
__device__ __forceinline__ size_t part_index(int64_t wave, int slot, int G, int g) {
  return ((size_t)wave * 2 + slot) * G + g;
}

template <typename E, class F>
__global__ __launch_bounds__(kBlock) void decode_stream(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const typename E::storage *__restrict__ q, int32_t hq,
    const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t batch, int32_t max_seq_len, float qscale,
    typename E::storage *__restrict__ out, float *__restrict__ lse,
    float2 *__restrict__ part_ml, float *__restrict__ part_acc,
    const typename E::storage *__restrict__ k_new, const typename E::storage *__restrict__ v_new,
    uint4 *kb_w, uint4 *vb_w, LatestArgs la) {
  constexpr int G = F::kGroup, D = F::kHeadDim;
  extern __shared__ int cum[];  // [batch + 1]
  row_prefix(seq_lens, batch, max_seq_len, hkv, cum);

  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t total = cum[batch];
  int64_t s = range_start(gw, total, nw);
  const int64_t e = range_start(gw + 1, total, nw);
  if (s >= e) return;

  // Unit holding entry s: the first r with cum[r + 1] > s.
  int lo_r = 0, hi_r = batch - 1;
  while (lo_r < hi_r) {
    const int mid = (lo_r + hi_r) >> 1;
    if (cum[mid + 1] > s) hi_r = mid; else lo_r = mid + 1;
  }
  int r = lo_r;
  int pr = (cum[r + 1] - cum[r]) / hkv;
  int kvh = (int)((s - cum[r]) / pr);
  int p = (int)((s - cum[r]) % pr);
  int slot = 0;
  while (s < e) {
    const int len = (int)min((int64_t)(pr - p), e - s);
    const int n = min(max(seq_lens[r], 0), max_seq_len);
    const size_t row0 = (size_t)r * hq + (size_t)kvh * G;
    F f(q + row0 * D, qscale);
    if constexpr (F::kLatest) f.la = la;
    typename F::State st;
    f.reset(st);
    const int32_t *pt_row = page_table + (size_t)r * pt_stride;
    if (k_new && n > 0) {
      const int pa = (n - 1) / kPage;  // page of the newest token
      if (pa >= p && pa < p + len)
        f.set_append(k_new + ((size_t)r * hkv + kvh) * D, v_new + ((size_t)r * hkv + kvh) * D,
                     n - 1, kb_w, vb_w, min(max(pt_row[pa], 0), num_pages - 1), hkv, kvh);
    }
    stream_pages(f, st, kb, vb, pt_row, num_pages, hkv, kvh, p, len, 1, 0, n,
                 F::kLatest ? la.depth + (size_t)r * la.stride : nullptr);
    f.finish_wave(st);
    if (p == 0 && len == pr) {  // the whole unit: finish here
      emit_final<F, E>(f, st, out, lse, row0);
    } else {
      f.emit(st, [&](int g, int d0, int cnt, float m, float l, const float *acc) {
        const size_t pi = part_index(gw, slot, G, g);
        for (int e2 = 0; e2 < cnt; e2 += 4)
          *reinterpret_cast<float4 *>(part_acc + pi * D + d0 + e2) =
              make_float4(acc[e2], acc[e2 + 1], acc[e2 + 2], acc[e2 + 3]);
        if (d0 == 0) part_ml[pi] = make_float2(m, l);
      });
    }
    s += len;
    slot = 1;
    p += len;
    if (p == pr) {
      p = 0;
      if (++kvh == hkv) {
        kvh = 0;
        do { ++r; } while (r < batch && cum[r + 1] == cum[r]);
        if (r < batch) pr = (cum[r + 1] - cum[r]) / hkv;
      }
    }
  }
}

// Finishes the units the stream kernel split across waves, and the units of
// empty requests (out 0, lse -inf). One block per unit; segments are folded
// in wave order. The (m, l) of up to kSegChunk segments at a time are staged
// in LDS, so each thread's acc loads are independent of one another.
constexpr int kSegChunk = 64;

// The units of row r are count(r) entries per kv head (pages for the
// balanced split, partitions for decode_parts).
template <typename E, int G, class Count>
__device__ __forceinline__ void combine_units(Count count, int32_t hkv, int32_t D, int32_t batch,
                                              int64_t nw, const float2 *__restrict__ part_ml,
                                              const float *__restrict__ part_acc,
                                              typename E::storage *__restrict__ out,
                                              float *__restrict__ lse) {
  __shared__ int sums[2][kBlock];
  __shared__ int seg_part[kSegChunk];  // part_index(wave, slot, G, 0) / G
  __shared__ float2 seg_ml[kSegChunk][G];
  const int u = blockIdx.x, r = u / hkv, kvh = u % hkv, tid = threadIdx.x;
  int before = 0, all = 0;
  for (int i = tid; i < batch; i += kBlock) {
    const int v = hkv * count(i);
    all += v;
    if (i < r) before += v;
  }
  sums[0][tid] = before;
  sums[1][tid] = all;
  __syncthreads();
  for (int off = kBlock / 2; off > 0; off >>= 1) {
    if (tid < off) {
      sums[0][tid] += sums[0][tid + off];
      sums[1][tid] += sums[1][tid + off];
    }
    __syncthreads();
  }
  const int64_t total = sums[1][0];
  const int pr = count(r);
  const int64_t a = (int64_t)sums[0][0] + (int64_t)kvh * pr, b = a + pr;
  const size_t row0 = (size_t)r * hkv * G + (size_t)kvh * G;
  if (pr == 0) {
    for (int idx = tid; idx < G * D; idx += kBlock) {
      const float z = 0.f;
      store_row<E>(out + (row0 + idx / D) * D + idx % D, &z, 1);
      if (lse && idx % D == 0) lse[row0 + idx / D] = -INFINITY;
    }
    return;
  }
  // Wave holding entry t: the last w with range_start(w) <= t.
  const int64_t w0 = ((a + 1) * nw - 1) / total, w1 = (b * nw - 1) / total;
  if (w0 == w1) return;  // finished by the stream kernel

  // Per-(g, d) running fold; chunks of segments are staged in LDS.
  const int per_thread = (G * D + kBlock - 1) / kBlock;  // <= 4 (G * D <= 1024)
  float M[4], L[4], A[4];
  for (int i = 0; i < 4; ++i) { M[i] = -INFINITY; L[i] = 0.f; A[i] = 0.f; }
  // range_start(w) = w*q + floor(w*rm / nw), stepped without divisions.
  const int64_t qt = total / nw, rm = total % nw;
  int64_t w = w0, start = range_start(w0, total, nw), frac = (w0 * rm) % nw;
  while (w <= w1) {
    // Collect up to kSegChunk non-empty waves (thread 0), in order.
    __shared__ int nseg;
    __shared__ int64_t next_w, next_start, next_frac;
    if (tid == 0) {
      int k = 0;
      while (w <= w1 && k < kSegChunk) {
        int64_t f2 = frac + rm, st2 = start + qt;
        if (f2 >= nw) { f2 -= nw; st2 += 1; }
        if (st2 > start) {  // non-empty range
          const int slot = start >= a ? 0 : 1;
          seg_part[k++] = (int)(w * 2 + slot);
        }
        ++w; start = st2; frac = f2;
      }
      nseg = k; next_w = w; next_start = start; next_frac = frac;
    }
    __syncthreads();
    for (int i = tid; i < nseg * G; i += kBlock)
      seg_ml[i / G][i % G] = part_ml[(size_t)seg_part[i / G] * G + i % G];
    __syncthreads();
    for (int i = 0; i < per_thread; ++i) {
      const int idx = tid + i * kBlock;
      if (idx >= G * D) break;
      const int g = idx / D, d = idx % D;
      float m = M[i];
      for (int k = 0; k < nseg; ++k) m = fmaxf(m, seg_ml[k][g].x);
      const float ms = (m == -INFINITY) ? 0.f : m;
      const float old = fast_exp2(M[i] - ms);  // rescale what was folded so far
      float l = L[i] * old, acc = A[i] * old;
      for (int k = 0; k < nseg; ++k) {
        const float f = fast_exp2(seg_ml[k][g].x - ms);
        l = fmaf(seg_ml[k][g].y, f, l);
        acc = fmaf(part_acc[((size_t)seg_part[k] * G + g) * D + d], f, acc);
      }
      M[i] = m; L[i] = l; A[i] = acc;
    }
    w = next_w; start = next_start; frac = next_frac;
    __syncthreads();
  }
  for (int i = 0; i < per_thread; ++i) {
    const int idx = tid + i * kBlock;
    if (idx >= G * D) break;
    const int g = idx / D, d = idx % D;
    const float o = (L[i] > 0.f) ? A[i] / L[i] : 0.f;
    store_row<E>(out + (row0 + g) * D + d, &o, 1);
    if (lse && d == 0) lse[row0 + g] = (L[i] > 0.f) ? (M[i] + log2f(L[i])) * kLn2 : -INFINITY;
  }
}

template <typename E, int G>
__global__ __launch_bounds__(kBlock) void decode_stream_combine(
    int32_t hkv, int32_t D, const int32_t *__restrict__ seq_lens, int32_t batch,
    int32_t max_seq_len, int64_t nw, const float2 *__restrict__ part_ml,
    const float *__restrict__ part_acc, typename E::storage *__restrict__ out,
    float *__restrict__ lse) {
  combine_units<E, G>([&](int r) { return pages_of(seq_lens, r, max_seq_len); }, hkv, D, batch,
                      nw, part_ml, part_acc, out, lse);
}

// The combine of decode_parts: a (request, kv head)'s segments in wave order.
template <typename E, int G>
__global__ __launch_bounds__(kBlock) void decode_parts_combine(
    int32_t hkv, int32_t D, const int32_t *__restrict__ seq_lens, int32_t batch,
    int32_t max_seq_len, int32_t partition, int32_t max_parts, int64_t nw,
    const float2 *__restrict__ part_ml, const float *__restrict__ part_acc,
    typename E::storage *__restrict__ out, float *__restrict__ lse) {
  const int pp = partition / kPage;
  combine_units<E, G>([&](int r) { return parts_of(seq_lens, r, max_seq_len, pp, max_parts); },
                      hkv, D, batch, nw, part_ml, part_acc, out, lse);
}

// Fixed partitions, streamed. The work of a call is the sequence of
// (request, kv head, partition) triples in request-major order; request r
// owns hkv * max(1, ceil(n_r / partition)) of them (an empty context still
// owns one, whose output is 0 and lse -inf). Every wave of a fully occupied
// grid takes one contiguous, equal-sized range of partitions and folds their
// pages as one pipelined stream per (request, kv head). Each partition is
// folded from a fresh state by one wave, in page order; at its end the wave
// combines it into the (request, kv head)'s running result in partition
// order (the fp32 split-K reduction), so no partition's partial leaves the
// registers. A (request, kv head) inside one wave's range is finished by that
// wave; one split between waves leaves a partial per wave (at most two per
// wave, slots 0 and 1, as in the balanced split) for decode_parts_combine.
// Steps must not straddle partitions: a partition's pages are a multiple of
// the fold's pages per step.
template <typename E, class F>
__global__ __launch_bounds__(kBlock) void decode_parts(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const typename E::storage *__restrict__ q, int32_t hq,
    const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t batch, int32_t max_seq_len, float qscale,
    int32_t partition, int32_t max_parts, typename E::storage *__restrict__ out,
    float *__restrict__ lse, float2 *__restrict__ part_ml, float *__restrict__ part_acc,
    const typename E::storage *__restrict__ k_new, const typename E::storage *__restrict__ v_new,
    uint4 *kb_w, uint4 *vb_w, LatestArgs la) {
  constexpr int G = F::kGroup, D = F::kHeadDim;
  extern __shared__ int cum[];  // [batch + 1]
  const int pp = partition / kPage;  // pages per partition
  row_prefix_of([&](int r) { return parts_of(seq_lens, r, max_seq_len, pp, max_parts); }, batch,
                hkv, cum);

  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t total = cum[batch];
  int64_t s = range_start(gw, total, nw);
  const int64_t e = range_start(gw + 1, total, nw);
  if (s >= e) return;

  // Row holding entry s: the first r with cum[r + 1] > s.
  int lo_r = 0, hi_r = batch - 1;
  while (lo_r < hi_r) {
    const int mid = (lo_r + hi_r) >> 1;
    if (cum[mid + 1] > s) hi_r = mid; else lo_r = mid + 1;
  }
  int r = lo_r;
  int np = (cum[r + 1] - cum[r]) / hkv;
  int kvh = (int)((s - cum[r]) / np);
  int j = (int)((s - cum[r]) % np);
  int slot = 0;
  while (s < e) {
    const int len = (int)min((int64_t)(np - j), e - s);  // partitions of this (r, kvh)
    const int n = min(max(seq_lens[r], 0), max_seq_len);
    const int p0 = j * pp, p1 = min((j + len) * pp, (n + kPage - 1) / kPage);
    const size_t row0 = (size_t)r * hq + (size_t)kvh * G;
    F f(q + row0 * D, qscale);
    if constexpr (F::kLatest) f.la = la;
    typename F::State st, run;
    f.reset(st);
    f.reset(run);  // the combine of no partition: m = -inf, l = 0, acc = 0
    const int32_t *pt_row = page_table + (size_t)r * pt_stride;
    if (k_new && n > 0) {
      const int pa = (n - 1) / kPage;  // page of the newest token
      if (pa >= p0 && pa < p1)
        f.set_append(k_new + ((size_t)r * hkv + kvh) * D, v_new + ((size_t)r * hkv + kvh) * D,
                     n - 1, kb_w, vb_w, min(max(pt_row[pa], 0), num_pages - 1), hkv, kvh);
    }
    if (p1 > p0) {
      const int cnt = p1 - p0;
      stream_pages(f, st, kb, vb, pt_row, num_pages, hkv, kvh, p0, cnt, 1, 0, n,
                   F::kLatest ? la.depth + (size_t)r * la.stride : nullptr, [&](int k) {
                     if (k % pp == 0 || k == cnt) {  // a partition ends
                       f.finish_wave(st);
                       F::merge(run, st);
                       f.reset(st);
                     }
                   });
    }
    if (j == 0 && len == np) {  // the whole (request, kv head): finish here
      emit_final<F, E>(f, run, out, lse, row0);
    } else {
      f.emit(run, [&](int g, int d0, int c, float m, float l, const float *acc) {
        const size_t pi = part_index(gw, slot, G, g);
        for (int e2 = 0; e2 < c; e2 += 4)
          *reinterpret_cast<float4 *>(part_acc + pi * D + d0 + e2) =
              make_float4(acc[e2], acc[e2 + 1], acc[e2 + 2], acc[e2 + 3]);
        if (d0 == 0) part_ml[pi] = make_float2(m, l);
      });
    }
    s += len;
    slot = 1;
    j += len;
    if (j == np) {
      j = 0;
      if (++kvh == hkv) {
        kvh = 0;
        if (++r < batch) np = (cum[r + 1] - cum[r]) / hkv;
      }
    }
  }
}

// Workgroups per compute unit of the balanced split: as many as fit, or a
// fixed count when built with -DPKV_STREAM_BLOCKS_PER_CU=n (tuning).
template <typename E, int D, int G>
static int stream_blocks_per_cu() {
#ifdef PKV_STREAM_BLOCKS_PER_CU
  return PKV_STREAM_BLOCKS_PER_CU;
#endif
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_stream<E, typename FoldFor<E, D, G>::type>, kBlock,
                                                   0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

template <typename E, int D>
static int blocks_by_group(int g) {
  switch (g) {
    case 1: return stream_blocks_per_cu<E, D, 1>();
    case 2: return stream_blocks_per_cu<E, D, 2>();
    case 4: return stream_blocks_per_cu<E, D, 4>();
    case 8: return stream_blocks_per_cu<E, D, 8>();
  }
  return 1;
}

int stream_waves(int dtype, int head_dim, int group, int num_cus) {
  // [dtype][head_dim 64/128][group]: blocks per CU. Occupancy is a property
  // of the kernel binary (gfx950 only), the same on every device; host
  // threads that race to fill an entry store the same value.
  static std::atomic<int> cache[2][2][9];
  std::atomic<int> &slot = cache[dtype == 1][head_dim == 128][group & 7 ? group : 8];
  int bpc = slot.load(std::memory_order_relaxed);
  if (bpc == 0) {
    bpc = dtype == 1 ? (head_dim == 128 ? blocks_by_group<BF16, 128>(group)
                                        : blocks_by_group<BF16, 64>(group))
                     : (head_dim == 128 ? blocks_by_group<F32, 128>(group)
                                        : blocks_by_group<F32, 64>(group));
    slot.store(bpc, std::memory_order_relaxed);
  }
  return num_cus * bpc * kWaves;
}

template <typename E, int D, int G, class F = typename FoldFor<E, D, G>::type>
static hipError_t stream_launch(const DecodeArgs &a, int64_t nw, hipStream_t stream) {
  const unsigned blocks = (unsigned)(nw / kWaves);
  const size_t lds = sizeof(int) * ((size_t)a.batch + 1);
  hipLaunchKernelGGL((decode_stream<E, F>), dim3(blocks), dim3(kBlock), lds, stream,
                     static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                     a.bank.num_pages, a.bank.num_kv_heads,
                     static_cast<const typename E::storage *>(a.q), a.num_q_heads, a.page_table,
                     a.pt_stride, a.seq_lens, a.batch, a.max_seq_len, a.scale * kLog2e,
                     static_cast<typename E::storage *>(a.out), a.lse,
                     reinterpret_cast<float2 *>(a.part_m), a.part_acc,
                     static_cast<const typename E::storage *>(a.k_new),
                     static_cast<const typename E::storage *>(a.v_new),
                     static_cast<uint4 *>(a.bank.k), static_cast<uint4 *>(a.bank.v), a.latest);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_stream_combine<E, G>), dim3(a.batch * a.bank.num_kv_heads),
                     dim3(kBlock), 0, stream, a.bank.num_kv_heads, D, a.seq_lens, a.batch,
                     a.max_seq_len, nw, reinterpret_cast<const float2 *>(a.part_m), a.part_acc,
                     static_cast<typename E::storage *>(a.out), a.lse);
  return hipGetLastError();
}

template <typename E, class F>
static hipError_t parts_launch(const DecodeArgs &a, hipStream_t stream) {
  constexpr int G = F::kGroup;
  const int64_t nw = a.nw;
  const unsigned blocks = (unsigned)(nw / kWaves);
  // The segment partials sit where the balanced split keeps its own.
  const size_t slots = (size_t)nw * 2 * G;
  float2 *part_ml = reinterpret_cast<float2 *>(a.part_m);
  float *part_acc = reinterpret_cast<float *>(reinterpret_cast<char *>(a.part_m) +
                                              (slots * 2 * sizeof(float) + 255) / 256 * 256);
  const size_t lds = sizeof(int) * ((size_t)a.batch + 1);
  hipLaunchKernelGGL((decode_parts<E, F>), dim3(blocks), dim3(kBlock), lds, stream,
                     static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                     a.bank.num_pages, a.bank.num_kv_heads,
                     static_cast<const typename E::storage *>(a.q), a.num_q_heads, a.page_table,
                     a.pt_stride, a.seq_lens, a.batch, a.max_seq_len, a.scale * kLog2e,
                     a.partition, a.max_parts, static_cast<typename E::storage *>(a.out), a.lse,
                     part_ml, part_acc, static_cast<const typename E::storage *>(a.k_new),
                     static_cast<const typename E::storage *>(a.v_new),
                     static_cast<uint4 *>(a.bank.k), static_cast<uint4 *>(a.bank.v), a.latest);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_parts_combine<E, G>), dim3(a.batch * a.bank.num_kv_heads),
                     dim3(kBlock), 0, stream, a.bank.num_kv_heads, F::kHeadDim, a.seq_lens,
                     a.batch, a.max_seq_len, a.partition, a.max_parts, nw, part_ml, part_acc,
                     static_cast<typename E::storage *>(a.out), a.lse);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t parts_by_group(const DecodeArgs &a, hipStream_t stream) {
  if (a.latest.depth) {
    switch (a.num_q_heads / a.bank.num_kv_heads) {
      case 1: return parts_launch<E, typename FoldFor<E, D, 1, true>::type>(a, stream);
      case 2: return parts_launch<E, typename FoldFor<E, D, 2, true>::type>(a, stream);
      case 4: return parts_launch<E, typename FoldFor<E, D, 4, true>::type>(a, stream);
      case 8: return parts_launch<E, typename FoldFor<E, D, 8, true>::type>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (a.num_q_heads / a.bank.num_kv_heads) {
    case 1: return parts_launch<E, typename FoldFor<E, D, 1>::type>(a, stream);
    case 2: return parts_launch<E, typename FoldFor<E, D, 2>::type>(a, stream);
    case 4: return parts_launch<E, typename FoldFor<E, D, 4>::type>(a, stream);
    case 8: return parts_launch<E, typename FoldFor<E, D, 8>::type>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename E, int D, bool L>
static int pages_per_step(int group) {
  switch (group) {
    case 1: return FoldFor<E, D, 1, L>::type::kPagesPerStep;
    case 2: return FoldFor<E, D, 2, L>::type::kPagesPerStep;
    case 4: return FoldFor<E, D, 4, L>::type::kPagesPerStep;
    case 8: return FoldFor<E, D, 8, L>::type::kPagesPerStep;
  }
  return 0;
}
template <typename E, int D>
static int pages_per_step(int group, bool latest) {
  return latest ? pages_per_step<E, D, true>(group) : pages_per_step<E, D, false>(group);
}

bool decode_parts_supported(const DecodeArgs &a) {
  const int g = a.num_q_heads / a.bank.num_kv_heads;
  const bool latest = a.latest.depth != nullptr;
  const int s = a.bank.dtype == 1
                    ? (a.bank.head_dim == 128 ? pages_per_step<BF16, 128>(g, latest)
                                              : pages_per_step<BF16, 64>(g, latest))
                    : (a.bank.head_dim == 128 ? pages_per_step<F32, 128>(g, latest)
                                              : pages_per_step<F32, 64>(g, latest));
  return a.max_parts > 1 && a.nw >= kWaves && a.nw % kWaves == 0 && a.batch <= kPartsMaxBatch &&
         s > 0 && a.partition % kPage == 0 && (a.partition / kPage) % s == 0;
}

hipError_t launch_decode_parts(const DecodeArgs &a, hipStream_t stream) {
  if (a.bank.dtype == 1)
    return a.bank.head_dim == 128 ? parts_by_group<BF16, 128>(a, stream)
                                  : parts_by_group<BF16, 64>(a, stream);
  return a.bank.head_dim == 128 ? parts_by_group<F32, 128>(a, stream)
                                : parts_by_group<F32, 64>(a, stream);
}

template <typename E, int D>
static hipError_t stream_by_group(const DecodeArgs &a, int64_t nw, hipStream_t stream) {
  if (a.latest.depth) {  // early exit
    switch (a.num_q_heads / a.bank.num_kv_heads) {
      case 1: return stream_launch<E, D, 1, typename FoldFor<E, D, 1, true>::type>(a, nw, stream);
      case 2: return stream_launch<E, D, 2, typename FoldFor<E, D, 2, true>::type>(a, nw, stream);
      case 4: return stream_launch<E, D, 4, typename FoldFor<E, D, 4, true>::type>(a, nw, stream);
      case 8: return stream_launch<E, D, 8, typename FoldFor<E, D, 8, true>::type>(a, nw, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (a.num_q_heads / a.bank.num_kv_heads) {
    case 1: return stream_launch<E, D, 1>(a, nw, stream);
    case 2: return stream_launch<E, D, 2>(a, nw, stream);
    case 4: return stream_launch<E, D, 4>(a, nw, stream);
    case 8: return stream_launch<E, D, 8>(a, nw, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_stream(const DecodeArgs &a, int64_t nw, hipStream_t stream) {
  if (a.bank.dtype == 1)
    return a.bank.head_dim == 128 ? stream_by_group<BF16, 128>(a, nw, stream)
                                  : stream_by_group<BF16, 64>(a, nw, stream);
  return a.bank.head_dim == 128 ? stream_by_group<F32, 128>(a, nw, stream)
                                : stream_by_group<F32, 64>(a, nw, stream);
}

}  // namespace pkv
