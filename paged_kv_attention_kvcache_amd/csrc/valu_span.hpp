// Vector-ALU attention of a group of query heads over a span of paged keys.
//
// Used where the contraction is too skinny for matrix cores (a GQA group of
// 1 or 2 query heads, or fp32 data). A workgroup of 4 wavefronts takes one
// (request, kv head, key span); wave w streams pages w, w+4, ... of the span.
// Within a wave, LPT = head_dim*bytes/16 consecutive lanes hold one token row
// of a (page, kv head) tile, 16 bytes each, so every load instruction of a
// wave reads 1 KiB of the 4 KiB tile contiguously. A q.k dot product is an
// in-lane FMA chain plus a DPP butterfly over the LPT lanes of the row; each
// row then keeps its own online-softmax state (m, l, acc) over the tokens it
// sees, so no cross-row traffic happens inside the page loop. At the end the
// rows are merged with lane shuffles and the four waves through LDS, in a
// fixed order (bitwise repeatable, independent of physical page ids).
//
// Scores are kept in base-2 units: each reduced q.k is multiplied by
// scale*log2(e) so the softmax uses exp2. For bf16, q.k runs on packed pairs
// with v_dot2_f32_bf16 (fp32 accumulation); fp32 data uses FMAs.
#pragma once
#include "common.hpp"

namespace pkv {

template <typename E, int D> struct Tile {
  static constexpr int kVecN = Vec<E>::kN;     // elements per 16-byte chunk
  static constexpr int kLPT = D / kVecN;       // lanes per token row
  static constexpr int kRPW = 64 / kLPT;       // token rows per wave load
  static constexpr int kNI = kPage / kRPW;     // wave loads per tile
  static constexpr int kTileVec = kPage * kLPT;  // 16-byte chunks per tile
  static_assert(kLPT == 8 || kLPT == 16 || kLPT == 32, "unsupported head_dim");
};

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;

template <typename E, int D, int G> struct SpanState {
  static constexpr int N = Tile<E, D>::kVecN;
  float m[G], l[G], acc[G][N];
};

// Loads the (page, kv head) K and V tile rows this lane owns.
template <typename E, int D>
__device__ __forceinline__ void load_tile(const uint4 *__restrict__ kb,
                                          const uint4 *__restrict__ vb, int page,
                                          int hkv, int kvh, int lane_off,
                                          uint4 (&kr)[Tile<E, D>::kNI],
                                          uint4 (&vr)[Tile<E, D>::kNI]) {
  using TL = Tile<E, D>;
  // page and kvh are wave-uniform: the tile base is a scalar address and each
  // lane adds a 32-bit offset.
  const size_t tile = ((size_t)page * hkv + kvh) * TL::kTileVec;
  const char *kt = reinterpret_cast<const char *>(kb + tile);
  const char *vt = reinterpret_cast<const char *>(vb + tile);
  const uint32_t off = (uint32_t)lane_off * 16u;
#pragma unroll
  for (int i = 0; i < TL::kNI; ++i) kr[i] = load_stream(kt + off + i * TL::kRPW * TL::kLPT * 16u);
#pragma unroll
  for (int i = 0; i < TL::kNI; ++i) vr[i] = load_stream(vt + off + i * TL::kRPW * TL::kLPT * 16u);
}

// Folds one loaded page (page index pi of the request) into the row state.
template <typename E, int D, int G>
__device__ __forceinline__ void fold_page(SpanState<E, D, G> &st, const QChunk<E> (&q)[G],
                                          float qscale, const uint4 (&kr)[Tile<E, D>::kNI],
                                          const uint4 (&vr)[Tile<E, D>::kNI], int pi,
                                          int row, int lo, int hi) {
  using TL = Tile<E, D>;
  constexpr int N = TL::kVecN, LPT = TL::kLPT, RPW = TL::kRPW, NI = TL::kNI;
  const int pos0 = pi * kPage + row;  // token of load i: pos0 + i * RPW
  const bool full = (pi * kPage >= lo) && (pi * kPage + kPage <= hi);

  float s[G][NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int g = 0; g < G; ++g) s[g][i] = q[g].dot(kr[i]);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NI; ++i) s[g][i] = group_sum<LPT>(s[g][i]) * qscale;

  bool valid[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int pos = pos0 + i * RPW;
    valid[i] = full || (pos >= lo && pos < hi);
    if (!valid[i]) {
#pragma unroll
      for (int g = 0; g < G; ++g) s[g][i] = -INFINITY;
    }
  }
  // One rescale per page and head, then the V rows one at a time (a masked
  // row is replaced by zeros so that poison in unused slots cannot leak).
  float ms[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = s[g][0];
#pragma unroll
    for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[g][i]);
    const float mn = fmaxf(st.m[g], mx);
    ms[g] = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(st.m[g] - ms[g]);
    st.l[g] *= alpha;
#pragma unroll
    for (int e = 0; e < N; ++e) st.acc[g][e] *= alpha;
    st.m[g] = mn;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float vf[N];
    Vec<E>::widen(vr[i], vf);
    if (!valid[i]) {
#pragma unroll
      for (int e = 0; e < N; ++e) vf[e] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = fast_exp2(s[g][i] - ms[g]);
      st.l[g] += p;
#pragma unroll
      for (int e = 0; e < N; ++e) st.acc[g][e] = fmaf(p, vf[e], st.acc[g][e]);
    }
  }
}

// Streams `count` pages of one (request, kv head) into this wave's row state:
// page indices p_first + stride * k, k = 0 .. count-1 (keys outside [lo, hi)
// masked). The page ids are fetched up front, one per lane, 64 at a time, and
// the loop is software-pipelined two deep: the next page's K/V loads are in
// flight while the current page is folded, so no load waits on a page-table
// read or on the previous page's math.
template <typename E, int D, int G>
__device__ __forceinline__ void wave_span(SpanState<E, D, G> &st, const uint4 *__restrict__ kb,
                                          const uint4 *__restrict__ vb,
                                          const int32_t *__restrict__ pt_row,
                                          int32_t num_pages, int32_t hkv, int32_t kvh,
                                          int p_first, int count, int stride, int lo, int hi,
                                          const QChunk<E> (&q)[G], float qscale) {
  using TL = Tile<E, D>;
  constexpr int LPT = TL::kLPT, NI = TL::kNI;
  const int lane = threadIdx.x & 63;
  const int row = lane / LPT, c = lane % LPT;
  const int lane_off = row * LPT + c;
  for (int base = 0; base < count; base += 64) {
    const int cnt = min(64, count - base);
    int pid = 0;
    if (lane < cnt) pid = min(max(pt_row[p_first + stride * (base + lane)], 0), num_pages - 1);
    const int pi0 = p_first + stride * base;  // page index of k = 0
    uint4 ka[NI], va[NI], kb2[NI], vb2[NI];
    auto page_of = [&](int k) { return __builtin_amdgcn_readlane(pid, k); };
    load_tile<E, D>(kb, vb, page_of(0), hkv, kvh, lane_off, ka, va);
    int k = 0;
    // Steady state: pages k+1 and k+2 both exist, so the prefetches are
    // unconditional and each fold only waits for its own page's loads.
    for (; k + 2 < cnt; k += 2) {
      load_tile<E, D>(kb, vb, page_of(k + 1), hkv, kvh, lane_off, kb2, vb2);
      fold_page<E, D, G>(st, q, qscale, ka, va, pi0 + stride * k, row, lo, hi);
      load_tile<E, D>(kb, vb, page_of(k + 2), hkv, kvh, lane_off, ka, va);
      fold_page<E, D, G>(st, q, qscale, kb2, vb2, pi0 + stride * (k + 1), row, lo, hi);
    }
    if (k + 1 < cnt) {  // two pages left
      load_tile<E, D>(kb, vb, page_of(k + 1), hkv, kvh, lane_off, kb2, vb2);
      fold_page<E, D, G>(st, q, qscale, ka, va, pi0 + stride * k, row, lo, hi);
      fold_page<E, D, G>(st, q, qscale, kb2, vb2, pi0 + stride * (k + 1), row, lo, hi);
    } else {  // one page left
      fold_page<E, D, G>(st, q, qscale, ka, va, pi0 + stride * k, row, lo, hi);
    }
  }
}

template <typename E, int D, int G>
__device__ __forceinline__ void reset(SpanState<E, D, G> &st) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < Tile<E, D>::kVecN; ++e) st.acc[g][e] = 0.f;
  }
}

// Merge the RPW row states of this wave (rows sit LPT lanes apart) with a
// fixed butterfly; afterwards the lanes of row 0 hold the wave's state.
template <typename E, int D, int G>
__device__ __forceinline__ void merge_rows(SpanState<E, D, G> &st) {
  constexpr int N = Tile<E, D>::kVecN, LPT = Tile<E, D>::kLPT;
#pragma unroll
  for (int mask = LPT; mask < 64; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(st.m[g], mask);
      const float lo_ = __shfl_xor(st.l[g], mask);
      const float mn = fmaxf(st.m[g], mo);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float a = fast_exp2(st.m[g] - ms), b = fast_exp2(mo - ms);
      st.l[g] = st.l[g] * a + lo_ * b;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float ao = __shfl_xor(st.acc[g][e], mask);
        st.acc[g][e] = st.acc[g][e] * a + ao * b;
      }
      st.m[g] = mn;
    }
  }
}

// Streams keys [lo, hi) with the 4 waves of the block (wave w takes pages
// w, w+4, ...) and leaves each wave's merged state in LDS:
// lds_ml[w][g] = (m, l), lds_acc[w][g][d].
template <typename E, int D, int G>
__device__ __forceinline__ void valu_span(const uint4 *__restrict__ kb,
                                          const uint4 *__restrict__ vb,
                                          const int32_t *__restrict__ pt_row,
                                          int32_t num_pages, int32_t hkv,
                                          int32_t kvh, int32_t lo, int32_t hi,
                                          const QChunk<E> (&q)[G], float qscale,
                                          float2 *lds_ml, float *lds_acc) {
  using TL = Tile<E, D>;
  constexpr int N = TL::kVecN, LPT = TL::kLPT;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / LPT, c = lane % LPT;

  SpanState<E, D, G> st;
  reset(st);
  const int p_first = lo / kPage;
  const int n_pages = hi > lo ? (hi - 1) / kPage - p_first + 1 : 0;
  const int npw = n_pages > w ? (n_pages - w + kWaves - 1) / kWaves : 0;
  if (npw > 0)
    wave_span<E, D, G>(st, kb, vb, pt_row, num_pages, hkv, kvh, p_first + w, npw, kWaves, lo, hi,
                       q, qscale);
  merge_rows(st);
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < N; ++e) lds_acc[(w * G + g) * D + c * N + e] = st.acc[g][e];
      if (c == 0) lds_ml[w * G + g] = make_float2(st.m[g], st.l[g]);
    }
  }
  __syncthreads();
}

// Combine the kWaves wave states of head g, dim d (in wave order).
template <int G, int D>
__device__ __forceinline__ void combine_waves(const float2 *lds_ml, const float *lds_acc,
                                              int g, int d, float &M, float &L, float &A) {
  M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_ml[w * G + g].x);
  const float ms = (M == -INFINITY) ? 0.f : M;
  L = 0.f;
  A = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = fast_exp2(lds_ml[w * G + g].x - ms);
    L = fmaf(lds_ml[w * G + g].y, f, L);
    A = fmaf(lds_acc[(w * G + g) * D + d], f, A);
  }
}

// Load this lane's 16-byte chunk of q for heads h0 .. h0+G-1.
template <typename E, int D, int G>
__device__ __forceinline__ void load_q(const typename E::storage *__restrict__ qrow,
                                       QChunk<E> (&q)[G]) {
  using TL = Tile<E, D>;
  const int c = (threadIdx.x & 63) % TL::kLPT;
  const uint4 *qv = reinterpret_cast<const uint4 *>(qrow);
#pragma unroll
  for (int g = 0; g < G; ++g) q[g].set(qv[g * TL::kLPT + c]);
}

}  // namespace pkv
