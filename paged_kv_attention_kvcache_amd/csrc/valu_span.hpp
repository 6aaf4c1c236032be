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
// Scores are kept in base-2 units: q is pre-multiplied by scale*log2(e) so
// the softmax uses exp2.
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

// Streams keys [lo, hi) and leaves each wave's merged state in LDS:
// lds_ml[w][g] = (m, l), lds_acc[w][g][d].
template <typename E, int D, int G>
__device__ __forceinline__ void valu_span(const uint4 *__restrict__ kb,
                                          const uint4 *__restrict__ vb,
                                          const int32_t *__restrict__ pt_row,
                                          int32_t num_pages, int32_t hkv,
                                          int32_t kvh, int32_t lo, int32_t hi,
                                          const float (&q)[G][Tile<E, D>::kVecN],
                                          float2 *lds_ml, float *lds_acc) {
  using TL = Tile<E, D>;
  constexpr int N = TL::kVecN, LPT = TL::kLPT, RPW = TL::kRPW, NI = TL::kNI;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / LPT, c = lane % LPT;

  SpanState<E, D, G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) st.acc[g][e] = 0.f;
  }

  if (hi > lo) {
    const int p_first = lo / kPage, p_last = (hi - 1) / kPage;
    for (int pi = p_first + w; pi <= p_last; pi += kWaves) {
      int page = pt_row[pi];
      page = min(max(page, 0), num_pages - 1);
      const size_t tile = ((size_t)page * hkv + kvh) * TL::kTileVec + row * LPT + c;
      uint4 kr[NI], vr[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) kr[i] = kb[tile + i * RPW * LPT];
#pragma unroll
      for (int i = 0; i < NI; ++i) vr[i] = vb[tile + i * RPW * LPT];

      const int pos0 = pi * kPage + row;  // token of load i: pos0 + i * RPW
      const bool full = (pi * kPage >= lo) && (pi * kPage + kPage <= hi);

      float s[G][NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float kf[N];
        Vec<E>::widen(kr[i], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < N; ++e) a = fmaf(q[g][e], kf[e], a);
          s[g][i] = a;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NI; ++i) s[g][i] = group_sum<LPT>(s[g][i]);

      float vf[NI][N];
#pragma unroll
      for (int i = 0; i < NI; ++i) Vec<E>::widen(vr[i], vf[i]);
      if (!full) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int pos = pos0 + i * RPW;
          if (pos < lo || pos >= hi) {
#pragma unroll
            for (int g = 0; g < G; ++g) s[g][i] = -INFINITY;
#pragma unroll
            for (int e = 0; e < N; ++e) vf[i][e] = 0.f;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = s[g][0];
#pragma unroll
        for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[g][i]);
        const float mn = fmaxf(st.m[g], mx);
        const float ms = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(st.m[g] - ms);
        float l = st.l[g] * alpha;
#pragma unroll
        for (int e = 0; e < N; ++e) st.acc[g][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const float p = fast_exp2(s[g][i] - ms);
          l += p;
#pragma unroll
          for (int e = 0; e < N; ++e) st.acc[g][e] = fmaf(p, vf[i][e], st.acc[g][e]);
        }
        st.l[g] = l;
        st.m[g] = mn;
      }
    }
  }

  // Merge the RPW row states of this wave (rows sit LPT lanes apart).
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

// Load this lane's 16-byte chunk of q for heads h0 .. h0+G-1, scaled.
template <typename E, int D, int G>
__device__ __forceinline__ void load_q(const typename E::storage *__restrict__ qrow,
                                       float qscale, float (&q)[G][Tile<E, D>::kVecN]) {
  using TL = Tile<E, D>;
  const int c = (threadIdx.x & 63) % TL::kLPT;
  const uint4 *qv = reinterpret_cast<const uint4 *>(qrow);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Vec<E>::widen(qv[g * TL::kLPT + c], q[g]);
#pragma unroll
    for (int e = 0; e < TL::kVecN; ++e) q[g][e] *= qscale;
  }
}

}  // namespace pkv
