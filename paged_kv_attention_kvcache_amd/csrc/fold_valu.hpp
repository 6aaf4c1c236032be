// Vector-ALU fold of paged K/V tiles for a GQA group of G query heads.
//
// Used where the contraction is too skinny for matrix cores (a group of 1 or
// 2 query heads, fp32 data, or head_dim 64). Within a wave, LPT =
// head_dim*bytes/16 consecutive lanes hold one token row of a (page, kv head)
// tile, 16 bytes each, so every load instruction of a wave reads 1 KiB of
// the 4 KiB tile contiguously. A q.k dot product is an in-lane chain (packed
// v_dot2_f32_bf16 for bf16, FMAs for fp32) plus a DPP butterfly over the LPT
// lanes of the row; each row then keeps its own online-softmax state (m, l,
// acc) over the tokens it sees, so no cross-row traffic happens inside the
// page loop. finish_wave() merges the rows with lane shuffles in a fixed
// order (bitwise repeatable, independent of physical page ids).
//
// Scores are in base-2 units: each reduced q.k is multiplied by
// scale*log2(e) and the softmax uses exp2.
#pragma once
#include "span.hpp"

namespace pkv {

template <typename E, int D> struct Tile {
  static constexpr int kVecN = Vec<E>::kN;       // elements per 16-byte chunk
  static constexpr int kLPT = D / kVecN;         // lanes per token row
  static constexpr int kRPW = 64 / kLPT;         // token rows per wave load
  static constexpr int kNI = kPage / kRPW;       // wave loads per tile
  static constexpr int kTileVec = kPage * kLPT;  // 16-byte chunks per tile
  static_assert(kLPT == 8 || kLPT == 16 || kLPT == 32, "unsupported head_dim");
};

// L: early-exit decode, each token row loaded from its own plane's bank.
template <typename E, int D, int G, bool L = false>
struct ValuFold {
  using TL = Tile<E, D>;
  static constexpr bool kLatest = L;
  static constexpr int N = TL::kVecN, LPT = TL::kLPT, RPW = TL::kRPW, NI = TL::kNI;
  static constexpr int kPagesPerStep = 1;
  static constexpr int kDepth = 2;  // steps in flight per wave (3 measured slower)
  static constexpr int kGroup = G;
  static constexpr int kHeadDim = D;
  static constexpr float kLazy = 8.f;  // rescale threshold, log2 units

  struct State {
    float m[G], l[G], acc[G][N];
  };
  struct Regs {
    uint4 k[NI], v[NI];
  };

  QChunk<E> q[G];
  float qscale;
  int row, c;
  uint32_t lane_off;  // bytes into a tile
  // Appended token (decode step): its page index in the request, its offset
  // in that page (-1: none) and this lane's 16-byte chunk of its K and V rows.
  int app_page = -1, app_tok = -1;
  uint4 app_k, app_v;
  LatestArgs la{};  // early-exit decode (L only)

  // qrow: the first of the G query rows (contiguous, head_dim each).
  __device__ __forceinline__ ValuFold(const typename E::storage *__restrict__ qrow, float qs)
      : qscale(qs) {
    const int lane = threadIdx.x & 63;
    row = lane / LPT;
    c = lane % LPT;
    lane_off = (uint32_t)(row * LPT + c) * 16u;
    const uint4 *qv = reinterpret_cast<const uint4 *>(qrow);
#pragma unroll
    for (int g = 0; g < G; ++g) q[g].set(qv[g * LPT + c]);
  }

  // Makes this wave the writer of the request's newest token: position pos
  // (page pos / 16) gets k_row / v_row (head_dim elements each) in the tile of
  // page id `page`, and the fold uses these values for that position.
  __device__ __forceinline__ void set_append(const typename E::storage *__restrict__ k_row,
                                             const typename E::storage *__restrict__ v_row,
                                             int pos, uint4 *__restrict__ kb,
                                             uint4 *__restrict__ vb, int page, int hkv,
                                             int kvh) {
    app_page = pos / kPage;
    app_tok = pos % kPage;
    app_k = reinterpret_cast<const uint4 *>(k_row)[c];
    app_v = reinterpret_cast<const uint4 *>(v_row)[c];
    if (row == app_tok % RPW) {
      const size_t at = ((size_t)page * hkv + kvh) * TL::kTileVec + (size_t)app_tok * LPT + c;
      kb[at] = app_k;
      vb[at] = app_v;
    }
  }

  __device__ __forceinline__ void reset(State &st) const {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      st.m[g] = -INFINITY;
      st.l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) st.acc[g][e] = 0.f;
    }
  }

  // The (page, kv head) tile rows this lane owns; page and kvh are
  // wave-uniform, so the tile base is a scalar address.
  template <bool C = false>
  __device__ __forceinline__ void load(Regs &r, const uint4 *__restrict__ kb,
                                       const uint4 *__restrict__ vb, int page, int,
                                       int hkv, int kvh) const {
    const size_t tile = ((size_t)page * hkv + kvh) * TL::kTileVec;
    const char *kt = reinterpret_cast<const char *>(kb + tile);
    const char *vt = reinterpret_cast<const char *>(vb + tile);
#pragma unroll
    for (int i = 0; i < NI; ++i) r.k[i] = load_kv<C>(kt + lane_off + i * RPW * LPT * 16u);
#pragma unroll
    for (int i = 0; i < NI; ++i) r.v[i] = load_kv<C>(vt + lane_off + i * RPW * LPT * 16u);
  }

  // Early-exit variant of load: `ex` holds the 16 exit depths of the page's
  // tokens (byte t = token t). The row of token t is read from the bank of
  // plane min(la.plane, depth); bytes past the plane (and ones that would be
  // negative as int8) read the query's own plane, so every address stays in
  // a bank the call was validated for.
  // (One page per step: the second page and its depths are not used.)
  __device__ __forceinline__ void load_latest(Regs &r, const uint4 *__restrict__ kb,
                                              const uint4 *__restrict__ vb, int page,
                                              const uint4 &ex, int, const uint4 &, int hkv,
                                              int kvh) const {
    const size_t tile = ((size_t)page * hkv + kvh) * TL::kTileVec;
    const char *kt = reinterpret_cast<const char *>(kb + tile);
    const char *vt = reinterpret_cast<const char *>(vb + tile);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = row + i * RPW;  // token of load i within the page
      const uint32_t w = (t >> 2) == 0 ? ex.x : (t >> 2) == 1 ? ex.y : (t >> 2) == 2 ? ex.z : ex.w;
      const int e = min((int)((w >> (8 * (t & 3))) & 0xffu), la.plane);
      const int64_t delta = e == 0 ? la.d0 : la.d1 + (int64_t)(e - 1) * la.step;
      const uint32_t off = lane_off + i * RPW * LPT * 16u;
      r.k[i] = load_stream(kt + delta + off);
      r.v[i] = load_stream(vt + delta + off);
    }
  }

  // Folds page pi of the request (keys outside [lo, hi) masked). The page
  // registers are only read (the loop that streams them keeps them in
  // place); on the appended token's page a local copy carries its row.
  __device__ __forceinline__ void fold(State &st, const Regs &r, int pi, int, int lo,
                                       int hi) const {
    if (pi == app_page) {
      Regs x = r;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (row + i * RPW == app_tok) {
          x.k[i] = app_k;
          x.v[i] = app_v;
        }
      fold_regs(st, x, pi, lo, hi);
    } else {
      fold_regs(st, r, pi, lo, hi);
    }
  }

  __device__ __forceinline__ void fold_regs(State &st, const Regs &r, int pi, int lo,
                                            int hi) const {
    const int pos0 = pi * kPage + row;  // token of load i: pos0 + i * RPW
    const bool full = (pi * kPage >= lo) && (pi * kPage + kPage <= hi);
    float s[G][NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint4 k = r.k[i];
#pragma unroll
      for (int g = 0; g < G; ++g) s[g][i] = q[g].dot(k);
    }
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
    // Each row state keeps a reference max m; it moves (and l, acc are
    // rescaled) only when a score exceeds it by more than 2^kLazy, so the
    // weights exp2(s - m) stay at most 2^kLazy (exact in fp32 and within
    // bf16's range) and most pages skip the rescale. The branch is taken by
    // the whole wave when any of its rows needs it.
    float mx[G];
    bool grow = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mx[g] = s[g][0];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx[g] = fmaxf(mx[g], s[g][i]);
      grow |= mx[g] > st.m[g] + kLazy;
    }
    if (__any(grow)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(st.m[g], mx[g]);
        const float alpha = fast_exp2(st.m[g] - ((mn == -INFINITY) ? 0.f : mn));
        st.l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < N; ++e) st.acc[g][e] *= alpha;
        st.m[g] = mn;
      }
    }
    float p[G][NI];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float nm = (st.m[g] == -INFINITY) ? 0.f : -st.m[g];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        p[g][i] = fast_exp2(s[g][i] + nm);
        st.l[g] += p[g][i];  // the denominator sums the fp32 weights
      }
    }
    if constexpr (N == 8) {
      // bf16: V of two token rows interleaved per dim (v_perm_b32) meets the
      // weights of those rows rounded to bf16 in one v_dot2_f32_bf16 (fp32
      // accumulation). Rows outside [lo, hi) contribute exact zeros, so
      // poison in unused slots cannot leak.
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      uint4 v[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) v[i] = valid[i] ? r.v[i] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const uint32_t a[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        const uint32_t b[4] = {v[i + 1].x, v[i + 1].y, v[i + 1].z, v[i + 1].w};
        uint32_t pp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g] = pack_bf16x2(p[g][i], p[g][i + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo16 = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
          const uint32_t hi16 = __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const bf16x2 w = __builtin_bit_cast(bf16x2, pp[g]);
            st.acc[g][2 * j] = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2, lo16), w, st.acc[g][2 * j], false);
            st.acc[g][2 * j + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2, hi16), w, st.acc[g][2 * j + 1], false);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[N];
        Vec<E>::widen(r.v[i], vf);
        if (!valid[i]) {
#pragma unroll
          for (int e = 0; e < N; ++e) vf[e] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < N; ++e) st.acc[g][e] = fmaf(p[g][i], vf[e], st.acc[g][e]);
      }
    }
  }

  // Merge the RPW row states (rows sit LPT lanes apart) with a fixed
  // butterfly; afterwards the lanes of row 0 hold the wave's state.
  __device__ __forceinline__ void finish_wave(State &st) const {
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

  // Folds finished state p (after finish_wave) into `into`, as the combine of
  // two partitions in order: each is rescaled to the larger max.
  __device__ __forceinline__ static void merge(State &into, const State &p) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(into.m[g], p.m[g]);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float a = fast_exp2(into.m[g] - ms), b = fast_exp2(p.m[g] - ms);
      into.l[g] = into.l[g] * a + p.l[g] * b;
#pragma unroll
      for (int e = 0; e < N; ++e) into.acc[g][e] = into.acc[g][e] * a + p.acc[g][e] * b;
      into.m[g] = mn;
    }
  }

  template <class Fn>
  __device__ __forceinline__ void emit(const State &st, Fn &&fn) const {
    if (row != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) fn(g, c * N, N, st.m[g], st.l[g], st.acc[g]);
  }
};

}  // namespace pkv
