// Page pipeline shared by every attention kernel, and the hand-off of
// per-wave online-softmax states.
//
// A "fold" policy F decides how a wave holds one step of pages in registers
// (F::Regs, F::kPagesPerStep pages), how it loads them (F::load) and how it
// folds them into its online-softmax state (F::fold). stream_pages() drives
// any fold over a list of pages of one (request, kv head): page ids are
// fetched one per lane, 64 at a time, ahead of the loop, and the loop is
// software-pipelined F::kDepth steps deep (the next steps' K/V loads are in
// flight while the current step is folded), so no load waits on a page-table read or
// on the previous step's math. After F::finish_wave(), F::emit() hands the
// wave's state to a callback as (head g, first dim d0, count, m, l, acc[count])
// slices, which the kernels route to LDS, to the output, or to split-K
// partials.
#pragma once
#include "common.hpp"

namespace pkv {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;

// No action after a step (stream_pages' default).
struct NoStepHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// Streams `count` pages p_first + stride * k (k = 0 .. count-1) of one
// (request, kv head) through fold f; keys outside [lo, hi) are masked. After
// each step, after(k) runs with k = the pages folded so far (a multiple of
// F::kPagesPerStep, or count); it may hand the state on and reset it. C:
// cached K/V loads (pages other requests read too) instead of non-temporal.
template <class F, class After = NoStepHook, bool C = false>
__device__ __forceinline__ void stream_pages(F &f, typename F::State &st,
                                             const uint4 *__restrict__ kb,
                                             const uint4 *__restrict__ vb,
                                             const int32_t *__restrict__ pt_row,
                                             int32_t num_pages, int32_t hkv, int32_t kvh,
                                             int p_first, int count, int stride, int lo, int hi,
                                             const uint8_t *__restrict__ ex_row = nullptr,
                                             After after = After()) {
  constexpr int S = F::kPagesPerStep;
  const int lane = threadIdx.x & 63;
  for (int base = 0; base < count; base += 64) {
    const int cnt = min(64, count - base);
    int pid = 0;
    uint4 ex = make_uint4(0u, 0u, 0u, 0u);  // early exit: the page's 16 exit depths
    if (lane < cnt) {
      const int pi = p_first + stride * (base + lane);
      pid = min(max(pt_row[pi], 0), num_pages - 1);
      if constexpr (F::kLatest) ex = *reinterpret_cast<const uint4 *>(ex_row + 16 * (size_t)pi);
    }
    const int pi0 = p_first + stride * base;  // page index of k = 0
    const int steps = (cnt + S - 1) / S;
    // Page id and page index of the k-th page of this chunk; a page past the
    // chunk (odd tail of a 2-page step) reloads the last page and is masked.
    auto page = [&](int k) { return __builtin_amdgcn_readlane(pid, min(k, cnt - 1)); };
    auto index = [&](int k) { return k < cnt ? pi0 + stride * k : -1; };
    // The 16 exit depths of the k-th page of this chunk (early exit).
    auto exits = [&](int k) {
      k = min(k, cnt - 1);
      return make_uint4(__builtin_amdgcn_readlane(ex.x, k), __builtin_amdgcn_readlane(ex.y, k),
                        __builtin_amdgcn_readlane(ex.z, k), __builtin_amdgcn_readlane(ex.w, k));
    };
    auto load = [&](typename F::Regs &r, int s) {
      if constexpr (F::kLatest) {
        f.load_latest(r, kb, vb, page(s * S), exits(s * S), page(s * S + S - 1),
                      exits(s * S + S - 1), hkv, kvh);
      } else {
        f.template load<C>(r, kb, vb, page(s * S), page(s * S + S - 1), hkv, kvh);
      }
    };
    // A fold ends with a compiler-only barrier: the next load into the same
    // registers must not be hoisted above it (that needs a second register
    // set, and the copy between the two sets at the loop's back edge waits
    // for every load in flight).
    auto fold = [&](typename F::Regs &r, int s) {
      f.fold(st, r, index(s * S), S > 1 ? index(s * S + 1) : -1, lo, hi);
      asm volatile("" ::: "memory");
      after(base + min(s * S + S, cnt));
    };
    if constexpr (F::kDepth >= 3) {
      // Three steps in flight: the steady state (all prefetches exist) runs
      // unconditionally; at most four steps remain for the tail.
      typename F::Regs ra, rb, rc;
      load(ra, 0);
      if (steps > 1) load(rb, 1);
      int s = 0;
      for (; s + 4 < steps; s += 3) {
        load(rc, s + 2);
        fold(ra, s);
        load(ra, s + 3);
        fold(rb, s + 1);
        load(rb, s + 4);
        fold(rc, s + 2);
      }
      if (s + 2 < steps) load(rc, s + 2);
      fold(ra, s);
      if (s + 3 < steps) load(ra, s + 3);
      if (s + 1 < steps) fold(rb, s + 1);
      if (s + 2 < steps) fold(rc, s + 2);
      if (s + 3 < steps) fold(ra, s + 3);
    } else {
      typename F::Regs ra, rb;
      load(ra, 0);
      int s = 0;
      // Steady state: steps s+1 and s+2 both exist, so the prefetches are
      // unconditional and each fold waits only for its own step's loads.
      for (; s + 2 < steps; s += 2) {
        load(rb, s + 1);
        fold(ra, s);
        load(ra, s + 2);
        fold(rb, s + 1);
      }
      if (s + 1 < steps) {
        load(rb, s + 1);
        fold(ra, s);
        fold(rb, s + 1);
      } else {
        fold(ra, s);
      }
    }
  }
}

// Per-wave states of a block in LDS: lds_ml[w][g] = (m, l), lds_acc[w][g][d].
template <class F>
__device__ __forceinline__ void emit_to_lds(F &f, const typename F::State &st, int w,
                                            float2 *lds_ml, float *lds_acc) {
  constexpr int G = F::kGroup, D = F::kHeadDim;
  f.emit(st, [&](int g, int d0, int cnt, float m, float l, const float *acc) {
    for (int e = 0; e < cnt; ++e) lds_acc[(w * G + g) * D + d0 + e] = acc[e];
    if (d0 == 0) lds_ml[w * G + g] = make_float2(m, l);
  });
}

// Combine the W wave states of head g, dim d (in wave order).
template <int G, int D, int W = kWaves>
__device__ __forceinline__ void combine_waves(const float2 *lds_ml, const float *lds_acc,
                                              int g, int d, float &M, float &L, float &A) {
  M = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, lds_ml[w * G + g].x);
  const float ms = (M == -INFINITY) ? 0.f : M;
  L = 0.f;
  A = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float f = fast_exp2(lds_ml[w * G + g].x - ms);
    L = fmaf(lds_ml[w * G + g].y, f, L);
    A = fmaf(lds_acc[(w * G + g) * D + d], f, A);
  }
}

// Normalised output of one (row, dim) from a folded (M, L, A); lse in
// natural log. L == 0 (nothing visible) gives 0 and -inf.
template <typename E>
__device__ __forceinline__ void finish(typename E::storage *__restrict__ out,
                                       float *__restrict__ lse, size_t rowh, int D, int d,
                                       float M, float L, float A) {
  const float o = (L > 0.f) ? A / L : 0.f;
  store_row<E>(out + rowh * D + d, &o, 1);
  if (lse && d == 0) lse[rowh] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Writes a wave's finished slices straight to the output.
template <class F, typename E>
__device__ __forceinline__ void emit_final(F &f, const typename F::State &st,
                                           typename E::storage *__restrict__ out,
                                           float *__restrict__ lse, size_t row0) {
  constexpr int D = F::kHeadDim;
  f.emit(st, [&](int g, int d0, int cnt, float m, float l, const float *acc) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float o[32];
    for (int e = 0; e < cnt; ++e) o[e] = acc[e] * inv;
    store_row<E>(out + (row0 + g) * D + d0, o, cnt);
    if (lse && d0 == 0) lse[row0 + g] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  });
}

}  // namespace pkv
