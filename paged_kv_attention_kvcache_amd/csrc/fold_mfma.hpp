// Matrix-core fold of paged K/V tiles for a GQA group (bf16, head_dim 128,
// G = 4 or 8 query heads sharing one kv head).
//
// The group's G query rows times a 16-token tile is a small dense
// contraction, so it runs on v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16,
// fp32 C 16x16; lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16] and
// C[4(l/16)+i][l%16]). Queries are padded to the 16 columns (columns >= G
// carry zeros and are never emitted). One step takes two pages (32 tokens):
//   S^T = K Q^T   : per page, 4 MFMAs over head_dim (A = K tile rows, k
//                   permuted so that lane l loads token l%16, 16-byte chunk
//                   4c + l/16 of slice c: contiguous 64-byte runs);
//   online softmax per query column n = l%16: each lane holds 8 scores
//                   (tokens 4(l/16)+i of both pages), the column max is a
//                   2-step lane shuffle;
//   O^T += V^T P^T: 8 MFMAs, one per dim slice j (A row m <-> dim 8m + j).
//                   The k index (token) is permuted the same way for P^T and
//                   V^T: k-group l/16 holds tokens 4(l/16)..+3 of page A and
//                   of page B, which is exactly the lane's own 8 scores, so
//                   P^T needs no data movement; V^T comes from 16-byte loads
//                   of whole token rows (8 dims) transposed in registers.
// Each lane ends with, for query n, the dims 32(l/16) .. +31.
//
// PC (per column): the 16 columns are up to 16 query rows of a short prefill
// chunk (column n = query row n / gh of head kvh * gh + n % gh, gh = query
// heads per kv head), each with its own causal end: column n sees keys below
// col_hi. Keys at or past the context end still zero their V rows for every
// column; keys inside the context but past a column's end only get
// probability 0 in that column.
//
// L (early exit): each token row is read from the bank of plane
// min(query plane, the token's exit depth) of the same layer; the fold math
// is unchanged.
#pragma once
#include <climits>

#include "span.hpp"

namespace pkv {

template <int G, bool PC = false, bool L = false>
struct MfmaFold {
  static_assert(PC ? G == 16 && !L : (G == 4 || G == 8),
                "MFMA fold covers GQA groups of 4 and 8, or 16 prefill columns");
  static constexpr int kPagesPerStep = 2;
  static constexpr bool kLatest = L;
  static constexpr int kDepth = 2;  // steps in flight per wave
  static constexpr int kGroup = G;
  static constexpr int kHeadDim = 128;
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));

  struct State {
    f32x4 acc[8];  // O^T tiles: acc[j][i] = dim 32(l/16) + 8i + j of query l%16
    float m, l;    // online-softmax state of query l%16 (l: this lane's tokens)
  };
  struct Regs {
    uint4 k[2][4];  // [page][c]: token l%16, chunk 4c + l/16
    uint4 v[2][4];  // [page][i]: token 4(l/16) + i, dims 8(l%16) .. +7
  };

  uint4 qb[4];  // B operand of S^T: query l%16, chunk 4c + l/16
  float qscale;
  int n, g4;
  int ncols = G;                       // columns emitted
  int col_hi = INT_MAX, hi_min = INT_MAX;  // PC: column n's key end; the smallest one
  uint32_t koff, voff;
  // Appended token (decode step): page index in the request, offset in the
  // page (-1: none), this lane's K chunks (as in Regs::k) and V chunk.
  int app_page = -1, app_tok = -1;
  uint4 app_k[4], app_v;
  LatestArgs la{};  // early-exit decode (L only)

  __device__ __forceinline__ static bf16x8 as_bf16(const uint4 &x) {
    return __builtin_bit_cast(bf16x8, x);
  }

  // qrow: the first of the G query rows (contiguous, 128 bf16 each).
  __device__ __forceinline__ MfmaFold(const uint16_t *__restrict__ qrow, float qs) : qscale(qs) {
    const int lane = threadIdx.x & 63;
    n = lane & 15;
    g4 = lane >> 4;
    koff = (uint32_t)(n * 256 + g4 * 16);
    voff = (uint32_t)(g4 * 1024 + n * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qb[c] = n < G ? *reinterpret_cast<const uint4 *>(qrow + n * 128 + (4 * c + g4) * 8)
                    : make_uint4(0, 0, 0, 0);
  }

  // PC: columns n < ncols are query rows q0 + n / gh, heads kvh * gh + n % gh
  // of the packed q [rows][hq][128]; row j's keys end at p0 + j + 1.
  __device__ __forceinline__ MfmaFold(const uint16_t *__restrict__ q, int q0, int hq, int kvh,
                                      int gh, int cols, int p0, float qs)
      : qscale(qs), ncols(cols), hi_min(p0 + 1) {
    static_assert(PC, "the per-column constructor is for prefill columns");
    const int lane = threadIdx.x & 63;
    n = lane & 15;
    g4 = lane >> 4;
    koff = (uint32_t)(n * 256 + g4 * 16);
    voff = (uint32_t)(g4 * 1024 + n * 16);
    const int j = n / gh, g = n % gh;
    col_hi = n < cols ? p0 + j + 1 : 0;
    const uint16_t *qrow = q + ((size_t)(q0 + (n < cols ? j : 0)) * hq + (size_t)kvh * gh + g) * 128;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qb[c] = n < cols ? *reinterpret_cast<const uint4 *>(qrow + (4 * c + g4) * 8)
                       : make_uint4(0, 0, 0, 0);
  }

  // Makes this wave the writer of the request's newest token at position pos:
  // its rows go to the tile of page id `page`, and the fold uses them for
  // that position.
  __device__ __forceinline__ void set_append(const uint16_t *__restrict__ k_row,
                                             const uint16_t *__restrict__ v_row, int pos,
                                             uint4 *__restrict__ kb, uint4 *__restrict__ vb,
                                             int page, int hkv, int kvh) {
    app_page = pos / kPage;
    app_tok = pos % kPage;
    const uint4 *kr = reinterpret_cast<const uint4 *>(k_row);
#pragma unroll
    for (int c = 0; c < 4; ++c) app_k[c] = kr[4 * c + g4];
    app_v = reinterpret_cast<const uint4 *>(v_row)[n];
    const size_t row = ((size_t)page * hkv + kvh) * 256 + (size_t)app_tok * 16;
    if (n == app_tok) {
#pragma unroll
      for (int c = 0; c < 4; ++c) kb[row + 4 * c + g4] = app_k[c];
    }
    if (g4 == 0) vb[row + n] = app_v;
  }

  __device__ __forceinline__ void reset(State &st) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
  }

  template <bool C = false>
  __device__ __forceinline__ void load(Regs &r, const uint4 *__restrict__ kb,
                                       const uint4 *__restrict__ vb, int page0, int page1,
                                       int hkv, int kvh) const {
    const size_t t0 = ((size_t)page0 * hkv + kvh) * 256, t1 = ((size_t)page1 * hkv + kvh) * 256;
    const char *k0 = reinterpret_cast<const char *>(kb + t0);
    const char *k1 = reinterpret_cast<const char *>(kb + t1);
    const char *v0 = reinterpret_cast<const char *>(vb + t0);
    const char *v1 = reinterpret_cast<const char *>(vb + t1);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.k[0][c] = load_kv<C>(k0 + koff + c * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.k[1][c] = load_kv<C>(k1 + koff + c * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[0][i] = load_kv<C>(v0 + voff + i * 256);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[1][i] = load_kv<C>(v1 + voff + i * 256);
  }

  // Byte offset from the query's own bank to the bank that holds token t of
  // a page whose 16 exit depths are `ex` (byte t = token t): plane
  // min(la.plane, depth); bytes past the plane (and ones that would be
  // negative as int8) give the query's own plane, so every address stays in
  // a bank the call was validated for.
  __device__ __forceinline__ int64_t exit_delta(const uint4 &ex, int t) const {
    const uint32_t w = (t >> 2) == 0 ? ex.x : (t >> 2) == 1 ? ex.y : (t >> 2) == 2 ? ex.z : ex.w;
    const int e = min((int)((w >> (8 * (t & 3))) & 0xffu), la.plane);
    return e == 0 ? la.d0 : la.d1 + (int64_t)(e - 1) * la.step;
  }

  // Early-exit variant of load: page0 / page1 with exit depths ex0 / ex1.
  // This lane's K chunks are all of token l%16; its V rows are tokens
  // 4(l/16) + i.
  __device__ __forceinline__ void load_latest(Regs &r, const uint4 *__restrict__ kb,
                                              const uint4 *__restrict__ vb, int page0,
                                              const uint4 &ex0, int page1, const uint4 &ex1,
                                              int hkv, int kvh) const {
    const size_t t0 = ((size_t)page0 * hkv + kvh) * 256, t1 = ((size_t)page1 * hkv + kvh) * 256;
    const char *kt[2] = {reinterpret_cast<const char *>(kb + t0),
                         reinterpret_cast<const char *>(kb + t1)};
    const char *vt[2] = {reinterpret_cast<const char *>(vb + t0),
                         reinterpret_cast<const char *>(vb + t1)};
    const uint4 ex[2] = {ex0, ex1};
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const char *k = kt[P] + exit_delta(ex[P], n) + koff;
#pragma unroll
      for (int c = 0; c < 4; ++c) r.k[P][c] = load_stream(k + c * 64);
    }
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.v[P][i] = load_stream(vt[P] + exit_delta(ex[P], 4 * g4 + i) + voff + i * 256);
  }

  // Folds pages piA and piB (piB = -1: absent) of the request; keys outside
  // [lo, hi) are masked.
  __device__ __forceinline__ void fold(State &st, const Regs &r, int piA, int piB, int lo,
                                       int hi) const {
    // The page registers are only read (the loop that streams them keeps
    // them in place); on the appended token's page a local copy carries its
    // row.
    if (piA == app_page || piB == app_page) {
      Regs x = r;
#pragma unroll
      for (int P = 0; P < 2; ++P) {
        if ((P == 0 ? piA : piB) != app_page) continue;
        if (n == app_tok) {
#pragma unroll
          for (int c = 0; c < 4; ++c) x.k[P][c] = app_k[c];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g4 + i == app_tok) x.v[P][i] = app_v;
      }
      fold_regs(st, x, piA, piB, lo, hi);
    } else {
      fold_regs(st, r, piA, piB, lo, hi);
    }
  }

  __device__ __forceinline__ void fold_regs(State &st, const Regs &r, int piA, int piB, int lo,
                                            int hi) const {
    auto kk = [&](int P, int c) { return r.k[P][c]; };
    auto vv = [&](int P, int i) { return r.v[P][i]; };
    f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(kk(0, c)), as_bf16(qb[c]), sA, 0, 0, 0);
      sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(kk(1, c)), as_bf16(qb[c]), sB, 0, 0, 0);
    }
    // hf: keys below it are visible to every column; hc: this lane's column.
    const int hf = PC ? min(hi, hi_min) : hi, hc = PC ? min(hi, col_hi) : hi;
    const bool full = piA >= 0 && piB >= 0 && piA * kPage >= lo && piA * kPage + kPage <= hf &&
                      piB * kPage >= lo && piB * kPage + kPage <= hf;
    float sv[8];
    bool ok[8], in[8];  // ok: visible to this column; in: inside [lo, hi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pa = piA * kPage + 4 * g4 + i, pb = piB * kPage + 4 * g4 + i;
      in[i] = full || (piA >= 0 && pa >= lo && pa < hi);
      in[4 + i] = full || (piB >= 0 && pb >= lo && pb < hi);
      ok[i] = PC ? (full || (in[i] && pa < hc)) : in[i];
      ok[4 + i] = PC ? (full || (in[4 + i] && pb < hc)) : in[4 + i];
      sv[i] = ok[i] ? sA[i] * qscale : -INFINITY;
      sv[4 + i] = ok[4 + i] ? sB[i] * qscale : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(st.m, mx);
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(st.m - ms);
    float p[8], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(sv[e] - ms);
      lsum += p[e];
    }
    st.l = st.l * alpha + lsum;
    st.m = mn;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] *= alpha;

    uint4 pw;
    pw.x = pack_bf16x2(p[0], p[1]);
    pw.y = pack_bf16x2(p[2], p[3]);
    pw.z = pack_bf16x2(p[4], p[5]);
    pw.w = pack_bf16x2(p[6], p[7]);
    const bf16x8 pb = as_bf16(pw);

    uint4 vr[8] = {vv(0, 0), vv(0, 1), vv(0, 2), vv(0, 3), vv(1, 0), vv(1, 1), vv(1, 2), vv(1, 3)};
    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!in[e]) vr[e] = make_uint4(0, 0, 0, 0);
    }
    auto word = [](const uint4 &x, int w) { return w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w; };
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t a[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t x = word(vr[2 * kk], j >> 1), y = word(vr[2 * kk + 1], j >> 1);
        a[kk] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      const uint4 av = make_uint4(a[0], a[1], a[2], a[3]);
      st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(av), pb, st.acc[j], 0, 0, 0);
    }
  }

  // The four lanes of a query column (l/16 = 0..3) share m; sum their l.
  __device__ __forceinline__ void finish_wave(State &st) const {
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
  }

  // Folds finished state p (after finish_wave) into `into`, as the combine of
  // two partitions in order: each is rescaled to the larger max.
  __device__ __forceinline__ static void merge(State &into, const State &p) {
    const float mn = fmaxf(into.m, p.m);
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    const float a = fast_exp2(into.m - ms), b = fast_exp2(p.m - ms);
    into.l = into.l * a + p.l * b;
#pragma unroll
    for (int j = 0; j < 8; ++j) into.acc[j] = into.acc[j] * a + p.acc[j] * b;
    into.m = mn;
  }

  template <class Fn>
  __device__ __forceinline__ void emit(const State &st, Fn &&fn) const {
    if (n >= (PC ? ncols : G)) return;
    float o[32];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[8 * i + j] = st.acc[j][i];
    fn(n, 32 * g4, 32, st.m, st.l, o);
  }
};

}  // namespace pkv
