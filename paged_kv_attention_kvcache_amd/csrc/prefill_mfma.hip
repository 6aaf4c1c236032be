// Chunked causal prefill over paged K/V on matrix cores (bf16, head_dim 128).
//
// An extend-prefill of a span ("Faster fuzzy minds", section "LOTUS"; a
// prefix-cache hit prefills only the suffix, section "When scheduler does
// the work"): the chunk's own K/V are already in the pool (write-then-
// attend); packed query row j of request r sits at position seq_len - q_len
// + j and sees keys 0..that position.
//
// Work: the tiles of 128 query rows of a (request, q head) see 1..T steps of
// keys, so one workgroup folds the pair of tiles T-1-p and p, one after the
// other, and every workgroup carries about the same number of keys; wave w
// owns rows 32w..32w+31 of a tile as two blocks of 16 query columns. Chunks
// of at most 64 rows per request take tiles of 64 rows instead (one block of
// 16 columns per wave), so that no wave of a tile sits idle. The contraction runs on
// v_mfma_f32_16x16x32_bf16 in the transposed form
//   S^T = K Q^T   (A = 16 keys x 32 dims from a row-major K tile),
//   O^T += V^T P^T (A = 16 dims x 32 keys, B = 32 keys x 16 queries),
// where the key index of P^T and V^T is permuted so that P^T is each lane's
// own scores (lane l: keys 4(l/16)+i of two pages, query l%16) and V^T comes
// straight from a row-major V tile through ds_read_b64_tr_b16 (lane j of a
// 16-lane group receives element j%4 of the 8-byte runs that lanes 4e + j/4
// address, e = 0..3: four consecutive keys of one dim).
//
// Keys go in steps of four pages (64 keys). Each step's 4 K and 4 V tiles
// (32 KiB) are copied from HBM straight into LDS with global_load_lds_dwordx4
// (no register staging), into a ring of stages: with two stages (two
// workgroups per CU) the next step is in flight while one is folded, with
// three or four (one workgroup per CU, longer contexts) the next two or three
// are. Each wave waits for its own copies with an
// explicit vmcnt and one barrier per step publishes the stage (the compiler
// does not track these copies, so the waits are written out). Within a
// 256-byte token row the 16-byte chunk c of token t sits at c ^ t in a K
// tile and at c ^ rot(t) in a V tile (rot: 4-bit left rotation). The
// 16-byte K reads conflict as if LDS served them eight lanes at a time over
// 32 four-byte banks: with the rotation on K, SQ_LDS_BANK_CONFLICT counted
// four cycles per K read, and with the plain XOR it reads 0. The rotation
// keeps the transposing 8-byte V reads (four tokens, two chunks per sixteen
// lanes) conflict-free, where the plain XOR would not.
//
// Softmax: scores in base 2; the column max is a lane-swap reduction
// (v_permlane32_swap, v_permlane16_swap); the output accumulators are
// rescaled only when a column's max grows by more than 2^8 over the max in
// use (the probabilities are then at most 256, exact in fp32 and bf16's
// range), so most steps do no rescaling at all.
#include <cfloat>
#include <utility>

#include "common.hpp"
#include "launch.hpp"
#include "span.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kXcds = 8;          // accelerator dies; workgroups are dealt to them round-robin
constexpr int kTileBytes = 4096;  // one (page, kv head) tile
constexpr float kLazy = 8.f;      // rescale threshold (log2 units)

__device__ __forceinline__ bf16x8 as_bf16(const uint4 &x) { return __builtin_bit_cast(bf16x8, x); }

// 4-bit left rotation: the chunk swizzle of token t within a tile row.
__device__ __forceinline__ int rot4(int t) { return ((t << 1) | (t >> 3)) & 15; }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_char *)p;
}

// 16 bytes per lane from global memory (base + voff) to LDS (m0 + 16 * lane).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const void *base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds));
}

// Waits until at most N of this wave's copies are outstanding (and its LDS
// reads are done), then meets the other waves.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with N = PER * min(ahead, A) (a wait count must be an immediate).
template <int PER, int A>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (A == 0) {
    wait_barrier<0>();
  } else {
    if (ahead >= A)
      wait_barrier<PER * A>();
    else
      wait_ahead<PER, A - 1>(ahead);
  }
}

__device__ __forceinline__ bf16x4 read_tr(const lds_char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
}

// max(a, b, c) as one v_max3_f32. fmaxf would first quiet possible
// signalling NaNs of every operand (one more instruction each); the scores
// here are finite or -inf.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Max / sum over the four lanes of a query column (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float col_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max3(__uint_as_float(a[0]), __uint_as_float(a[1]), -INFINITY);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(b[0]), __uint_as_float(b[1]), -INFINITY);
}
__device__ __forceinline__ float col_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace

// SP: pages per step; RING: LDS stages; MAXP: page ids held in LDS; NB:
// blocks of 16 query rows per wave (tiles of 64 NB rows).
template <int SP, int RING, int MAXP, int NB>
__global__ __launch_bounds__(kBlock) void prefill_mfma(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const uint16_t *__restrict__ q, int32_t hq, int32_t batch, int32_t tiles,
    const int32_t *__restrict__ cu_q_lens, int32_t total_q,
    const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t max_seq_len, float qscale,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  constexpr int kTileRows = 64 * NB;  // query rows per tile
  constexpr int kStepKeys = SP * kPage;
  constexpr int kStageBytes = 2 * SP * kTileBytes;  // K and V tiles of a step
  constexpr int kTPW = 2 * SP / kWaves;             // tiles each wave copies per step
  static_assert(kTPW >= 1 && SP % 2 == 0, "a step is an even number of pages");
  __shared__ __attribute__((aligned(1024))) uint4 ring[RING * kStageBytes / 16];
  __shared__ int32_t pids[MAXP];

  // Causal tiles see 1, 2, ..., T steps of keys, so they are paired: the
  // workgroup of pair p folds tile T-1-p and then tile p of its (request,
  // head), and every pair carries about the same number of keys.
  //
  // Workgroup i runs on XCD i % 8 (round-robin dispatch), and each XCD has
  // its own L2. The pairs of one (request, head) are given ids on the same
  // XCD and next to each other in its dispatch order (id / 8), so they run
  // at the same time, stream the same K/V steps from key 0 up at about the
  // same pace, and read them through one L2. Each XCD takes a contiguous
  // block of (request, head) units, so the q heads of a GQA group (which
  // read the same K/V) share an L2 too.
  const int npairs = (tiles + 1) / 2;
  const int per_xcd = (hq * batch + kXcds - 1) / kXcds;
  const int id = (int)blockIdx.x;
  const int slot = id / kXcds;
  const int pr = slot % npairs;
  const int unit = (id % kXcds) * per_xcd + slot / npairs;  // (request, head) = (r, h)
  if (slot / npairs >= per_xcd || unit >= hq * batch) return;
  const int h = unit % hq, r = unit / hq;
  const int kvh = h / (hq / hkv);
  // Rows stay inside the packed [total_q] arrays and the launched tiles
  // whatever cu_q_lens holds.
  const int q0 = min(max(cu_q_lens[r], 0), total_q);
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  const int q_len = min(min(max(cu_q_lens[r + 1] - q0, 0), n),
                        (int)min((long long)total_q - q0, (long long)tiles * kTileRows));
  const int tiles_r = (q_len + kTileRows - 1) / kTileRows;
  if (pr >= (tiles_r + 1) / 2) return;
  const int p0 = n - q_len;  // position of query row 0
  const int t_hi = tiles_r - 1 - pr;  // the pair's later tile
  const int kpages = min((p0 + min((t_hi + 1) * kTileRows, q_len) + kPage - 1) / kPage, MAXP);
  const int32_t *pt_row = page_table + (size_t)r * pt_stride;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g4 = lane >> 4;

  for (int i = tid; i < kpages; i += kBlock) pids[i] = min(max(pt_row[i], 0), num_pages - 1);
  __syncthreads();

  // Copies: wave w moves tiles kTPW w .. kTPW w + kTPW - 1 of every stage
  // (tiles 0..SP-1 are the step's K pages, SP..2SP-1 its V pages), 1 KiB
  // (four token rows) per instruction; lane l of copy qq lands in LDS slot 64 qq + l, i.e. token
  // 4 qq + l/16, swizzled chunk l%16, and so reads chunk (l%16) ^ token (K tile) or
  // (l%16) ^ rot(token) (V tile).
  static_assert(SP % kTPW == 0, "a wave copies K tiles only or V tiles only");
  const bool copies_k = kTPW * w < SP;
  uint32_t goff[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int tt = 4 * qq + (lane >> 4);
    goff[qq] = (uint32_t)(tt * 16 + ((lane & 15) ^ (copies_k ? tt : rot4(tt)))) * 16u;
  }
  const uint32_t ring0 = lds_addr(ring);
  // Step j into ring slot `slot` (= j % RING, a compile-time constant).
  auto issue = [&](int j, auto slot) {
    const uint32_t dst = ring0 + (uint32_t)decltype(slot)::value * kStageBytes;
    int pid[kTPW];
#pragma unroll
    for (int u = 0; u < kTPW; ++u)
      pid[u] = pids[min(j * SP + (kTPW * w + u) % SP, kpages - 1)];
#pragma unroll
    for (int u = 0; u < kTPW; ++u) {
      const int tile = kTPW * w + u;
      const uint4 *src = (tile < SP ? kb : vb) +
                         ((size_t)__builtin_amdgcn_readfirstlane(pid[u]) * hkv + kvh) * 256;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) dma16(dst + tile * kTileBytes + qq * 1024, goff[qq], src);
    }
  };

  // LDS read offsets within a tile. K: token nl, chunk 4c + g4. V (transposed
  // read for dims 16 sl .. +15): token 4 g4 + nl/4, dims 16 sl + 4 (nl%4) .. +3.
  uint32_t koff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) koff[c] = (uint32_t)(nl * 16 + ((4 * c + g4) ^ nl)) * 16u;
  const int tv = 4 * g4 + (nl >> 2);
  const int gv = rot4(tv);
  uint32_t voff[8];
#pragma unroll
  for (int sl = 0; sl < 8; ++sl)
    voff[sl] = (uint32_t)(tv * 16 + ((2 * sl + ((nl >> 1) & 1)) ^ gv)) * 16u + (nl & 1) * 8u;

  // Q operands (B of S^T): block b, query row wrow0 + 16b + nl, chunk 4c + g4.
  // A negative scale moves into Q's sign bits (exact), so the scale applied
  // to scores is positive; a zero scale becomes the smallest normal float
  // (scores of at most ~1e4 then give exp2 of exactly 1).
  float qs = qscale;
  uint32_t sgn = 0;
  if (qs < 0.f) {
    qs = -qs;
    sgn = 0x80008000u;
  }
  if (!(qs > 0.f)) qs = FLT_MIN;
  for (int pass = 0; pass < 2; ++pass) {
    const int t = pass == 0 ? t_hi : pr;
    if (pass == 1 && t == t_hi) break;  // the middle tile of an odd count
    if (pass == 1) __syncthreads();  // the second tile refills the ring
    const int row_lo = t * kTileRows, row_hi = min(row_lo + kTileRows, q_len);
    const int key_end = p0 + row_hi;  // keys [0, key_end) are visible to the tile
    const int steps = (key_end + kStepKeys - 1) / kStepKeys;
    const int wrow0 = row_lo + w * 16 * NB;
    uint4 qb[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int row = wrow0 + 16 * b + nl;
      const bool ok = row < row_hi;
      const uint4 *qr =
          reinterpret_cast<const uint4 *>(q + ((size_t)(q0 + (ok ? row : 0)) * hq + h) * 128);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 x = qr[4 * c + g4];
        qb[b][c] = ok ? make_uint4(x.x ^ sgn, x.y ^ sgn, x.z ^ sgn, x.w ^ sgn)
                      : make_uint4(0, 0, 0, 0);
      }
    }

    // acc[b][sl]: O^T tiles; l[b]: this lane's part of the softmax denominator
    // (its keys), summed in fp32 before the probabilities are rounded to bf16.
    f32x4 acc[NB][8];
    float m[NB], l[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[b] = -INFINITY;
      l[b] = 0.f;
    }
    const int wave_rows = max(0, min(16 * NB, row_hi - wrow0));
    const int wave_last = p0 + wrow0 + wave_rows - 1;  // last query position of the wave

    static_for<RING - 1>([&](auto j) {
      if (decltype(j)::value < steps) issue(decltype(j)::value, j);
    });

    const lds_char *ringb = (const lds_char *)ring;
    // One step; the stage index is a compile-time constant (the loop below is
    // unrolled by RING), so every LDS address is a per-lane base plus an
    // immediate offset.
    auto step = [&](int s, auto stage) {
      // stages issued after this one, each kTPW * 4 copies per wave
      wait_ahead<kTPW * 4, RING - 2>(min(RING - 2, steps - 1 - s));
      if (s + RING - 1 < steps)
        issue(s + RING - 1, std::integral_constant<int, (decltype(stage)::value + RING - 1) % RING>{});

      const int k0 = s * kStepKeys;
      const lds_char *st = ringb + decltype(stage)::value * kStageBytes;
      const bool tail = k0 + kStepKeys > n;
      if (tail) {
        // Token rows at or beyond the context end may hold anything (NaN
        // included) and meet probability 0 in the PV product: zero their V.
        lds_u32x4 *vst = (lds_u32x4 *)(st + SP * kTileBytes);
#pragma unroll
        for (int i = 0; i < SP; ++i) {
          const int chunk = tid + kBlock * i;  // V tile i, token tid / 16
          if (k0 + 16 * i + (tid >> 4) >= n) vst[chunk] = u32x4{0u, 0u, 0u, 0u};
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      if (wave_rows == 0 || k0 > wave_last) return;  // nothing visible to this wave

      // S^T for the step's pages, every query block of the wave (K reads
      // shared), two pages at a time with the dim chunk outermost:
      // consecutive MFMAs update 2 NB different accumulators.
      f32x4 S[NB][SP];
#pragma unroll
      for (int P2 = 0; P2 < SP; P2 += 2) {
        uint4 kr[2][4];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            kr[pp][c] = __builtin_bit_cast(
                uint4, *(const lds_u32x4 *)(st + (P2 + pp) * kTileBytes + koff[c]));
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int b = 0; b < NB; ++b)
              S[b][P2 + pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  as_bf16(kr[pp][c]), as_bf16(qb[b][c]),
                  c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[b][P2 + pp], 0, 0, 0);
      }
      // Keys after a query or beyond the context are masked (only on steps
      // that cross the diagonal or the end of the context).
      if (tail || k0 + kStepKeys - 1 > p0 + wrow0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          // key k0 + 4 g4 + (16 P + i) is visible iff 16 P + i <= lim
          const int lim = min(p0 + wrow0 + 16 * b + nl, n - 1) - k0 - 4 * g4;
#pragma unroll
          for (int P = 0; P < SP; ++P)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * P + i > lim) S[b][P][i] = -INFINITY;
        }
      }

      uint4 pb[NB][SP / 2];  // P^T operands [block][half step]: keys 4 g4 + i of pages 2hs, 2hs+1
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4 * SP; e += 2) mx = max3(mx, S[b][e >> 2][e & 3], S[b][e >> 2][(e & 3) + 1]);
        const float mxs = col_max(mx) * qs;
        if (__any(mxs > m[b] + kLazy)) {
          const float mn = fmaxf(m[b], mxs);
          const float alpha = fast_exp2(m[b] - ((mn == -INFINITY) ? 0.f : mn));
          l[b] *= alpha;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[b][j] *= alpha;
          m[b] = mn;
        }
        const float nms = (m[b] == -INFINITY) ? 0.f : -m[b];
        float p[SP][4], lsum = 0.f;
#pragma unroll
        for (int P = 0; P < SP; ++P)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[P][i] = fast_exp2(fmaf(S[b][P][i], qs, nms));
            lsum += p[P][i];
          }
        l[b] += lsum;
#pragma unroll
        for (int hs = 0; hs < SP / 2; ++hs) {
          pb[b][hs].x = pack_bf16x2(p[2 * hs][0], p[2 * hs][1]);
          pb[b][hs].y = pack_bf16x2(p[2 * hs][2], p[2 * hs][3]);
          pb[b][hs].z = pack_bf16x2(p[2 * hs + 1][0], p[2 * hs + 1][1]);
          pb[b][hs].w = pack_bf16x2(p[2 * hs + 1][2], p[2 * hs + 1][3]);
        }
      }

      // O^T += V^T P^T, 32 keys (pages 2hs, 2hs+1) at a time.
#pragma unroll
      for (int hs = 0; hs < SP / 2; ++hs) {
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const uint2 a = __builtin_bit_cast(uint2, read_tr(st + (SP + 2 * hs) * kTileBytes + voff[sl]));
          const uint2 c = __builtin_bit_cast(uint2, read_tr(st + (SP + 2 * hs + 1) * kTileBytes + voff[sl]));
          const uint4 v = make_uint4(a.x, a.y, c.x, c.y);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[b][sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(v), as_bf16(pb[b][hs]),
                                                                 acc[b][sl], 0, 0, 0);
        }
      }
    };
    for (int s0 = 0; s0 < steps; s0 += RING)
      static_for<RING>([&](auto i) {
        if (s0 + decltype(i)::value < steps) step(s0 + decltype(i)::value, i);
      });

    // Sum each column's l over its four lane groups, then write O and lse.
    // Lane (nl, g4) holds dims 16 sl + 4 g4 + i of query nl.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float lt = col_sum(l[b]);
      const int row = wrow0 + 16 * b + nl;
      if (row >= row_hi) continue;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const size_t rowh = (size_t)(q0 + row) * hq + h;
      uint2 *orow = reinterpret_cast<uint2 *>(out + rowh * 128 + 4 * g4);
#pragma unroll
      for (int sl = 0; sl < 8; ++sl)
        orow[4 * sl] = make_uint2(pack_bf16x2(acc[b][sl][0] * inv, acc[b][sl][1] * inv),
                                  pack_bf16x2(acc[b][sl][2] * inv, acc[b][sl][3] * inv));
      if (lse && g4 == 0) lse[rowh] = lt > 0.f ? (m[b] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

namespace {
// Two workgroups per CU: two 64-key stages (64 KiB) and page ids for 32k
// tokens each. One per CU: four stages (128 KiB) and page ids for 64k
// tokens, or three stages (96 KiB) and page ids for 256k tokens (64 KiB;
// 160 KiB in all, the whole LDS of a CU).
constexpr int kNarrowMaxPages = 2048, kWideMaxPages = 4096, kDeepMaxPages = 16384;
}  // namespace

bool prefill_mfma_supported(const PrefillArgs &a) {
  return a.bank.dtype == 1 && a.bank.head_dim == 128 && a.max_seq_len <= kDeepMaxPages * kPage;
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
  const bool narrow = a.max_seq_len <= kNarrowMaxPages * kPage;
  // A chunk of at most 64 rows per request would leave half of a 128-row
  // tile's waves without rows: 64-row tiles (measured 9% faster per pass of
  // a 64-row block over 512 cached tokens). Longer chunks keep 128 rows,
  // whose waves read each K and V operand for two query blocks.
  const int nb = narrow && a.max_q_len <= 64 ? 1 : 2;
  const int tiles = (a.max_q_len + 64 * nb - 1) / (64 * nb);
  if (tiles == 0) return hipSuccess;
  const long long units = (long long)a.num_q_heads * a.batch;
  const long long blocks = (long long)((tiles + 1) / 2) * ((units + kXcds - 1) / kXcds * kXcds);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                       a.bank.num_pages, a.bank.num_kv_heads, static_cast<const uint16_t *>(a.q),
                       a.num_q_heads, a.batch, tiles, a.cu_q_lens, a.total_q, a.page_table,
                       a.pt_stride, a.seq_lens, a.max_seq_len, a.scale * kLog2e,
                       static_cast<uint16_t *>(a.out), a.lse);
    return hipGetLastError();
  };
  // Two workgroups per CU (72 KiB of LDS each) hide one another's copy
  // waits and softmax; the single-workgroup kernels cover longer contexts.
  if (narrow)
    return nb == 1 ? go(prefill_mfma<4, 2, kNarrowMaxPages, 1>)
                   : go(prefill_mfma<4, 2, kNarrowMaxPages, 2>);
  if (a.max_seq_len <= kWideMaxPages * kPage) return go(prefill_mfma<4, 4, kWideMaxPages, 2>);
  return go(prefill_mfma<4, 3, kDeepMaxPages, 2>);
}

}  // namespace pkv
