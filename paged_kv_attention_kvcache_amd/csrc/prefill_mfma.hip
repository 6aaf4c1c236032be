// Chunked causal prefill over paged K/V on matrix cores (bf16, head_dim 128).
//
// An extend-prefill of a span ("Faster fuzzy minds", section "LOTUS"; a
// prefix-cache hit prefills only the suffix, section "When scheduler does
// the work"): the chunk's own K/V are already in the pool (write-then-
// attend); packed query row j of request r sits at position seq_len - q_len
// + j and sees keys 0..that position.
//
// Work: one workgroup per (tile of 128 query rows, q head, request); wave w
// owns rows 32w .. 32w+31 of the tile as two blocks of 16 query columns. The
// contraction runs on v_mfma_f32_16x16x32_bf16 in the transposed form
//   S^T = K Q^T (A = 16 keys x 32 dims, B = 32 dims x 16 queries),
//   O^T += V^T P^T (A = 16 dims x 32 keys, B = 32 keys x 16 queries),
// with the key index of P^T and V^T permuted so that P^T is each lane's own
// scores (lane l: keys 4(l/16)+i of both pages of a step, query l%16).
// Keys go by steps of two pages (32 keys): the workgroup copies the step's
// K and V tiles (4 x 4 KiB) from HBM into LDS once, with the 16-byte chunk
// index of each token row XOR-swizzled by the token so that the MFMA-layout
// reads below are bank-conflict free, double-buffered (the next step's
// global loads are in flight during the current step's math) with one
// barrier per step. Both query blocks of a wave share each K and V read.
// Steps past a wave's last query are skipped; only steps that cross the
// diagonal are masked. Tiles are launched heaviest (latest rows) first.
#include "common.hpp"
#include "launch.hpp"
#include "span.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 128;   // query rows per workgroup
constexpr int kBlocksPerWave = 2;  // 16-query column blocks per wave
constexpr int kStepKeys = 32;    // keys per step (two pages)
constexpr int kTileChunks = 256;  // 16-byte chunks in a (page, kv head) tile
constexpr int kStage = 4 * kTileChunks;  // K page A, K page B, V page A, V page B

__device__ __forceinline__ bf16x8 as_bf16(const uint4 &x) { return __builtin_bit_cast(bf16x8, x); }

// LDS slot of chunk c of token t in a tile (c ^ t spreads a column of the
// tile over all 16 four-bank groups).
__device__ __forceinline__ int swz(int t, int c) { return t * 16 + (c ^ t); }

}  // namespace

__global__ __launch_bounds__(kBlock) void prefill_mfma(
    const uint4 *__restrict__ kb, const uint4 *__restrict__ vb, int32_t num_pages, int32_t hkv,
    const uint16_t *__restrict__ q, int32_t hq, const int32_t *__restrict__ cu_q_lens,
    const int32_t *__restrict__ page_table, int32_t pt_stride,
    const int32_t *__restrict__ seq_lens, int32_t max_seq_len, float qscale,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  __shared__ uint4 stage[2][kStage];

  const int r = blockIdx.z, h = blockIdx.y;
  const int G = hq / hkv, kvh = h / G;
  const int q0 = cu_q_lens[r];
  const int n = min(max(seq_lens[r], 0), max_seq_len);
  const int q_len = min(max(cu_q_lens[r + 1] - q0, 0), n);
  const int tiles = (q_len + kTileRows - 1) / kTileRows;
  const int t = (int)gridDim.x - 1 - (int)blockIdx.x;  // heaviest tiles first
  if (t >= tiles) return;
  const int p0 = n - q_len;  // position of query row 0
  const int row_lo = t * kTileRows, row_hi = min(row_lo + kTileRows, q_len);
  const int key_end = p0 + row_hi;  // keys [0, key_end) are visible to the tile
  const int steps = (key_end + kStepKeys - 1) / kStepKeys;
  const int kpages = (key_end + kPage - 1) / kPage;
  const int32_t *pt_row = page_table + (size_t)r * pt_stride;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g4 = lane >> 4;
  const int wrow0 = row_lo + w * 32;  // first row of this wave
  const int wave_rows = max(0, min(32, row_hi - wrow0));
  const int wave_last_pos = p0 + wrow0 + wave_rows - 1;  // last query position of the wave

  // Q operands (B of S^T): block b, query row wrow0 + 16b + nl, chunk 4c + g4.
  uint4 qb[kBlocksPerWave][4];
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    const int row = wrow0 + 16 * b + nl;
    const bool ok = row < row_hi;
    const uint4 *qr = reinterpret_cast<const uint4 *>(q + ((size_t)(q0 + (ok ? row : 0)) * hq + h) * 128);
#pragma unroll
    for (int c = 0; c < 4; ++c) qb[b][c] = ok ? qr[4 * c + g4] : make_uint4(0, 0, 0, 0);
  }
  f32x4 acc[kBlocksPerWave][8];
  float m[kBlocksPerWave], l[kBlocksPerWave];
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[b] = -INFINITY;
    l[b] = 0.f;
  }

  // Global -> register copy of step s: thread tid moves chunk tid of each of
  // the four tiles (token tid / 16, chunk tid % 16).
  auto fetch = [&](int s, uint4 (&g)[4]) {
    const int pa = min(2 * s, kpages - 1), pb = min(2 * s + 1, kpages - 1);
    const int ida = min(max(pt_row[pa], 0), num_pages - 1);
    const int idb = min(max(pt_row[pb], 0), num_pages - 1);
    const size_t ta = ((size_t)ida * hkv + kvh) * kTileChunks + tid;
    const size_t tb = ((size_t)idb * hkv + kvh) * kTileChunks + tid;
    g[0] = load_stream(kb + ta);
    g[1] = load_stream(kb + tb);
    g[2] = load_stream(vb + ta);
    g[3] = load_stream(vb + tb);
  };
  auto put = [&](int buf, const uint4 (&g)[4]) {
    const int slot = swz(tid >> 4, tid & 15);
#pragma unroll
    for (int p = 0; p < 4; ++p) stage[buf][p * kTileChunks + slot] = g[p];
  };

  uint4 g[4];
  if (steps > 0) {
    fetch(0, g);
    put(0, g);
  }
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < steps;
    if (more) fetch(s + 1, g);  // in flight during this step's math
    const int k0 = s * kStepKeys;
    if (wave_rows > 0 && k0 <= wave_last_pos) {
      const uint4 *st = stage[buf];
      // S^T for both pages; K rows of this lane: token nl, chunk 4c + g4.
      uint4 kr[2][4];
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int c = 0; c < 4; ++c) kr[P][c] = st[P * kTileChunks + swz(nl, 4 * c + g4)];
      // V rows of this lane: token 4 g4 + i of each page, dims chunk nl.
      uint4 vr[8];
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[4 * P + i] = st[(2 + P) * kTileChunks + swz(4 * g4 + i, nl)];
      // Keys of this lane: k0 + 16 P + 4 g4 + i. Beyond the context they may
      // hold anything: zero their V rows.
      const bool diag = k0 + kStepKeys - 1 > p0 + wrow0;  // some key after some row
      if (k0 + kStepKeys > n) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + 16 * (e >> 2) + 4 * g4 + (e & 3) >= n) vr[e] = make_uint4(0, 0, 0, 0);
      }
      // V^T operands (shared by both query blocks): dim slice j.
      uint4 va[8];
      auto word = [](const uint4 &x, int i) { return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w; };
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t a[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t x = word(vr[2 * kk], j >> 1), y = word(vr[2 * kk + 1], j >> 1);
          a[kk] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
        va[j] = make_uint4(a[0], a[1], a[2], a[3]);
      }
#pragma unroll
      for (int b = 0; b < kBlocksPerWave; ++b) {
        const int qpos = p0 + wrow0 + 16 * b + nl;  // this lane's query position
        if (p0 + wrow0 + 16 * b > wave_last_pos) continue;  // block past the tile
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(kr[0][c]), as_bf16(qb[b][c]), sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(kr[1][c]), as_bf16(qb[b][c]), sb, 0, 0, 0);
        }
        float sv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = sa[i] * qscale;
          sv[4 + i] = sb[i] * qscale;
        }
        if (diag || k0 + kStepKeys > n) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kpos = k0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
            if (kpos > qpos || kpos >= n) sv[e] = -INFINITY;
          }
        }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[b], mx);
        const float ms = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m[b] - ms);
        float p[8], lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(sv[e] - ms);
          lsum += p[e];
        }
        l[b] = l[b] * alpha + lsum;
        m[b] = mn;
        uint4 pw;
        pw.x = pack_bf16x2(p[0], p[1]);
        pw.y = pack_bf16x2(p[2], p[3]);
        pw.z = pack_bf16x2(p[4], p[5]);
        pw.w = pack_bf16x2(p[6], p[7]);
        const bf16x8 pb = as_bf16(pw);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc[b][j] *= alpha;
          acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(va[j]), pb, acc[b][j], 0, 0, 0);
        }
      }
    }
    if (more) put(buf ^ 1, g);
    __syncthreads();
  }

  // Sum each column's l over its four lane groups, then write O and lse.
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    float lt = l[b] + __shfl_xor(l[b], 16);
    lt += __shfl_xor(lt, 32);
    const int row = wrow0 + 16 * b + nl;
    if (row >= row_hi) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float o[32];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[8 * i + j] = acc[b][j][i] * inv;
    const size_t rowh = (size_t)(q0 + row) * hq + h;
    store_row<BF16>(out + rowh * 128 + 32 * g4, o, 32);
    if (lse && g4 == 0) lse[rowh] = lt > 0.f ? (m[b] + log2f(lt)) * kLn2 : -INFINITY;
  }
}

bool prefill_mfma_supported(const PrefillArgs &a) {
  return a.bank.dtype == 1 && a.bank.head_dim == 128;
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
  const int tiles = (a.max_q_len + kTileRows - 1) / kTileRows;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(tiles, a.num_q_heads, a.batch);
  hipLaunchKernelGGL(prefill_mfma, grid, dim3(kBlock), 0, stream,
                     static_cast<const uint4 *>(a.bank.k), static_cast<const uint4 *>(a.bank.v),
                     a.bank.num_pages, a.bank.num_kv_heads, static_cast<const uint16_t *>(a.q),
                     a.num_q_heads, a.cu_q_lens, a.page_table, a.pt_stride, a.seq_lens,
                     a.max_seq_len, a.scale * kLog2e, static_cast<uint16_t *>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace pkv
