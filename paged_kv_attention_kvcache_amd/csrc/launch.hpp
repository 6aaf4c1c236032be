// Internal launchers (host side) for the gfx950 kernels. Arguments are
// validated by the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "args.hpp"
#include "pagedkv.h"

namespace pkv {

// Sets the thread's last-error message (pkv_last_error) and returns code.
int set_error(int code, const char *msg);

// One bank of the pool: K and V base pointers already offset to the bank.
struct Bank {
  void *k;
  void *v;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;  // 0 = fp32, 1 = bf16
};

hipError_t launch_kv_write(const Bank &b, const void *k, const void *v,
                           const int32_t *slots, int32_t num_tokens,
                           hipStream_t stream);

struct DecodeArgs {
  Bank bank;
  const void *q;
  int32_t num_q_heads;
  const int32_t *page_table;
  int32_t pt_stride;
  const int32_t *seq_lens;
  int32_t batch;
  int32_t max_seq_len;
  float scale;
  int32_t partition;  // tokens, multiple of 16
  int32_t max_parts;
  void *out;
  float *lse;
  float *part_m, *part_l, *part_acc;
  // Decode step with append: each request's newest token (position
  // seq_len - 1), [batch][num_kv_heads][head_dim], written and attended in
  // the same kernel. NULL: the pool already holds it.
  const void *k_new = nullptr, *v_new = nullptr;
  int32_t num_cus = 256;  // compute units of the device (sizes persistent grids)
  // Waves of decode_parts' grid (a multiple of 4; 0: that kernel is not
  // used). The workspace then also holds 2 * nw * G segment partials
  // ((m, l) pairs, then acc at the next 256-byte boundary).
  int64_t nw = 0;
  LatestArgs latest{};    // early-exit decode when latest.depth != null
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// Balanced split ("stream-K"): nw waves take equal page ranges; part_m holds
// float2 (m, l) per [wave][slot][head] and part_acc [wave][slot][head][D].
hipError_t launch_decode_stream(const DecodeArgs &a, int64_t nw, hipStream_t stream);
// Waves of the stream kernel that fit on num_cus compute units at once.
int stream_waves(int dtype, int head_dim, int group, int num_cus);
// Fixed partitions streamed by a persistent grid (each partition folded by
// one wave and combined in order in its registers), then the combine of
// (request, kv head)s split between waves; launch_decode takes it whenever
// it applies.
constexpr int kPartsMaxBatch = 4096;  // rows whose prefix the kernel keeps in LDS
bool decode_parts_supported(const DecodeArgs &a);
hipError_t launch_decode_parts(const DecodeArgs &a, hipStream_t stream);

hipError_t launch_reduce(int32_t dtype, int32_t batch, int32_t num_q_heads,
                         int32_t head_dim, const int32_t *seq_lens,
                         int32_t max_seq_len, int32_t partition,
                         int32_t max_parts, const float *part_m,
                         const float *part_l, const float *part_acc, void *out,
                         float *lse, bool skip_single, hipStream_t stream);

struct PrefillArgs {
  Bank bank;
  const void *q;
  int32_t num_q_heads;
  const int32_t *cu_q_lens;
  int32_t total_q;
  const int32_t *page_table;
  int32_t pt_stride;
  const int32_t *seq_lens;
  int32_t batch;
  int32_t max_q_len;
  int32_t max_seq_len;
  float scale;
  void *out;
  float *lse;
};

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
// Matrix-core prefill (bf16, head_dim 128); launch_prefill picks it when it applies.
bool prefill_mfma_supported(const PrefillArgs &a);
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream);
// Short chunks (bf16, head_dim 128, rows x GQA group <= 16 per request) as one
// 16-column decode-style pass per (request, kv head); launch_prefill picks it first.
bool prefill_cols_supported(const PrefillArgs &a);
hipError_t launch_prefill_cols(const PrefillArgs &a, hipStream_t stream);

// paged_decode_attn with its split-K workspace supplied by `scratch` (which
// stores a device pointer of scratch_bytes bytes and returns 0, or returns a
// negative code), called only after every argument has been validated and
// the sizes found to fit in scratch_bytes.
int decode_scratch(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                   const void *q, int32_t num_q_heads, const int32_t *page_table,
                   int32_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                   int32_t max_seq_len, float scale, int32_t partition, void *out, float *lse,
                   int (*scratch)(void **), size_t scratch_bytes, void *stream);

}  // namespace pkv
