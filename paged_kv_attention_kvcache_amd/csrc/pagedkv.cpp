// C-ABI of the paged-KV attention library: host-side validation, bank
// addressing and launch. See include/pagedkv.h for the contract of each
// entry point.
#include "pagedkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return PKV_OK;
}

// Re-raises the current error with "call i" in front of its message.
int fail_call(int code, int32_t i) {
  char msg[sizeof g_err];
  memcpy(msg, g_err, sizeof msg);
  return fail(code, "call %d of the step: %s", i, msg);
}

constexpr int kDefaultPartition = 512;  // fixed partitions when the balanced split is off
constexpr int kStreamMaxBatch = 4096;   // rows the balanced split indexes in LDS
constexpr int kWholeMaxSeq = 4096;      // longest context one workgroup reads whole
constexpr int kWholeMinPairs = 512;     // (request, kv head) pairs that fill the GPU
constexpr int kWholeShortSeq = 256;     // contexts this short take one launch at any batch
constexpr size_t kAlign = 256;

enum class Mode { kWhole, kStream, kFixed };

// partition 0: one workgroup per (request, kv head) reading its whole
// context when there are enough pairs to fill the GPU and contexts are short
// (no partials, no combine launch, and requests that share prefix pages read
// them at about the same time), or when every context is so short (at most
// 16 pages) that the call is launch-bound and one launch beats the balanced
// split's two; otherwise the balanced split. partition > 0: fixed partitions
// of that many tokens.
Mode decode_mode(int32_t batch, int32_t hkv, int32_t max_seq_len, int32_t partition) {
  if (partition > 0) return Mode::kFixed;
  if (max_seq_len <= kWholeShortSeq) return Mode::kWhole;
  if (max_seq_len <= kWholeMaxSeq && (int64_t)batch * hkv >= kWholeMinPairs) return Mode::kWhole;
  // the balanced split indexes the call's pages with 32-bit prefix sums
  const int64_t pages = (int64_t)batch * hkv * ((max_seq_len + 15) / 16);
  return batch <= kStreamMaxBatch && pages <= INT32_MAX ? Mode::kStream : Mode::kFixed;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : 4; }

// Validates the pool descriptor and resolves (plane, layer) to a bank.
int resolve_bank(const pkv_pool *p, int32_t plane, int32_t layer, pkv::Bank *bank) {
  if (!p) return fail(PKV_EINVAL, "pool is NULL");
  if (p->dtype != PKV_F32 && p->dtype != PKV_BF16)
    return fail(PKV_EUNSUPPORTED, "dtype %d not supported (0 = fp32, 1 = bf16)", p->dtype);
  if (p->page_size != 16) return fail(PKV_EUNSUPPORTED, "page_size %d not supported (16)", p->page_size);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim %d not supported (64, 128)", p->head_dim);
  if (p->num_pages <= 0 || p->num_kv_heads <= 0 || p->num_planes <= 0 || p->num_layers <= 0 ||
      p->num_banks <= 0)
    return fail(PKV_EINVAL, "pool sizes must be positive");
  if (!p->bank_of || !p->k_base || !p->v_base)
    return fail(PKV_EINVAL, "pool bank_of / k_base / v_base is NULL");
  if ((reinterpret_cast<uintptr_t>(p->k_base) | reinterpret_cast<uintptr_t>(p->v_base)) & 15)
    return fail(PKV_EINVAL, "pool arrays must be 16-byte aligned");
  if (plane < 0 || plane >= p->num_planes || layer < 0 || layer >= p->num_layers)
    return fail(PKV_EINVAL, "(plane %d, layer %d) outside %d x %d", plane, layer, p->num_planes,
                p->num_layers);
  const int32_t b = p->bank_of[(size_t)plane * p->num_layers + layer];
  if (b < 0) return fail(PKV_ENOTHELD, "plane %d does not hold layer %d", plane, layer);
  if (b >= p->num_banks) return fail(PKV_EINVAL, "bank %d >= num_banks %d", b, p->num_banks);
  const size_t bank_elems =
      (size_t)p->num_pages * p->num_kv_heads * p->page_size * p->head_dim;
  const size_t off = (size_t)b * bank_elems * elem_bytes(p->dtype);
  bank->k = static_cast<char *>(p->k_base) + off;
  bank->v = static_cast<char *>(p->v_base) + off;
  bank->num_pages = p->num_pages;
  bank->num_kv_heads = p->num_kv_heads;
  bank->head_dim = p->head_dim;
  bank->dtype = p->dtype;
  return PKV_OK;
}

int check_heads(const pkv_pool *p, int32_t hq) {
  if (hq <= 0 || hq % p->num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", hq,
                p->num_kv_heads);
  const int g = hq / p->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PKV_EUNSUPPORTED, "GQA group %d not supported (1, 2, 4, 8)", g);
  return PKV_OK;
}

// Compute units of the current device (cached per device; host threads may
// race to fill an entry, with the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Waves of the balanced split for this call: as many as are resident at once,
// but no more than there are pages to stream (a multiple of 4).
int64_t stream_wave_count(const pkv_pool *p, int32_t batch, int32_t hq, int32_t max_seq_len) {
  const int g = hq / p->num_kv_heads;
  int64_t nw = pkv::stream_waves(p->dtype, p->head_dim, g, device_cus());
  const int64_t pages = (int64_t)batch * p->num_kv_heads * ((max_seq_len + 15) / 16);
  nw = std::min<int64_t>(nw, (pages + 3) / 4 * 4);
  return std::max<int64_t>(nw, 4);
}

// Tokens per workgroup in the fixed and whole modes.
// Waves of the streamed fixed-partition grid: as for the balanced split, and
// no more than the call's partitions (rounded up to whole workgroups).
int64_t parts_wave_count(const pkv_pool *p, int32_t batch, int32_t hq, int32_t max_seq_len,
                         int64_t max_parts) {
  const int64_t parts = (int64_t)batch * p->num_kv_heads * max_parts;
  return std::max<int64_t>(4, std::min(stream_wave_count(p, batch, hq, max_seq_len),
                                       (parts + 3) / 4 * 4));
}

int32_t fixed_partition(Mode m, int32_t max_seq_len, int32_t partition) {
  if (m == Mode::kWhole) return max_seq_len <= 16 ? 16 : (max_seq_len + 15) / 16 * 16;
  return partition > 0 ? partition : kDefaultPartition;
}

int launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(PKV_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

int pkv::set_error(int code, const char *msg) {
  snprintf(g_err, sizeof g_err, "%s", msg);
  return code;
}

extern "C" {

int pkv_bank_map(int32_t num_planes, int32_t num_layers, int32_t rec_first, int32_t rec_count,
                 int32_t *bank_of) {
  if (num_planes <= 0 || num_layers <= 0 || rec_first < 0 || rec_count < 0 ||
      (int64_t)rec_first + rec_count > num_layers || !bank_of)
    return fail(PKV_EINVAL, "bad bank map request");
  if ((int64_t)num_planes * num_layers > INT32_MAX)
    return fail(PKV_EINVAL, "%d planes x %d layers is too many banks", num_planes, num_layers);
  int32_t next = 0;
  for (int32_t plane = 0; plane < num_planes; ++plane)
    for (int32_t layer = 0; layer < num_layers; ++layer) {
      const bool held = plane == 0 || (layer >= rec_first && layer < rec_first + rec_count);
      bank_of[(size_t)plane * num_layers + layer] = held ? next++ : -1;
    }
  ok();
  return next;
}

size_t pkv_pool_bytes(const pkv_pool *p) {
  if (!p || p->num_banks <= 0 || p->num_pages <= 0) return 0;
  return (size_t)p->num_banks * p->num_pages * p->num_kv_heads * p->page_size * p->head_dim *
         elem_bytes(p->dtype);
}

int paged_kv_write(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *k,
                   const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                   void *stream) {
  pkv::Bank bank;
  int rc = resolve_bank(pool, plane_id, layer_id, &bank);
  if (rc) return rc;
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(PKV_EINVAL, "k / v / slot_mapping is NULL");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(PKV_EINVAL, "k and v must be 16-byte aligned");
  return launched(pkv::launch_kv_write(bank, k, v, slot_mapping, num_tokens,
                                       static_cast<hipStream_t>(stream)),
                  "paged_kv_write");
}

size_t paged_decode_workspace_bytes(const pkv_pool *pool, int32_t batch, int32_t num_q_heads,
                                    int32_t max_seq_len, int32_t partition) {
  if (!pool || batch <= 0 || num_q_heads <= 0 || pool->num_kv_heads <= 0 ||
      num_q_heads % pool->num_kv_heads != 0 || pool->head_dim <= 0 || max_seq_len < 0 ||
      partition < 0)
    return 0;
  const size_t D = (size_t)pool->head_dim;
  const size_t G = (size_t)(num_q_heads / pool->num_kv_heads);
  const Mode mode = decode_mode(batch, pool->num_kv_heads, max_seq_len, partition);
  // Segment partials: two (m, l, acc) slots per wave and head of the group.
  auto seg = [&](int64_t nw) {
    const size_t slots = (size_t)nw * 2 * G;
    return align_up(slots * 2 * sizeof(float)) + align_up(slots * D * sizeof(float));
  };
  if (mode == Mode::kStream) return seg(stream_wave_count(pool, batch, num_q_heads, max_seq_len));
  partition = fixed_partition(mode, max_seq_len, partition);
  const size_t parts = max_seq_len > 0 ? (size_t)(max_seq_len + partition - 1) / partition : 1;
  const size_t rows = (size_t)batch * num_q_heads;
  const size_t fixed =
      2 * align_up(rows * parts * sizeof(float)) + align_up(rows * parts * D * sizeof(float));
  if (mode != Mode::kFixed) return fixed;
  // the streamed kernel's segment partials share the space
  return std::max(fixed, seg(parts_wave_count(pool, batch, num_q_heads, max_seq_len,
                                              (int64_t)parts)));
}

namespace {

int decode_impl(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *k_new,
                const void *v_new, const void *q, int32_t num_q_heads,
                const int32_t *page_table, int32_t page_table_stride, const int32_t *seq_lens,
                int32_t batch, int32_t max_seq_len, float scale, int32_t partition, void *out,
                float *lse, void *workspace, size_t workspace_bytes, void *stream,
                const pkv::LatestArgs *latest = nullptr,
                int (*scratch)(void **) = nullptr) {
  pkv::Bank bank;
  int rc = resolve_bank(pool, plane_id, layer_id, &bank);
  if (rc) return rc;
  if ((rc = check_heads(pool, num_q_heads))) return rc;
  if (batch <= 0) return fail(PKV_EINVAL, "batch %d <= 0", batch);
  if (!q || !page_table || !seq_lens || !out) return fail(PKV_EINVAL, "q / page_table / seq_lens / out is NULL");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(PKV_EINVAL, "q and out must be 16-byte aligned");
  if (page_table_stride <= 0) return fail(PKV_EINVAL, "page_table_stride %d <= 0", page_table_stride);
  if (max_seq_len < 0 || (int64_t)max_seq_len > (int64_t)page_table_stride * pool->page_size)
    return fail(PKV_EINVAL, "max_seq_len %d outside [0, stride * page_size = %lld]", max_seq_len,
                (long long)page_table_stride * pool->page_size);
  if (partition < 0 || partition % 16 != 0)
    return fail(PKV_EINVAL, "partition %d must be 0 or a positive multiple of 16", partition);
  const size_t need = paged_decode_workspace_bytes(pool, batch, num_q_heads, max_seq_len,
                                                   partition);
  if (scratch) {
    // The library's own scratch array: bounded, looked up only once every
    // argument has been validated.
    if (workspace_bytes < need)
      return fail(PKV_EWORKSPACE,
                  "these sizes need %zu bytes of split-K scratch, more than the library's %zu "
                  "(use paged_decode_attn with a workspace)",
                  need, workspace_bytes);
    if ((rc = scratch(&workspace))) return rc;
  }
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  const Mode mode = decode_mode(batch, pool->num_kv_heads, max_seq_len, partition);
  const bool stream_mode = mode == Mode::kStream;
  if (!stream_mode) partition = fixed_partition(mode, max_seq_len, partition);
  const int32_t max_parts =
      stream_mode || max_seq_len == 0 ? 1 : (max_seq_len + partition - 1) / partition;
  if (max_parts > 65535) return fail(PKV_EINVAL, "too many partitions (%d)", max_parts);

  pkv::DecodeArgs a{};
  a.bank = bank;
  a.q = q;
  a.num_q_heads = num_q_heads;
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.scale = scale;
  a.partition = partition;
  a.max_parts = max_parts;
  a.out = out;
  a.lse = lse;
  a.k_new = k_new;
  a.v_new = v_new;
  a.num_cus = device_cus();
  if (latest) a.latest = *latest;
  char *ws = static_cast<char *>(workspace);
  if (stream_mode) {
    const int64_t nw = stream_wave_count(pool, batch, num_q_heads, max_seq_len);
    const size_t slots = (size_t)nw * 2 * (num_q_heads / pool->num_kv_heads);
    a.part_m = reinterpret_cast<float *>(ws);
    a.part_acc = reinterpret_cast<float *>(ws + align_up(slots * 2 * sizeof(float)));
    return launched(pkv::launch_decode_stream(a, nw, static_cast<hipStream_t>(stream)),
                    "decode");
  }
  const size_t rows = (size_t)batch * num_q_heads;
  const size_t ml = align_up(rows * max_parts * sizeof(float));
  // streamed fixed partitions index the call's partitions with 32-bit sums
  if (mode == Mode::kFixed && (int64_t)batch * pool->num_kv_heads * max_parts <= INT32_MAX)
    a.nw = parts_wave_count(pool, batch, num_q_heads, max_seq_len, max_parts);
  a.part_m = reinterpret_cast<float *>(ws);
  a.part_l = reinterpret_cast<float *>(ws + ml);
  a.part_acc = reinterpret_cast<float *>(ws + 2 * ml);
  return launched(pkv::launch_decode(a, static_cast<hipStream_t>(stream)), "decode");
}

}  // namespace

int paged_decode_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *q,
                      int32_t num_q_heads, const int32_t *page_table, int32_t page_table_stride,
                      const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, float scale,
                      int32_t partition, void *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return decode_impl(pool, plane_id, layer_id, nullptr, nullptr, q, num_q_heads, page_table,
                     page_table_stride, seq_lens, batch, max_seq_len, scale, partition, out, lse,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

int pkv::decode_scratch(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *q,
                        int32_t num_q_heads, const int32_t *page_table,
                        int32_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                        int32_t max_seq_len, float scale, int32_t partition, void *out,
                        float *lse, int (*scratch)(void **), size_t scratch_bytes,
                        void *stream) {
  return decode_impl(pool, plane_id, layer_id, nullptr, nullptr, q, num_q_heads, page_table,
                     page_table_stride, seq_lens, batch, max_seq_len, scale, partition, out, lse,
                     nullptr, scratch_bytes, stream, nullptr, scratch);
}

extern "C" {

int paged_decode_append_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                             const void *k_new, const void *v_new, const void *q,
                             int32_t num_q_heads, const int32_t *page_table,
                             int32_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                             int32_t max_seq_len, float scale, int32_t partition, void *out,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  if (!k_new || !v_new) return fail(PKV_EINVAL, "k_new / v_new is NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  return decode_impl(pool, plane_id, layer_id, k_new, v_new, q, num_q_heads, page_table,
                     page_table_stride, seq_lens, batch, max_seq_len, scale, partition, out, lse,
                     workspace, workspace_bytes, stream);
}

int paged_decode_step(const pkv_pool *pool, int32_t num_calls, const int32_t *plane_ids,
                      const int32_t *layer_ids, const void *const *k_new,
                      const void *const *v_new, const void *const *q, int32_t num_q_heads,
                      const int32_t *page_table, int32_t page_table_stride,
                      const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, float scale,
                      int32_t partition, void *const *out, float *const *lse, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (num_calls < 0) return fail(PKV_EINVAL, "num_calls %d < 0", num_calls);
  if (num_calls == 0) return ok();
  if (!plane_ids || !layer_ids || !q || !out)
    return fail(PKV_EINVAL, "plane_ids / layer_ids / q / out is NULL");
  if (!k_new != !v_new) return fail(PKV_EINVAL, "k_new and v_new must both be given or both NULL");
  // Validate every call before enqueuing any (all or nothing).
  for (int32_t i = 0; i < num_calls; ++i) {
    pkv::Bank bank;
    int rc = resolve_bank(pool, plane_ids[i], layer_ids[i], &bank);
    if (rc) return fail_call(rc, i);
    if (!q[i] || !out[i]) return fail(PKV_EINVAL, "call %d: q / out is NULL", i);
    if ((reinterpret_cast<uintptr_t>(q[i]) | reinterpret_cast<uintptr_t>(out[i])) & 15)
      return fail(PKV_EINVAL, "call %d: q and out must be 16-byte aligned", i);
    if (k_new && (!k_new[i] || !v_new[i]))
      return fail(PKV_EINVAL, "call %d: k_new / v_new is NULL", i);
    if (k_new && ((reinterpret_cast<uintptr_t>(k_new[i]) | reinterpret_cast<uintptr_t>(v_new[i])) & 15))
      return fail(PKV_EINVAL, "call %d: k_new and v_new must be 16-byte aligned", i);
  }
  for (int32_t i = 0; i < num_calls; ++i) {
    const int rc = decode_impl(pool, plane_ids[i], layer_ids[i], k_new ? k_new[i] : nullptr,
                               v_new ? v_new[i] : nullptr, q[i], num_q_heads, page_table,
                               page_table_stride, seq_lens, batch, max_seq_len, scale, partition,
                               out[i], lse ? lse[i] : nullptr, workspace, workspace_bytes, stream);
    if (rc) return fail_call(rc, i);
  }
  return ok();
}

struct pkv_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

int paged_decode_step_capture(const pkv_pool *pool, int32_t num_calls, const int32_t *plane_ids,
                              const int32_t *layer_ids, const void *const *k_new,
                              const void *const *v_new, const void *const *q,
                              int32_t num_q_heads, const int32_t *page_table,
                              int32_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                              int32_t max_seq_len, float scale, int32_t partition,
                              void *const *out, float *const *lse, void *workspace,
                              size_t workspace_bytes, void *capture_stream,
                              pkv_step_graph **graph) {
  if (!graph) return fail(PKV_EINVAL, "graph is NULL");
  *graph = nullptr;
  if (!capture_stream) return fail(PKV_EINVAL, "capture_stream must not be the null stream");
  hipStream_t cs = static_cast<hipStream_t>(capture_stream);
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return fail(PKV_ELAUNCH, "hipStreamBeginCapture failed");
  int rc = paged_decode_step(pool, num_calls, plane_ids, layer_ids, k_new, v_new, q, num_q_heads,
                             page_table, page_table_stride, seq_lens, batch, max_seq_len, scale,
                             partition, out, lse, workspace, workspace_bytes, capture_stream);
  char saved[sizeof g_err];
  memcpy(saved, g_err, sizeof saved);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(cs, &g);
  if (rc) {
    if (g) (void)hipGraphDestroy(g);
    memcpy(g_err, saved, sizeof saved);
    return rc;
  }
  if (e != hipSuccess || !g)
    return fail(PKV_ELAUNCH, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  hipGraphExec_t x = nullptr;
  const hipError_t ei = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (ei != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(PKV_ELAUNCH, "hipGraphInstantiate failed: %s", hipGetErrorString(ei));
  }
  *graph = new (std::nothrow) pkv_step_graph{g, x};
  if (!*graph) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return fail(PKV_ELAUNCH, "out of host memory");
  }
  return ok();
}

int paged_decode_step_graph_launch(pkv_step_graph *graph, void *stream) {
  if (!graph) return fail(PKV_EINVAL, "graph is NULL");
  const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ELAUNCH, "hipGraphLaunch failed: %s", hipGetErrorString(e));
  return ok();
}

void paged_decode_step_graph_destroy(pkv_step_graph *graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
}

int paged_decode_latest_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                             const int8_t *exit_depth, int32_t exit_stride, const void *k_new,
                             const void *v_new, const void *q, int32_t num_q_heads,
                             const int32_t *page_table, int32_t page_table_stride,
                             const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                             float scale, int32_t partition, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream) {
  pkv::Bank bank;
  int rc = resolve_bank(pool, plane_id, layer_id, &bank);
  if (rc) return rc;
  if (!exit_depth) return fail(PKV_EINVAL, "exit_depth is NULL");
  if (reinterpret_cast<uintptr_t>(exit_depth) & 15)
    return fail(PKV_EINVAL, "exit_depth must be 16-byte aligned");
  if (exit_stride <= 0 || exit_stride % 16 != 0 || exit_stride < (max_seq_len + 15) / 16 * 16)
    return fail(PKV_EINVAL, "exit_stride %d must be a multiple of 16 covering max_seq_len %d",
                exit_stride, max_seq_len);
  if (!k_new != !v_new) return fail(PKV_EINVAL, "k_new and v_new must both be given or both NULL");
  if (k_new && ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15))
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  // Every plane up to the query's must hold the layer; the banks of planes
  // 1..plane_id must be evenly spaced (true of every per-plane map).
  const int32_t *row = pool->bank_of;
  auto bank_at = [&](int32_t p) { return row[(size_t)p * pool->num_layers + layer_id]; };
  for (int32_t p = 0; p <= plane_id; ++p)
    if (bank_at(p) < 0 || bank_at(p) >= pool->num_banks)
      return fail(PKV_ENOTHELD, "plane %d does not hold layer %d", p, layer_id);
  for (int32_t p = 3; p <= plane_id; ++p)
    if (bank_at(p) - bank_at(p - 1) != bank_at(2) - bank_at(1))
      return fail(PKV_EUNSUPPORTED, "banks of layer %d are not evenly spaced over planes 1..%d",
                  layer_id, plane_id);
  const int64_t bank_bytes = (int64_t)pool->num_pages * pool->num_kv_heads * pool->page_size *
                             pool->head_dim * elem_bytes(pool->dtype);
  pkv::LatestArgs la{};
  la.depth = reinterpret_cast<const uint8_t *>(exit_depth);
  la.stride = exit_stride;
  la.plane = plane_id;
  la.d0 = (int64_t)(bank_at(0) - bank_at(plane_id)) * bank_bytes;
  la.d1 = plane_id >= 1 ? (int64_t)(bank_at(1) - bank_at(plane_id)) * bank_bytes : 0;
  la.step = plane_id >= 2 ? (int64_t)(bank_at(2) - bank_at(1)) * bank_bytes : 0;
  return decode_impl(pool, plane_id, layer_id, k_new, v_new, q, num_q_heads, page_table,
                     page_table_stride, seq_lens, batch, max_seq_len, scale, partition, out, lse,
                     workspace, workspace_bytes, stream, &la);
}

int paged_decode_split_mode(const pkv_pool *pool, int32_t batch, int32_t num_q_heads,
                            int32_t max_seq_len, int32_t partition) {
  if (!pool || pool->num_kv_heads <= 0 || batch <= 0 || num_q_heads <= 0 || partition < 0)
    return fail(PKV_EINVAL, "bad sizes");
  switch (decode_mode(batch, pool->num_kv_heads, max_seq_len, partition)) {
    case Mode::kWhole: return 0;
    case Mode::kStream: return 1;
    case Mode::kFixed: return 2;
  }
  return 2;
}

int paged_decode_reduce(int32_t dtype, int32_t batch, int32_t num_q_heads, int32_t head_dim,
                        const int32_t *seq_lens, int32_t partition, int32_t max_parts,
                        const float *part_m, const float *part_l, const float *part_acc,
                        void *out, float *lse, void *stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim %d", head_dim);
  if (batch <= 0 || num_q_heads <= 0 || partition <= 0 || max_parts <= 0)
    return fail(PKV_EINVAL, "sizes must be positive");
  if (!seq_lens || !part_m || !part_l || !part_acc || !out)
    return fail(PKV_EINVAL, "NULL pointer");
  const int64_t max_seq = (int64_t)partition * max_parts;
  return launched(pkv::launch_reduce(dtype, batch, num_q_heads, head_dim, seq_lens,
                                     (int32_t)(max_seq > 0x7fffffff ? 0x7fffffff : max_seq),
                                     partition, max_parts, part_m, part_l, part_acc, out, lse,
                                     false, static_cast<hipStream_t>(stream)),
                  "paged_decode_reduce");
}

namespace {

// Validates a prefill call and fills its launch arguments (nothing enqueued).
int prefill_args(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *q,
                 int32_t num_q_heads, const int32_t *cu_q_lens, int32_t total_q,
                 const int32_t *page_table, int32_t page_table_stride, const int32_t *seq_lens,
                 int32_t batch, int32_t max_q_len, int32_t max_seq_len, float scale, void *out,
                 float *lse, pkv::PrefillArgs *a) {
  pkv::Bank bank;
  int rc = resolve_bank(pool, plane_id, layer_id, &bank);
  if (rc) return rc;
  if ((rc = check_heads(pool, num_q_heads))) return rc;
  if (batch <= 0) return fail(PKV_EINVAL, "batch %d <= 0", batch);
  if (total_q < 0) return fail(PKV_EINVAL, "total_q %d < 0", total_q);
  if (total_q == 0) return ok();
  if (!q || !cu_q_lens || !page_table || !seq_lens || !out)
    return fail(PKV_EINVAL, "q / cu_q_lens / page_table / seq_lens / out is NULL");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(PKV_EINVAL, "q and out must be 16-byte aligned");
  if (page_table_stride <= 0) return fail(PKV_EINVAL, "page_table_stride %d <= 0", page_table_stride);
  if (max_seq_len < 0 || (int64_t)max_seq_len > (int64_t)page_table_stride * pool->page_size)
    return fail(PKV_EINVAL, "max_seq_len %d outside [0, stride * page_size]", max_seq_len);
  if (max_q_len < 0 || max_q_len > max_seq_len)
    return fail(PKV_EINVAL, "max_q_len %d outside [0, max_seq_len]", max_q_len);
  *a = pkv::PrefillArgs{};
  a->bank = bank;
  a->q = q;
  a->num_q_heads = num_q_heads;
  a->cu_q_lens = cu_q_lens;
  a->total_q = total_q;
  a->page_table = page_table;
  a->pt_stride = page_table_stride;
  a->seq_lens = seq_lens;
  a->batch = batch;
  a->max_q_len = max_q_len;
  a->max_seq_len = max_seq_len;
  a->scale = scale;
  a->out = out;
  a->lse = lse;
  return ok();
}

}  // namespace

int paged_prefill_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *q,
                       int32_t num_q_heads, const int32_t *cu_q_lens, int32_t total_q,
                       const int32_t *page_table, int32_t page_table_stride,
                       const int32_t *seq_lens, int32_t batch, int32_t max_q_len,
                       int32_t max_seq_len, float scale, void *out, float *lse, void *stream) {
  pkv::PrefillArgs a;
  int rc = prefill_args(pool, plane_id, layer_id, q, num_q_heads, cu_q_lens, total_q, page_table,
                        page_table_stride, seq_lens, batch, max_q_len, max_seq_len, scale, out,
                        lse, &a);
  if (rc || total_q == 0) return rc;
  return launched(pkv::launch_prefill(a, static_cast<hipStream_t>(stream)), "paged_prefill_attn");
}

int paged_extend_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *k,
                      const void *v, const int32_t *slot_mapping, const void *q,
                      int32_t num_q_heads, const int32_t *cu_q_lens, int32_t total_q,
                      const int32_t *page_table, int32_t page_table_stride,
                      const int32_t *seq_lens, int32_t batch, int32_t max_q_len,
                      int32_t max_seq_len, float scale, void *out, float *lse, void *stream) {
  pkv::PrefillArgs a;
  int rc = prefill_args(pool, plane_id, layer_id, q, num_q_heads, cu_q_lens, total_q, page_table,
                        page_table_stride, seq_lens, batch, max_q_len, max_seq_len, scale, out,
                        lse, &a);
  if (rc || total_q == 0) return rc;
  if (!k || !v || !slot_mapping) return fail(PKV_EINVAL, "k / v / slot_mapping is NULL");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(PKV_EINVAL, "k and v must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launched(pkv::launch_kv_write(a.bank, k, v, slot_mapping, total_q, s), "paged_extend_attn");
  if (rc) return rc;
  return launched(pkv::launch_prefill(a, s), "paged_extend_attn");
}

const char *pkv_last_error(void) { return g_err; }

}  // extern "C"
