/*
 * pagedkv -- paged-KV attention over a multi-plane page pool, for AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow two pages:
 *   [FFM]   "Faster fuzzy minds" (dibbla.space, fast_subconscious)
 *           - section "When scheduler does the work": the KV cache is a flat
 *             pool of fixed-size slots addressed through
 *             page_table[request, position]; a sequence's KV need not be
 *             contiguous and two sequences may point at the same slots;
 *             requests sharing a prompt prefix inherit its KV;
 *           - section "So why is this hard for latent / looped models?":
 *             each decode step appends one slot per request and runs one
 *             query per request;
 *           - section "LOTUS -- the one place I opened the scheduler":
 *             store_kv scatters each token's K/V to the slots it is handed
 *             (out_loc), so handing the same slots again overwrites in
 *             place; re-running a span is an extend-prefill;
 *           - section "Recurrent depth -- a deep model in a trench coat":
 *             loop iteration t of weight layer l writes its own KV bank
 *             t*L + l; a token keeps one position across all its banks.
 *   [PR152] vllm-rlt pull 152, "[Huginn] Opt-in prefix caching with
 *           position-keyed noise", section "Summary": each plane (loop
 *           depth) holds only the layers it runs -- all layers at depth 0,
 *           the recurrent layers deeper -- and banks are allocated only for
 *           held layers (section "Notes", item #147).
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every buffer. The library allocates no
 *     device memory and keeps no state between calls except a thread-local
 *     error string (and, for paged_decode_attn_noalloc, one fixed scratch
 *     array per GPU, placed when its code is loaded).
 *   - Asynchrony: device work is enqueued on `stream` (a hipStream_t passed
 *     as void*; NULL = the null stream) and the call returns without
 *     synchronising. Buffers must stay valid until the stream reaches the
 *     work.
 *   - Errors: a negative return means nothing was enqueued (except
 *     PKV_ELAUNCH, which reports a failed launch). pkv_last_error() then
 *     describes it. Device-resident tables (page ids, slots, seq_lens,
 *     cu_q_lens) are not read on the host; values outside their contract
 *     give unspecified results, but kernels clamp every index so that no
 *     access leaves the buffers described here.
 *
 * Pool layout (device memory, one array for K and one for V):
 *   element (bank, page, kv_head, offset, dim) of K is at
 *   k_base[(((bank * num_pages + page) * num_kv_heads + kv_head)
 *           * page_size + offset) * head_dim + dim]
 *   and likewise for V. Banks are plane-major (bank ids come from bank_of).
 *   A (page, kv_head) tile is page_size x head_dim contiguous elements
 *   (4 KiB for bf16 at head_dim 128 and page_size 16).
 *   Position pos of request r lives at page page_table[r * stride + pos /
 *   page_size], offset pos % page_size, in every bank: one page table and
 *   one slot mapping serve all planes and layers.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* null pointer, bad size or shape            */
  PKV_EUNSUPPORTED = -2,  /* dtype / head_dim / page_size / group size  */
  PKV_ENOTHELD = -3,      /* (plane, layer) owns no bank                */
  PKV_EWORKSPACE = -4,    /* workspace too small                        */
  PKV_ELAUNCH = -5,       /* a kernel launch failed                     */
  PKV_ENOSPACE = -6       /* page manager: not enough free pages        */
};

/* The pool descriptor. dtype is shared by the pool, q, k/v inputs and out.
 * Supported: page_size 16; head_dim 64 or 128; num_q_heads / num_kv_heads
 * in {1, 2, 4, 8}. bank_of is a HOST array [num_planes * num_layers] whose
 * entry is the bank of (plane, layer) or -1 if the plane does not hold the
 * layer. k_base / v_base are DEVICE pointers to num_banks * num_pages *
 * num_kv_heads * page_size * head_dim elements each, 16-byte aligned. */
typedef struct {
  int32_t dtype;          /* pkv_dtype */
  int32_t page_size;
  int32_t num_pages;      /* pages per bank; ids in [0, num_pages) */
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_planes;
  int32_t num_layers;
  int32_t num_banks;
  const int32_t *bank_of; /* HOST */
  void *k_base;           /* DEVICE */
  void *v_base;           /* DEVICE */
} pkv_pool;

/* Per-plane layer map ([FFM] recurrent depth; [PR152] summary). Plane 0
 * holds every layer; planes >= 1 hold layers [rec_first, rec_first +
 * rec_count), packed in plane-major order. rec_first = 0 and rec_count =
 * num_layers gives bank = plane * num_layers + layer. Host only: fills the
 * caller's bank_of [num_planes * num_layers] and returns the bank count, or a
 * negative code. */
int pkv_bank_map(int32_t num_planes, int32_t num_layers, int32_t rec_first,
                 int32_t rec_count, int32_t *bank_of);

/* Bytes of one of the pool's two arrays (K or V) for this descriptor. Host only. */
size_t pkv_pool_bytes(const pkv_pool *pool);

/* store_kv ([FFM] LOTUS): for every token t with slot s = slot_mapping[t] >=
 * 0, copy k[t][h][:] and v[t][h][:] for every kv head h to page s / page_size,
 * offset s % page_size of bank bank_of[plane_id][layer_id]. A byte copy: k and
 * v are DEVICE [num_tokens][num_kv_heads][head_dim] in the pool dtype. A
 * negative slot is skipped (padding). Writing a slot again in a later call
 * overwrites it; the same slot twice in one call is unspecified; slots at or
 * past num_pages * page_size are skipped. num_tokens 0 enqueues nothing. */
int paged_kv_write(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                   const void *k, const void *v, const int32_t *slot_mapping,
                   int32_t num_tokens, void *stream);

/* Workspace bytes paged_decode_attn needs for these sizes on the current
 * device. Host only (it may query the device's compute-unit count and the
 * decode kernel's occupancy). 0 for invalid sizes. */
size_t paged_decode_workspace_bytes(const pkv_pool *pool, int32_t batch,
                                    int32_t num_q_heads, int32_t max_seq_len,
                                    int32_t partition);

/* Decode attention through the page table ([FFM] scheduler and looped-model
 * sections: one query per request, the KV read through page_table). For each
 * request r with n = seq_lens[r] and each q head h: the query q[r][h][:] sits
 * at position n - 1 and attends keys 0..n-1 of kv head h / (num_q_heads /
 * num_kv_heads) in bank bank_of[plane_id][layer_id]:
 *   out[r][h][:] = sum_k softmax_k(scale * q . K_k) V_k, lse[r][h] = ln sum_k exp(scale q.K_k).
 * Work split (the fp32 partials (m, l, acc) of a split context are folded in
 * position order by a combine kernel, so results are bitwise repeatable and
 * independent of physical page placement):
 *   partition > 0 (a multiple of 16): fixed partitions of that many tokens.
 *     Each partition is folded from a fresh state, and a row's partitions
 *     are combined in partition order with the fp32 merge (rescale each to
 *     the larger max). When a partition holds a whole number of the fold's
 *     steps (two pages for bf16 head_dim 128 with GQA groups 4 and 8, one
 *     page otherwise) and batch <= 4096, a persistent grid deals the
 *     partitions to its waves in equal contiguous ranges and merges each
 *     row's partitions in registers (rows split between waves are finished
 *     by a combine kernel); otherwise one workgroup per (partition, kv head,
 *     request) writes partials that a reduction combines as
 *     paged_decode_reduce does.
 *   partition 0 (library default), chosen per call:
 *     - whole contexts, one workgroup per (request, kv head), when
 *       batch * num_kv_heads >= 512 and max_seq_len <= 4096 (no partials,
 *       no combine);
 *     - otherwise a balanced split: the (request, kv head, page) sequence is
 *       cut into one equal contiguous range per wave of the grid, so every
 *       wave streams the same number of pages whatever the spread of
 *       lengths (falls back to partition 512 when batch > 4096).
 * Calls that share a workspace must not run concurrently.
 *   q:          DEVICE [batch][num_q_heads][head_dim], pool dtype
 *   page_table: DEVICE int32 [batch][page_table_stride] page ids
 *   seq_lens:   DEVICE int32 [batch], each in [0, max_seq_len]
 *   max_seq_len: HOST bound, <= page_table_stride * page_size
 *   out:        DEVICE [batch][num_q_heads][head_dim], pool dtype (RNE from fp32)
 *   lse:        DEVICE fp32 [batch][num_q_heads] natural log, or NULL
 *   workspace:  DEVICE scratch, >= paged_decode_workspace_bytes(...) bytes
 * seq_len 0 gives out 0 and lse -inf. */
int paged_decode_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                      const void *q, int32_t num_q_heads,
                      const int32_t *page_table, int32_t page_table_stride,
                      const int32_t *seq_lens, int32_t batch,
                      int32_t max_seq_len, float scale, int32_t partition,
                      void *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream);

/* paged_decode_attn for callers that cannot allocate device memory: code
 * under HIP stream capture, tight serving loops, harnesses that forbid
 * allocation. It takes no workspace; the split-K partials go to a
 * library-held device array of PKV_SCRATCH_BYTES on each GPU (placed when
 * the library's code is loaded on that GPU, held until the process ends).
 * The call allocates nothing. Every other argument, the results and the
 * errors are those of paged_decode_attn, and the results are bitwise equal
 * to paged_decode_attn's with a workspace of its own. Sizes whose
 * paged_decode_workspace_bytes exceeds PKV_SCRATCH_BYTES return
 * PKV_EWORKSPACE with nothing enqueued (e.g. many long contexts on small
 * fixed partitions). All calls on one GPU share its array, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams, other
 * host threads) race and give unspecified results; calls on one stream are
 * ordered and safe. */
#define PKV_SCRATCH_BYTES (32 << 20)
int paged_decode_attn_noalloc(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                              const void *q, int32_t num_q_heads, const int32_t *page_table,
                              int32_t page_table_stride, const int32_t *seq_lens,
                              int32_t batch, int32_t max_seq_len, float scale,
                              int32_t partition, void *out, float *lse, void *stream);

/* Which split paged_decode_attn takes for these sizes: 0 = whole contexts
 * (one workgroup per request and kv head), 1 = balanced split + combine,
 * 2 = fixed partitions (+ combine when a context spans several). Host only;
 * negative on invalid sizes. */
int paged_decode_split_mode(const pkv_pool *pool, int32_t batch, int32_t num_q_heads,
                            int32_t max_seq_len, int32_t partition);

/* One decode step of a layer in one call: store_kv of each request's newest
 * token followed by decode attention ([FFM] "So why is this hard...": a
 * decode step appends exactly one slot per request). For each request r with
 * n = seq_lens[r] > 0, k_new[r][h][:] and v_new[r][h][:] (DEVICE
 * [batch][num_kv_heads][head_dim], pool dtype, 16-byte aligned) are written
 * to position n - 1, i.e. page page_table[r][(n - 1) / 16], offset
 * (n - 1) % 16, of bank bank_of[plane_id][layer_id], and then attended
 * exactly as paged_decode_attn would after a paged_kv_write of the same rows:
 * the results and the pool contents are bitwise identical to that pair of
 * calls. The page holding position n - 1 must not be shared with another
 * request of the same call (the newest token's page is private). All other
 * arguments as for paged_decode_attn. */
int paged_decode_append_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                             const void *k_new, const void *v_new, const void *q,
                             int32_t num_q_heads, const int32_t *page_table,
                             int32_t page_table_stride, const int32_t *seq_lens,
                             int32_t batch, int32_t max_seq_len, float scale,
                             int32_t partition, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Decode with early exit: the "latest bank" ([FFM] "Can we actually stop
 * early?": when the recurrent state converges, a token that halted at depth
 * e keeps its depth-e KV, and later tokens attend that latest bank).
 * exit_depth is DEVICE int8 [batch][exit_stride]: exit_depth[r][pos] is the
 * deepest plane position pos of request r holds. The query of request r at
 * plane_id reads position pos of layer layer_id from plane
 * min(plane_id, exit_depth[r][pos]) -- the same page and slot in that
 * plane's bank -- and otherwise this is paged_decode_attn (k_new, v_new
 * NULL) or paged_decode_append_attn (k_new, v_new given; the newest token is
 * written to and read from plane_id's bank). Requirements (checked, nothing
 * enqueued otherwise): exit_depth 16-byte aligned; exit_stride a multiple of
 * 16 and >= max_seq_len; every plane 0..plane_id holds layer_id
 * (PKV_ENOTHELD), with the banks of planes 1..plane_id evenly spaced (true of
 * every pkv_bank_map layout; PKV_EUNSUPPORTED otherwise); GQA groups as for
 * paged_decode_attn (1, 2, 4, 8). Device depths are not validated: a depth
 * at or past plane_id (or negative) reads plane_id's own bank. */
int paged_decode_latest_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                             const int8_t *exit_depth, int32_t exit_stride, const void *k_new,
                             const void *v_new, const void *q, int32_t num_q_heads,
                             const int32_t *page_table, int32_t page_table_stride,
                             const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                             float scale, int32_t partition, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream);

/* One decode step of a looped model: the decode calls of every (plane,
 * layer) the step visits, in the given order, enqueued by one host call
 * ([FFM] "Recurrent depth": loop iteration t of layer l is one attention
 * call on bank t*L + l, and the loop runs inside the model's forward; [PR152]
 * "Notes" #148 submits a fixed-depth decode loop as one unit). Call i is
 * paged_decode_append_attn on (plane_ids[i], layer_ids[i]) with k_new[i],
 * v_new[i], q[i], out[i], lse[i] -- or paged_decode_attn when k_new and
 * v_new are NULL (the arrays themselves, not their entries). plane_ids,
 * layer_ids and the pointer arrays are HOST arrays of num_calls entries
 * (lse may be NULL: no lse for any call); every other argument is shared by
 * all calls and means what it means for paged_decode_attn. Every call is
 * validated before the first is enqueued. The calls run one after another
 * on `stream` and share the workspace. */
int paged_decode_step(const pkv_pool *pool, int32_t num_calls, const int32_t *plane_ids,
                      const int32_t *layer_ids, const void *const *k_new,
                      const void *const *v_new, const void *const *q, int32_t num_q_heads,
                      const int32_t *page_table, int32_t page_table_stride,
                      const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, float scale,
                      int32_t partition, void *const *out, float *const *lse, void *workspace,
                      size_t workspace_bytes, void *stream);

/* A decode step recorded once and replayed as one submission ([FFM] "When
 * scheduler does the work": a decode step has a fixed shape, so it is
 * captured once as a graph and replayed; [PR152] "Notes" #148: the decode
 * loop of a fixed-depth model as one submission). paged_decode_step_capture
 * records paged_decode_step with these arguments into a HIP graph (stream
 * capture on capture_stream, which must not be the null stream; nothing
 * runs during capture) and returns it in *graph. A launch replays the whole
 * step on `stream`, reading the device buffers' contents at replay time:
 * q, k_new, v_new, page_table and seq_lens may change between replays
 * (seq_lens within the captured max_seq_len), pointers and host sizes may
 * not. The graph holds HIP runtime objects (host memory, and whatever the
 * runtime allocates to instantiate it) until paged_decode_step_graph_destroy;
 * the device buffers stay the caller's. Replays that share a workspace must
 * not overlap. */
typedef struct pkv_step_graph pkv_step_graph;
int paged_decode_step_capture(const pkv_pool *pool, int32_t num_calls, const int32_t *plane_ids,
                              const int32_t *layer_ids, const void *const *k_new,
                              const void *const *v_new, const void *const *q,
                              int32_t num_q_heads, const int32_t *page_table,
                              int32_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                              int32_t max_seq_len, float scale, int32_t partition,
                              void *const *out, float *const *lse, void *workspace,
                              size_t workspace_bytes, void *capture_stream,
                              pkv_step_graph **graph);
int paged_decode_step_graph_launch(pkv_step_graph *graph, void *stream);
void paged_decode_step_graph_destroy(pkv_step_graph *graph);

/* The split-K combine for fixed partitions on its own (the second kernel of
 * paged_decode_attn with partition > 0, usable on partials gathered from
 * elsewhere, e.g. other devices). For each row i = r *
 * num_q_heads + h with n = seq_lens[r], combines partials j = 0 ..
 * ceil(n / partition) - 1 in order. Partials are in base-2 units: part_m =
 * log2(e) * (max score of the partition), part_l = sum 2^(log2(e) s - part_m),
 * part_acc = sum 2^(log2(e) s - part_m) V. Output:
 *   M = max_j m_j, L = sum_j l_j 2^(m_j - M), out = sum_j acc_j 2^(m_j - M) / L,
 *   lse = ln(2) (M + log2 L).
 * The arrays are laid out rows x max_parts [x head_dim].
 * A row with no partial gets out 0, lse -inf. */
int paged_decode_reduce(int32_t dtype, int32_t batch, int32_t num_q_heads,
                        int32_t head_dim, const int32_t *seq_lens,
                        int32_t partition, int32_t max_parts,
                        const float *part_m, const float *part_l,
                        const float *part_acc, void *out, float *lse,
                        void *stream);

/* Chunked causal prefill over paged context ([FFM] LOTUS: an extend-prefill;
 * [FFM] scheduler: a cache hit prefills only the suffix). Write-then-attend:
 * the chunk's own K/V must already be in the pool (paged_kv_write first).
 * Request r owns packed query rows cu_q_lens[r] .. cu_q_lens[r+1]-1; with
 * q_len = cu_q_lens[r+1] - cu_q_lens[r] and n = seq_lens[r] (context held
 * after this chunk, so q_len <= n), row j sits at position n - q_len + j and
 * attends keys 0..n - q_len + j (inclusive causal mask) of its kv head:
 *   q:          DEVICE [total_q][num_q_heads][head_dim], pool dtype
 *   cu_q_lens:  DEVICE int32 [batch + 1], cu_q_lens[0] = 0, cu_q_lens[batch] = total_q
 *   page_table, seq_lens: as for decode
 *   max_q_len, max_seq_len: HOST bounds on q_len and n
 *   out:        DEVICE [total_q][num_q_heads][head_dim]; lse fp32 [total_q][num_q_heads] or NULL
 * max_q_len also picks the kernel: with bf16 and head_dim 128, a call whose
 * max_q_len times the GQA group is at most 16 runs as one decode-style pass
 * per (request, kv head) (all its rows share one 16-column matrix-core
 * operand); longer chunks take 128-row query tiles on matrix cores. A q_len
 * above max_q_len is outside the contract (unspecified rows, no access
 * outside the buffers). */
int paged_prefill_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id,
                       const void *q, int32_t num_q_heads,
                       const int32_t *cu_q_lens, int32_t total_q,
                       const int32_t *page_table, int32_t page_table_stride,
                       const int32_t *seq_lens, int32_t batch,
                       int32_t max_q_len, int32_t max_seq_len, float scale,
                       void *out, float *lse, void *stream);

/* One extend pass over a span in one call ([FFM] "LOTUS": a pass over the
 * latent block writes the block's K/V to the slots it was handed -- the same
 * slots on every pass, so each pass overwrites the last in place -- and is
 * one parallel extend-prefill over all block positions). Exactly
 * paged_kv_write(k, v, slot_mapping, total_q tokens) followed by
 * paged_prefill_attn with the other arguments, on `stream`, with results
 * and pool bytes bitwise identical to that pair of calls:
 *   k, v:          DEVICE [total_q][num_kv_heads][head_dim], pool dtype,
 *                  16-byte aligned; row i is the K/V of packed query row i
 *   slot_mapping:  DEVICE int32 [total_q]; row i's slot, normally the slot
 *                  of its own position n - q_len + j (negative: not written)
 * Every argument is validated before anything is enqueued. */
int paged_extend_attn(const pkv_pool *pool, int32_t plane_id, int32_t layer_id, const void *k,
                      const void *v, const int32_t *slot_mapping, const void *q,
                      int32_t num_q_heads, const int32_t *cu_q_lens, int32_t total_q,
                      const int32_t *page_table, int32_t page_table_stride,
                      const int32_t *seq_lens, int32_t batch, int32_t max_q_len,
                      int32_t max_seq_len, float scale, void *out, float *lse, void *stream);

/* ------------------------------------------------------------------------
 * Host page manager (no device work). One page-id space serves every bank
 * ([FFM] "When scheduler does the work": slots are addressed through a page
 * table and sequences may share them; a shared prefix is inherited). Pages
 * carry reference counts -- a page is free again when its last reference is
 * released -- and the free count is O(1) ([PR152] "Notes" #151). A page may
 * be published as a reusable prefix page once every one of its slots has
 * been written in every layer that each plane in use holds ([PR152]
 * "Summary": coverage is checked per plane over the layers it holds, all
 * layers at depth 0 and the recurrent layers deeper). Not thread-safe: one
 * manager per scheduler thread. */
typedef struct pkv_page_mgr pkv_page_mgr;

/* A manager of num_pages pages of page_size slots (<= 64) for the plane map
 * bank_of [num_planes * num_layers] (HOST, copied; -1 = not held; each bank
 * id at most once). Every page starts free. NULL on invalid arguments. */
pkv_page_mgr *pkv_mgr_create(int32_t num_pages, int32_t page_size, int32_t num_planes,
                             int32_t num_layers, const int32_t *bank_of);
void pkv_mgr_destroy(pkv_page_mgr *mgr);
/* Free pages (constant time), or PKV_EINVAL for a NULL manager. */
int32_t pkv_mgr_free_count(const pkv_page_mgr *mgr);
/* Takes n free pages into page_ids[n] (HOST), each with one reference and no
 * slot marked written; all or nothing (PKV_ENOSPACE when fewer are free). */
int pkv_mgr_alloc(pkv_page_mgr *mgr, int32_t n, int32_t *page_ids);
/* One more reference to each listed page (a request that aliases a shared
 * prefix page); every page must be in use. All or nothing. */
int pkv_mgr_retain(pkv_page_mgr *mgr, int32_t n, const int32_t *page_ids);
/* Drops one reference per listed entry (an id may repeat); a page whose
 * count reaches 0 is free. All or nothing: no page may be released more
 * times than it is held. */
int pkv_mgr_release(pkv_page_mgr *mgr, int32_t n, const int32_t *page_ids);
/* References held on page (0 = free), or PKV_EINVAL. */
int32_t pkv_mgr_refcount(const pkv_page_mgr *mgr, int32_t page);
/* Records that store_kv wrote these slots (HOST [n], the slot_mapping of a
 * paged_kv_write; negative = padding, skipped) in bank (plane, layer).
 * PKV_ENOTHELD if the plane does not hold the layer; PKV_EINVAL for a slot
 * at or past num_pages * page_size (nothing recorded then). */
int pkv_mgr_note_write(pkv_page_mgr *mgr, int32_t plane, int32_t layer, int32_t n,
                       const int32_t *slots);
/* The number of leading pages of page_ids [n_pages] (a request's page-table
 * row) that may be published: in use, and every slot written in every layer
 * held by each of planes 0 .. planes_used - 1. Negative on invalid arguments. */
int32_t pkv_mgr_published_prefix(const pkv_page_mgr *mgr, int32_t planes_used,
                                 const int32_t *page_ids, int32_t n_pages);

/* The slots of a span of positions of each request ([FFM] "When scheduler
 * does the work": position pos of a request lives in slot page_table[r][pos /
 * page_size] * page_size + pos % page_size; [FFM] "LOTUS": a latent block's
 * slots are handed out once and every pass writes the same ones). Host only:
 * page_table [batch][stride], starts [batch] and slots [batch][span] are HOST
 * arrays. For r < batch and j < span, with pos = starts[r] + j:
 *   slots[r * span + j] = page_table[r * stride + pos / page_size] * page_size
 *                         + pos % page_size.
 * PKV_EINVAL, with nothing written, for a negative start, a span that runs
 * past stride * page_size, or a page id of the span outside [0, num_pages). */
int pkv_span_slots(const int32_t *page_table, int32_t stride, int32_t page_size,
                   int32_t num_pages, const int32_t *starts, int32_t batch, int32_t span,
                   int32_t *slots);

/* Message for the last non-zero return on this thread ("" if none). */
const char *pkv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
