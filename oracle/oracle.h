/*
 * Reference oracle for paged-KV attention over a multi-plane page pool.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain, fp64 CPU
 * definition that the GPU library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it. It shares no code, header or constant with
 * the GPU library.
 *
 * Sources (the pages this follows):
 *   [FFM]  "Faster fuzzy minds" (dibbla.space, fast_subconscious):
 *          section "When scheduler does the work" -- paged KV: a flat pool of
 *          fixed-size slots addressed through page_table[request, position];
 *          section "LOTUS -- the one place I opened the scheduler" -- store_kv
 *          scatters each token's K/V to the slots it is handed (out_loc), so
 *          handing the same slots again overwrites in place, and a span is
 *          re-run as an extend-prefill;
 *          section "Recurrent depth -- a deep model in a trench coat" --
 *          loop iteration t of weight layer l owns KV bank t*L + l, and one
 *          token keeps one position (hence one slot) across all banks.
 *   [PR152] "[Huginn] Opt-in prefix caching with position-keyed noise"
 *          (vllm-rlt pull 152), section "Summary" -- per-plane layer map:
 *          depth 0 holds every layer, deeper planes only the recurrent ones;
 *          section "Notes", item #147 -- packing those planes.
 *
 * Readings where the pages are silent (each is listed with its reason in
 * the project design notes):
 *   - page_table is page-granular: slot(r, pos) = pt[r][pos / P] * P + pos % P
 *     (equals the per-position table of [FFM] when P = 1);
 *   - pool layout: K and V are each [bank][page][kv_head][P][head_dim];
 *   - the decode query sits at position seq_len - 1 (seq_len counts the token
 *     just written); prefill row j of a request with q_len rows sits at
 *     seq_len - q_len + j; a query sees every key at a position <= its own;
 *   - q head h reads kv head h / (Hq / Hkv);
 *   - seq_len 0 gives out 0 and lse -inf;
 *   - a negative slot is skipped; a duplicate slot inside one write and an
 *     out-of-range slot or page id are errors.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_EINVAL = -1,     /* bad shape / pointer / dtype */
  ORC_ENOTHELD = -3,   /* (plane, layer) owns no bank */
  ORC_ESLOT = -10,     /* slot outside the pool */
  ORC_EDUP = -11,      /* same slot twice in one write */
  ORC_EPAGE = -12,     /* page id outside the pool */
  ORC_ELEN = -13       /* seq_len beyond the page-table row, or q_len > seq_len */
};

/* Host pool. elem_bytes 4 = fp32, 2 = bf16 (raw bits). k and v each hold
 * num_banks * num_pages * num_kv_heads * page_size * head_dim elements. */
typedef struct {
  int32_t elem_bytes;
  int32_t page_size;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_planes;
  int32_t num_layers;
  int32_t num_banks;
  const int32_t *bank_of;   /* [num_planes * num_layers], -1 = not held */
  void *k;
  void *v;
} orc_pool;

/* Per-plane layer map ([FFM] recurrent depth; [PR152] summary). Plane 0
 * holds every layer; planes >= 1 hold layers [rec_first, rec_first+rec_count).
 * rec_first = 0, rec_count = num_layers gives bank = plane*L + layer.
 * Writes bank_of and returns the bank count, or a negative code. */
int orc_bank_map(int32_t num_planes, int32_t num_layers, int32_t rec_first,
                 int32_t rec_count, int32_t *bank_of);

/* store_kv ([FFM] LOTUS): k, v are [T][Hkv][D] in the pool dtype. */
int orc_kv_write(const orc_pool *pool, int32_t plane, int32_t layer,
                 const void *k, const void *v, const int32_t *slots, int32_t T);

/* Attention over the gathered context. cu_q_lens == NULL means decode (one
 * query per request, q is [B][Hq][D]); otherwise q is packed
 * [cu_q_lens[B]][Hq][D]. out is [rows][Hq][D] fp64, lse is [rows][Hq]. */
int orc_attend(const orc_pool *pool, int32_t plane, int32_t layer,
               const void *q, int32_t num_q_heads, const int32_t *cu_q_lens,
               const int32_t *page_table, int32_t pt_stride,
               const int32_t *seq_lens, int32_t batch, double scale,
               double *out, double *lse);

/* Decode with early exit ([FFM] "Can we actually stop early?": a token that
 * halts at an earlier depth keeps its last, converged KV, and later tokens
 * attend that latest bank). exit_depth[r * exit_stride + pos] is the deepest
 * plane position pos of request r holds; the query of request r at plane
 * `plane` reads position pos from plane min(plane, exit_depth) of the same
 * layer, then attends exactly as decode does. Every such plane must hold
 * the layer (ORC_ENOTHELD otherwise); a depth outside [0, num_planes) is
 * ORC_EINVAL. */
int orc_decode_latest(const orc_pool *pool, int32_t plane, int32_t layer,
                      const int8_t *exit_depth, int32_t exit_stride,
                      const void *q, int32_t num_q_heads,
                      const int32_t *page_table, int32_t pt_stride,
                      const int32_t *seq_lens, int32_t batch, double scale,
                      double *out, double *lse);

/* Split-K partials of decode: partition j covers positions
 * [j*partition, min((j+1)*partition, seq_len)). Per (request, q head, j):
 * m = max score, l = sum exp(s - m), acc = sum exp(s - m) * v.
 * Arrays are [B][Hq][max_parts] (acc has a trailing [D]); a partition that
 * holds no position gets m = -inf, l = 0, acc = 0. */
int orc_decode_partials(const orc_pool *pool, int32_t plane, int32_t layer,
                        const void *q, int32_t num_q_heads,
                        const int32_t *page_table, int32_t pt_stride,
                        const int32_t *seq_lens, int32_t batch, double scale,
                        int32_t partition, int32_t max_parts,
                        double *pm, double *pl, double *pacc);

/* Combine n_parts[i] partials of each row i (rows = B*Hq): M = max m,
 * L = sum l*exp(m-M), out = sum acc*exp(m-M) / L, lse = M + ln L. */
int orc_combine(int32_t rows, int32_t max_parts, int32_t head_dim,
                const int32_t *n_parts, const double *pm, const double *pl,
                const double *pacc, double *out, double *lse);

#ifdef __cplusplus
}
#endif
#endif
