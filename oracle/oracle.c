/*
 * fp64 reference oracle for paged-KV attention over a multi-plane page pool.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. See oracle.h for
 * the pages each function follows and the readings taken where they are
 * silent. Everything here is the plain definition written out: gather the
 * context through the page table into contiguous arrays, then textbook
 * softmax attention in fp64. The only parallelism is an OpenMP loop over
 * independent (request, kv head) pairs; no arithmetic is blocked, fused or
 * reordered.
 *
 * Parity pins (in the CPU test suite): brute-force dense masked attention on
 * the logical (never paged) K/V, closed forms (V = 1, K = 0, one key,
 * hand-computed two-key weights), and invariants (page permutation, page
 * size, shared vs copied prefix pages, chunking, decode == prefill with one
 * row, GQA == MHA with repeated heads, plane isolation, split/combine).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Decode one stored element exactly. bf16 is the top half of an IEEE fp32,
 * so shifting its 16 bits left by 16 gives that fp32 exactly. */
static double load_elem(int32_t elem_bytes, const void *base, size_t idx) {
  if (elem_bytes == 4) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Element index of pool[bank][page][kv_head][offset][dim]. */
static size_t pool_index(const orc_pool *p, int32_t bank, int32_t page,
                         int32_t kvh, int32_t off, int32_t d) {
  size_t i = (size_t)bank;
  i = i * (size_t)p->num_pages + (size_t)page;
  i = i * (size_t)p->num_kv_heads + (size_t)kvh;
  i = i * (size_t)p->page_size + (size_t)off;
  i = i * (size_t)p->head_dim + (size_t)d;
  return i;
}

static int check_pool(const orc_pool *p) {
  if (!p || !p->k || !p->v || !p->bank_of) return ORC_EINVAL;
  if (p->elem_bytes != 4 && p->elem_bytes != 2) return ORC_EINVAL;
  if (p->page_size <= 0 || p->num_pages <= 0 || p->num_kv_heads <= 0 ||
      p->head_dim <= 0 || p->num_planes <= 0 || p->num_layers <= 0 ||
      p->num_banks <= 0)
    return ORC_EINVAL;
  return ORC_OK;
}

/* Bank owned by (plane, layer), per the per-plane layer map. */
static int bank_for(const orc_pool *p, int32_t plane, int32_t layer) {
  if (plane < 0 || plane >= p->num_planes || layer < 0 ||
      layer >= p->num_layers)
    return ORC_EINVAL;
  int32_t b = p->bank_of[plane * p->num_layers + layer];
  if (b < 0) return ORC_ENOTHELD;
  if (b >= p->num_banks) return ORC_EINVAL;
  return b;
}

int orc_bank_map(int32_t num_planes, int32_t num_layers, int32_t rec_first,
                 int32_t rec_count, int32_t *bank_of) {
  if (num_planes <= 0 || num_layers <= 0 || rec_first < 0 || rec_count < 0 ||
      rec_first + rec_count > num_layers || !bank_of)
    return ORC_EINVAL;
  int32_t next = 0;
  /* Depth 0 holds every layer. */
  for (int32_t l = 0; l < num_layers; ++l) bank_of[l] = next++;
  /* Deeper planes hold only the recurrent layers, in plane-major order. */
  for (int32_t t = 1; t < num_planes; ++t)
    for (int32_t l = 0; l < num_layers; ++l) {
      int held = (l >= rec_first && l < rec_first + rec_count);
      bank_of[t * num_layers + l] = held ? next++ : -1;
    }
  return next;
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

int orc_kv_write(const orc_pool *p, int32_t plane, int32_t layer,
                 const void *k, const void *v, const int32_t *slots,
                 int32_t T) {
  int rc = check_pool(p);
  if (rc) return rc;
  if (T < 0 || (T > 0 && (!k || !v || !slots))) return ORC_EINVAL;
  int bank = bank_for(p, plane, layer);
  if (bank < 0) return bank;

  /* Preconditions: every slot inside the pool, no slot twice. */
  int64_t cap = (int64_t)p->num_pages * p->page_size;
  int32_t *sorted = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  if (!sorted) return ORC_EINVAL;
  int32_t n = 0;
  for (int32_t t = 0; t < T; ++t) {
    if (slots[t] < 0) continue; /* padding row */
    if ((int64_t)slots[t] >= cap) { free(sorted); return ORC_ESLOT; }
    sorted[n++] = slots[t];
  }
  qsort(sorted, (size_t)n, sizeof(int32_t), cmp_i32);
  for (int32_t i = 1; i < n; ++i)
    if (sorted[i] == sorted[i - 1]) { free(sorted); return ORC_EDUP; }
  free(sorted);

  /* The scatter: token t, head h goes to page s / P, offset s % P. */
  size_t eb = (size_t)p->elem_bytes, row = (size_t)p->head_dim * eb;
  for (int32_t t = 0; t < T; ++t) {
    int32_t s = slots[t];
    if (s < 0) continue;
    int32_t page = s / p->page_size, off = s % p->page_size;
    for (int32_t h = 0; h < p->num_kv_heads; ++h) {
      size_t dst = pool_index(p, bank, page, h, off, 0) * eb;
      size_t src = ((size_t)t * p->num_kv_heads + h) * row;
      memcpy((char *)p->k + dst, (const char *)k + src, row);
      memcpy((char *)p->v + dst, (const char *)v + src, row);
    }
  }
  return ORC_OK;
}

/* Checks shared by the attention entry points. */
static int check_tables(const orc_pool *p, const int32_t *page_table,
                        int32_t pt_stride, const int32_t *seq_lens,
                        int32_t batch, const int32_t *cu_q_lens) {
  for (int32_t r = 0; r < batch; ++r) {
    int32_t n = seq_lens[r];
    if (n < 0 || (int64_t)n > (int64_t)pt_stride * p->page_size)
      return ORC_ELEN;
    int32_t npages = (n + p->page_size - 1) / p->page_size;
    for (int32_t i = 0; i < npages; ++i) {
      int32_t page = page_table[(size_t)r * pt_stride + i];
      if (page < 0 || page >= p->num_pages) return ORC_EPAGE;
    }
    if (cu_q_lens) {
      int32_t ql = cu_q_lens[r + 1] - cu_q_lens[r];
      if (ql < 0 || ql > n) return ORC_ELEN;
    }
  }
  if (cu_q_lens && cu_q_lens[0] != 0) return ORC_EINVAL;
  return ORC_OK;
}

/* Gather positions [0, n) of kv head kvh of request r into contiguous
 * Kc[n][D], Vc[n][D] (fp64): position pos lives at page pt[r][pos / P],
 * offset pos % P, of bank `bank` -- or, given the request's exit depths
 * (early-exit decode), of the bank of (min(plane, depth[pos]), layer).
 * Returns 0 or an error code. */
static int gather(const orc_pool *p, int32_t bank, const int8_t *depth,
                  int32_t plane, int32_t layer, const int32_t *pt_row,
                  int32_t kvh, int32_t n, double *Kc, double *Vc) {
  int32_t D = p->head_dim;
  for (int32_t pos = 0; pos < n; ++pos) {
    if (depth) {
      int32_t e = depth[pos];
      if (e < 0 || e >= p->num_planes) return ORC_EINVAL;
      bank = bank_for(p, e < plane ? e : plane, layer);
      if (bank < 0) return bank;
    }
    int32_t page = pt_row[pos / p->page_size];
    int32_t off = pos % p->page_size;
    for (int32_t d = 0; d < D; ++d) {
      size_t i = pool_index(p, bank, page, kvh, off, d);
      Kc[(size_t)pos * D + d] = load_elem(p->elem_bytes, p->k, i);
      Vc[(size_t)pos * D + d] = load_elem(p->elem_bytes, p->v, i);
    }
  }
  return ORC_OK;
}

/* Textbook softmax attention of one query over keys [lo, hi) of the gathered
 * context: s_k = scale * q.K_k, w_k = exp(s_k - max s), o = sum w_k V_k / sum w_k,
 * lse = max s + ln(sum w_k). Returns m, l and the unnormalised acc too, which
 * are the split-K partials when [lo, hi) is one partition. */
static void attend_span(const double *qv, const double *Kc, const double *Vc,
                        int32_t lo, int32_t hi, int32_t D, double scale,
                        double *w, double *m_out, double *l_out,
                        double *acc, double *o, double *lse) {
  for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
  if (hi <= lo) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    if (o) for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    if (lse) *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int32_t k = lo; k < hi; ++k) {
    double s = 0.0;
    for (int32_t d = 0; d < D; ++d) s += qv[d] * Kc[(size_t)k * D + d];
    w[k - lo] = scale * s;
    if (w[k - lo] > m) m = w[k - lo];
  }
  double l = 0.0;
  for (int32_t k = lo; k < hi; ++k) {
    w[k - lo] = exp(w[k - lo] - m);
    l += w[k - lo];
  }
  for (int32_t k = lo; k < hi; ++k)
    for (int32_t d = 0; d < D; ++d) acc[d] += w[k - lo] * Vc[(size_t)k * D + d];
  *m_out = m;
  *l_out = l;
  if (o) for (int32_t d = 0; d < D; ++d) o[d] = acc[d] / l;
  if (lse) *lse = m + log(l);
}

int orc_attend(const orc_pool *p, int32_t plane, int32_t layer,
               const void *q, int32_t Hq, const int32_t *cu_q_lens,
               const int32_t *page_table, int32_t pt_stride,
               const int32_t *seq_lens, int32_t batch, double scale,
               double *out, double *lse) {
  int rc = check_pool(p);
  if (rc) return rc;
  if (batch < 0 || Hq <= 0 || Hq % p->num_kv_heads != 0 || pt_stride < 0)
    return ORC_EINVAL;
  if (batch == 0) return ORC_OK;
  if (!q || !page_table || !seq_lens || !out || !lse) return ORC_EINVAL;
  int bank = bank_for(p, plane, layer);
  if (bank < 0) return bank;
  rc = check_tables(p, page_table, pt_stride, seq_lens, batch, cu_q_lens);
  if (rc) return rc;

  const int32_t D = p->head_dim, Hkv = p->num_kv_heads, G = Hq / Hkv;
  const int32_t pairs = batch * Hkv;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t pr = 0; pr < pairs; ++pr) {
    int32_t r = pr / Hkv, kvh = pr % Hkv;
    int32_t n = seq_lens[r];
    int32_t row0 = cu_q_lens ? cu_q_lens[r] : r;
    int32_t qlen = cu_q_lens ? cu_q_lens[r + 1] - cu_q_lens[r] : 1;
    size_t nn = (size_t)(n > 0 ? n : 1);
    double *Kc = (double *)malloc(nn * D * sizeof(double));
    double *Vc = (double *)malloc(nn * D * sizeof(double));
    double *w = (double *)malloc(nn * sizeof(double));
    double *qv = (double *)malloc((size_t)D * sizeof(double));
    double *acc = (double *)malloc((size_t)D * sizeof(double));
    if (!Kc || !Vc || !w || !qv || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
      gather(p, bank, NULL, plane, layer, page_table + (size_t)r * pt_stride, kvh, n, Kc, Vc);
      for (int32_t j = 0; j < qlen; ++j) {
        /* Query row j sits at position n - qlen + j and sees keys 0..pos. */
        int32_t pos = n - qlen + j;
        int32_t row = row0 + j;
        for (int32_t g = 0; g < G; ++g) {
          int32_t h = kvh * G + g;
          size_t qo = ((size_t)row * Hq + h) * D;
          for (int32_t d = 0; d < D; ++d) qv[d] = load_elem(p->elem_bytes, q, qo + d);
          double m, l;
          attend_span(qv, Kc, Vc, 0, pos + 1, D, scale, w, &m, &l, acc,
                      out + qo, lse + (size_t)row * Hq + h);
        }
      }
    }
    free(Kc); free(Vc); free(w); free(qv); free(acc);
  }
  return failed ? ORC_EINVAL : ORC_OK;
}

int orc_decode_latest(const orc_pool *p, int32_t plane, int32_t layer,
                      const int8_t *exit_depth, int32_t exit_stride,
                      const void *q, int32_t Hq,
                      const int32_t *page_table, int32_t pt_stride,
                      const int32_t *seq_lens, int32_t batch, double scale,
                      double *out, double *lse) {
  int rc = check_pool(p);
  if (rc) return rc;
  if (batch < 0 || Hq <= 0 || Hq % p->num_kv_heads != 0 || pt_stride < 0)
    return ORC_EINVAL;
  if (batch == 0) return ORC_OK;
  if (!q || !page_table || !seq_lens || !out || !lse || !exit_depth) return ORC_EINVAL;
  int bank = bank_for(p, plane, layer);
  if (bank < 0) return bank;
  rc = check_tables(p, page_table, pt_stride, seq_lens, batch, NULL);
  if (rc) return rc;
  for (int32_t r = 0; r < batch; ++r)
    if (seq_lens[r] > exit_stride) return ORC_ELEN;

  const int32_t D = p->head_dim, Hkv = p->num_kv_heads, G = Hq / Hkv;
  const int32_t pairs = batch * Hkv;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t pr = 0; pr < pairs; ++pr) {
    int32_t r = pr / Hkv, kvh = pr % Hkv;
    int32_t n = seq_lens[r];
    size_t nn = (size_t)(n > 0 ? n : 1);
    double *Kc = (double *)malloc(nn * D * sizeof(double));
    double *Vc = (double *)malloc(nn * D * sizeof(double));
    double *w = (double *)malloc(nn * sizeof(double));
    double *qv = (double *)malloc((size_t)D * sizeof(double));
    double *acc = (double *)malloc((size_t)D * sizeof(double));
    int err = (!Kc || !Vc || !w || !qv || !acc) ? ORC_EINVAL : ORC_OK;
    if (!err)
      err = gather(p, bank, exit_depth + (size_t)r * exit_stride, plane, layer,
                   page_table + (size_t)r * pt_stride, kvh, n, Kc, Vc);
    if (err) {
#pragma omp critical
      failed = failed ? failed : err;
    } else {
      for (int32_t g = 0; g < G; ++g) {
        int32_t h = kvh * G + g;
        size_t qo = ((size_t)r * Hq + h) * D;
        for (int32_t d = 0; d < D; ++d) qv[d] = load_elem(p->elem_bytes, q, qo + d);
        double m, l;
        attend_span(qv, Kc, Vc, 0, n, D, scale, w, &m, &l, acc, out + qo,
                    lse + (size_t)r * Hq + h);
      }
    }
    free(Kc); free(Vc); free(w); free(qv); free(acc);
  }
  return failed;
}

int orc_decode_partials(const orc_pool *p, int32_t plane, int32_t layer,
                        const void *q, int32_t Hq,
                        const int32_t *page_table, int32_t pt_stride,
                        const int32_t *seq_lens, int32_t batch, double scale,
                        int32_t partition, int32_t max_parts,
                        double *pm, double *pl, double *pacc) {
  int rc = check_pool(p);
  if (rc) return rc;
  if (batch < 0 || Hq <= 0 || Hq % p->num_kv_heads != 0 || partition <= 0 ||
      max_parts <= 0)
    return ORC_EINVAL;
  if (batch == 0) return ORC_OK;
  if (!q || !page_table || !seq_lens || !pm || !pl || !pacc) return ORC_EINVAL;
  int bank = bank_for(p, plane, layer);
  if (bank < 0) return bank;
  rc = check_tables(p, page_table, pt_stride, seq_lens, batch, NULL);
  if (rc) return rc;
  for (int32_t r = 0; r < batch; ++r)
    if ((int64_t)seq_lens[r] > (int64_t)partition * max_parts) return ORC_ELEN;

  const int32_t D = p->head_dim, Hkv = p->num_kv_heads, G = Hq / Hkv;
  const int32_t pairs = batch * Hkv;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t pr = 0; pr < pairs; ++pr) {
    int32_t r = pr / Hkv, kvh = pr % Hkv;
    int32_t n = seq_lens[r];
    size_t nn = (size_t)(n > 0 ? n : 1);
    double *Kc = (double *)malloc(nn * D * sizeof(double));
    double *Vc = (double *)malloc(nn * D * sizeof(double));
    double *w = (double *)malloc(nn * sizeof(double));
    double *qv = (double *)malloc((size_t)D * sizeof(double));
    if (!Kc || !Vc || !w || !qv) {
#pragma omp atomic write
      failed = 1;
    } else {
      gather(p, bank, NULL, plane, layer, page_table + (size_t)r * pt_stride, kvh, n, Kc, Vc);
      for (int32_t g = 0; g < G; ++g) {
        int32_t h = kvh * G + g;
        size_t qo = ((size_t)r * Hq + h) * D;
        for (int32_t d = 0; d < D; ++d) qv[d] = load_elem(p->elem_bytes, q, qo + d);
        for (int32_t j = 0; j < max_parts; ++j) {
          int32_t lo = j * partition;
          int32_t hi = lo + partition < n ? lo + partition : n;
          size_t i = ((size_t)r * Hq + h) * max_parts + j;
          attend_span(qv, Kc, Vc, lo, hi, D, scale, w, pm + i, pl + i,
                      pacc + i * D, NULL, NULL);
        }
      }
    }
    free(Kc); free(Vc); free(w); free(qv);
  }
  return failed ? ORC_EINVAL : ORC_OK;
}

int orc_combine(int32_t rows, int32_t max_parts, int32_t D,
                const int32_t *n_parts, const double *pm, const double *pl,
                const double *pacc, double *out, double *lse) {
  if (rows < 0 || max_parts <= 0 || D <= 0) return ORC_EINVAL;
  if (rows == 0) return ORC_OK;
  if (!n_parts || !pm || !pl || !pacc || !out || !lse) return ORC_EINVAL;
  for (int32_t i = 0; i < rows; ++i)
    if (n_parts[i] < 0 || n_parts[i] > max_parts) return ORC_EINVAL;
  for (int32_t i = 0; i < rows; ++i) {
    const double *m = pm + (size_t)i * max_parts;
    const double *l = pl + (size_t)i * max_parts;
    const double *a = pacc + (size_t)i * max_parts * D;
    double *o = out + (size_t)i * D;
    double M = -INFINITY;
    for (int32_t j = 0; j < n_parts[i]; ++j)
      if (m[j] > M) M = m[j];
    if (M == -INFINITY) {
      for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
      lse[i] = -INFINITY;
      continue;
    }
    double L = 0.0;
    for (int32_t j = 0; j < n_parts[i]; ++j) L += l[j] * exp(m[j] - M);
    for (int32_t d = 0; d < D; ++d) {
      double s = 0.0;
      for (int32_t j = 0; j < n_parts[i]; ++j)
        s += a[(size_t)j * D + d] * exp(m[j] - M);
      o[d] = s / L;
    }
    lse[i] = M + log(L);
  }
  return ORC_OK;
}
