// Host-side page manager of the multi-plane pool: page allocation with
// reference counts for shared prefix pages, a constant-time free count, and
// per-plane prefix publication.
//
// Pages are one id space shared by every bank ("Faster fuzzy minds", section
// "When scheduler does the work": sequences address slots through a page
// table and may point at the same slots; a shared prefix is inherited, not
// recomputed). A page returns to the free list when its last reference is
// released. A page may be published as a reusable prefix page once every
// slot of it has been written in every layer each plane holds (vllm-rlt pull
// 152, section "Summary": coverage checked per plane over the layers that
// plane holds, all layers at depth 0 and only the recurrent layers deeper;
// with every layer held by every plane this is the all-layers rule). Section
// "Notes" item #151 asks for the free count in constant time.
//
// Bookkeeping: free ids in a min-heap (lowest id first, O(log n) per page;
// the count is its size); a bit mask of written slots per (bank, page) and,
// per (plane, page), the number of held layers whose mask is full, so a
// publication check is one comparison per plane.
#include <algorithm>
#include <cstdint>
#include <climits>
#include <functional>
#include <memory>
#include <vector>

#include "launch.hpp"
#include "pagedkv.h"

struct pkv_page_mgr {
  int32_t num_pages, page_size, num_planes, num_layers, num_banks;
  std::vector<int32_t> bank_of;        // [plane * layers + layer]
  std::vector<int32_t> plane_of_bank;  // [bank]
  std::vector<int32_t> held;           // [plane]: layers the plane holds
  std::vector<int32_t> free_ids;       // free page ids, a min-heap (lowest id handed out first)
  std::vector<int32_t> refs;           // [page]
  std::vector<uint64_t> mask;          // [bank * pages + page]: written slots
  std::vector<int32_t> full;           // [plane * pages + page]: held layers fully written
  uint64_t all = 0;                    // mask of a fully written page
};

namespace {

int mfail(int code, const char *msg) { return pkv::set_error(code, msg); }

bool valid_ids(const pkv_page_mgr *m, int32_t n, const int32_t *ids) {
  if (n < 0 || (n > 0 && !ids)) return false;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= m->num_pages) return false;
  return true;
}

// Clears the written state of `page` in every bank.
void clear_page(pkv_page_mgr *m, int32_t page) {
  for (int32_t b = 0; b < m->num_banks; ++b) m->mask[(size_t)b * m->num_pages + page] = 0;
  for (int32_t p = 0; p < m->num_planes; ++p) m->full[(size_t)p * m->num_pages + page] = 0;
}

pkv_page_mgr *create_mgr(int32_t num_pages, int32_t page_size, int32_t num_planes,
                         int32_t num_layers, const int32_t *bank_of) {
  std::unique_ptr<pkv_page_mgr> holder(new pkv_page_mgr);
  pkv_page_mgr *m = holder.get();
  m->num_pages = num_pages;
  m->page_size = page_size;
  m->num_planes = num_planes;
  m->num_layers = num_layers;
  m->bank_of.assign(bank_of, bank_of + (size_t)num_planes * num_layers);
  int32_t nb = 0;
  for (int32_t b : m->bank_of) nb = b + 1 > nb ? b + 1 : nb;
  m->num_banks = nb;
  m->plane_of_bank.assign(nb, -1);
  m->held.assign(num_planes, 0);
  for (int32_t p = 0; p < num_planes; ++p)
    for (int32_t l = 0; l < num_layers; ++l) {
      const int32_t b = m->bank_of[(size_t)p * num_layers + l];
      if (b < 0) continue;
      if (m->plane_of_bank[b] >= 0) return nullptr;  // a bank belongs to one (plane, layer)
      m->plane_of_bank[b] = p;
      ++m->held[p];
    }
  m->free_ids.resize(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) m->free_ids[i] = i;  // sorted: already a min-heap
  m->refs.assign(num_pages, 0);
  m->mask.assign((size_t)nb * num_pages, 0);
  m->full.assign((size_t)num_planes * num_pages, 0);
  m->all = page_size == 64 ? ~0ull : ((1ull << page_size) - 1);
  return holder.release();
}

}  // namespace

extern "C" {

pkv_page_mgr *pkv_mgr_create(int32_t num_pages, int32_t page_size, int32_t num_planes,
                             int32_t num_layers, const int32_t *bank_of) {
  if (num_pages <= 0 || page_size <= 0 || page_size > 64 || num_planes <= 0 ||
      num_layers <= 0 || !bank_of || (int64_t)num_planes * num_layers > INT32_MAX)
    return nullptr;
  // A bank belongs to one (plane, layer), so ids run below planes x layers.
  const int64_t max_banks = (int64_t)num_planes * num_layers;
  for (int64_t i = 0; i < max_banks; ++i)
    if (bank_of[i] >= max_banks) return nullptr;
  try {
    return create_mgr(num_pages, page_size, num_planes, num_layers, bank_of);
  } catch (...) {  // out of host memory: nothing escapes the C interface
    return nullptr;
  }
}
void pkv_mgr_destroy(pkv_page_mgr *m) { delete m; }

int32_t pkv_mgr_free_count(const pkv_page_mgr *m) {
  return m ? (int32_t)m->free_ids.size() : PKV_EINVAL;
}

int pkv_mgr_alloc(pkv_page_mgr *m, int32_t n, int32_t *page_ids) {
  if (!m || n < 0 || (n > 0 && !page_ids)) return mfail(PKV_EINVAL, "bad arguments");
  if ((size_t)n > m->free_ids.size()) return mfail(PKV_ENOSPACE, "not enough free pages");
  for (int32_t i = 0; i < n; ++i) {
    std::pop_heap(m->free_ids.begin(), m->free_ids.end(), std::greater<int32_t>());
    const int32_t id = m->free_ids.back();
    m->free_ids.pop_back();
    m->refs[id] = 1;
    clear_page(m, id);
    page_ids[i] = id;
  }
  return pkv::set_error(PKV_OK, "");
}

int pkv_mgr_retain(pkv_page_mgr *m, int32_t n, const int32_t *page_ids) {
  if (!m || !valid_ids(m, n, page_ids)) return mfail(PKV_EINVAL, "bad page ids");
  for (int32_t i = 0; i < n; ++i)
    if (m->refs[page_ids[i]] <= 0) return mfail(PKV_EINVAL, "retain of a free page");
  for (int32_t i = 0; i < n; ++i) ++m->refs[page_ids[i]];
  return pkv::set_error(PKV_OK, "");
}

int pkv_mgr_release(pkv_page_mgr *m, int32_t n, const int32_t *page_ids) {
  if (!m || !valid_ids(m, n, page_ids)) return mfail(PKV_EINVAL, "bad page ids");
  // all or nothing: no id may be released more times than it is held
  try {
    std::vector<int32_t> ids(page_ids, page_ids + n);
    std::sort(ids.begin(), ids.end());
    for (int32_t i = 0, j = 0; i < n; i = j) {
      while (j < n && ids[j] == ids[i]) ++j;
      if (j - i > m->refs[ids[i]]) return mfail(PKV_EINVAL, "release of a free page");
    }
  } catch (...) {
    return mfail(PKV_EINVAL, "out of host memory");
  }
  for (int32_t i = 0; i < n; ++i)
    if (--m->refs[page_ids[i]] == 0) {
      m->free_ids.push_back(page_ids[i]);
      std::push_heap(m->free_ids.begin(), m->free_ids.end(), std::greater<int32_t>());
    }
  return pkv::set_error(PKV_OK, "");
}

int32_t pkv_mgr_refcount(const pkv_page_mgr *m, int32_t page) {
  if (!m || page < 0 || page >= m->num_pages) return PKV_EINVAL;
  return m->refs[page];
}

int pkv_mgr_note_write(pkv_page_mgr *m, int32_t plane, int32_t layer, int32_t n,
                       const int32_t *slots) {
  if (!m || n < 0 || (n > 0 && !slots)) return mfail(PKV_EINVAL, "bad arguments");
  if (plane < 0 || plane >= m->num_planes || layer < 0 || layer >= m->num_layers)
    return mfail(PKV_EINVAL, "(plane, layer) outside the pool");
  const int32_t b = m->bank_of[(size_t)plane * m->num_layers + layer];
  if (b < 0) return mfail(PKV_ENOTHELD, "the plane does not hold the layer");
  const int64_t cap = (int64_t)m->num_pages * m->page_size;
  for (int32_t i = 0; i < n; ++i)
    if (slots[i] >= cap) return mfail(PKV_EINVAL, "slot outside the pool");
  for (int32_t i = 0; i < n; ++i) {
    if (slots[i] < 0) continue;  // padding
    const int32_t page = slots[i] / m->page_size, off = slots[i] % m->page_size;
    uint64_t &mk = m->mask[(size_t)b * m->num_pages + page];
    const bool was_full = mk == m->all;
    mk |= 1ull << off;
    if (!was_full && mk == m->all) ++m->full[(size_t)plane * m->num_pages + page];
  }
  return pkv::set_error(PKV_OK, "");
}

int32_t pkv_mgr_published_prefix(const pkv_page_mgr *m, int32_t planes_used,
                                 const int32_t *page_ids, int32_t n_pages) {
  if (!m || planes_used <= 0 || planes_used > m->num_planes || !valid_ids(m, n_pages, page_ids))
    return mfail(PKV_EINVAL, "bad arguments");
  int32_t k = 0;
  for (; k < n_pages; ++k) {
    const int32_t page = page_ids[k];
    bool ok = m->refs[page] > 0;
    for (int32_t p = 0; ok && p < planes_used; ++p)
      ok = m->full[(size_t)p * m->num_pages + page] == m->held[p];
    if (!ok) break;
  }
  pkv::set_error(PKV_OK, "");
  return k;
}

int pkv_span_slots(const int32_t *page_table, int32_t stride, int32_t page_size,
                   int32_t num_pages, const int32_t *starts, int32_t batch, int32_t span,
                   int32_t *slots) {
  if (!page_table || !starts || !slots || stride <= 0 || page_size <= 0 || num_pages <= 0 ||
      batch < 0 || span < 0)
    return mfail(PKV_EINVAL, "pkv_span_slots: bad arguments");
  if ((int64_t)num_pages * page_size > INT32_MAX)
    return mfail(PKV_EINVAL, "pkv_span_slots: slots of this pool overflow int32");
  // Check everything first: nothing is written on failure.
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t lo = starts[r], hi = lo + span;
    if (lo < 0 || (span > 0 && hi > (int64_t)stride * page_size))
      return mfail(PKV_EINVAL, "pkv_span_slots: span outside the page-table row");
    for (int64_t p = lo; p < hi; p += page_size - p % page_size) {
      const int32_t id = page_table[(size_t)r * stride + p / page_size];
      if (id < 0 || id >= num_pages) return mfail(PKV_EINVAL, "pkv_span_slots: bad page id");
    }
  }
  for (int32_t r = 0; r < batch; ++r)
    for (int32_t j = 0; j < span; ++j) {
      const int64_t p = (int64_t)starts[r] + j;
      slots[(size_t)r * span + j] =
          page_table[(size_t)r * stride + p / page_size] * page_size + (int32_t)(p % page_size);
    }
  return pkv::set_error(PKV_OK, "");
}

}  // extern "C"
