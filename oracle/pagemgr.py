"""Plain model of the host page manager (TEST INFRASTRUCTURE ONLY; only the
test suite may import it).

Pages, reference counts and per-plane prefix publication, written with Python
sets and dicts straight from the pages:

* "Faster fuzzy minds", section "When scheduler does the work": slots are
  addressed through a page table and two sequences may point at the same
  slots; a request that shares a prompt prefix inherits its KV. So a page
  has owners (a reference count) and is free when it has none.
* vllm-rlt pull 152, section "Summary": a prefix may be published only if it
  is written; coverage is checked per plane over the layers that plane
  holds (all layers at depth 0, only the recurrent layers deeper), not over
  every layer of every plane. ``rule="every_layer"`` gives the rule the pull
  replaced, for the pins.

Free pages are handed out lowest id first, as the library does, so that page
ids can be compared between the two.
"""
from __future__ import annotations


class PageModel:
    def __init__(self, num_pages: int, page_size: int, bank_of):
        self.num_pages, self.page_size = num_pages, page_size
        self.bank_of = [list(row) for row in bank_of]  # [plane][layer] -> bank or -1
        self.refs = {}                                  # page -> count (> 0)
        self.written = {}                               # (plane, layer, page) -> set of offsets

    def free_count(self) -> int:
        return self.num_pages - len(self.refs)

    def alloc(self, n: int):
        free = [p for p in range(self.num_pages) if p not in self.refs]
        if n > len(free):
            return None
        got = free[:n]
        for p in got:
            self.refs[p] = 1
            for key in [k for k in self.written if k[2] == p]:
                del self.written[key]
        return got

    def retain(self, ids) -> bool:
        if any(p not in self.refs for p in ids):
            return False
        for p in ids:
            self.refs[p] += 1
        return True

    def release(self, ids) -> bool:
        for p in set(ids):
            if list(ids).count(p) > self.refs.get(p, 0):
                return False
        for p in ids:
            self.refs[p] -= 1
            if self.refs[p] == 0:
                del self.refs[p]
        return True

    def note_write(self, plane: int, layer: int, slots) -> bool:
        if self.bank_of[plane][layer] < 0:
            return False
        for s in slots:
            if s >= 0:
                key = (plane, layer, s // self.page_size)
                self.written.setdefault(key, set()).add(s % self.page_size)
        return True

    def page_written(self, plane: int, layer: int, page: int) -> bool:
        return len(self.written.get((plane, layer, page), ())) == self.page_size

    def published_prefix(self, planes_used: int, ids, rule: str = "per_plane") -> int:
        k = 0
        for page in ids:
            ok = page in self.refs
            for plane in range(planes_used):
                for layer, bank in enumerate(self.bank_of[plane]):
                    needed = bank >= 0 if rule == "per_plane" else True
                    if needed and not self.page_written(plane, layer, page):
                        ok = False
            if not ok:
                break
            k += 1
        return k
