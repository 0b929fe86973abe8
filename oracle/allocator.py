"""Reference multi-level split/merge page allocator (test infrastructure).

Written from the Rimuru pages: the paper summary's abstract (a shared page
pool; memory views, each with its own page size and page table; huge-page
alignment with a multi-level allocator that splits and merges pages),
Figures 6 and 7 of that summary, and the explainer's paragraph on moving the
fence (huge pages are a common multiple of the expert and state page sizes;
a huge page splits into expert-sized pages, which may split into KV-sized
pages; reclaiming merges back along the same path; a huge page is never cut
straight into KV blocks; one request's small pages come from one parent when
possible).

Where the pages leave the policy open, this is the reading (the product's
allocator must make the same decisions):

* Page of view v for owner o, one page at a time:
  1. the lowest-address parent of v that already holds a page of o and has a
     free slot;
  2. else the lowest-address parent of v with a free slot;
  3. else a new parent: the lowest-address free huge page when v is cut from
     huge pages, otherwise one page of the parent view allocated (by these same
     rules) to a reserved split owner of v.
  Within a parent, the lowest free slot. A parent of size S yields
  floor(S / page) slots; the remainder is tail waste.
* A multi-page request is all or nothing: on failure the pages taken by the
  call are released again and the pool is left as it was.
* A parent whose last slot is freed merges back into its own parent level.
* Budgets: each view may carry a byte budget on the pages its real owners
  hold; a request that would exceed it fails with ENOMEM. A transfer moves
  budget between two views and fails with EBUSY when the source would drop
  below what its owners hold. Nothing resident ever moves.

Parity status: pinned by property tests (no overlap, alignment, byte
conservation, full merge back, the two rules above, deterministic replay,
error codes) in tests/test_oracle_allocator.py.
"""
from __future__ import annotations

from sortedcontainers import SortedList

OK, EINVAL, ENOMEM, ERANGE, EDTYPE, EHIP, EBUSY = 0, -1, -2, -3, -4, -5, -6
KIND_EXPERT, KIND_KV, KIND_SSM, KIND_CONV = 0, 1, 2, 3
SPLIT = 1 << 63          # owners >= SPLIT are reserved: SPLIT | child view id


class _Parent:
    __slots__ = ("base", "slots", "used")

    def __init__(self, base, n):
        self.base = base
        self.slots = [None] * n
        self.used = 0


class _View:
    def __init__(self, vid, kind, page, parent, parent_size):
        self.vid = vid
        self.kind = kind
        self.page = page
        self.parent = parent                 # None (huge) or view id
        self.parent_size = parent_size
        self.nslots = parent_size // page
        self.parents = {}                    # base -> _Parent
        self.avail = SortedList()            # bases of parents with a free slot
        self.owner_pages = {}                # owner -> [offsets] in allocation order
        self.owner_parents = {}              # owner -> {base: count}
        self.page_parent = {}                # offset -> parent base
        self.used = 0                        # pages held by real owners
        self.budget = None                   # None = unlimited


class Allocator:
    def __init__(self, pool_bytes: int, huge_bytes: int):
        if huge_bytes <= 0 or huge_bytes % 128 or pool_bytes < huge_bytes:
            raise ValueError("bad pool or huge page size")
        self.pool_bytes = pool_bytes
        self.huge = huge_bytes
        self.n_huge = pool_bytes // huge_bytes
        self.free_huge = SortedList(range(self.n_huge))
        self.views: list[_View] = []

    # ------------------------------------------------------------ views
    def map_view(self, kind: int, page_bytes: int, parent: int | None = None):
        """Register a view; returns (status, view id)."""
        if kind not in (0, 1, 2, 3) or page_bytes <= 0 or page_bytes % 128:
            return EINVAL, -1
        if parent is None:
            psize = self.huge
            if psize % page_bytes:
                return EINVAL, -1            # huge pages must divide evenly
            if kind == KIND_KV and page_bytes != self.huge:
                return EINVAL, -1            # never cut a huge page straight into KV
        else:
            if not 0 <= parent < len(self.views):
                return EINVAL, -1
            psize = self.views[parent].page
            if page_bytes > psize:
                return EINVAL, -1
        v = _View(len(self.views), kind, page_bytes, parent, psize)
        self.views.append(v)
        return OK, v.vid

    # ------------------------------------------------------------ pages
    def _new_parent(self, v: _View):
        if v.parent is None:
            if not self.free_huge:
                return None
            base = self.free_huge.pop(0) * self.huge
        else:
            base = self._take(self.views[v.parent], SPLIT | v.vid)
            if base is None:
                return None
        v.parents[base] = _Parent(base, v.nslots)
        v.avail.add(base)
        return base

    def _take(self, v: _View, owner: int):
        base = None
        held = v.owner_parents.get(owner)
        if held:
            for b in sorted(held):
                if v.parents[b].used < v.nslots:
                    base = b
                    break
        if base is None and v.avail:
            base = v.avail[0]
        if base is None:
            base = self._new_parent(v)
            if base is None:
                return None
        par = v.parents[base]
        slot = par.slots.index(None)
        par.slots[slot] = owner
        par.used += 1
        if par.used == v.nslots:
            v.avail.remove(base)
        v.owner_parents.setdefault(owner, {})
        v.owner_parents[owner][base] = v.owner_parents[owner].get(base, 0) + 1
        off = base + slot * v.page
        v.page_parent[off] = base
        if owner >= SPLIT:
            v.owner_pages.setdefault(owner, []).append(off)
        return off

    def _release(self, v: _View, off: int, owner: int):
        base = v.page_parent.pop(off)
        par = v.parents[base]
        slot = (off - base) // v.page
        assert par.slots[slot] == owner
        par.slots[slot] = None
        if par.used == v.nslots:
            v.avail.add(base)
        par.used -= 1
        cnt = v.owner_parents[owner]
        cnt[base] -= 1
        if cnt[base] == 0:
            del cnt[base]
            if not cnt:
                del v.owner_parents[owner]
        if par.used == 0:                                   # merge back
            del v.parents[base]
            v.avail.remove(base)
            if v.parent is None:
                self.free_huge.add(base // self.huge)
            else:
                pv = self.views[v.parent]
                pv.owner_pages[SPLIT | v.vid].remove(base)
                if not pv.owner_pages[SPLIT | v.vid]:
                    del pv.owner_pages[SPLIT | v.vid]
                self._release(pv, base, SPLIT | v.vid)

    def alloc(self, vid: int, owner: int, n: int):
        """Allocate n pages of view vid for owner; returns (status, offsets)."""
        if not 0 <= vid < len(self.views) or owner < 0 or owner >= SPLIT or n <= 0:
            return EINVAL, []
        v = self.views[vid]
        if v.budget is not None and (v.used + n) * v.page > v.budget:
            return ENOMEM, []
        got = []
        for _ in range(n):
            off = self._take(v, owner)
            if off is None:
                for o in reversed(got):
                    self._release(v, o, owner)
                return ENOMEM, []
            got.append(off)
        v.owner_pages.setdefault(owner, []).extend(got)
        v.used += n
        return OK, got

    def free(self, vid: int, owner: int):
        if not 0 <= vid < len(self.views) or owner >= SPLIT:
            return EINVAL
        v = self.views[vid]
        pages = v.owner_pages.pop(owner, None)
        if not pages:
            return EINVAL
        for off in pages:
            self._release(v, off, owner)
        v.used -= len(pages)
        return OK

    def pages(self, vid: int, owner: int):
        return list(self.views[vid].owner_pages.get(owner, []))

    # ------------------------------------------------------------ budgets
    def set_budget(self, vid: int, nbytes):
        v = self.views[vid]
        if nbytes is not None and nbytes < v.used * v.page:
            return EBUSY
        v.budget = nbytes
        return OK

    def transfer(self, src: int, dst: int, nbytes: int):
        if src == dst or nbytes < 0:
            return EINVAL
        a, b = self.views[src], self.views[dst]
        if a.budget is None or b.budget is None:
            return EINVAL
        if a.budget - nbytes < a.used * a.page:
            return EBUSY
        a.budget -= nbytes
        b.budget += nbytes
        return OK

    def used_bytes(self, vid: int) -> int:
        v = self.views[vid]
        return v.used * v.page

    # ------------------------------------------------------------ stats
    def stats(self):
        per_kind = [0, 0, 0, 0]
        free = len(self.free_huge) * self.huge
        waste = self.pool_bytes - self.n_huge * self.huge
        nparents = 0
        for v in self.views:
            per_kind[v.kind] += v.used * v.page
            nparents += len(v.parents)
            for par in v.parents.values():
                free += (v.nslots - par.used) * v.page
                waste += v.parent_size - v.nslots * v.page
        return {"huge_pages": self.n_huge, "huge_free": len(self.free_huge),
                "bytes_per_kind": per_kind, "bytes_free": free,
                "waste_bytes": waste, "split_parents": nparents}
