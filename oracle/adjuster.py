"""Workload-aware adjuster policy (test infrastructure).

Written from the Rimuru pages: the paper summary's abstract (a workload-aware
adjuster reallocates pages across tensor types by runtime demand), its
Figure 8 (expert prefetch overlapped with execution) and the explainer's
paragraph on the two pieces that make the moving fence usable. What those
say, in this module's terms: more concurrent requests move budget from the
expert view to the KV view; finished requests release KV blocks whose budget
returns to the experts; and an expert being uploaded by the prefetch path is
never chosen for eviction. The pages give no rule beyond that; this is the
plain reading (the product's adjuster must take the same decisions):

* State: which experts are resident (all three projections, P pages each, as
  expert-view owners 3e + p), which have an upload in flight (loaded, not
  yet reported done), and an integer popularity score per expert,
  s <- s - (s >> shift) + (routed << 16) each step.
* A step gets the KV blocks demanded (D), the routed slots per expert, and
  the experts the next layer call reads ("needed"). Pinned = needed or in
  flight: a pinned expert is never evicted.
  1. Demand loads, ascending expert id: a needed expert that is not resident
     gets pages. While the expert view's free budget is short, evict the
     coldest unpinned resident expert; with none left, take the shortfall
     from the KV view's unused budget; else the step fails (ENOMEM). If the
     pool itself has no room although the budget allows (KV blocks sit in
     expert-sized pages), evict the next coldest and retry.
  2. KV target W = (D + headroom) blocks. Below it: the KV view may take
     the shortfall, but never so much that the expert view's budget drops
     below min_resident experts (the room the next steps' needed experts
     load into); evict coldest unpinned experts until the expert view's
     free budget covers that amount or nothing is left to evict, then move
     what is free. Above W by more than return_blocks blocks: give back
     everything above max(W, KV bytes held).
  3. Prefetch: while the expert view has a whole expert of free budget and
     fewer than max_prefetch prefetches were made this step, load the most
     popular non-resident expert with a positive score that was not evicted
     in this step (ties: lower id); stop at the first that does not fit.
  "Coldest" is the lowest score, ties to the lower id. Loads (demand, then
  prefetch) are reported in order; the caller uploads into their pages and
  reports each upload done.

Parity status: pinned by tests/test_oracle_adjuster.py (hand-worked steps,
the pages' stated behaviour on ramps and drains, and invariants on seeded
traces).
"""
from __future__ import annotations

from .allocator import EINVAL, ENOMEM, OK, Allocator


class AdjusterError(Exception):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Adjuster:
    def __init__(self, alloc: Allocator, expert_view: int, kv_view: int, E: int, P: int,
                 min_resident: int = 0, headroom_blocks: int = 0, return_blocks: int = 0,
                 shift: int = 3, max_prefetch: int = 1):
        xv, kv = alloc.views[expert_view], alloc.views[kv_view]
        if xv.budget is None or kv.budget is None:
            raise AdjusterError(EINVAL, "both views need a finite budget")
        if E <= 0 or P <= 0 or min_resident < 0 or headroom_blocks < 0 or return_blocks < 0 \
                or not 0 <= shift <= 16 or max_prefetch < 0:
            raise AdjusterError(EINVAL, "bad adjuster parameter")
        self.a, self.xv, self.kv = alloc, expert_view, kv_view
        self.E, self.P = E, P
        self.min_resident, self.headroom, self.ret = min_resident, headroom_blocks, return_blocks
        self.shift, self.max_prefetch = shift, max_prefetch
        self.kpage = kv.page
        self.expert_bytes = 3 * P * xv.page
        self.resident = [False] * E
        self.inflight = [False] * E
        self.score = [0] * E
        for e in range(E):
            held = [len(alloc.pages(expert_view, 3 * e + p)) for p in range(3)]
            if held == [P, P, P]:
                self.resident[e] = True
            elif any(held):
                raise AdjusterError(EINVAL, f"expert {e} is partly resident")

    # ------------------------------------------------------------ helpers
    def _budget(self, vid):
        return self.a.views[vid].budget

    def _free_x(self):
        return self._budget(self.xv) - self.a.used_bytes(self.xv)

    def _coldest(self, pinned):
        best = None
        for e in range(self.E):
            if self.resident[e] and not pinned[e]:
                if best is None or self.score[e] < self.score[best]:
                    best = e
        return best

    def _evict(self, e, evicted):
        for p in range(3):
            assert self.a.free(self.xv, 3 * e + p) == OK
        self.resident[e] = False
        evicted.append(e)

    def _load(self, e):
        """Pages for the three projections of e, all or nothing."""
        done = []
        for p in range(3):
            st, _ = self.a.alloc(self.xv, 3 * e + p, self.P)
            if st != OK:
                for q in done:
                    self.a.free(self.xv, 3 * e + q)
                return st
            done.append(p)
        return OK

    # ------------------------------------------------------------ policy
    def step(self, demand_blocks: int, routed, needed):
        E = self.E
        for e in range(E):
            s = self.score[e]
            self.score[e] = s - (s >> self.shift) + (int(routed[e]) << 16)
        pinned = [bool(needed[e]) or self.inflight[e] for e in range(E)]
        evicted, loaded = [], []
        out = {"evicted": evicted, "loaded": loaded, "kv_moved": 0}

        # 1. demand loads
        for e in range(E):
            if not needed[e] or self.resident[e]:
                continue
            while True:
                if self._free_x() < self.expert_bytes:
                    v = self._coldest(pinned)
                    if v is not None:
                        self._evict(v, evicted)
                        continue
                    short = self.expert_bytes - self._free_x()
                    if self._budget(self.kv) - self.a.used_bytes(self.kv) < short:
                        raise AdjusterError(ENOMEM, f"no room for needed expert {e}")
                    assert self.a.transfer(self.kv, self.xv, short) == OK
                    out["kv_moved"] -= short
                if self._load(e) == OK:
                    break
                v = self._coldest(pinned)
                if v is None:
                    raise AdjusterError(ENOMEM, f"pool has no room for needed expert {e}")
                self._evict(v, evicted)
            self.resident[e] = True
            self.inflight[e] = True
            loaded.append(e)

        # 2. KV budget toward the demand
        want = (demand_blocks + self.headroom) * self.kpage
        bk = self._budget(self.kv)
        if bk < want:
            goal = min(want - bk, max(0, self._budget(self.xv) - self.min_resident * self.expert_bytes))
            while self._free_x() < goal:
                v = self._coldest(pinned)
                if v is None:
                    break
                self._evict(v, evicted)
            take = min(goal, self._free_x())
            if take > 0:
                assert self.a.transfer(self.xv, self.kv, take) == OK
                out["kv_moved"] += take
        elif bk - want > self.ret * self.kpage:
            give = bk - max(want, self.a.used_bytes(self.kv))
            if give > 0:
                assert self.a.transfer(self.kv, self.xv, give) == OK
                out["kv_moved"] -= give

        # 3. prefetch into free expert budget
        n = 0
        while n < self.max_prefetch and self._free_x() >= self.expert_bytes:
            best = None
            for e in range(E):
                if not self.resident[e] and self.score[e] > 0 and e not in evicted:
                    if best is None or self.score[e] > self.score[best]:
                        best = e
            if best is None or self._load(best) != OK:
                break
            self.resident[best] = True
            self.inflight[best] = True
            loaded.append(best)
            n += 1
        return out

    def upload_done(self, e: int):
        if not 0 <= e < self.E or not self.inflight[e]:
            raise AdjusterError(EINVAL, f"expert {e} has no upload in flight")
        self.inflight[e] = False
