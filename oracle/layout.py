"""Reference layout production: seeded request streams run through the
reference allocator, then the expert-view page table (test infrastructure).

The recipes (the product's layout runner follows the same rules):

* scatter (tiny layer): every expert page is its own single-page owner; the
  expert pages and the KV blocks are allocated in one seeded order.
  Page q of projection p of expert e is owner (e*3 + p)*P + q.
* fill_then_place (decode and hybrid prefill layers): filler requests (KV,
  SSM, conv) are allocated in stream order until the first ENOMEM; then the
  projections (owner e*3 + p, P pages each) are allocated in a seeded order,
  and each that fails frees a victim filler request and retries. The victim
  is live[floor(u * len(live))], live the granted filler requests in grant
  order, u the next uniform draw.
* churn (fragmented prefill): the seeded alloc/free stream runs as issued
  (frees of owners that hold nothing return EINVAL and are recorded); then
  every projection not resident is allocated in the seeded projection order,
  freeing KV victims as above on failure.
* adjuster steps (decode sweep), on top of fill_then_place: budgets start at
  what each view holds plus half of the free bytes each. A step (f, d)
  moves b = floor(f * usable / kv_page) * kv_page bytes of budget.
  d = 0 (expert -> KV): b is clamped to the expert view's unused budget
  (rounded down to whole KV pages), moved, then new KV requests are granted
  in stream order while they fit the KV budget, stopping at the first that
  does not fit or fails. d = 1 (KV -> expert): b is clamped to the KV budget
  (rounded down to whole KV pages), victims are freed until the KV view
  holds at most its budget minus b, then b is moved. Expert pages never move.

Expert-view page table: pt[e, p, q] = (offset of page q of projection (e, p))
// page_bytes, int32 [E, 3, P].

Parity status: pinned through the allocator's property tests and the
per-recipe invariants in tests/test_oracle_layout.py.
"""
from __future__ import annotations

import numpy as np

from moe_inputs import gen
from moe_inputs.configs import MoEConfig

from .allocator import ENOMEM, OK, Allocator


class Layout:
    def __init__(self, cfg: MoEConfig):
        self.cfg = cfg
        self.alloc = Allocator(cfg.pool_bytes, cfg.huge_bytes)
        self.vid = {}
        for v in cfg.views:
            parent = None if v.parent is None else self.vid[v.parent]
            st, vid = self.alloc.map_view(v.kind, v.page_bytes, parent)
            assert st == OK, (v, st)
            self.vid[v.name] = vid
        self.statuses = []
        self.live_filler = []          # (view name, owner) in grant order
        self._u = gen.uniforms(cfg)
        self._ui = 0

    def _next_u(self):
        u = self._u[self._ui]
        self._ui += 1
        return u

    def _free_victim(self):
        if not self.live_filler:
            raise RuntimeError("layout: nothing left to free")
        i = int(np.floor(self._next_u() * len(self.live_filler)))
        name, owner = self.live_filler.pop(i)
        st = self.alloc.free(self.vid[name], owner)
        assert st == OK
        return name, owner

    def _place(self, owner, n):
        ev = self.vid["expert"]
        while True:
            st, _ = self.alloc.alloc(ev, owner, n)
            if st == OK:
                return
            assert st == ENOMEM
            self._free_victim()

    # --------------------------------------------------------- recipes
    def run_scatter(self):
        for op, name, owner, n in gen.scatter_events(self.cfg):
            st, _ = self.alloc.alloc(self.vid[name], owner, n)
            assert st == OK
        return self

    def run_fill_then_place(self):
        for name, owner, n in gen.filler_requests(self.cfg):
            st, _ = self.alloc.alloc(self.vid[name], owner, n)
            if st == ENOMEM:
                break
            self.live_filler.append((name, owner))
        for o in gen.projection_order(self.cfg):
            self._place(o, self.cfg.P)
        return self

    def run_churn(self):
        resident = set()
        for op, name, owner, n in gen.churn_events(self.cfg):
            vid = self.vid[name]
            if op == "alloc":
                st, _ = self.alloc.alloc(vid, owner, n)
                if st == OK:
                    if name == "expert":
                        resident.add(owner)
                    else:
                        self.live_filler.append((name, owner))
            else:
                st = self.alloc.free(vid, owner)
                if st == OK:
                    if name == "expert":
                        resident.discard(owner)
                    else:
                        self.live_filler.remove((name, owner))
            self.statuses.append(st)
        for o in gen.projection_order(self.cfg):
            if o not in resident:
                self._place(o, self.cfg.P)
        return self

    def run(self):
        return {"scatter": self.run_scatter, "fill_then_place": self.run_fill_then_place,
                "churn": self.run_churn}[self.cfg.layout]()

    # --------------------------------------------------------- adjuster
    def init_budgets(self):
        a = self.alloc
        ev, kv = self.vid["expert"], self.vid["kv"]
        usable = a.n_huge * a.huge
        free = usable - a.used_bytes(ev) - a.used_bytes(kv)
        assert a.set_budget(ev, a.used_bytes(ev) + free // 2) == OK
        assert a.set_budget(kv, a.used_bytes(kv) + (free - free // 2)) == OK
        self._kv_req = []
        self._kv_next = 1 << 40

    def adjuster_step(self, f: float, d: int, kv_sizes: list):
        """One boundary move; kv_sizes is consumed from the front."""
        a = self.alloc
        ev, kv = self.vid["expert"], self.vid["kv"]
        kvp = self.cfg.view("kv").page_bytes
        usable = a.n_huge * a.huge
        b = int(np.floor(f * usable / kvp)) * kvp
        if d == 0:
            b = min(b, (a.views[ev].budget - a.used_bytes(ev)) // kvp * kvp)
            assert a.transfer(ev, kv, b) == OK
            while kv_sizes:
                n = kv_sizes[0]
                if a.used_bytes(kv) + n * kvp > a.views[kv].budget:
                    break
                st, _ = a.alloc(kv, self._kv_next, n)
                if st != OK:
                    break
                kv_sizes.pop(0)
                self.live_filler.append(("kv", self._kv_next))
                self._kv_next += 1
        else:
            b = min(b, a.views[kv].budget // kvp * kvp)
            while a.used_bytes(kv) > a.views[kv].budget - b:
                self._free_victim()
            assert a.transfer(kv, ev, b) == OK
        return b

    # --------------------------------------------------------- outputs
    def page_table(self) -> np.ndarray:
        cfg = self.cfg
        ev = self.vid["expert"]
        pt = np.zeros((cfg.E, 3, cfg.P), dtype=np.int32)
        for e in range(cfg.E):
            for p in range(3):
                if cfg.layout == "scatter":
                    offs = [self.alloc.pages(ev, (e * 3 + p) * cfg.P + q)[0] for q in range(cfg.P)]
                else:
                    offs = self.alloc.pages(ev, e * 3 + p)
                assert len(offs) == cfg.P
                pt[e, p] = np.asarray(offs, dtype=np.int64) // cfg.page_bytes
        return pt


def build_pool(cfg: MoEConfig, pt: np.ndarray, weight_bits: np.ndarray,
               poison: bool = True) -> np.ndarray:
    """Host image of the pool: expert pages hold the weights, every other byte
    holds a quiet-NaN pattern (0x7FC07FC0 read as fp32 or as two bf16) so a
    stray read turns the output non-finite."""
    from .moe import place_weights
    if poison:
        pool = np.empty(cfg.pool_bytes, dtype=np.uint8)
        pool.view(np.uint32)[:] = np.uint32(0x7FC07FC0)
    else:
        pool = np.zeros(cfg.pool_bytes, dtype=np.uint8)
    place_weights(pool, pt, weight_bits, cfg.page_bytes)
    return pool
