"""Layout production through librimuru's allocator: seeded request streams in,
expert-view page table out (host only, before any kernel runs).

Recipes (the same rules the reference recipes state):
  scatter          single-page owners for every expert page plus KV blocks, in
                   one seeded order; page q of projection (e, p) is owner
                   (e*3 + p)*P + q.
  fill_then_place  filler requests in stream order until the first ENOMEM,
                   then projections (owner e*3 + p) in seeded order; each
                   failure frees victim live[floor(u * len(live))] and retries.
  churn            the seeded alloc/free stream as issued, then every missing
                   projection in seeded order, freeing KV victims on ENOMEM.
  adjuster step    budgets start at what each view holds plus half the free
                   bytes each; a step moves floor(f*usable/kv_page) KV pages of
                   budget toward KV (then grows KV requests while they fit) or
                   toward the experts (after freeing KV victims). Resident
                   expert pages never move.
"""
from __future__ import annotations

import math

import numpy as np

from moe_inputs import gen
from moe_inputs.configs import MoEConfig

from . import rimuru as R


class DeviceLayout:
    def __init__(self, cfg: MoEConfig):
        self.cfg = cfg
        self.pool = R.pool_create(cfg.pool_bytes, cfg.huge_bytes)
        self.views = {}
        for v in cfg.views:
            parent = self.views[v.parent] if v.parent is not None else None
            self.views[v.name] = R.view_map(self.pool, v.kind, v.page_bytes, parent)
        self.statuses = []
        self.live = []                       # granted filler (view name, owner), grant order
        self._u = gen.uniforms(cfg)
        self._ui = 0

    def _victim(self):
        if not self.live:
            raise RuntimeError("layout: no filler request left to free")
        u = self._u[self._ui]
        self._ui += 1
        name, owner = self.live.pop(int(math.floor(u * len(self.live))))
        R.view_free(self.views[name], owner)

    def _place(self, owner: int, n: int):
        v = self.views["expert"]
        while True:
            st, _ = R.view_alloc_status(v, owner, n)
            if st == R.OK:
                return
            if st != R.ENOMEM:
                R.check(st, "layout place")
            self._victim()

    def run(self):
        cfg = self.cfg
        if cfg.layout == "scatter":
            for _, name, owner, n in gen.scatter_events(cfg):
                R.view_alloc(self.views[name], owner, n)
        elif cfg.layout == "fill_then_place":
            for name, owner, n in gen.filler_requests(cfg):
                st, _ = R.view_alloc_status(self.views[name], owner, n)
                if st == R.ENOMEM:
                    break
                R.check(st, "layout fill")
                self.live.append((name, owner))
            for o in gen.projection_order(cfg):
                self._place(o, cfg.P)
        elif cfg.layout == "churn":
            resident = set()
            for op, name, owner, n in gen.churn_events(cfg):
                v = self.views[name]
                if op == "alloc":
                    st, _ = R.view_alloc_status(v, owner, n)
                    if st == R.OK:
                        if name == "expert":
                            resident.add(owner)
                        else:
                            self.live.append((name, owner))
                else:
                    st = R.view_free_status(v, owner)
                    if st == R.OK:
                        if name == "expert":
                            resident.discard(owner)
                        else:
                            self.live.remove((name, owner))
                self.statuses.append(st)
            for o in gen.projection_order(cfg):
                if o not in resident:
                    self._place(o, cfg.P)
        else:
            raise ValueError(cfg.layout)
        return self

    # ------------------------------------------------------------ adjuster
    def init_budgets(self):
        ev, kv = self.views["expert"], self.views["kv"]
        usable = self.pool.huge_bytes * R.pool_stats(self.pool)["huge_pages"]
        ue, _ = R.view_usage(ev)
        uk, _ = R.view_usage(kv)
        free = usable - ue - uk
        R.check(R.view_set_budget(ev, ue + free // 2), "budget")
        R.check(R.view_set_budget(kv, uk + (free - free // 2)), "budget")
        self._kv_next = 1 << 40

    def adjuster_step(self, f: float, d: int, kv_sizes: list) -> int:
        ev, kv = self.views["expert"], self.views["kv"]
        kvp = self.cfg.view("kv").page_bytes
        usable = self.pool.huge_bytes * R.pool_stats(self.pool)["huge_pages"]
        b = int(math.floor(f * usable / kvp)) * kvp
        if d == 0:
            ue, be = R.view_usage(ev)
            b = min(b, (be - ue) // kvp * kvp)
            R.check(R.pool_transfer(self.pool, ev, kv, b), "transfer")
            while kv_sizes:
                n = kv_sizes[0]
                uk, bk = R.view_usage(kv)
                if uk + n * kvp > bk:
                    break
                st, _ = R.view_alloc_status(kv, self._kv_next, n)
                if st != R.OK:
                    break
                kv_sizes.pop(0)
                self.live.append(("kv", self._kv_next))
                self._kv_next += 1
        else:
            _, bk = R.view_usage(kv)
            b = min(b, bk // kvp * kvp)
            while R.view_usage(kv)[0] > bk - b:
                self._victim()
            R.check(R.pool_transfer(self.pool, kv, ev, b), "transfer")
        return b

    # ------------------------------------------------------------ outputs
    def page_table(self) -> np.ndarray:
        cfg = self.cfg
        v = self.views["expert"]
        pt = np.zeros((cfg.E, 3, cfg.P), dtype=np.int32)
        for e in range(cfg.E):
            for p in range(3):
                if cfg.layout == "scatter":
                    offs = np.array([R.view_pages(v, (e * 3 + p) * cfg.P + q)[0] for q in range(cfg.P)])
                else:
                    offs = R.view_pages(v, e * 3 + p)
                if len(offs) != cfg.P:
                    raise RuntimeError(f"projection ({e}, {p}) holds {len(offs)} pages, not {cfg.P}")
                pt[e, p] = offs // cfg.page_bytes
        return pt


def contiguous_page_table(cfg: MoEConfig) -> np.ndarray:
    """Pages of each projection consecutive and in order, projections in
    (expert, projection) order: the layout of one contiguous weight tensor."""
    return np.arange(cfg.E * 3 * cfg.P, dtype=np.int32).reshape(cfg.E, 3, cfg.P)
