"""The product's adjuster policy (C++, through the C ABI) against the oracle
(oracle/adjuster.py over oracle/allocator.py) on seeded synthetic serving
traces: every step's evictions, loads, budget moves, residency, in-flight
set and scores, and the pool offsets of every expert and KV owner, must be
identical. Host only."""
import numpy as np
import pytest

from moe_inputs import gen
from oracle.adjuster import Adjuster as OAdjuster, AdjusterError
from oracle.allocator import OK, Allocator
from paged_moe_expert_amd import rimuru as R

KIB, MIB = 1024, 1024 * 1024


class Native:
    def __init__(self, pool_bytes, huge, xpage, kpage, E, P, xb, kb, prm):
        self.p = R.pool_create(pool_bytes, huge)
        self.xv = R.view_map(self.p, 0, xpage)
        self.kv = R.view_map(self.p, 1, kpage, self.xv)
        for e in range(E):
            for q in range(3):
                R.view_alloc(self.xv, 3 * e + q, P)
        assert R.view_set_budget(self.xv, xb) == OK and R.view_set_budget(self.kv, kb) == OK
        self.adj = R.adjuster_create(self.p, self.xv, self.kv, E, P, **prm)

    def step(self, d, routed, needed):
        st, ev, ld, mv = R.adjuster_step_status(self.adj, d, routed, needed)
        return st, ev, ld, mv

    def done(self, e):
        R.adjuster_upload_done(self.adj, e)

    def kv_alloc(self, owner, n):
        return R.view_alloc_status(self.kv, owner, n)[0]

    def kv_free(self, owner):
        R.view_free(self.kv, owner)

    def snapshot(self, E):
        res, fl, sc = R.adjuster_state(self.adj)
        xu, xb = R.view_usage(self.xv)
        ku, kb = R.view_usage(self.kv)
        pages = [tuple(R.view_pages(self.xv, o).tolist()) for o in range(3 * E)]
        return res.tolist(), fl.tolist(), [int(v) for v in sc], (xu, xb, ku, kb), pages

    def kv_pages(self, owner):
        return tuple(R.view_pages(self.kv, owner).tolist())


class Oracle:
    def __init__(self, pool_bytes, huge, xpage, kpage, E, P, xb, kb, prm):
        self.a = Allocator(pool_bytes, huge)
        _, self.xv = self.a.map_view(0, xpage, None)
        _, self.kv = self.a.map_view(1, kpage, self.xv)
        for e in range(E):
            for q in range(3):
                assert self.a.alloc(self.xv, 3 * e + q, P)[0] == OK
        assert self.a.set_budget(self.xv, xb) == OK and self.a.set_budget(self.kv, kb) == OK
        self.adj = OAdjuster(self.a, self.xv, self.kv, E, P, **prm)

    def step(self, d, routed, needed):
        try:
            r = self.adj.step(d, routed, needed)
            return OK, r["evicted"], r["loaded"], r["kv_moved"]
        except AdjusterError as err:
            return err.status, None, None, None

    def done(self, e):
        self.adj.upload_done(e)

    def kv_alloc(self, owner, n):
        return self.a.alloc(self.kv, owner, n)[0]

    def kv_free(self, owner):
        assert self.a.free(self.kv, owner) == OK

    def snapshot(self, E):
        xv, kv = self.a.views[self.xv], self.a.views[self.kv]
        pages = [tuple(self.a.pages(self.xv, o)) for o in range(3 * E)]
        return (list(self.adj.resident), list(self.adj.inflight), list(self.adj.score),
                (self.a.used_bytes(self.xv), xv.budget, self.a.used_bytes(self.kv), kv.budget), pages)

    def kv_pages(self, owner):
        return tuple(self.a.pages(self.kv, owner))


def run_both(geom, prm, trace, check_every=1):
    E = geom["E"]
    sides = [Native(**geom, prm=prm), Oracle(**geom, prm=prm)]
    kpage = geom["kpage"]
    blocks, routed, _ = trace
    owners = [[], []]               # KV owners per side: [owner, blocks], newest last
    next_owner = 1 << 40
    counts = {"evicted": 0, "loaded": 0, "grew": 0, "gave": 0, "failed": 0}
    for s in range(len(blocks)):
        d = int(blocks[s])
        needed = (routed[s] > 0).astype(np.uint8)
        outs = [side.step(d, routed[s], needed) for side in sides]
        assert outs[0][0] == outs[1][0], f"step {s}: status {outs[0][0]} vs {outs[1][0]}"
        if outs[0][0] == OK:
            assert outs[0][1:] == outs[1][1:], f"step {s}: {outs[0][1:]} vs {outs[1][1:]}"
            counts["evicted"] += len(outs[0][1])
            counts["loaded"] += len(outs[0][2])
            counts["grew"] += outs[0][3] > 0
            counts["gave"] += outs[0][3] < 0
        else:
            counts["failed"] += 1
        if s % check_every == 0 or outs[0][0] != OK:
            snaps = [side.snapshot(E) for side in sides]
            assert snaps[0] == snaps[1], f"step {s}: state differs"
        if outs[0][0] != OK:
            break
        # the requests' KV blocks follow the demand within the budget: newest
        # owners leave first, a new owner takes what grew
        for i, side in enumerate(sides):
            budget = side.snapshot(E)[3][3] if i == 1 else R.view_usage(side.kv)[1]
            held = sum(n for _, n in owners[i])
            target = min(d, budget // kpage)
            while owners[i] and held > target:
                o, n = owners[i].pop()
                side.kv_free(o)
                held -= n
            grow = target - held
            while grow > 0:
                if side.kv_alloc(next_owner + s, grow) == OK:
                    owners[i].append((next_owner + s, grow))
                    break
                grow -= max(1, grow // 4)
        assert owners[0] == owners[1]
        for o, _ in owners[0]:
            assert sides[0].kv_pages(o) == sides[1].kv_pages(o)
        for e in outs[0][2]:
            for side in sides:
                side.done(e)
    return counts


def exercised(c):
    return c["evicted"] > 0 and c["loaded"] > 0 and c["grew"] > 0 and c["gave"] > 0


SMALL = dict(pool_bytes=160 * 64 * KIB, huge=64 * KIB, xpage=64 * KIB, kpage=16 * KIB, E=24, P=1,
             xb=24 * 3 * 64 * KIB, kb=(160 - 72) * 64 * KIB)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_parity_small_pool(seed):
    prm = dict(min_resident=14, headroom_blocks=8, return_blocks=16, shift=2, max_prefetch=2)
    trace = gen.serving_trace(seed, 300, 24, 2, mean_arrivals=0.3, prompt_mu=5.0, output_mu=4.5,
                              max_step_tokens=6, phase_steps=60, period=100)
    assert exercised(run_both(SMALL, prm, trace))


def test_parity_small_pool_tight_floor_reaches_enomem():
    """A floor too low for what a step needs: both sides fail on the same
    step with the same partial state."""
    prm = dict(min_resident=2, headroom_blocks=8, return_blocks=4, shift=1, max_prefetch=3)
    trace = gen.serving_trace(11, 300, 24, 2, mean_arrivals=0.6, prompt_mu=5.0, output_mu=4.5,
                              max_step_tokens=8, phase_steps=40, period=80)
    assert run_both(SMALL, prm, trace)["failed"] == 1


def test_parity_multi_page_experts():
    """P = 3 pages per projection of 32 KiB, KV blocks of 8 KiB, 1 MiB huge pages."""
    geom = dict(pool_bytes=64 * MIB, huge=MIB, xpage=32 * KIB, kpage=8 * KIB, E=32, P=3,
                xb=32 * 9 * 32 * KIB, kb=64 * MIB - 32 * 9 * 32 * KIB)
    prm = dict(min_resident=20, headroom_blocks=16, return_blocks=64, shift=3, max_prefetch=2)
    trace = gen.serving_trace(21, 250, 32, 4, mean_arrivals=5.0, prompt_mu=5.5, output_mu=4.5,
                              max_step_tokens=4, phase_steps=50, period=120)
    assert exercised(run_both(geom, prm, trace))


def test_parity_decode_pool():
    """The Qwen3-30B-A3B decode pool: 4 GiB of 3 MiB huge pages, 128 experts of
    three 3 MiB pages, 32 KiB KV blocks cut from expert pages (states
    checked every 10 steps)."""
    geom = dict(pool_bytes=4096 * MIB, huge=3 * MIB, xpage=3 * MIB, kpage=32 * KIB, E=128, P=1,
                xb=128 * 9 * MIB, kb=1365 * 3 * MIB - 128 * 9 * MIB)
    prm = dict(min_resident=96, headroom_blocks=256, return_blocks=2048, shift=3, max_prefetch=4)
    trace = gen.serving_trace(31, 200, 128, 8, mean_arrivals=30.0, prompt_mu=5.5, output_mu=4.8,
                              max_step_tokens=8, phase_steps=60, period=100)
    assert exercised(run_both(geom, prm, trace, check_every=10))


def test_native_argument_errors():
    p = R.pool_create(16 * 64 * KIB, 64 * KIB)
    xv = R.view_map(p, 0, 64 * KIB)
    kv = R.view_map(p, 1, 16 * KIB, xv)
    for q in range(3):
        R.view_alloc(xv, q, 1)
    with pytest.raises(R.RimuruError, match="finite budget"):
        R.adjuster_create(p, xv, kv, 2, 1)                  # no budgets yet
    assert R.view_set_budget(xv, 6 * 64 * KIB) == OK and R.view_set_budget(kv, 8 * 64 * KIB) == OK
    with pytest.raises(R.RimuruError, match="two views"):
        R.adjuster_create(p, xv, xv, 2, 1)
    other = R.pool_create(16 * 64 * KIB, 64 * KIB)
    ov = R.view_map(other, 1, 64 * KIB)                      # a whole huge page per KV block
    with pytest.raises(R.RimuruError, match="two views"):
        R.adjuster_create(p, xv, ov, 2, 1)
    with pytest.raises(R.RimuruError, match="bad parameter"):
        R.adjuster_create(p, xv, kv, 2, 1, shift=17)
    R.view_alloc(xv, 3, 1)                                   # expert 1: one projection only
    with pytest.raises(R.RimuruError, match="partly resident"):
        R.adjuster_create(p, xv, kv, 2, 1)
    R.view_free(xv, 3)
    a = R.adjuster_create(p, xv, kv, 2, 1)
    assert R.adjuster_state(a)[0].tolist() == [True, False]
    st, *_ = R.adjuster_step_status(a, 0, np.array([-1, 0]), np.zeros(2))
    assert st == R.EINVAL
    with pytest.raises(R.RimuruError, match="no upload"):
        R.adjuster_upload_done(a, 1)
    r = R.adjuster_step(a, 0, np.array([0, 3]), np.array([0, 1]))   # demand load of expert 1
    assert r["loaded"] == [1]
    R.adjuster_upload_done(a, 1)
