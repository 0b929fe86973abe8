"""Pins of the oracle adjuster policy (oracle/adjuster.py) against the
behaviour the Rimuru pages state for it (paper summary, abstract and
Figure 8; explainer, paragraph on the two pieces that make the moving fence
usable) and against hand-worked steps and invariants."""
import pytest

from moe_inputs import gen
from oracle.adjuster import Adjuster, AdjusterError
from oracle.allocator import ENOMEM, OK, Allocator

KIB = 1024
HUGE = 64 * KIB
KVB = 16 * KIB            # KV block cut from 64 KiB expert pages
EXPERT = 3 * HUGE         # P = 1: three 64 KiB pages per expert


def small_pool(E=4, n_huge=16, x_budget=None, k_budget=None, **kw):
    """n_huge huge pages of 64 KiB; expert view of 64 KiB pages straight from
    huge pages; KV view of 16 KiB blocks cut from expert pages; E experts
    resident (owners 3e + p), then budgets."""
    a = Allocator(n_huge * HUGE, HUGE)
    _, xv = a.map_view(0, HUGE, None)
    _, kv = a.map_view(1, KVB, xv)
    for e in range(E):
        for p in range(3):
            assert a.alloc(xv, 3 * e + p, 1)[0] == OK
    xb = E * EXPERT if x_budget is None else x_budget
    assert a.set_budget(xv, xb) == OK
    assert a.set_budget(kv, n_huge * HUGE - xb if k_budget is None else k_budget) == OK
    return a, xv, kv, Adjuster(a, xv, kv, E, 1, **kw)


def budgets(a, xv, kv):
    return a.views[xv].budget, a.views[kv].budget


def test_hand_worked_ramp_and_drain():
    a, xv, kv, adj = small_pool(min_resident=1, headroom_blocks=2, return_blocks=2, shift=3,
                                max_prefetch=2)
    total = sum(budgets(a, xv, kv))
    # step 1: demand 10 blocks + 2 headroom = 192 KiB < the KV budget of 256 KiB,
    # surplus 64 KiB > 2 blocks: everything above max(192 KiB, 0 held) goes back
    r = adj.step(10, [5, 0, 3, 1], [1, 0, 0, 0])
    assert r == {"evicted": [], "loaded": [], "kv_moved": -64 * KIB}
    assert budgets(a, xv, kv) == (4 * EXPERT + 64 * KIB, 192 * KIB)
    assert adj.score == [5 << 16, 0, 3 << 16, 1 << 16]
    # step 2: want 22 blocks = 352 KiB, short 160 KiB, 64 KiB free in the expert
    # view: evict the coldest unpinned expert (1, score 0), then move 160 KiB
    r = adj.step(20, [0, 0, 0, 0], [1, 0, 0, 0])
    assert r == {"evicted": [1], "loaded": [], "kv_moved": 160 * KIB}
    assert budgets(a, xv, kv) == (4 * EXPERT + 64 * KIB - 160 * KIB, 352 * KIB)
    # step 3: want 42 blocks = 672 KiB, short 320 KiB with 96 KiB free: expert 3
    # (score 7 << 13) then expert 2 go; expert 0 is needed (and the last one)
    r = adj.step(40, [0, 0, 0, 0], [1, 0, 0, 0])
    assert r == {"evicted": [3, 2], "loaded": [], "kv_moved": 320 * KIB}
    assert adj.resident == [True, False, False, False]
    # step 4: demand falls to 4 blocks: the KV budget shrinks to 6 blocks and
    # the expert view prefetches the two most popular evicted experts (2, then
    # 3); expert 1 never received a slot and stays out
    r = adj.step(4, [0, 0, 0, 0], [1, 0, 0, 0])
    assert r == {"evicted": [], "loaded": [2, 3], "kv_moved": -576 * KIB}
    assert adj.resident == [True, False, True, True]
    assert adj.inflight == [False, False, True, True]
    assert sum(budgets(a, xv, kv)) == total
    # the pages the loads got are the lowest free ones (allocator rule)
    assert a.pages(xv, 3 * 2 + 0) and len(a.pages(xv, 3 * 3 + 2)) == 1


def test_uploads_in_flight_are_never_evicted():
    a, xv, kv, adj = small_pool(max_prefetch=2, return_blocks=0)
    adj.step(0, [0, 4, 2, 0], [0, 0, 0, 0])      # all resident; KV gives back its spare
    # a spike evicts the coldest unpinned experts: 0 and 3 (score 0), then 2
    r = adj.step(48, [0, 0, 0, 0], [0, 1, 0, 0])
    assert r["evicted"] == [0, 3, 2]
    r = adj.step(0, [0, 0, 0, 0], [0, 1, 0, 0])  # drain: expert 2 (the only one with a score) returns
    assert r["loaded"] == [2] and adj.inflight[2]
    # a new spike cannot take expert 2 while its upload is in flight ...
    r = adj.step(48, [0, 0, 0, 0], [0, 1, 0, 0])
    assert r["evicted"] == [] and adj.resident[2]
    # ... but can once the upload is reported done
    adj.upload_done(2)
    r = adj.step(48, [0, 0, 0, 0], [0, 1, 0, 0])
    assert r["evicted"] == [2]
    with pytest.raises(AdjusterError):
        adj.upload_done(2)                        # nothing in flight any more


def test_demand_load_evicts_coldest_then_borrows_from_kv():
    a, xv, kv, adj = small_pool(E=4, max_prefetch=0)
    # evict experts 2 and 3 by a KV spike (1 is needed, 0 colder)
    adj.step(0, [9, 9, 1, 0], [0, 0, 0, 0])
    adj.step(32, [0, 0, 0, 0], [1, 1, 0, 0])
    assert adj.resident == [True, True, False, False]
    held_x = a.used_bytes(xv)
    # expert 3 is needed now: the expert view has no free budget and both
    # residents are pinned, so its pages come out of KV's unused budget
    r = adj.step(32, [0, 0, 0, 5], [1, 1, 0, 1])
    assert r["loaded"] == [3] and r["evicted"] == []
    assert a.used_bytes(xv) == held_x + EXPERT
    # needed experts are resident after every step
    assert all(adj.resident[e] for e in (0, 1, 3))


def test_step_fails_when_needed_experts_cannot_fit():
    a, xv, kv, _ = small_pool(E=4, n_huge=12, max_prefetch=0)   # the pool holds exactly 4 experts
    assert a.views[kv].budget == 0
    adj5 = Adjuster(a, xv, kv, 5, 1)              # expert 4 has no pages yet
    assert adj5.resident == [True] * 4 + [False]
    adj5.step(0, [0] * 5, [1, 1, 1, 0, 1])        # room for 4 by evicting the unneeded expert 3
    assert adj5.resident == [True, True, True, False, True]
    with pytest.raises(AdjusterError) as ei:
        adj5.step(0, [0] * 5, [1] * 5)            # five needed, room for four
    assert ei.value.status == ENOMEM


def test_min_resident_floor_and_hysteresis():
    a, xv, kv, adj = small_pool(E=4, min_resident=3, return_blocks=4, max_prefetch=0)
    # want 64 blocks = 1 MiB, but the expert budget keeps 3 experts: one goes
    r = adj.step(64, [0, 0, 0, 0], [0, 0, 0, 0])
    assert r["evicted"] == [0] and sum(adj.resident) == 3
    assert budgets(a, xv, kv) == (3 * EXPERT, 256 * KIB + EXPERT)
    # 28 blocks of budget: a dip to 25 blocks (3 over, within 4) gives nothing back
    r = adj.step(25, [0] * 4, [0] * 4)
    assert r["kv_moved"] == 0
    # a dip to 20 (8 over) gives back everything above 20 blocks
    r = adj.step(20, [0] * 4, [0] * 4)
    assert r["kv_moved"] == -8 * KVB and budgets(a, xv, kv)[1] == 20 * KVB
    # never below what the KV owners hold
    assert a.alloc(kv, 77, 18)[0] == OK
    r = adj.step(0, [0] * 4, [0] * 4)
    assert budgets(a, xv, kv)[1] == 18 * KVB


def _drive(adj, a, xv, kv, trace, kv_owner=1 << 40):
    """Run a trace; after each step the KV view's owners hold min(demand,
    budget) blocks (one owner standing for all running requests) and the
    step's uploads finish. Returns one record per step, taken right after
    the adjuster's step."""
    blocks, routed, _ = trace
    log = []
    for s in range(len(blocks)):
        needed = [1 if c > 0 else 0 for c in routed[s]]
        pinned = [bool(needed[e]) or adj.inflight[e] for e in range(adj.E)]
        r = adj.step(int(blocks[s]), routed[s], needed)
        log.append({"r": r, "needed": needed, "pinned": pinned, "resident": list(adj.resident),
                    "want": (int(blocks[s]) + adj.headroom) * adj.kpage,
                    "bx": a.views[xv].budget, "bk": a.views[kv].budget,
                    "ux": a.used_bytes(xv), "uk": a.used_bytes(kv), "score": list(adj.score)})
        if a.pages(kv, kv_owner):
            a.free(kv, kv_owner)
        n = min(int(blocks[s]), a.views[kv].budget // a.views[kv].page)
        while n > 0 and a.alloc(kv, kv_owner, n)[0] != OK:
            n -= max(1, n // 8)
        for e in r["loaded"]:
            adj.upload_done(e)
    return log


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_invariants_on_seeded_traces(seed):
    E, floor_experts, ret, maxp = 24, 14, 16, 2
    a, xv, kv, adj = small_pool(E=E, n_huge=160, min_resident=floor_experts, headroom_blocks=8,
                                return_blocks=ret, shift=2, max_prefetch=maxp)
    total = sum(budgets(a, xv, kv))
    trace = gen.serving_trace(seed, 300, E, 2, mean_arrivals=0.3, prompt_mu=5.0, output_mu=4.5,
                              max_step_tokens=6, phase_steps=60, period=100)
    log = _drive(adj, a, xv, kv, trace)
    grew = gave = 0
    for st in log:
        r, pinned, res = st["r"], st["pinned"], st["resident"]
        free_x = st["bx"] - st["ux"]
        # budgets are conserved and respected
        assert st["bx"] + st["bk"] == total
        assert st["ux"] <= st["bx"] and st["uk"] <= st["bk"]
        # pinned experts (needed, or upload in flight) are never evicted
        assert not [e for e in r["evicted"] if pinned[e]]
        # every needed expert is resident for the layer call
        assert all(res[e] for e in range(E) if st["needed"][e])
        # below the KV target only when the expert side is at its floor or
        # has nothing left to give
        if st["bk"] < st["want"]:
            assert st["bx"] <= floor_experts * EXPERT or \
                (free_x == 0 and all(pinned[e] for e in range(E) if res[e]))
        # above it by more than the hysteresis only while KV holds that much
        if st["bk"] - st["want"] > ret * KVB and r["kv_moved"] <= 0:
            assert st["bk"] <= max(st["want"], st["uk"]) or r["kv_moved"] == 0
        # prefetch leaves no whole expert of budget idle while a popular one is out
        demand = sum(1 for e in r["loaded"] if st["needed"][e])
        if free_x >= EXPERT and len(r["loaded"]) - demand < maxp:
            waiting = [e for e in range(E) if not res[e] and st["score"][e] > 0 and e not in r["evicted"]]
            assert not waiting
        grew += r["kv_moved"] > 0
        gave += r["kv_moved"] < 0
    assert grew > 10 and gave > 3                 # the trace moves the fence both ways


def test_kv_budget_tracks_demand_when_experts_can_go():
    """With a generous expert floor of 0 and nothing needed, the KV budget
    reaches the demand (plus headroom) whenever the pool can hold it."""
    a, xv, kv, adj = small_pool(E=8, n_huge=64, headroom_blocks=4, return_blocks=0, max_prefetch=8)
    cap = 64 * HUGE // KVB
    for d in (10, 50, 100, 180, 60, 5, 0):
        adj.step(d, [1] * 8, [0] * 8)
        want = min((d + 4) * KVB, 64 * HUGE)
        assert a.views[kv].budget == want or a.views[kv].budget == 64 * HUGE - a.used_bytes(xv)
        assert a.views[kv].budget <= cap * KVB


def test_replay_is_deterministic():
    outs = []
    for _ in range(2):
        a, xv, kv, adj = small_pool(E=16, n_huge=96, min_resident=10, headroom_blocks=4,
                                    return_blocks=8, max_prefetch=1)
        trace = gen.serving_trace(9, 120, 16, 2, mean_arrivals=1.0, max_step_tokens=4)
        log = _drive(adj, a, xv, kv, trace)
        outs.append([(st["r"]["evicted"], st["r"]["loaded"], st["r"]["kv_moved"]) for st in log])
    assert outs[0] == outs[1]
