"""Pins for the reference page allocator: invariants the pages fix (views over
one pool, huge pages split into expert-sized pages that may split into KV
pages, merge back in reverse, no huge page cut straight into KV blocks, one
request's pages from one parent when possible) checked on seeded and
hypothesis-generated request streams."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import (EBUSY, EINVAL, ENOMEM, OK, SPLIT, Allocator, KIND_CONV,
                              KIND_EXPERT, KIND_KV, KIND_SSM)

KB = 1024


def three_level(pool=48 * 4 * 64 * KB, huge=4 * 64 * KB, expert=64 * KB, kv=32 * KB):
    a = Allocator(pool, huge)
    assert a.map_view(KIND_EXPERT, expert) == (OK, 0)
    assert a.map_view(KIND_KV, kv, 0) == (OK, 1)
    return a


def all_pages(a):
    """(view, owner, offset, size) of every page held by a real owner."""
    out = []
    for v in a.views:
        for o, offs in v.owner_pages.items():
            if o >= SPLIT:
                continue
            out += [(v.vid, o, off, v.page) for off in offs]
    return out


def check_invariants(a):
    pages = all_pages(a)
    # 1. no overlap between any two pages held by real owners
    iv = sorted((off, off + sz) for _, _, off, sz in pages)
    for (s0, e0), (s1, e1) in zip(iv, iv[1:]):
        assert e0 <= s1
    # 2. each page sits at parent base + slot*page inside a live parent, and
    #    each parent sits inside a huge page or inside a split page of its parent view
    for v in a.views:
        for base, par in v.parents.items():
            assert par.used == sum(s is not None for s in par.slots) > 0
            if v.parent is None:
                assert base % a.huge == 0 and base // a.huge not in set(a.free_huge)
            else:
                pv = a.views[v.parent]
                assert base in pv.owner_pages[SPLIT | v.vid]
            for i, s in enumerate(par.slots):
                if s is not None:
                    off = base + i * v.page
                    assert v.page_parent[off] == base
                    assert off + v.page <= base + v.parent_size
    for vid, o, off, sz in pages:
        v = a.views[vid]
        base = v.page_parent[off]
        assert (off - base) % v.page == 0
        assert v.parents[base].slots[(off - base) // v.page] == o
    # 3. byte conservation
    s = a.stats()
    assert sum(s["bytes_per_kind"]) + s["bytes_free"] + s["waste_bytes"] == a.pool_bytes
    # 4. used counts
    for v in a.views:
        n = sum(len(p) for o, p in v.owner_pages.items() if o < SPLIT)
        assert n == v.used


def snapshot(a):
    return (tuple(a.free_huge),
            tuple((v.vid, tuple(sorted((b, tuple(p.slots)) for b, p in v.parents.items())),
                   tuple(sorted((o, tuple(p)) for o, p in v.owner_pages.items())), v.used)
                  for v in a.views))


def test_huge_split_into_expert_then_kv():
    a = three_level()
    st_, offs = a.alloc(1, 7, 3)             # three KV blocks
    assert st_ == OK
    # the first huge page became expert-sized pages; one of those became KV blocks
    assert offs == [0, 32 * KB, 64 * KB]
    assert set(a.views[0].parents) == {0}
    assert a.views[0].owner_pages[SPLIT | 1] == [0, 64 * KB]
    check_invariants(a)


def test_never_cut_huge_straight_into_kv():
    a = Allocator(1 << 20, 256 * KB)
    assert a.map_view(KIND_KV, 32 * KB, None)[0] == EINVAL
    assert a.map_view(KIND_KV, 256 * KB, None)[0] == OK     # a KV block the size of a huge page


def test_view_validation():
    a = Allocator(1 << 20, 256 * KB)
    assert a.map_view(KIND_EXPERT, 100)[0] == EINVAL          # not a multiple of 128
    assert a.map_view(KIND_EXPERT, 96 * KB)[0] == EINVAL      # does not divide the huge page
    assert a.map_view(7, 64 * KB)[0] == EINVAL
    assert a.map_view(KIND_EXPERT, 64 * KB)[0] == OK
    assert a.map_view(KIND_CONV, 128 * KB, 0)[0] == EINVAL    # larger than its parent
    assert a.map_view(KIND_CONV, 48 * KB, 0)[0] == OK         # 1 slot + 16 KiB tail
    assert a.map_view(KIND_CONV, 48 * KB, 5)[0] == EINVAL


def test_same_parent_for_one_request():
    a = three_level()
    a.alloc(1, 1, 1)                          # another owner takes a KV block first
    st_, offs = a.alloc(1, 2, 2)
    assert st_ == OK
    bases = {a.views[1].page_parent[o] for o in offs}
    # the second owner's two blocks: one fills the partial parent, the next
    # comes from a new parent; afterwards owner 2 keeps using its own parent
    st_, more = a.alloc(1, 2, 1)
    assert a.views[1].page_parent[more[0]] in bases
    check_invariants(a)


def test_request_prefers_parent_it_already_uses():
    a = three_level()
    _, o1 = a.alloc(0, 10, 1)                 # expert page, huge 0 slot 0
    _, o2 = a.alloc(0, 11, 2)                 # slots 1, 2
    a.free(0, 10)                             # slot 0 free again
    _, o3 = a.alloc(0, 11, 1)                 # owner 11 extends in huge 0 (lowest slot)
    assert o3 == [0]
    check_invariants(a)


def test_reclaim_merges_back_in_reverse():
    a = three_level()
    a.alloc(0, 1, 3)
    a.alloc(1, 2, 5)
    a.alloc(1, 3, 4)
    check_invariants(a)
    for vid, o in ((1, 2), (0, 1), (1, 3)):
        assert a.free(vid, o) == OK
        check_invariants(a)
    assert list(a.free_huge) == list(range(a.n_huge))
    assert all(not v.parents for v in a.views)
    assert a.stats()["bytes_free"] == a.n_huge * a.huge


def test_enomem_is_all_or_nothing():
    a = three_level(pool=2 * 4 * 64 * KB)     # two huge pages = 8 expert pages
    assert a.alloc(0, 1, 5)[0] == OK
    before = snapshot(a)
    assert a.alloc(0, 2, 4) == (ENOMEM, [])
    assert snapshot(a) == before
    assert a.alloc(1, 3, 6)[0] == OK          # the 3 free expert pages as 6 KV blocks
    assert a.alloc(1, 4, 1)[0] == ENOMEM
    check_invariants(a)


def test_error_codes():
    a = three_level()
    assert a.free(0, 5) == EINVAL             # owner holds nothing
    assert a.alloc(0, 1, 0)[0] == EINVAL
    assert a.alloc(0, SPLIT, 1)[0] == EINVAL  # reserved owner id
    assert a.alloc(9, 1, 1)[0] == EINVAL
    assert a.alloc(0, 1, 1)[0] == OK
    assert a.free(0, 1) == OK and a.free(0, 1) == EINVAL   # double free


def test_budgets_and_transfer():
    a = three_level()
    assert a.set_budget(0, 4 * 64 * KB) == OK
    assert a.set_budget(1, 0) == OK
    assert a.alloc(1, 1, 1)[0] == ENOMEM       # KV has no budget yet
    assert a.transfer(0, 1, 64 * KB) == OK
    assert a.alloc(1, 1, 2)[0] == OK
    assert a.alloc(1, 2, 1)[0] == ENOMEM
    assert a.alloc(0, 3, 3)[0] == OK          # 3 of the 3 remaining expert pages
    assert a.transfer(0, 1, 64 * KB) == EBUSY  # would leave the experts short
    assert a.set_budget(1, 32 * KB) == EBUSY   # below what KV holds
    assert a.transfer(1, 0, 64 * KB) == EBUSY
    a.free(1, 1)
    assert a.transfer(1, 0, 64 * KB) == OK
    check_invariants(a)


def test_tail_waste_counted():
    a = Allocator(5 * 2 * 1024 * KB + 123 * 128, 2 * 1024 * KB)
    a.map_view(KIND_EXPERT, 2 * 1024 * KB)
    a.map_view(KIND_CONV, 48 * KB, 0)
    a.map_view(KIND_SSM, 1024 * KB)
    assert a.alloc(1, 1, 50)[0] == OK          # 42 in the first parent, 8 in a second
    assert a.alloc(2, 2, 1)[0] == OK
    s = a.stats()
    assert s["waste_bytes"] == 123 * 128 + 2 * (2048 - 42 * 48) * KB
    check_invariants(a)


ops = st.lists(st.tuples(st.integers(0, 2), st.integers(0, 11), st.integers(1, 9), st.booleans()),
               min_size=1, max_size=120)


@settings(max_examples=150, deadline=None)
@given(ops)
def test_random_streams_keep_invariants_and_replay(stream):
    def run():
        a = Allocator(6 * 256 * KB + 5 * 128, 256 * KB)
        a.map_view(KIND_EXPERT, 64 * KB)
        a.map_view(KIND_KV, 16 * KB, 0)
        a.map_view(KIND_SSM, 128 * KB)
        log = []
        for vid, owner, n, is_free in stream:
            if is_free:
                log.append(a.free(vid, owner))
            else:
                before = snapshot(a)
                st_, offs = a.alloc(vid, owner, n)
                if st_ == ENOMEM:
                    assert snapshot(a) == before
                log.append((st_, tuple(offs)))
            check_invariants(a)
        return a, log

    a, log1 = run()
    _, log2 = run()
    assert log1 == log2
    # freeing everything merges the pool back to whole huge pages
    for v in a.views:
        for o in [o for o in list(v.owner_pages) if o < SPLIT]:
            assert a.free(v.vid, o) == OK
            check_invariants(a)
    assert list(a.free_huge) == list(range(a.n_huge))


def test_kv_requests_fill_whole_parents_first():
    # U{1..128}-block requests on 96-slot parents: every parent but the
    # newest is full while only grants happen (lowest address first).
    a = Allocator(64 * 3 * 1024 * KB, 3 * 1024 * KB)
    a.map_view(KIND_EXPERT, 3 * 1024 * KB)
    a.map_view(KIND_KV, 32 * KB, 0)
    r = np.random.default_rng(0)
    for i in range(40):
        assert a.alloc(1, 100 + i, int(r.integers(1, 129)))[0] == OK
    v = a.views[1]
    bases = sorted(v.parents)
    assert all(v.parents[b].used == v.nslots for b in bases[:-1])
    check_invariants(a)
