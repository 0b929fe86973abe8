"""The C++ allocator makes exactly the decisions of the reference allocator:
same statuses, same offsets, same statistics (bit-exact integer parity)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from moe_inputs import CONFIGS, gen
from oracle.allocator import Allocator
from oracle.layout import Layout
from paged_moe_expert_amd import rimuru as R
from paged_moe_expert_amd.layouts import DeviceLayout

KB = 1024

ops = st.lists(st.tuples(st.integers(0, 3), st.integers(0, 9), st.integers(1, 12),
                         st.sampled_from(["alloc", "free", "budget", "transfer"]),
                         st.integers(0, 40)),
               min_size=1, max_size=150)


def _pair():
    ref = Allocator(5 * 512 * KB + 3 * 128, 512 * KB)
    dev = R.pool_create(5 * 512 * KB + 3 * 128, 512 * KB)
    spec = [(0, 64 * KB, None), (1, 16 * KB, 0), (2, 256 * KB, None), (3, 48 * KB, 0)]
    views = []
    for kind, page, parent in spec:
        assert ref.map_view(kind, page, parent)[0] == 0
        views.append(R.view_map(dev, kind, page, None if parent is None else views[parent]))
    return ref, dev, views


@settings(max_examples=120, deadline=None)
@given(ops)
def test_random_streams_bit_exact(stream):
    ref, dev, views = _pair()
    for vid, owner, n, op, amount in stream:
        v = views[vid]
        if op == "alloc":
            s1, o1 = ref.alloc(vid, owner, n)
            s2, o2 = R.view_alloc_status(v, owner, n)
            assert s1 == s2 and list(o1) == o2.tolist()
        elif op == "free":
            assert ref.free(vid, owner) == R.view_free_status(v, owner)
        elif op == "budget":
            b = None if amount == 0 else amount * 16 * KB
            assert ref.set_budget(vid, b) == R.view_set_budget(v, b)
        else:
            dst = (vid + 1) % 4
            assert ref.transfer(vid, dst, amount * 16 * KB) == R.pool_transfer(dev, v, views[dst], amount * 16 * KB)
        assert ref.stats() == R.pool_stats(dev)
    R.pool_check(dev)
    for vid in range(4):
        for owner in range(10):
            assert ref.pages(vid, owner) == R.view_pages(views[vid], owner).tolist()


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_config_layouts_bit_exact(cid):
    cfg = CONFIGS[cid]
    ref = Layout(cfg).run()
    dev = DeviceLayout(cfg).run()
    assert np.array_equal(ref.page_table(), dev.page_table())
    assert ref.alloc.stats() == R.pool_stats(dev.pool)
    assert ref._ui == dev._ui
    R.pool_check(dev.pool)


@pytest.mark.slow
def test_churn_layout_bit_exact():
    cfg = CONFIGS[4]
    ref = Layout(cfg).run()
    dev = DeviceLayout(cfg).run()
    assert ref.statuses == dev.statuses
    assert np.array_equal(ref.page_table(), dev.page_table())
    assert ref.alloc.stats() == R.pool_stats(dev.pool)
    R.pool_check(dev.pool)


def test_adjuster_steps_bit_exact():
    cfg = CONFIGS[5]
    ref = Layout(cfg).run()
    dev = DeviceLayout(cfg).run()
    ref.init_budgets()
    dev.init_budgets()
    for B in (1, 256):
        s1, s2 = gen.adjuster_kv_requests(cfg, B), gen.adjuster_kv_requests(cfg, B)
        for f, d in gen.adjuster_plan(cfg, B):
            assert ref.adjuster_step(f, d, s1) == dev.adjuster_step(f, d, s2)
            assert ref.alloc.stats() == R.pool_stats(dev.pool)
            assert np.array_equal(ref.page_table(), dev.page_table())
    R.pool_check(dev.pool)


def test_enomem_leaves_pool_unchanged_and_double_free_fails():
    dev = R.pool_create(2 * 256 * KB, 256 * KB)
    ev = R.view_map(dev, 0, 64 * KB)
    kv = R.view_map(dev, 1, 32 * KB, ev)
    R.view_alloc(ev, 1, 5)
    before = R.pool_stats(dev)
    st_, offs = R.view_alloc_status(ev, 2, 4)
    assert st_ == R.ENOMEM and offs.size == 0
    assert R.pool_stats(dev) == before
    assert R.view_alloc(kv, 3, 6).size == 6
    R.view_free(kv, 3)
    assert R.view_free_status(kv, 3) == R.EINVAL
    with pytest.raises(R.RimuruError):
        R.view_map(dev, 1, 32 * KB, None)         # KV cut straight from huge pages
    R.pool_check(dev)
