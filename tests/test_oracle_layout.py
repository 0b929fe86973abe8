"""Pins for the reference layout recipes and the workload registry."""
import json
import os

import numpy as np
import pytest

from moe_inputs import CONFIGS, gen
from moe_inputs.configs import lcm
from oracle.allocator import SPLIT
from oracle.layout import Layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table1_shapes.json")


def test_configs_follow_table1():
    t1 = json.load(open(GOLDEN))
    q3, q35 = t1["Qwen3-30B-A3B"], t1["Qwen3.5-35B-A3B"]
    for cid in (2, 4, 5):
        c = CONFIGS[cid]
        assert [c.H, c.I] == q3["w1"] == q3["w3"] and [c.I, c.H] == q3["w2"]
        kv = c.view("kv").page_bytes
        assert kv == 16 * np.prod(q3["kv"]) * 2         # 16-token bf16 blocks
        assert q3["ssm"] is None and q3["conv"] is None
    c = CONFIGS[3]
    assert [c.H, c.I] == q35["w1"] and [c.I, c.H] == q35["w2"]
    assert c.view("kv").page_bytes == 16 * np.prod(q35["kv"]) * 2
    assert c.view("ssm").page_bytes == np.prod(q35["ssm"]) * 2
    assert c.view("conv").page_bytes == np.prod(q35["conv"]) * 2
    # huge pages are a common multiple of the expert and state page sizes
    assert c.huge_bytes == lcm(c.page_bytes, c.view("ssm").page_bytes)
    for cid in (1, 2, 4, 5):
        c = CONFIGS[cid]
        assert c.huge_bytes % lcm(c.page_bytes, c.view("kv").page_bytes) == 0
    assert CONFIGS[4].P == 48 and CONFIGS[1].P == 8


def _check_layout(L):
    cfg = L.cfg
    pt = L.page_table()
    a = L.alloc
    # expert pages: distinct, inside the pool, never shared with another view
    pages = pt.reshape(-1).astype(np.int64)
    assert len(np.unique(pages)) == pages.size
    assert pages.min() >= 0 and (pages.max() + 1) * cfg.page_bytes <= a.n_huge * a.huge
    ev = L.vid["expert"]
    expert_ranges = set(int(p) * cfg.page_bytes for p in pages)
    for v in a.views:
        for o, offs in v.owner_pages.items():
            if o >= SPLIT or v.vid == ev:
                continue
            for off in offs:
                base = off - off % cfg.page_bytes
                assert base not in expert_ranges
    s = a.stats()
    assert sum(s["bytes_per_kind"]) + s["bytes_free"] + s["waste_bytes"] == cfg.pool_bytes
    assert s["bytes_per_kind"][0] == cfg.E * 3 * cfg.proj_bytes
    return pt


def test_tiny_layout_is_a_seeded_scatter():
    cfg = CONFIGS[1]
    pt = _check_layout(Layout(cfg).run())
    # 192 of the 256 pages hold expert weights, the other 64 pages are 16 KV blocks
    assert sorted(pt.reshape(-1).tolist()) != list(range(192))
    assert len(set(pt.reshape(-1).tolist())) == 192 and pt.max() < 256
    # pages of one projection are not consecutive
    assert not all(np.all(np.diff(pt[e, p]) == 1) for e in range(8) for p in range(3))
    pt2 = Layout(cfg).run().page_table()
    assert np.array_equal(pt, pt2)                      # deterministic replay


@pytest.mark.parametrize("cid", [2, 3])
def test_fill_then_place_layouts(cid):
    L = Layout(CONFIGS[cid]).run()
    pt = _check_layout(L)
    s = L.alloc.stats()
    assert s["bytes_per_kind"][1] > 0                   # KV filler remains interleaved
    if cid == 3:
        assert s["bytes_per_kind"][2] > 0 and s["bytes_per_kind"][3] > 0
    # expert pages are spread over the pool, not packed at the front
    assert pt.max() > 0.9 * L.alloc.n_huge


@pytest.mark.slow
def test_churn_layout_fragments_projections():
    cfg = CONFIGS[4]
    L = Layout(cfg).run()
    pt = _check_layout(L)
    breaks = sum(int(np.sum(np.diff(pt[e, p]) != 1)) for e in range(cfg.E) for p in range(3))
    assert breaks > cfg.E                                # projections are split across runs
    s = L.alloc.stats()
    assert s["bytes_per_kind"][1] > 0


def test_adjuster_steps_never_move_experts():
    cfg = CONFIGS[5]
    L = Layout(cfg).run()
    pt0 = L.page_table()
    L.init_budgets()
    sizes = gen.adjuster_kv_requests(cfg, 16)
    moved = []
    for f, d in gen.adjuster_plan(cfg, 16):
        moved.append(L.adjuster_step(f, d, sizes))
        assert np.array_equal(L.page_table(), pt0)
        a = L.alloc
        for v in a.views:
            assert v.budget is not None and v.used * v.page <= v.budget
    assert sum(moved) > 0.1 * cfg.pool_bytes
