"""The layer under the workload-aware adjuster (Rimuru paper summary,
abstract and Figure 8; explainer, paragraph on the adjuster): over a
synthetic concurrency profile the KV view grows and shrinks, experts are
evicted and come back through uploads into fresh pages, KV blocks land on
pages experts gave up, and every step's layer call must still read exactly
its experts' weights.

Checks, on the GPU through the C ABI, at every step:
  - the needed experts are resident, their uploads done before the layer;
  - KV blocks allocated in the step are filled with a NaN pattern (any read
    of them by the layer would make y non-finite);
  - routing equals the oracle's and y matches the oracle layer computed from
    the host copy of the weights (contiguous layout, independent of the
    device pool);
  - the allocator stays consistent (pool check).
"""
import numpy as np
import pytest
import torch

from gpu_common import POISON, decode_dev, rel_err, say, to_dev_bits
from moe_inputs import gen
from moe_inputs.configs import MoEConfig, ViewSpec
from oracle.moe import moe_forward, route
from paged_moe_expert_amd import rimuru as R
from paged_moe_expert_amd._lib import VIEW_EXPERT, VIEW_KV

pytestmark = pytest.mark.gpu

KIB = 1024
PAGE = 64 * KIB            # one bf16 projection of 256 x 128
KVB = 16 * KIB
N_HUGE = 192
# KV blocks demanded per step: a rise past the KV budget, a drain, a second spike
DEMAND = [40, 200, 420, 640, 760, 700, 380, 120, 10, 0, 300, 720, 560, 90, 0]


def _cfg():
    return MoEConfig(cid=92, name="adjuster-small", T=2, E=32, k=4, H=256, I=128, dtype="bf16",
                     page_bytes=PAGE, huge_bytes=PAGE, pool_bytes=N_HUGE * PAGE,
                     views=(ViewSpec("expert", VIEW_EXPERT, PAGE, None),
                            ViewSpec("kv", VIEW_KV, KVB, "expert")),
                     layout="scatter", logits="zipf", zipf_s=1.2)


def test_layer_follows_the_adjuster():
    cfg = _cfg()
    E, k, H, I, T = cfg.E, cfg.k, cfg.H, cfg.I, cfg.T
    proj = H * I * 2
    assert proj == PAGE
    pool_h = R.pool_create(cfg.pool_bytes, PAGE)
    xv = R.view_map(pool_h, VIEW_EXPERT, PAGE, None)
    kv = R.view_map(pool_h, VIEW_KV, KVB, xv)
    for e in range(E):
        for p in range(3):
            R.view_alloc(xv, 3 * e + p, 1)
    xb_budget = E * 3 * PAGE
    assert R.view_set_budget(xv, xb_budget) == R.OK
    assert R.view_set_budget(kv, N_HUGE * PAGE - xb_budget) == R.OK
    adj = R.adjuster_create(pool_h, xv, kv, E, 1, min_resident=12, headroom_blocks=4,
                            return_blocks=8, shift=2, max_prefetch=2)

    wb = gen.all_weight_bits(cfg)                              # [E, 3, H*I] bf16 bits
    host_w = torch.from_numpy(wb.view(np.uint8).reshape(E, 3, proj).copy()).pin_memory()
    dev = torch.device("cuda:0")
    pool = torch.empty(cfg.pool_bytes, dtype=torch.uint8, device=dev)
    pool.view(torch.int32).fill_(POISON)
    side = torch.cuda.Stream(device=dev)

    def rows_of(e):
        return np.array([R.view_pages(xv, 3 * e + p) // PAGE for p in range(3)], dtype=np.int32)

    def upload(es):
        for e in es:
            R.expert_upload(pool, rows_of(e), PAGE, host_w[e], stream=side)
        side.synchronize()

    upload(range(E))                                           # initial residency
    # the oracle's weights: the host copy in the contiguous layout
    w_pool = wb.view(np.uint8).reshape(-1)
    pt_contig = np.arange(E * 3, dtype=np.int32).reshape(E, 3, 1)

    kv_owners = []                                             # (owner, offsets), newest last
    blocks_view = pool.view(torch.int32).view(-1, KVB // 4)
    stats = {"evicted": 0, "loaded": 0, "grew": 0, "gave": 0}
    for s, demand in enumerate(DEMAND):
        lg = gen.logits(cfg, T, seed_key=s)
        ids, _ = route(lg, k)
        routed = np.bincount(ids.ravel(), minlength=E).astype(np.int32)
        needed = (routed > 0).astype(np.uint8)
        r = R.adjuster_step(adj, demand, routed, needed)
        say(f"[adjuster] step {s}: demand {demand} blocks, evicted {r['evicted']}, "
            f"loaded {r['loaded']}, kv_moved {r['kv_moved'] // KVB} blocks")
        stats["evicted"] += len(r["evicted"])
        stats["loaded"] += len(r["loaded"])
        stats["grew"] += r["kv_moved"] > 0
        stats["gave"] += r["kv_moved"] < 0
        upload(r["loaded"])                                    # demand loads and prefetches
        for e in r["loaded"]:
            R.adjuster_upload_done(adj, e)
        resident = R.adjuster_state(adj)[0]
        assert all(resident[e] for e in range(E) if needed[e])

        # KV blocks follow the demand within the budget; new blocks get NaN
        _, kb = R.view_usage(kv)
        target = min(demand, kb // KVB)
        held = sum(len(o[1]) for o in kv_owners)
        while kv_owners and held > target:
            o, offs = kv_owners.pop()
            R.view_free(kv, o)
            held -= len(offs)
        if target > held:
            st, offs = R.view_alloc_status(kv, (1 << 40) + s, target - held)
            if st == R.OK:
                kv_owners.append(((1 << 40) + s, offs))
                idx = torch.from_numpy(offs // KVB).to(dev)
                blocks_view.index_fill_(0, idx, POISON)
        R.pool_check(pool_h)

        # the layer on this step's page table: resident experts' pages; the
        # rest point at page 0 and are never read (no token routes to them)
        pt = np.zeros((E, 3, 1), dtype=np.int32)
        for e in range(E):
            if resident[e]:
                pt[e] = rows_of(e)
        x = gen.x_bits(cfg, T, seed_key=s)
        b = R.fused_moe_paged(to_dev_bits(x, "bf16"), torch.from_numpy(lg).to(dev), pool,
                              torch.from_numpy(pt).to(dev), PAGE, k, I)
        torch.cuda.synchronize()
        y = decode_dev(b.y)
        assert np.isfinite(y).all(), f"step {s}: the layer read a non-expert page"
        assert np.array_equal(b.topk_ids.cpu().numpy(), ids)
        ref = moe_forward(x, lg, w_pool, pt_contig, PAGE, E=E, k=k, H=H, I=I, dtype="bf16")
        err = rel_err(y, ref["y"])
        assert err <= 1e-2, f"step {s}: rel_err {err:.3e}"
    say(f"[adjuster] totals {stats}")
    assert stats["evicted"] > 0 and stats["loaded"] > 0 and stats["grew"] > 0 and stats["gave"] > 0
