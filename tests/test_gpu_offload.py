"""Dual-buffer expert upload (Rimuru paper summary, Figure 8): an evicted
expert returns from pinned host memory directly into fresh expert-view pages
while the layer keeps running on the old pages, with no device-to-device copy.

Checks, on the GPU through the C ABI:
  - the fresh pages hold exactly the host bytes afterwards;
  - a layer run concurrently on another stream (old page table) is bitwise
    equal to the layer before the upload (the upload touches only new pages);
  - the layer on the new page table is bitwise equal to the layer before the
    eviction, and matches the oracle: weights moved, results unchanged;
  - the allocator state stays consistent when the old pages are freed.
"""
import numpy as np
import pytest
import torch

from gpu_common import decode_dev, host_pool, record, rel_err, say, to_dev_bits, weights_dev
from moe_inputs.configs import MoEConfig, ViewSpec
from moe_inputs import gen
from oracle.moe import moe_forward
from paged_moe_expert_amd import rimuru as R
from paged_moe_expert_amd._lib import VIEW_EXPERT, VIEW_KV

pytestmark = pytest.mark.gpu

KIB = 1024


def _cfg():
    page = 4 * KIB
    return MoEConfig(cid=91, name="upload-small", T=48, E=16, k=4, H=256, I=128, dtype="bf16",
                     page_bytes=page, huge_bytes=64 * KIB, pool_bytes=8 << 20,
                     views=(ViewSpec("expert", VIEW_EXPERT, page, None),
                            ViewSpec("kv", VIEW_KV, 8 * KIB, None)),
                     layout="scatter", logits="normal")


def _host_pool_bytes(pool_dev):
    return pool_dev.cpu().numpy()


def test_expert_upload_into_fresh_pages():
    cfg = _cfg()
    E, k, H, I, page = cfg.E, cfg.k, cfg.H, cfg.I, cfg.page_bytes
    proj = H * I * 2
    P = proj // page
    pool_h = R.pool_create(cfg.pool_bytes, cfg.huge_bytes)
    ev = R.view_map(pool_h, VIEW_EXPERT, page, None)
    pt = np.zeros((E, 3, P), dtype=np.int32)
    for e in range(E):
        for p in range(3):
            pt[e, p] = R.view_alloc(ev, e * 3 + p, P) // page
    wb = gen.all_weight_bits(cfg)                         # [E, 3, H*I] bf16 bits
    xb, lg = gen.x_bits(cfg, cfg.T), gen.logits(cfg, cfg.T)
    dev = torch.device("cuda:0")
    pool = torch.empty(cfg.pool_bytes, dtype=torch.uint8, device=dev)
    pool.view(torch.int32).fill_(0x7FC07FC0)
    ptd = torch.from_numpy(pt).to(dev)
    R.experts_store(pool, ptd, weights_dev(wb), page)
    x = to_dev_bits(xb, "bf16")
    lgd = torch.from_numpy(lg).to(dev)
    b0 = R.fused_moe_paged(x, lgd, pool, ptd, page, k, I)
    torch.cuda.synchronize()
    y0 = b0.y.clone()

    # evict the most-routed expert: fresh pages first (dual buffer), then the upload
    ids = b0.topk_ids.cpu().numpy()
    victim = int(np.bincount(ids.ravel(), minlength=E).argmax())
    new_rows = np.stack([R.view_alloc(ev, 1000 + p, P) // page for p in range(3)]).astype(np.int32)
    assert not set(new_rows.ravel()) & set(pt[victim].ravel())
    host = torch.from_numpy(wb[victim].view(np.uint8).reshape(3, proj).copy()).pin_memory()
    side = torch.cuda.Stream()
    say(f"[upload] victim expert {victim}, {3 * P} pages, layer on the old pages meanwhile")
    R.expert_upload(pool, new_rows, page, host, stream=side)
    b_during = R.fused_moe_paged(x, lgd, pool, ptd, page, k, I)   # current stream, old page table
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(b_during.y, y0)

    pool_host = _host_pool_bytes(pool)
    for p in range(3):
        got = np.concatenate([pool_host[q * page:(q + 1) * page] for q in new_rows[p]])[:proj]
        assert np.array_equal(got, wb[victim, p].view(np.uint8)), f"projection {p}"

    pt2 = pt.copy()
    pt2[victim] = new_rows
    b1 = R.fused_moe_paged(x, lgd, pool, torch.from_numpy(pt2).to(dev), page, k, I)
    torch.cuda.synchronize()
    assert torch.equal(b1.y, y0)                          # weights moved, results unchanged
    # the oracle's pool: the generator's weights placed on the host at the
    # new page table's pages (nothing read back from the device)
    ref = moe_forward(xb, lg, host_pool(cfg.pool_bytes, page, pt2, wb), pt2, page, E=E, k=k, H=H, I=I,
                      dtype="bf16")
    err = rel_err(decode_dev(b1.y), ref["y"])
    say(f"[upload] rel_err vs oracle {err:.3e}")
    record("expert upload, layer on the new pages", err, 1e-2)
    assert err <= 1e-2

    # eviction completes: the old pages return to the view
    for p in range(3):
        R.view_free(ev, victim * 3 + p)
    R.pool_check(pool_h)


def test_expert_upload_page_runs():
    """Destination pages in runs of several lengths, in descending order and
    with a partial last page: every page gets exactly its slice of the host
    bytes, the rest of the pool (the partial page's tail included) keeps its
    poison."""
    page, P = 4 * KIB, 6
    proj = 5 * page + page // 2                           # the last page half used
    pool_bytes = 64 * page
    rows = np.array([[10, 11, 12, 20, 21, 5],             # runs of 3, 2, 1
                     [40, 39, 38, 37, 36, 35],            # descending: six runs of one
                     [50, 51, 52, 53, 54, 55]],           # one run, crossing the projection's end
                    dtype=np.int32)
    rng = np.random.default_rng(77)
    src = rng.integers(0, 256, size=3 * proj, dtype=np.uint8)
    host = torch.from_numpy(src.reshape(3, proj).copy()).pin_memory()
    dev = torch.device("cuda:0")
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.view(torch.int32).fill_(0x7FC07FC0)
    poison = pool[:page].cpu().numpy().copy()
    say("[upload] page runs: 3+2+1, six descending, one run past the projection's end")
    side = torch.cuda.Stream()
    R.expert_upload(pool, rows, page, host, stream=side)
    side.synchronize()
    got = pool.cpu().numpy()
    expect = np.tile(poison, pool_bytes // page)
    for p in range(3):
        for q in range(P):
            off = q * page
            n = min(page, proj - off)
            expect[rows[p, q] * page:rows[p, q] * page + n] = src[p * proj + off:p * proj + off + n]
    assert np.array_equal(got, expect)
