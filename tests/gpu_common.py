"""Shared set-up for the GPU parity tests: device pools and the checks against
the oracle. Inputs come from moe_inputs only; the oracle gets its own layout
(reference allocator) and its own host pool."""
from __future__ import annotations

import sys

import numpy as np
import torch

from moe_inputs import gen
from oracle.layout import Layout, build_pool
from oracle.moe import moe_forward
from paged_moe_expert_amd import rimuru as R
from paged_moe_expert_amd.layouts import DeviceLayout

from margins import record  # noqa: F401  (re-exported for the GPU tests)

POISON = 0x7FC07FC0          # quiet NaN as fp32 and as two bf16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bits(bits: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).cuda()


def dev_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


def decode_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def weights_dev(wb: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(wb).view(np.int16 if wb.dtype == np.uint16 else np.int32)).cuda()


def paged_pool(pool_bytes: int, pt: np.ndarray, wdev: torch.Tensor, page_bytes: int):
    """Device pool: poison everywhere, expert weights on the pages pt names."""
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    pool.view(torch.int32).fill_(POISON)
    ptd = torch.from_numpy(pt).cuda()
    R.experts_store(pool, ptd, wdev, page_bytes)
    return pool, ptd


def host_pool(pool_bytes: int, page: int, pt: np.ndarray, wb: np.ndarray) -> np.ndarray:
    """The oracle's pool, built on the host from the generator's weight bits
    [E, 3, n] and a page table: zeros everywhere, page q of projection (e, p)
    at pt[e, p, q] * page (the last page of a projection may be partial).
    Nothing in it comes from the device."""
    pool = np.zeros(pool_bytes, dtype=np.uint8)
    raw = np.ascontiguousarray(wb).view(np.uint8).reshape(wb.shape[0], 3, -1)
    nbytes = raw.shape[2]
    for e in range(pt.shape[0]):
        for p in range(3):
            for q in range(pt.shape[2]):
                lo, hi = q * page, min((q + 1) * page, nbytes)
                if lo >= hi:
                    break
                a = int(pt[e, p, q]) * page
                pool[a:a + hi - lo] = raw[e, p, lo:hi]
    return pool


def contiguous_pool(cfg, wdev: torch.Tensor):
    """The contiguous layout: the weight tensor itself, pages in order."""
    pt = np.arange(cfg.E * 3 * cfg.P, dtype=np.int32).reshape(cfg.E, 3, cfg.P)
    return wdev.view(torch.uint8).reshape(-1), torch.from_numpy(pt).cuda()


def run(cfg, x, lg, pool, ptd, bufs=None):
    out = R.fused_moe_paged(x, lg, pool, ptd, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs)
    torch.cuda.synchronize()
    return out


def check_routing(bufs, ref, T, k, E, bm):
    ids = bufs.topk_ids.cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), "top-k ids differ from the oracle"
    w = bufs.topk_w.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(w - ref["w"]) <= 2e-6 * ref["w"]), np.abs(w - ref["w"]).max()
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-6)
    off = bufs.expert_off.cpu().numpy()
    srt = bufs.sorted_ids.cpu().numpy()
    TK = T * k
    assert off[0] == 0
    for e in range(E):
        lst = ref["lists"][e]
        seg = srt[off[e]:off[e + 1]]
        assert off[e + 1] - off[e] == (len(lst) + bm - 1) // bm * bm, f"padding of expert {e}"
        assert np.array_equal(seg[:len(lst)], lst), f"list of expert {e}"
        assert np.all(seg[len(lst):] == TK)


def rel_err(y, y_ref):
    scale = np.abs(y_ref).max(axis=1)
    scale[scale == 0] = 1.0
    return float((np.abs(y - y_ref).max(axis=1) / scale).max())


class Case:
    """One configuration set up on the device and for the oracle."""

    def __init__(self, cfg, T=None, seed_key=0, layout=True):
        self.cfg = cfg
        self.T = cfg.T if T is None else T
        self.xb = gen.x_bits(cfg, self.T, seed_key)
        self.lg = gen.logits(cfg, self.T, seed_key)
        self.wb = gen.all_weight_bits(cfg)
        self.x = to_dev_bits(self.xb, cfg.dtype)
        self.lgd = torch.from_numpy(self.lg).cuda()
        self.wdev = weights_dev(self.wb)
        if layout:
            self.dev_layout = DeviceLayout(cfg).run()
            self.pt = self.dev_layout.page_table()
            self.pool, self.ptd = paged_pool(cfg.pool_bytes, self.pt, self.wdev, cfg.page_bytes)
            self.ref_layout = Layout(cfg).run()
            self.pt_ref = self.ref_layout.page_table()
            self._ref_pool = None

    def ref_pool(self):
        if self._ref_pool is None:
            self._ref_pool = build_pool(self.cfg, self.pt_ref, self.wb, poison=False)
        return self._ref_pool

    def oracle(self, tokens=None):
        c = self.cfg
        return moe_forward(self.xb, self.lg, self.ref_pool(), self.pt_ref, c.page_bytes, E=c.E, k=c.k,
                           H=c.H, I=c.I, dtype=c.dtype, tokens=tokens)

    def run(self, bufs=None, pool=None, ptd=None):
        return run(self.cfg, self.x, self.lgd, self.pool if pool is None else pool,
                   self.ptd if ptd is None else ptd, bufs)
