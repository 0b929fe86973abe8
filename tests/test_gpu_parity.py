"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars: top-k ids and per-expert lists bit-exact; weights within 2e-6
(relative) and summing to one within 1e-6; y within a row-wise max-norm
relative error of 1e-2 for bf16 and 1e-4 for fp32; paged and contiguous
layouts bitwise equal; repeated runs bitwise equal.
"""
from dataclasses import replace

import numpy as np
import pytest

from moe_inputs import CONFIGS, gen
from moe_inputs.configs import CFG1, KIB

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    from gpu_common import (Case, check_routing, contiguous_pool, decode_dev, host_pool, paged_pool,
                            record, rel_err, run, say, to_dev_bits, weights_dev)
    from oracle.moe import moe_forward
    from paged_moe_expert_amd import rimuru as R

TOL = {"bf16": 1e-2, "f32": 1e-4}


# ---------------------------------------------------------------- custom shapes

def _custom(name, E, k, H, I, T, dtype, page, bias=None, seed=0):
    """A shape outside the registry, on a seeded random page permutation."""
    cfg = replace(CFG1, cid=100 + seed, name=name, E=E, k=k, H=H, I=I, T=T, dtype=dtype,
                  page_bytes=page, logits="normal")
    es = cfg.es
    P = -(-H * I * es // page)
    n_pages = E * 3 * P + 7
    r = np.random.default_rng(1000 + seed)
    pt = r.permutation(n_pages)[:E * 3 * P].astype(np.int32).reshape(E, 3, P)
    wb = gen.all_weight_bits(cfg)
    xb = gen.x_bits(cfg, T)
    lg = gen.logits(cfg, T)
    if bias is not None:
        lg = (lg + np.asarray(bias, dtype=np.float32)[None, :E]).astype(np.float32)
    return cfg, P, n_pages, pt, wb, xb, lg


def _padded_weights(wb, P, page):
    # weights tensor padded to P*page bytes per projection for the store call
    es = wb.dtype.itemsize
    E = wb.shape[0]
    padded = np.zeros((E, 3, P * page // es), dtype=wb.dtype)
    padded[:, :, :wb.shape[2]] = wb
    return padded


CUSTOM = [
    # name, E, k, H, I, T, dtype, page, bias
    ("bf16-decode-tiles", 16, 4, 256, 128, 40, "bf16", 4 * KIB, None),
    ("bf16-mid-tiles", 16, 4, 256, 128, 300, "bf16", 4 * KIB, None),
    ("bf16-mid-odd-page", 16, 4, 256, 128, 300, "bf16", 12 * KIB, None),
    ("bf16-big-tiles", 16, 4, 256, 128, 1000, "bf16", 4 * KIB, None),
    ("bf16-big-skewed", 16, 4, 256, 128, 1000, "bf16", 8 * KIB, [4, 3, 2.5, 2] + [0] * 10 + [-50, -50]),
    ("f32-mid-tiles", 8, 2, 128, 64, 500, "f32", 4 * KIB, None),
    ("f32-big-tiles", 8, 2, 128, 64, 1500, "f32", 4 * KIB, None),
    ("bf16-narrow-inter-big-tiles", 8, 2, 128, 64, 1500, "bf16", 4 * KIB, None),
    ("bf16-k1", 4, 1, 128, 64, 33, "bf16", 4 * KIB, None),
    ("bf16-k-equals-E", 8, 8, 128, 192, 19, "bf16", 4 * KIB, None),
    ("bf16-one-expert", 1, 1, 192, 64, 50, "bf16", 4 * KIB, None),
    ("bf16-128B-pages", 4, 2, 64, 64, 21, "bf16", 128, None),
    ("bf16-one-token", 16, 4, 256, 128, 1, "bf16", 4 * KIB, None),
    # 4 tokens x 8 experts of 40 on one 64 KiB page a projection: the gate/up
    # stream routes the batch itself with the page table staged in LDS, and
    # the expert count is not a multiple of the 64 lanes that select
    ("bf16-routed-stream-one-page", 40, 8, 256, 128, 4, "bf16", 64 * KIB, None),
    # 24576 pages per projection: too many to stage in LDS, read from global
    ("bf16-huge-page-table", 2, 1, 2048, 768, 300, "bf16", 128, None),
    ("bf16-huge-page-table-decode", 2, 1, 2048, 768, 8, "bf16", 128, None),
    # 128-row plan with 256-column gate/up and 512-column down tiles
    ("bf16-pipelined-tiles", 8, 2, 512, 256, 1200, "bf16", 4 * KIB, None),
    ("bf16-pipelined-odd-page-skewed", 8, 2, 512, 512, 1500, "bf16", 12 * KIB, [3, 2, 1, 0, 0, 0, -1, -40]),
    ("bf16-pipelined-many-experts", 32, 4, 512, 256, 1400, "bf16", 64 * KIB, None),
    # the persistent prefill GEMM: several tiles per workgroup (tile contexts
    # and copies running on from one tile into the next), the shortest K it
    # takes (6 stages), and 12 KiB pages whose boundaries cut 512-byte row
    # pieces under skewed routing
    ("bf16-pf-many-tiles", 8, 2, 512, 256, 40000, "bf16", 4 * KIB, None),
    ("bf16-pf-short-k", 4, 2, 192, 256, 3000, "bf16", 4 * KIB, None),
    ("bf16-pf-skewed-odd-page", 16, 4, 512, 512, 20000, "bf16", 12 * KIB, [4, 3, 2.5, 2, 1] + [0] * 9 + [-3, -50]),
    # the 128-row asynchronous-pipeline GEMM, where the persistent one does
    # not take the shape: gate/up over 768 pages a projection (more page
    # addresses than a persistent tile context holds), and a down GEMM of
    # K = 128 (four 32-deep stages, fewer than the persistent ring needs)
    ("bf16-pipelined-long-page-table", 8, 2, 1024, 1536, 1000, "bf16", 4 * KIB, None),
    ("bf16-pipelined-short-down", 8, 2, 512, 128, 1200, "bf16", 4 * KIB, None),
    # the persistent GEMM on 64-row tiles (few rows per expert, weight-bound)
    ("bf16-pf64-tiles", 64, 8, 512, 256, 1000, "bf16", 8 * KIB, None),
    ("bf16-pf64-skewed-odd-page", 32, 4, 512, 512, 1200, "bf16", 12 * KIB, [3, 2, 1.5, 1] + [0] * 26 + [-2, -40]),
    # the weight stream on 32-row tiles (9 to 24 routed rows an expert on
    # average): a fragmented page table, and one page a projection with
    # skewed routing (experts past 32 rows take several tiles, some none)
    ("bf16-stream32-tiles", 16, 4, 256, 128, 80, "bf16", 4 * KIB, None),
    ("bf16-stream32-skewed-one-page", 16, 4, 256, 128, 90, "bf16", 64 * KIB, [3, 2.5, 2] + [0] * 11 + [-40, -40]),
    # the 16-row weight stream's down GEMM over many pages with 12 steps a
    # wavefront (K = 1536), where it takes 128-column tiles
    ("bf16-decode-long-down", 64, 4, 512, 1536, 64, "bf16", 4 * KIB, None),
    # count and sort of many slots cut into ranges (two here), with T*k not a
    # multiple of 4 (the unvectorised scans)
    ("bf16-split-sort-odd-slots", 8, 3, 128, 64, 5001, "bf16", 4 * KIB, None),
    # the shape limits: 512 experts, top-32 (8 logits a lane in gating, a
    # 32-row combine), with a wavefront per token and with one-workgroup routing
    ("bf16-max-experts-and-k", 512, 32, 128, 64, 50, "bf16", 4 * KIB, None),
    ("bf16-max-experts-and-k-8-tokens", 512, 32, 128, 64, 8, "bf16", 4 * KIB, None),
]


@pytest.mark.parametrize("spec", CUSTOM, ids=[c[0] for c in CUSTOM])
def test_custom_shapes_against_oracle(spec):
    name, E, k, H, I, T, dtype, page, bias = spec
    say(f"[custom] {name}: E={E} k={k} H={H} I={I} T={T} {dtype} page={page}")
    cfg, P, n_pages, pt, wb, xb, lg = _custom(name, E, k, H, I, T, dtype, page, bias,
                                               seed=CUSTOM.index(spec))
    wdev = weights_dev(_padded_weights(wb, P, page))
    pool, ptd = paged_pool(n_pages * page, pt, wdev, page)
    x = to_dev_bits(xb, dtype)
    lgd = torch.from_numpy(lg).cuda()
    bufs = R.fused_moe_paged(x, lgd, pool, ptd, page, k, I)
    torch.cuda.synchronize()
    ref = moe_forward(xb, lg, host_pool(n_pages * page, page, pt, wb), pt, page, E=E, k=k, H=H, I=I,
                      dtype=dtype)
    check_routing(bufs, ref, T, k, E, bufs.block_m)
    y = decode_dev(bufs.y)
    assert np.isfinite(y).all()
    err = rel_err(y, ref["y"])
    say(f"[custom] {name}: block_m={bufs.block_m} rel_err={err:.3e}")
    record(f"custom {name} (block_m {bufs.block_m})", err, TOL[dtype])
    assert err <= TOL[dtype]
    # paged == contiguous, bitwise
    cpool = wdev.view(torch.uint8).reshape(-1)
    cpt = torch.arange(E * 3 * P, dtype=torch.int32, device="cuda").reshape(E, 3, P)
    b2 = R.fused_moe_paged(x, lgd, cpool, cpt, page, k, I)
    torch.cuda.synchronize()
    assert torch.equal(b2.y, bufs.y)


@pytest.mark.parametrize("T", [3, 8, 40, 4096],
                         ids=["routing-in-gate-up-stream", "one-workgroup-routing", "gating-and-sort", "gating-count-sort"])
def test_tied_and_signed_zero_logits(T):
    """Logits drawn from {-1, -0.0, +0.0, 0.5, 1} (seeded): most tokens have
    ties at the top-k boundary and between -0 and +0. The kernels must keep
    the lower expert index on a tie and treat -0 as +0, exactly as the
    oracle's route does (3 tokens: the gate/up stream routes the batch
    itself, over several pages a projection; 8 tokens: one-workgroup
    routing; 40: gating and the self-counting sort; 4096: gating, count and
    sort)."""
    E, k, H, I, page = 16, 4, 256, 128, 4 * KIB
    name = f"bf16-ties-T{T}"
    cfg, P, n_pages, pt, wb, xb, _ = _custom(name, E, k, H, I, T, "bf16", page, seed=50 + T)
    r = np.random.default_rng(77 + T)
    lg = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], dtype=np.float32)[r.integers(0, 5, size=(T, E))]
    assert np.signbit(lg).any() and (lg == 0).any()
    wdev = weights_dev(_padded_weights(wb, P, page))
    pool, ptd = paged_pool(n_pages * page, pt, wdev, page)
    x = to_dev_bits(xb, "bf16")
    bufs = R.fused_moe_paged(x, torch.from_numpy(lg).cuda(), pool, ptd, page, k, I)
    torch.cuda.synchronize()
    ref = moe_forward(xb, lg, host_pool(n_pages * page, page, pt, wb), pt, page, E=E, k=k, H=H, I=I, dtype="bf16")
    check_routing(bufs, ref, T, k, E, bufs.block_m)
    err = rel_err(decode_dev(bufs.y), ref["y"])
    say(f"[ties] T={T}: rel_err={err:.3e}")
    record(f"ties T={T}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------- registry configs

@pytest.fixture(scope="module")
def tiny():
    return Case(CONFIGS[1])


def test_tiny_fp32_full_parity(tiny):
    say("[cfg1] tiny fp32 layer, seeded scatter over a 256-page pool")
    c = tiny
    assert np.array_equal(c.pt, c.pt_ref)
    bufs = c.run()
    ref = c.oracle()
    check_routing(bufs, ref, c.T, c.cfg.k, c.cfg.E, bufs.block_m)
    err = rel_err(decode_dev(bufs.y), ref["y"])
    say(f"[cfg1] rel_err={err:.3e}")
    record("tiny fp32 layer, all tokens", err, TOL["f32"])
    assert err <= TOL["f32"]


def test_tiny_paged_equals_contiguous_and_repeats(tiny):
    c = tiny
    a = c.run()
    ya = a.y.clone()
    b = c.run()
    assert torch.equal(b.y, ya)                       # run to run
    pool, ptd = contiguous_pool(c.cfg, c.wdev)
    cc = c.run(pool=pool, ptd=ptd)
    assert torch.equal(cc.y, ya)                      # paged == contiguous


def test_tiny_token_permutation_equivariance(tiny):
    c = tiny
    base = c.run().y.clone()
    perm = torch.randperm(c.T, generator=torch.Generator().manual_seed(3)).cuda()
    out = R.fused_moe_paged(c.x[perm].contiguous(), c.lgd[perm].contiguous(), c.pool, c.ptd,
                            c.cfg.page_bytes, c.cfg.k, c.cfg.I)
    torch.cuda.synchronize()
    assert torch.equal(out.y, base[perm])


def test_poisoned_idle_expert_pages_never_reach_output(tiny):
    c = tiny
    lg = c.lg.copy()
    lg[:, 6:] = -1e30                                  # experts 6, 7 get no tokens
    lgd = torch.from_numpy(lg).cuda()
    out0 = R.fused_moe_paged(c.x, lgd, c.pool, c.ptd, c.cfg.page_bytes, c.cfg.k, c.cfg.I)
    torch.cuda.synchronize()
    y0 = out0.y.clone()
    pool = c.pool.clone()
    pv = pool.view(torch.int32)
    P, page = c.cfg.P, c.cfg.page_bytes
    for e in (6, 7):
        for p in range(3):
            for q in range(P):
                a = int(c.pt[e, p, q]) * page // 4
                pv[a:a + page // 4] = 0x7FC07FC0
    out1 = R.fused_moe_paged(c.x, lgd, pool, c.ptd, page, c.cfg.k, c.cfg.I)
    torch.cuda.synchronize()
    assert torch.isfinite(out1.y).all()
    assert torch.equal(out1.y, y0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_configs(cid):
    """Every output row of the full-size layers against the oracle: all 64
    decode tokens, all 2048 tokens of the Qwen3.5-shaped prefill and all 8192
    of the fragmented prefill (every row tile of every plan)."""
    cfg = CONFIGS[cid]
    say(f"[cfg{cid}] {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} page={cfg.page_bytes}")
    c = Case(cfg)
    assert np.array_equal(c.pt, c.pt_ref)
    bufs = c.run()
    y = decode_dev(bufs.y)
    assert np.isfinite(y).all()
    say(f"[cfg{cid}] oracle over all {c.T} tokens")
    ref = c.oracle()
    check_routing(bufs, ref, c.T, cfg.k, cfg.E, bufs.block_m)
    err = rel_err(y, ref["y"])
    say(f"[cfg{cid}] block_m={bufs.block_m} rel_err={err:.3e} over all {c.T} tokens")
    record(f"{cfg.name} (block_m {bufs.block_m}), all {c.T} tokens", err, TOL[cfg.dtype])
    assert err <= TOL[cfg.dtype]
    y0 = bufs.y.clone()
    pool, ptd = contiguous_pool(cfg, c.wdev)
    cc = c.run(pool=pool, ptd=ptd)
    assert torch.equal(cc.y, y0), "paged and contiguous layouts differ"
    again = c.run()
    assert torch.equal(again.y, y0), "run-to-run difference"
    if cfg.P > 1:
        # the same weights with one page per projection (page = the whole
        # projection): another page size, the same bytes, the same output
        pt1 = torch.from_numpy(np.arange(cfg.E * 3, dtype=np.int32).reshape(cfg.E, 3, 1)).cuda()
        one = R.fused_moe_paged(c.x, c.lgd, c.wdev.view(torch.uint8).reshape(-1), pt1, cfg.proj_bytes, cfg.k, cfg.I)
        torch.cuda.synchronize()
        assert torch.equal(one.y, y0), "one page per projection differs from the paged layout"


@pytest.mark.timeout(900)
def test_decode_sweep_under_adjuster_steps():
    cfg = CONFIGS[5]
    base = Case(cfg, T=1)
    dl, rl = base.dev_layout, base.ref_layout
    dl.init_budgets()
    rl.init_budgets()
    for B in cfg.batches:
        say(f"[cfg5] batch {B}")
        xb, lg = gen.x_bits(cfg, B), gen.logits(cfg, B)
        x, lgd = to_dev_bits(xb, cfg.dtype), torch.from_numpy(lg).cuda()
        bufs = R.MoeBuffers(B, cfg.E, cfg.k, cfg.H, cfg.I, cfg.P, R.BF16)
        out = run(cfg, x, lgd, base.pool, base.ptd, bufs)
        y0 = out.y.clone()
        ref = moe_forward(xb, lg, base.ref_pool(), base.pt_ref, cfg.page_bytes, E=cfg.E, k=cfg.k,
                          H=cfg.H, I=cfg.I, dtype=cfg.dtype)
        check_routing(out, ref, B, cfg.k, cfg.E, out.block_m)
        err = rel_err(decode_dev(out.y), ref["y"])
        say(f"[cfg5] B={B} rel_err={err:.3e} over all {B} tokens")
        record(f"decode sweep B={B} (block_m {out.block_m}), all tokens", err, TOL["bf16"])
        assert err <= TOL["bf16"]
        s1, s2 = gen.adjuster_kv_requests(cfg, B), gen.adjuster_kv_requests(cfg, B)
        for f, d in gen.adjuster_plan(cfg, B):
            assert dl.adjuster_step(f, d, s1) == rl.adjuster_step(f, d, s2)
            pt = dl.page_table()
            assert np.array_equal(pt, base.pt) and np.array_equal(rl.page_table(), pt)
            ptd = torch.from_numpy(pt.copy()).cuda()        # re-issued page table
            o = run(cfg, x, lgd, base.pool, ptd, bufs)
            assert torch.equal(o.y, y0)
