"""Pins for the fp64 MoE oracle: each test ties the oracle to something other
than itself (brute force, closed forms, library routines, invariants)."""
import math
import struct

import numpy as np
import pytest
from scipy.special import softmax

from moe_inputs import CONFIGS, gen
from oracle import brute
from oracle.layout import Layout, build_pool
from oracle.moe import decode, expert_lists, moe_forward, resolve_projection, route, silu


def _sorted_topk(row, k):
    vals = [float(v) + 0.0 for v in row]
    return sorted(range(len(vals)), key=lambda e: (-vals[e], e))[:k]


# ----------------------------------------------------------------- routing

@pytest.mark.parametrize("seed", range(6))
def test_route_ids_match_python_sort_with_ties(seed):
    r = np.random.default_rng(seed)
    T, E = 40, int(r.integers(2, 40))
    k = int(r.integers(1, E + 1))
    l = r.standard_normal((T, E)).astype(np.float32)
    # plant ties, signed zeros and repeated maxima
    l[::3, 1] = l[::3, 0]
    l[1::4, :] = np.round(l[1::4, :])
    l[2, :] = 0.0
    l[2, ::2] = -0.0
    ids, w = route(l, k)
    for t in range(T):
        assert list(ids[t]) == _sorted_topk(l[t], k)


def test_route_signed_zero_is_a_tie():
    l = np.array([[-0.0, 0.0, -1.0, 0.0]], dtype=np.float32)
    ids, w = route(l, 3)
    assert ids.tolist() == [[0, 1, 3]]
    assert np.allclose(w, 1 / 3, rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(4))
def test_route_invariants(seed):
    r = np.random.default_rng(100 + seed)
    T, E, k = 64, 32, 5
    l = (r.standard_normal((T, E)) * 4).astype(np.float32)
    ids, w = route(l, k)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        sel = l[t, ids[t]]
        rest = np.delete(l[t], ids[t])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(sel) <= 0)                 # rank order
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_route_weights_closed_form_small():
    # logits (ln 3, 0, ln 1/2) with k = 2 keep (ln 3, 0): weights 3/4, 1/4
    l = np.array([[math.log(3.0), 0.0, math.log(0.5)]], dtype=np.float64)
    ids, w = route(l, 2)
    assert ids.tolist() == [[0, 1]]
    assert abs(w[0, 0] - 0.75) < 1e-15 and abs(w[0, 1] - 0.25) < 1e-15


def test_route_k_equals_e_is_full_softmax():
    r = np.random.default_rng(7)
    l = r.standard_normal((16, 12)).astype(np.float32)
    ids, w = route(l, 12)
    ref = softmax(l.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids, w, axis=1)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)


def test_route_renormalised_equals_full_softmax_then_topk():
    r = np.random.default_rng(8)
    l = r.standard_normal((16, 20)).astype(np.float32)
    ids, w = route(l, 4)
    p = softmax(l.astype(np.float64), axis=1)
    kept = np.take_along_axis(p, ids, axis=1)
    assert np.allclose(w, kept / kept.sum(1, keepdims=True), rtol=1e-13, atol=0)


def test_expert_lists_invariants():
    r = np.random.default_rng(9)
    l = r.standard_normal((50, 10)).astype(np.float32)
    ids, _ = route(l, 3)
    lists = expert_lists(ids, 10)
    allf = np.concatenate(lists)
    assert sorted(allf.tolist()) == list(range(150))
    for e, L in enumerate(lists):
        assert np.all(np.diff(L) > 0)
        assert set((L // 3).tolist()) == {t for t in range(50) if e in ids[t]}
        assert np.all(ids.reshape(-1)[L] == e)


# ----------------------------------------------------------------- pages

def test_resolve_hand_built_page_table():
    # one fp32 projection [2, 4] = 32 bytes on two 16-byte pages; the page
    # table puts row 0 on pool page 3 and row 1 on pool page 1.
    pool = np.full(64, 0xFF, dtype=np.uint8)
    row0 = [1.0, 2.0, 3.0, 4.0]
    row1 = [-1.5, 0.25, 8.0, -0.0]
    pool[48:64] = np.frombuffer(struct.pack("<4f", *row0), dtype=np.uint8)
    pool[16:32] = np.frombuffer(struct.pack("<4f", *row1), dtype=np.uint8)
    pt = np.array([[[3, 1]]], dtype=np.int32)
    got = resolve_projection(pool, pt, 0, 0, 2, 4, "f32", 16)
    assert got.tolist() == [row0, row1]


def test_resolve_bf16_page_split_mid_row():
    # bf16 [3, 4] = 24 bytes over 8-byte pages: each row is one page, stored
    # in reverse page order; bf16 0x3F80 = 1.0, 0xC000 = -2.0.
    vals = np.array([[0x3F80, 0xC000, 0x0000, 0x4040],
                     [0x3F00, 0x3E80, 0xBF80, 0x4000],
                     [0x4080, 0x40A0, 0x40C0, 0x40E0]], dtype=np.uint16)
    pool = np.zeros(32, dtype=np.uint8)
    for r in range(3):
        pool[(2 - r) * 8:(3 - r) * 8] = vals[r].view(np.uint8)
    pt = np.array([[[2, 1, 0]]], dtype=np.int32)
    got = resolve_projection(pool, pt, 0, 0, 3, 4, "bf16", 8)
    assert got.tolist() == [[1.0, -2.0, 0.0, 3.0], [0.5, 0.25, -1.0, 2.0], [4.0, 5.0, 6.0, 7.0]]


def test_place_then_resolve_round_trip():
    cfg = CONFIGS[1]
    L = Layout(cfg).run()
    pt = L.page_table()
    wb = gen.all_weight_bits(cfg)
    pool = build_pool(cfg, pt, wb)
    for e in (0, 5):
        W2 = resolve_projection(pool, pt, e, 2, cfg.I, cfg.H, "f32", cfg.page_bytes)
        assert np.array_equal(W2.reshape(-1), decode(wb[e, 2], "f32"))


def _contiguous(cfg, wb):
    pt = np.arange(cfg.E * 3 * cfg.P, dtype=np.int32).reshape(cfg.E, 3, cfg.P)
    pool = np.ascontiguousarray(wb).view(np.uint8).reshape(-1).copy()
    return pool, pt


def test_layout_permutation_invariance_bitwise():
    cfg = CONFIGS[1]
    wb = gen.all_weight_bits(cfg)
    x, lg = gen.x_bits(cfg), gen.logits(cfg)
    kw = dict(E=cfg.E, k=cfg.k, H=cfg.H, I=cfg.I, dtype=cfg.dtype)
    pool_c, pt_c = _contiguous(cfg, wb)
    y_c = moe_forward(x, lg, pool_c, pt_c, cfg.page_bytes, **kw)["y"]
    pt_s = Layout(cfg).run().page_table()
    y_s = moe_forward(x, lg, build_pool(cfg, pt_s, wb), pt_s, cfg.page_bytes, **kw)["y"]
    assert np.array_equal(y_c, y_s)
    # any other permutation of the pool's pages, too
    perm = np.random.default_rng(3).permutation(256).astype(np.int32)
    pt_p = perm[:cfg.E * 3 * cfg.P].reshape(cfg.E, 3, cfg.P)
    y_p = moe_forward(x, lg, build_pool(cfg, pt_p, wb), pt_p, cfg.page_bytes, **kw)["y"]
    assert np.array_equal(y_c, y_p)
    assert np.isfinite(y_c).all()


# ----------------------------------------------------------------- expert MLP

def _one_expert_pool(W1, W3, W2):
    wb = np.stack([W1.reshape(-1), W3.reshape(-1), W2.reshape(-1)]).astype(np.float32)
    pool = wb.view(np.uint8).reshape(-1).copy()
    pt = np.array([[[0], [1], [2]]], dtype=np.int32)
    return pool, pt, wb.nbytes // 3


def test_silu_reference_values():
    a = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    got = silu(a)
    # SiLU(1) = 1 / (1 + 1/e); SiLU(-1) = -1 / (1 + e)
    assert got[0] == 0.0
    assert abs(got[1] - 0.7310585786300049) < 1e-16
    assert abs(got[2] + 0.2689414213699951) < 1e-16
    assert abs(got[3] - 30.0) < 1e-11 and abs(got[4]) < 1e-11


def test_identity_weights_closed_form_and_gate_operand():
    # H = I = 4, w1 = c*Id, w3 = Id, w2 = Id: y_i = SiLU(c x_i) * x_i.
    # Gating the wrong operand would give SiLU(x_i) * c x_i instead.
    c = 2.0
    Id = np.eye(4, dtype=np.float32)
    pool, pt, pb = _one_expert_pool(c * Id, Id, Id)
    x = np.array([[0.5, -1.0, 2.0, 0.0]], dtype=np.float32)
    out = moe_forward(x.view(np.uint32), np.zeros((1, 1), np.float32), pool, pt, pb,
                      E=1, k=1, H=4, I=4, dtype="f32")
    expect = [(c * v) / (1 + math.exp(-c * v)) * v for v in x[0].tolist()]
    assert np.allclose(out["y"][0], expect, rtol=1e-15, atol=0)
    assert out["w"].tolist() == [[1.0]]


def test_selection_weights_closed_form_non_square():
    # H = 4, I = 2: w1 picks x0, x1; w3 picks x2, x3; w2 sends h0 -> y1, h1 -> y3.
    W1 = np.zeros((4, 2), np.float32); W1[0, 0] = 1; W1[1, 1] = 1
    W3 = np.zeros((4, 2), np.float32); W3[2, 0] = 1; W3[3, 1] = 1
    W2 = np.zeros((2, 4), np.float32); W2[0, 1] = 1; W2[1, 3] = 1
    pool, pt, pb = _one_expert_pool(W1, W3, W2)
    x = np.array([[1.0, -2.0, 3.0, 0.5]], dtype=np.float32)
    y = moe_forward(x.view(np.uint32), np.zeros((1, 1), np.float32), pool, pt, pb,
                    E=1, k=1, H=4, I=2, dtype="f32")["y"][0]
    s = lambda a: a / (1 + math.exp(-a))
    assert np.allclose(y, [0.0, s(1.0) * 3.0, 0.0, s(-2.0) * 0.5], rtol=1e-15, atol=0)


def _tiny(seed, E=6, k=2, H=8, I=4, T=5):
    r = np.random.default_rng(seed)
    wb = (r.standard_normal((E, 3, H * I)) * 0.3).astype(np.float32)
    x = r.standard_normal((T, H)).astype(np.float32)
    lg = r.standard_normal((T, E)).astype(np.float32)
    pool = wb.view(np.uint8).reshape(-1).copy()
    pt = np.arange(E * 3, dtype=np.int32).reshape(E, 3, 1)
    return wb, x, lg, pool, pt, H * I * 4


def test_zero_up_projection_gives_zero():
    wb, x, lg, pool, pt, pb = _tiny(1)
    wb[:, 1] = 0.0
    pool = wb.view(np.uint8).reshape(-1).copy()
    y = moe_forward(x.view(np.uint32), lg, pool, pt, pb, E=6, k=2, H=8, I=4, dtype="f32")["y"]
    assert np.all(y == 0.0)


def test_identical_experts_make_routing_irrelevant():
    wb, x, lg, pool, pt, pb = _tiny(2)
    wb[:] = wb[0]
    pool = wb.view(np.uint8).reshape(-1).copy()
    y = moe_forward(x.view(np.uint32), lg, pool, pt, pb, E=6, k=2, H=8, I=4, dtype="f32")["y"]
    y1 = moe_forward(x.view(np.uint32), np.zeros((5, 1), np.float32), pool[:pb * 3], pt[:1], pb,
                     E=1, k=1, H=8, I=4, dtype="f32")["y"]
    assert np.allclose(y, y1, rtol=1e-14, atol=1e-15)


def test_power_of_two_down_scale_is_exact():
    wb, x, lg, pool, pt, pb = _tiny(3)
    kw = dict(E=6, k=2, H=8, I=4, dtype="f32")
    y = moe_forward(x.view(np.uint32), lg, pool, pt, pb, **kw)["y"]
    wb2 = wb.copy(); wb2[:, 2] *= 8.0
    y2 = moe_forward(x.view(np.uint32), lg, wb2.view(np.uint8).reshape(-1).copy(), pt, pb, **kw)["y"]
    assert np.array_equal(y2, 8.0 * y)


def test_token_permutation_equivariance_exact():
    wb, x, lg, pool, pt, pb = _tiny(4, T=9)
    kw = dict(E=6, k=2, H=8, I=4, dtype="f32")
    perm = np.random.default_rng(0).permutation(9)
    y = moe_forward(x.view(np.uint32), lg, pool, pt, pb, **kw)["y"]
    yp = moe_forward(x[perm].view(np.uint32), lg[perm], pool, pt, pb, **kw)["y"]
    assert np.array_equal(yp, y[perm])


def test_token_subset_matches_full():
    wb, x, lg, pool, pt, pb = _tiny(5, T=9)
    kw = dict(E=6, k=2, H=8, I=4, dtype="f32")
    y = moe_forward(x.view(np.uint32), lg, pool, pt, pb, **kw)["y"]
    ys = moe_forward(x.view(np.uint32), lg, pool, pt, pb, tokens=[7, 2, 4], **kw)["y"]
    assert np.allclose(ys, y[[7, 2, 4]], rtol=1e-14, atol=1e-16)


# ----------------------------------------------------------------- whole layer

@pytest.mark.parametrize("seed", range(3))
def test_oracle_matches_dense_brute_force_random(seed):
    E, k, H, I, T = 7, 3, 12, 6, 6
    wb, x, lg, _, _, pb = _tiny(10 + seed, E=E, k=k, H=H, I=I, T=T)
    # scatter the projections over a permuted page pool of 24-byte pages
    page = 24
    P = H * I * 4 // page
    perm = np.random.default_rng(seed).permutation(E * 3 * P + 5).astype(np.int32)
    pt = perm[:E * 3 * P].reshape(E, 3, P)
    pool = np.full((E * 3 * P + 5) * page, 0xFF, dtype=np.uint8)
    raw = wb.view(np.uint8).reshape(E, 3, -1)
    for e in range(E):
        for p in range(3):
            for q in range(P):
                pool[pt[e, p, q] * page:(pt[e, p, q] + 1) * page] = raw[e, p, q * page:(q + 1) * page]
    out = moe_forward(x.view(np.uint32), lg, pool, pt, page, E=E, k=k, H=H, I=I, dtype="f32")
    ids, mask, yb = brute.brute_moe(x.view(np.uint32), lg, wb.view(np.uint32), E=E, k=k, H=H, I=I,
                                   dtype="f32")
    assert np.array_equal(out["ids"], ids)
    assert np.allclose(out["w"], np.take_along_axis(mask, ids, 1), rtol=1e-13, atol=0)
    assert np.allclose(out["y"], yb, rtol=1e-12, atol=1e-14)


def test_oracle_matches_brute_force_on_tiny_layer():
    cfg = CONFIGS[1]
    wb = gen.all_weight_bits(cfg)
    x, lg = gen.x_bits(cfg), gen.logits(cfg)
    pt = Layout(cfg).run().page_table()
    out = moe_forward(x, lg, build_pool(cfg, pt, wb), pt, cfg.page_bytes,
                      E=cfg.E, k=cfg.k, H=cfg.H, I=cfg.I, dtype=cfg.dtype)
    ids, mask, yb = brute.brute_moe(x, lg, wb, E=cfg.E, k=cfg.k, H=cfg.H, I=cfg.I, dtype=cfg.dtype)
    assert np.array_equal(out["ids"], ids)
    scale = np.abs(yb).max(axis=1, keepdims=True)
    assert np.all(np.abs(out["y"] - yb) <= 1e-12 * scale)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    got = decode(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == float(np.float32(3.3895313892515355e38))
    assert got[3] == 2.0 ** -133                        # smallest bf16 subnormal
    assert got[4] == 0.0 and math.copysign(1.0, got[4]) == -1.0
    assert got[5] == 3.140625


def test_generated_bf16_rounding_is_nearest_even():
    # Ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 and rounds to even (1);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 and rounds up.
    a = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -(1 + 2 ** -7)], dtype=np.float32)
    b = gen.f32_to_bf16_bits(a)
    assert decode(b, "bf16").tolist() == [1.0, 1 + 2 ** -6, 1.0, -(1 + 2 ** -7)]


# ---------------------------------------------------------------- router projection

def _bits_f32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def test_router_logits_brute_force_loops():
    """logits[t, e] = sum_h x[t, h] * w_gate[e, h], checked with plain loops."""
    g = np.random.default_rng(7)
    x = g.standard_normal((3, 5)).astype(np.float32)
    wg = g.standard_normal((4, 5)).astype(np.float32)
    from oracle.moe import router_logits
    got = router_logits(_bits_f32(x), _bits_f32(wg), "f32")
    for t in range(3):
        for e in range(4):
            ref = math.fsum(float(x[t, h]) * float(wg[e, h]) for h in range(5))
            assert got[t, e] == pytest.approx(ref, rel=1e-15, abs=1e-15)


def test_router_logits_hand_values_and_structure():
    from oracle.moe import router_logits
    x = np.array([[1.0, 2.0, 0.5]], dtype=np.float32)
    wg = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 2.0], [-1.0, -1.0, -1.0]], dtype=np.float32)
    assert router_logits(_bits_f32(x), _bits_f32(wg), "f32").tolist() == [[1.0, 3.0, -3.5]]
    # permuting the experts (rows of w_gate) permutes the logit columns
    g = np.random.default_rng(3)
    xb = gen.encode(g.standard_normal((6, 64)).astype(np.float32), "bf16")
    wb = gen.encode(g.standard_normal((8, 64)).astype(np.float32), "bf16")
    perm = g.permutation(8)
    a = router_logits(xb, wb, "bf16")
    b = router_logits(xb, wb[perm], "bf16")
    assert np.array_equal(b, a[:, perm])
    # bf16 inputs decode exactly: the logits equal the fp64 dot products of the decoded values
    xd, wd = decode(xb.reshape(-1), "bf16").reshape(6, 64), decode(wb.reshape(-1), "bf16").reshape(8, 64)
    assert np.array_equal(a, xd @ wd.T)
