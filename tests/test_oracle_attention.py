"""Pins of the paged decode-attention oracle (oracle/attention.py): closed
forms, torch's scaled_dot_product_attention on dense tensors, layout read-back
against an independent array construction, block-table permutation
invariance and the grouped-query head mapping."""
import numpy as np
import pytest
import torch

from moe_inputs import gen
from oracle.attention import block_bytes, decode_attention, gather_kv

BT = 16


def pack_blocks(K, V, dtype="f32"):
    """Blocks of one request built with array transposes (not byte offsets):
    K [n_kv, L, D], V [n_kv, L, D] -> uint8 [n_blocks, block_bytes]."""
    n_kv, L, D = K.shape
    nb = -(-L // BT)
    Kp = np.zeros((n_kv, nb * BT, D), dtype=np.float32)
    Vp = np.zeros_like(Kp)
    Kp[:, :L], Vp[:, :L] = K, V
    out = []
    for b in range(nb):
        kb = Kp[:, b * BT:(b + 1) * BT, :]                     # [n_kv, 16, D]
        vb = Vp[:, b * BT:(b + 1) * BT, :].transpose(0, 2, 1)   # [n_kv, D, 16]
        bits = np.concatenate([gen.encode(np.ascontiguousarray(kb).reshape(-1), dtype),
                               gen.encode(np.ascontiguousarray(vb).reshape(-1), dtype)])
        out.append(bits.view(np.uint8))
    return np.stack(out)


def build(K, V, q, positions, dtype="f32"):
    """Pool with the request's blocks at the given block positions."""
    blocks = pack_blocks(K, V, dtype)
    bb = blocks.shape[1]
    pool = np.full((max(positions) + 2) * bb, 0xFF, dtype=np.uint8)
    for i, p in enumerate(positions):
        pool[p * bb:(p + 1) * bb] = blocks[i]
    return pool


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_layout_read_back_matches_array_construction():
    n_kv, L, D = 2, 37, 8
    K, V = rnd((n_kv, L, D), 1), rnd((n_kv, L, D), 2)
    pos = [5, 0, 3]
    pool = build(K, V, None, pos)
    assert block_bytes(n_kv, D, "f32") == pool.size // (max(pos) + 2)
    K2, V2 = gather_kv(pool, pos, L, n_kv, D, "f32")
    assert np.array_equal(K2, K.astype(np.float64)) and np.array_equal(V2, V.astype(np.float64))


def test_against_torch_sdpa_with_grouped_heads():
    n_q, n_kv, D = 8, 2, 16
    lens = [1, 15, 16, 17, 70]
    B = len(lens)
    q = rnd((B, n_q, D), 3)
    pools, tables = [], []
    bb = block_bytes(n_kv, D, "f32")
    pool = np.zeros(0, dtype=np.uint8)
    table = np.zeros((B, 8), dtype=np.int32)
    Ks, Vs = [], []
    nxt = 0
    for b, L in enumerate(lens):
        K, V = rnd((n_kv, L, D), 10 + b), rnd((n_kv, L, D), 20 + b)
        blocks = pack_blocks(K, V)
        table[b, :len(blocks)] = np.arange(nxt, nxt + len(blocks))[::-1]   # reversed placement
        pool = np.concatenate([pool, np.zeros(len(blocks) * bb, dtype=np.uint8)])
        for i in range(len(blocks)):
            p = table[b, i]
            pool[p * bb:(p + 1) * bb] = blocks[i]
        nxt += len(blocks)
        Ks.append(K)
        Vs.append(V)
    scale = 1.0 / np.sqrt(D)
    out = decode_attention(gen.encode(q.reshape(-1), "f32"), pool, table, lens, n_q=n_q, n_kv=n_kv,
                           head_dim=D, dtype="f32", scale=scale)
    for b, L in enumerate(lens):
        qt = torch.from_numpy(q[b].astype(np.float64)).reshape(1, n_q, 1, D)
        kt = torch.from_numpy(Ks[b].astype(np.float64)).repeat_interleave(n_q // n_kv, 0).unsqueeze(0)
        vt = torch.from_numpy(Vs[b].astype(np.float64)).repeat_interleave(n_q // n_kv, 0).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        assert np.allclose(out[b], ref.reshape(n_q, D).numpy(), rtol=1e-12, atol=1e-12)


def test_closed_forms():
    n_kv, D = 1, 4
    # one token: the output is that token's V
    K, V = rnd((1, 1, D), 4), rnd((1, 1, D), 5)
    pool = build(K, V, None, [0])
    q = gen.encode(rnd((1, 1, D), 6).reshape(-1), "f32")
    out = decode_attention(q, pool, [[0]], [1], n_q=1, n_kv=1, head_dim=D, dtype="f32", scale=0.5)
    assert np.array_equal(out[0, 0], V[0, 0].astype(np.float64))
    # equal keys: uniform weights, the mean of V
    L = 40
    K = np.tile(rnd((1, 1, D), 7), (1, L, 1))
    V = rnd((1, L, D), 8)
    pool = build(K, V, None, [2, 0, 1])
    out = decode_attention(q, pool, [[2, 0, 1]], [L], n_q=1, n_kv=1, head_dim=D, dtype="f32", scale=1.0)
    assert np.allclose(out[0, 0], V[0].astype(np.float64).mean(0), rtol=1e-13, atol=1e-13)
    # one key far ahead of the rest: its V
    K = np.zeros((1, L, D), dtype=np.float32)
    K[0, 23] = 1000.0
    qv = np.ones((1, 1, D), dtype=np.float32)
    pool = build(K, V, None, [0, 1, 2])
    out = decode_attention(gen.encode(qv.reshape(-1), "f32"), pool, [[0, 1, 2]], [L], n_q=1, n_kv=1,
                           head_dim=D, dtype="f32", scale=1.0)
    assert np.allclose(out[0, 0], V[0, 23], rtol=1e-12, atol=1e-12)
    # no context: zeros
    out = decode_attention(q, pool, [[0]], [0], n_q=1, n_kv=1, head_dim=D, dtype="f32", scale=1.0)
    assert not out.any()


def test_block_permutation_invariance_and_group_mapping():
    n_q, n_kv, D, L = 4, 2, 8, 50
    K, V = rnd((n_kv, L, D), 30), rnd((n_kv, L, D), 31)
    q = gen.encode(rnd((1, n_q, D), 32).reshape(-1), "bf16")
    Kb = gen.encode(K.reshape(-1), "bf16")
    K16 = np.ascontiguousarray(Kb).view(np.uint16).astype(np.uint32) << 16
    K = K16.view(np.float32).reshape(K.shape)
    Vb = gen.encode(V.reshape(-1), "bf16").view(np.uint16).astype(np.uint32) << 16
    V = Vb.view(np.float32).reshape(V.shape)
    a = decode_attention(q, build(K, V, None, [0, 1, 2, 3], "bf16"), [[0, 1, 2, 3]], [L], n_q=n_q,
                         n_kv=n_kv, head_dim=D, dtype="bf16", scale=0.3)
    b = decode_attention(q, build(K, V, None, [6, 2, 4, 0], "bf16"), [[6, 2, 4, 0]], [L], n_q=n_q,
                         n_kv=n_kv, head_dim=D, dtype="bf16", scale=0.3)
    assert np.array_equal(a, b)
    # heads 2 and 3 read KV head 1: zeroing its V zeroes exactly those heads
    V0 = V.copy()
    V0[1] = 0.0
    c = decode_attention(q, build(K, V0, None, [0, 1, 2, 3], "bf16"), [[0, 1, 2, 3]], [L], n_q=n_q,
                         n_kv=n_kv, head_dim=D, dtype="bf16", scale=0.3)
    assert np.array_equal(c[0, :2], a[0, :2]) and not c[0, 2:].any() and a[0, 2:].any()
