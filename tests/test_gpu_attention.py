"""Paged decode attention over the KV view (explainer "Rimuru unifies serving
memory", paragraph on moving the fence; paper summary, Table 1 KV shapes)
against the oracle, on the GPU through the C ABI.

The KV blocks come from the allocator's KV view cut from expert-sized pages;
the pages between them hold NaN "expert weights", so a read outside a
request's blocks turns its output non-finite. Cases cover ragged context
lengths (1, a block minus one, exact blocks, long), several context splits,
empty contexts, grouped-query ratios 1, 8 and 16, head_dim 128 and 256, and
the Qwen3-30B-A3B decode shape at full size on sampled requests.
"""
import numpy as np
import pytest
import torch

from gpu_common import POISON, decode_dev, record, say
from moe_inputs import gen
from oracle.attention import block_bytes, decode_attention
from paged_moe_expert_amd import rimuru as R
from paged_moe_expert_amd._lib import VIEW_EXPERT, VIEW_KV

pytestmark = pytest.mark.gpu

KIB = 1024
BT = 16


def pack_blocks(K, V):
    """uint8 [n_blocks, block_bytes] of one request: per block, K of every KV
    head [16][D], then V of every KV head [D][16] (array transposes)."""
    n_kv, L, D = K.shape
    nb = -(-L // BT)
    Kp = np.zeros((n_kv, nb * BT, D), dtype=np.float32)
    Vp = np.zeros_like(Kp)
    Kp[:, :L], Vp[:, :L] = K, V
    kb = Kp.reshape(n_kv, nb, BT, D).transpose(1, 0, 2, 3).reshape(nb, -1)      # [nb][n_kv][16][D]
    vb = Vp.reshape(n_kv, nb, BT, D).transpose(1, 0, 3, 2).reshape(nb, -1)      # [nb][n_kv][D][16]
    bits = gen.encode(np.ascontiguousarray(np.concatenate([kb, vb], axis=1)), "bf16")
    return np.ascontiguousarray(bits).view(np.uint8).reshape(nb, -1)


def poison_tail(block: np.ndarray, L: int, n_kv: int, D: int) -> None:
    """Fill the token slots at or past the context end L of a request's last
    block (K rows and V columns of every KV head) with the pool's NaN filler."""
    t0 = L % BT
    if t0 == 0:
        return
    u = block.view(np.uint16)
    kpart = u[:n_kv * BT * D].reshape(n_kv, BT, D)
    vpart = u[n_kv * BT * D:].reshape(n_kv, D, BT)
    kpart[:, t0:, :] = POISON & 0xFFFF
    vpart[:, :, t0:] = POISON & 0xFFFF


def setup(lens, n_kv, D, seed, expert_page=None, expert_every=1, stale_tails=False):
    """Allocator pool with an expert view and a KV view cut from it; expert
    owners (NaN pages) interleaved with the requests' KV blocks (one before
    every expert_every-th request). stale_tails: the slots past each context
    in its last block hold NaN instead of zeros."""
    bb = block_bytes(n_kv, D, "bf16")
    xp = expert_page or 4 * bb
    need = sum(-(-L // BT) for L in lens)
    n_huge = -(-need * bb // xp) + len(lens) // expert_every + len(lens) + 5   # KV, expert pages, partials
    pool_h = R.pool_create(n_huge * xp, xp)
    xv = R.view_map(pool_h, VIEW_EXPERT, xp, None)
    kv = R.view_map(pool_h, VIEW_KV, bb, xv)
    max_blocks = max(1, max(-(-L // BT) for L in lens))
    table = np.zeros((len(lens), max_blocks), dtype=np.int32)
    rng = np.random.default_rng(seed)
    host = np.empty(n_huge * xp, dtype=np.uint8)
    host.view(np.uint32)[:] = POISON
    for b, L in enumerate(lens):
        if b % expert_every == 0:
            R.view_alloc(xv, 1000 + b, 1)               # an expert page between requests
        nb = -(-L // BT)
        if nb == 0:
            continue
        offs = R.view_alloc(kv, b, nb)
        table[b, :nb] = offs // bb
        K = rng.standard_normal((n_kv, L, D), dtype=np.float32)
        V = rng.standard_normal((n_kv, L, D), dtype=np.float32)
        blocks = pack_blocks(K, V)
        if stale_tails:
            poison_tail(blocks[-1], L, n_kv, D)
        for i, o in enumerate(offs):
            host[o:o + bb] = blocks[i]
    R.block_table_check(table, lens, bb, host.size)
    return host, table, max_blocks


def run_case(lens, n_q, n_kv, D, seed, sample=None, **kw):
    host, table, max_blocks = setup(lens, n_kv, D, seed, **kw)
    B = len(lens)
    qb = gen.encode(np.random.default_rng(seed + 1).standard_normal((B, n_q, D)).astype(np.float32), "bf16")
    dev = torch.device("cuda:0")
    pool = torch.from_numpy(host).to(dev)
    q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16).reshape(B, n_q, D)
    bt = torch.from_numpy(table).to(dev)
    lt = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev)
    scale = 1.0 / np.sqrt(D)
    ws, ns, _ = R.attn_sizes(B, n_q, n_kv, D, max_blocks)
    say(f"[attn] B={B} n_q={n_q} n_kv={n_kv} D={D} max_blocks={max_blocks} splits={ns} lens={lens[:8]}...")
    out = R.paged_decode_attention(q, pool, bt, lt, n_kv, scale)
    torch.cuda.synchronize()
    got = decode_dev(out)
    assert np.isfinite(got).all(), "read outside the request's blocks"
    reqs = list(range(B)) if sample is None else sample
    worst = 0.0
    ref = decode_attention(qb, host, table, lens, n_q=n_q, n_kv=n_kv, head_dim=D, dtype="bf16",
                           scale=scale, requests=reqs)
    for i, b in enumerate(reqs):
        if lens[b] == 0:
            assert not got[b].any()
            continue
        r = ref[i]
        err = (np.abs(got[b] - r).max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-30)).max()
        worst = max(worst, err)
        assert err <= 1e-2, f"request {b} (L={lens[b]}): rel_err {err:.3e}"
    record(f"attention B={B} n_q={n_q} n_kv={n_kv} D={D}{' stale tails' if kw.get('stale_tails') else ''}",
           worst, 1e-2)
    # a second call is bitwise equal (deterministic merge order)
    out2 = R.paged_decode_attention(q, pool, bt, lt, n_kv, scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    return ns


def test_ragged_lengths_qwen3_shape():
    lens = [1, 15, 16, 17, 33, 200, 700, 0, 5, 64, 129, 1000]
    assert run_case(lens, 32, 4, 128, seed=1) > 1


def test_stale_nan_tails_of_last_blocks():
    """The slots past each context in its last block hold the pool's NaN
    filler (a block cut from a page that held something else): the output
    stays finite and matches the oracle, with one split and with several."""
    lens = [1, 15, 17, 31, 200, 701, 5, 1000, 33, 2047]
    assert run_case(lens, 32, 4, 128, seed=21, stale_tails=True) > 1
    rng = np.random.default_rng(22)
    lens = np.clip(np.rint(rng.lognormal(4.5, 1.0, 256)), 1, 700).astype(int).tolist()
    assert run_case(lens, 32, 4, 128, seed=23, sample=[0, 5, 64, 128, 255], expert_every=8,
                    stale_tails=True) == 1
    run_case([3, 250, 17], 16, 2, 256, seed=24, stale_tails=True)


def test_one_long_request_many_splits():
    assert run_case([4095], 32, 4, 128, seed=2) >= 16


def test_head_dim_256_qwen35_shape():
    run_case([3, 16, 250, 600, 31], 16, 2, 256, seed=3)


@pytest.mark.parametrize("n_q,n_kv", [(4, 4), (16, 1), (24, 2)])
def test_group_ratios(n_q, n_kv):
    run_case([7, 48, 300, 1], n_q, n_kv, 128, seed=4 + n_q)


def test_context_beyond_one_split_table():
    """A context of 1100 blocks among many short requests: the split count is
    raised so that no split's block-table slice exceeds 1024 blocks."""
    lens = [17600] + [5] * 299
    ns = run_case(lens, 32, 4, 128, seed=11, sample=[0, 1, 150, 299])
    assert ns >= 2


def test_single_split_writes_output_directly():
    """256 requests over 4 KV heads take one split: the first kernel writes
    the normalised output itself (no merge launch), empty contexts included."""
    rng = np.random.default_rng(12)
    lens = np.clip(np.rint(rng.lognormal(4.5, 1.0, 256)), 1, 700).astype(int)
    lens[[3, 100, 255]] = 0
    lens = lens.tolist()
    ns = run_case(lens, 32, 4, 128, seed=13, sample=[0, 3, 7, 100, 128, 200, 255], expert_every=8)
    assert ns == 1


def test_no_requests_is_a_no_op():
    dev = torch.device("cuda:0")
    q = torch.zeros((0, 32, 128), dtype=torch.bfloat16, device=dev)
    pool = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    bt = torch.zeros((0, 1), dtype=torch.int32, device=dev)
    lt = torch.zeros(0, dtype=torch.int32, device=dev)
    out = R.paged_decode_attention(q, pool, bt, lt, 4, 0.1)
    assert out.shape == (0, 32, 128)


def test_qwen3_decode_batch_full_size_sampled():
    """64 requests with contexts up to 4096 tokens in a pool laid out like the
    decode layer's (3 MiB expert pages, 32 KiB KV blocks cut from them)."""
    rng = np.random.default_rng(7)
    lens = np.clip(np.rint(rng.lognormal(6.8, 0.8, 64)), 1, 4096).astype(int).tolist()
    run_case(lens, 32, 4, 128, seed=8, sample=[0, 1, 17, 40, 63, int(np.argmax(lens))],
             expert_page=3 * 1024 * KIB, expert_every=4)
