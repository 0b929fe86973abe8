"""fp64 reference of paged decode attention over the KV view (test
infrastructure).

What is computed, and where it comes from:

* The KV cache lives in the same shared page pool as the experts, in its own
  memory view: 16-token blocks reached through a per-request block table
  (PagedAttention's block-table idea, which the explainer's paragraph on
  moving the fence says Rimuru stretches across tensor types; blocks hold
  16 tokens there). One token's K and V have the shape [2, n_kv_heads,
  head_dim] (paper summary, Table 1: [2, 4, 128] for Qwen3-30B-A3B,
  [2, 2, 256] for Qwen3.5-35B-A3B).
* Inside a block the pages fix no order. Reading: all of K, then all of V;
  K per KV head token-major [16][head_dim]; V per KV head dim-major
  [head_dim][16] (the product's kernel reads both as contiguous runs). Byte
  offsets within a block of kv_head j, token t, dim i (es bytes per element):
    K: ((j * 16 + t) * head_dim + i) * es
    V: (n_kv * 16 * head_dim + (j * head_dim + i) * 16 + t) * es
* Decode attention, one query token per request, grouped-query heads: query
  head h uses KV head h // (n_q / n_kv);
    out[b, h] = softmax_t(scale * q[b, h] . K_b[t]) @ V_b,  t < context_len[b]
  (the plain definition; no causal mask is needed for the last token). A
  request with context length 0 gets zeros.

Parity status: pinned in tests/test_oracle_attention.py (closed forms:
one token, equal keys, a dominating key; torch's scaled_dot_product_attention
on the gathered dense K and V; block-table permutation invariance; a
hand-placed block read back by byte offsets; the group mapping).
"""
from __future__ import annotations

import numpy as np

from .moe import decode

ES = {"f32": 4, "bf16": 2}


def block_bytes(n_kv: int, head_dim: int, dtype: str, block_tokens: int = 16) -> int:
    return 2 * n_kv * block_tokens * head_dim * ES[dtype]


def gather_kv(pool: np.ndarray, table_row, length: int, n_kv: int, head_dim: int, dtype: str,
              block_tokens: int = 16):
    """Dense K, V [n_kv, length, head_dim] (fp64) of one request, read element
    by element through its block table (block indices in units of a block)."""
    es = ES[dtype]
    bb = block_bytes(n_kv, head_dim, dtype, block_tokens)
    half = n_kv * block_tokens * head_dim * es
    pool = np.asarray(pool).view(np.uint8)
    K = np.zeros((n_kv, length, head_dim))
    V = np.zeros((n_kv, length, head_dim))
    for tok in range(length):
        base = int(table_row[tok // block_tokens]) * bb
        t = tok % block_tokens
        for j in range(n_kv):
            k0 = base + (j * block_tokens + t) * head_dim * es
            K[j, tok] = decode(pool[k0:k0 + head_dim * es].copy(), dtype)
            v_offs = base + half + ((j * head_dim + np.arange(head_dim)) * block_tokens + t) * es
            raw = np.stack([pool[o:o + es] for o in v_offs]).reshape(-1).copy()
            V[j, tok] = decode(raw, dtype)
    return K, V


def decode_attention(q_bits, pool, block_table, context_lens, *, n_q: int, n_kv: int, head_dim: int,
                     dtype: str, scale: float, block_tokens: int = 16, requests=None):
    """out [len(requests), n_q, head_dim] fp64 (requests: optional subset)."""
    B = len(context_lens)
    requests = range(B) if requests is None else requests
    g = n_q // n_kv
    q = decode(np.asarray(q_bits).reshape(-1), dtype).reshape(B, n_q, head_dim)
    out = np.zeros((len(requests), n_q, head_dim))
    for r, b in enumerate(requests):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_kv(pool, block_table[b], L, n_kv, head_dim, dtype, block_tokens)
        for h in range(n_q):
            s = scale * (K[h // g] @ q[b, h])
            w = np.exp(s - s.max())
            out[r, h] = (w / w.sum()) @ V[h // g]
    return out
