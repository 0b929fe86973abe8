"""fp64 reference of the page-table-aware fused MoE layer (test infrastructure).

What is computed, and where it comes from:

* The layer reads each expert's weights where they sit in the shared pool,
  through the expert view's page table, with no contiguous copy (Rimuru paper
  summary, abstract; explainer "Rimuru unifies serving memory", paragraph on
  the two pieces that make the moving fence usable). ``resolve_projection``
  does that resolution explicitly, element by element.
* Each expert owns three projections w1, w3 [hidden, inter] and
  w2 [inter, hidden] (paper summary, Table 1). Reading: w1 is the gate, w3
  the up projection and w2 the down projection of a gated SiLU MLP,
  ``SiLU(x w1) * (x w3) @ w2``; the pages name the matrices, not the formula.
* Routing: softmax over the router logits, keep the top k, renormalise the k
  kept weights to sum to one. The pages are silent; this is the plainest
  reading. Ties in the logits go to the lower expert index, -0 equals +0.
* Combine: y[t] = sum over j of w[t, j] * expert_{ids[t, j]}(x[t]), j in
  rank order.
* Router projection (the step upstream of routing that the pages leave
  implicit): logits[t, e] = x[t] . w_gate[e], w_gate [E, H] in a Linear
  layer's layout. ``router_logits`` computes it in fp64.

Parity status: pinned. Routing by brute-force sorting, closed forms and the
k = E special case; page resolution by layout-permutation invariance and a
hand-built page table; the expert MLP by closed forms at special weights; the
whole layer by a dense brute force that evaluates every expert for every
token. The pins live in tests/test_oracle_moe.py.
"""
from __future__ import annotations

import numpy as np

ES = {"f32": 4, "bf16": 2}


# ---------------------------------------------------------------- decoding

def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bit patterns -> fp64. Both conversions are exact."""
    if dtype == "f32":
        return np.ascontiguousarray(bits).view(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- routing

def router_logits(x_bits: np.ndarray, w_gate_bits: np.ndarray, dtype: str) -> np.ndarray:
    """logits [T, E] = x [T, H] @ w_gate [E, H]^T in fp64 (inputs decoded
    exactly from their storage bits)."""
    x = decode(np.asarray(x_bits).reshape(-1), dtype).reshape(np.asarray(x_bits).shape)
    wg = decode(np.asarray(w_gate_bits).reshape(-1), dtype).reshape(np.asarray(w_gate_bits).shape)
    return x @ wg.T


def route(logits: np.ndarray, k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Experts are ranked by (logit descending, expert index ascending) on the
    raw logits; -0 is first made +0 so the two compare equal. The weights are
    exp(l_j - m) / sum_j' exp(l_j' - m) over the k kept logits, m the largest:
    the full softmax's denominator cancels in the renormalisation.

    Returns ids int64 [T, k] in rank order and w fp64 [T, k].
    """
    l = np.asarray(logits, dtype=np.float64) + 0.0       # -0 -> +0
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    idx = np.broadcast_to(np.arange(E), l.shape)
    order = np.lexsort((idx, -l), axis=-1)                # primary: -l, then index
    ids = order[:, :k].astype(np.int64)
    sel = np.take_along_axis(l, ids, axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


def expert_lists(ids: np.ndarray, E: int):
    """Per-expert lists of routed slots: flat ids t*k + j, ascending."""
    flat = np.asarray(ids).reshape(-1)
    return [np.nonzero(flat == e)[0].astype(np.int64) for e in range(E)]


# ---------------------------------------------------------------- pages

def resolve_projection(pool: np.ndarray, pt: np.ndarray, e: int, p: int,
                       R: int, C: int, dtype: str, page_bytes: int) -> np.ndarray:
    """Read projection p of expert e, logical [R, C] row-major, through the page
    table and return it as fp64.

    Element (r, c) sits at flat byte offset f = (r*C + c)*es of the
    projection; its page is q = f // page_bytes and its pool address
    pt[e, p, q]*page_bytes + f % page_bytes.
    """
    es = ES[dtype]
    f = np.arange(R * C, dtype=np.int64) * es
    q = f // page_bytes
    if q.max() >= pt.shape[2]:
        raise ValueError("projection spans more pages than the page table holds")
    addr = pt[e, p, q].astype(np.int64) * page_bytes + f % page_bytes
    if addr.min() < 0 or addr.max() + es > pool.size:
        raise ValueError("page table points outside the pool")
    raw = pool[addr[:, None] + np.arange(es)]             # [R*C, es] bytes
    bits = np.ascontiguousarray(raw).view(np.uint32 if es == 4 else np.uint16).reshape(-1)
    return decode(bits, dtype).reshape(R, C)


# ---------------------------------------------------------------- expert MLP

def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a), written to stay finite for large |a|."""
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = a[pos] / (1.0 + np.exp(-a[pos]))
    ea = np.exp(a[~pos])
    out[~pos] = a[~pos] * ea / (1.0 + ea)
    return out


def expert_mlp(X: np.ndarray, W1: np.ndarray, W3: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """Gated SiLU MLP of one expert on rows X [n, H]: (SiLU(X W1) * (X W3)) W2."""
    return (silu(X @ W1) * (X @ W3)) @ W2


# ---------------------------------------------------------------- the layer

def moe_forward(x_bits, logits, pool, pt, page_bytes: int, *, E: int, k: int,
                H: int, I: int, dtype: str, tokens=None):
    """The fused MoE layer in fp64, weights read through the page table.

    tokens: optional subset of token indices for which y is computed (routing
    and lists always cover every token). Returns a dict with ids, w, lists
    and y (fp64 [len(tokens), H]).
    """
    ids, w = route(logits, k)
    lists = expert_lists(ids, E)
    T = ids.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    X = decode(np.asarray(x_bits)[tokens].reshape(-1), dtype).reshape(len(tokens), H)
    slot = np.zeros((len(tokens), k, H))
    for e in np.unique(ids[tokens]):
        ti, jj = np.nonzero(ids[tokens] == e)             # rows of this expert
        W1 = resolve_projection(pool, pt, e, 0, H, I, dtype, page_bytes)
        W3 = resolve_projection(pool, pt, e, 1, H, I, dtype, page_bytes)
        W2 = resolve_projection(pool, pt, e, 2, I, H, dtype, page_bytes)
        slot[ti, jj] = expert_mlp(X[ti], W1, W3, W2)
    y = np.zeros((len(tokens), H))
    wt = w[tokens]
    for j in range(k):                                    # fixed rank order
        y += wt[:, j:j + 1] * slot[:, j]
    return {"ids": ids, "w": w, "lists": lists, "y": y}


def place_weights(pool: np.ndarray, pt: np.ndarray, weight_bits: np.ndarray,
                  page_bytes: int) -> None:
    """Write contiguous projections [E, 3, n] (storage bits) into the pool pages
    the page table names: page q of projection (e, p) holds its bytes
    [q*page_bytes, (q+1)*page_bytes)."""
    E, three, _ = weight_bits.shape
    raw = np.ascontiguousarray(weight_bits).view(np.uint8).reshape(E, three, -1)
    P = pt.shape[2]
    for e in range(E):
        for p in range(three):
            for q in range(P):
                a = int(pt[e, p, q]) * page_bytes
                pool[a:a + page_bytes] = raw[e, p, q * page_bytes:(q + 1) * page_bytes]
