"""Dense brute force of the MoE layer for tiny inputs (test infrastructure).

Shares nothing with oracle.moe beyond the bit decoding of inputs: it ranks
experts with Python's ``sorted``, takes the full softmax over all E experts,
keeps the top k and renormalises them, evaluates every expert on every token
from contiguous weights (no pages, no grouping, no lists) and combines with a
dense [T, E] weight mask. Pure Python loops: keep T*E small.

Parity status: this is itself a pin for oracle.moe (same definition, other
structure); its own formula is pinned by the closed-form tests.
"""
from __future__ import annotations

import math

import numpy as np

from .moe import decode


def _silu(a: float) -> float:
    return a / (1.0 + math.exp(-a)) if a >= 0 else a * math.exp(a) / (1.0 + math.exp(a))


def brute_moe(x_bits, logits, weight_bits, *, E, k, H, I, dtype):
    """x_bits [T, H], logits [T, E] fp32, weight_bits [E, 3, H*I] storage bits."""
    T = logits.shape[0]
    X = decode(np.asarray(x_bits).reshape(-1), dtype).reshape(T, H)
    W = decode(np.asarray(weight_bits).reshape(-1), dtype).reshape(E, 3, H * I)
    ids = np.zeros((T, k), dtype=np.int64)
    mask = np.zeros((T, E))
    for t in range(T):
        lt = [float(v) + 0.0 for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-lt[e], e))
        mx = max(lt)
        full = [math.exp(v - mx) for v in lt]
        z = sum(full)
        p = [v / z for v in full]                       # full softmax over E
        kept = order[:k]
        s = sum(p[e] for e in kept)
        for j, e in enumerate(kept):
            ids[t, j] = e
            mask[t, e] = p[e] / s
    y = np.zeros((T, H))
    for e in range(E):
        W1 = W[e, 0].reshape(H, I)
        W3 = W[e, 1].reshape(H, I)
        W2 = W[e, 2].reshape(I, H)
        for t in range(T):
            a = X[t] @ W1
            b = X[t] @ W3
            h = np.array([_silu(float(a[i])) * float(b[i]) for i in range(I)])
            y[t] += mask[t, e] * (h @ W2)
    return ids, mask, y
