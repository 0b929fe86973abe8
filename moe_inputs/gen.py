"""Seeded synthetic inputs for the paged fused-MoE workloads.

Every draw comes from numpy's PCG64 seeded by ``SeedSequence(entropy=cid,
spawn_key=(stream, ...))`` so each stream can be regenerated on its own.
This module draws random numbers and encodes them in the workload's dtype.
It computes nothing of the method itself (no routing, no page resolution, no
expert MLP, no allocation decisions) and is the only code the oracle and the
product share.

Distributions (none is fixed by the pages, which measure on real requests):
  x ~ N(0, 1); expert weights ~ N(0, 0.02); router logits ~ N(0, 1) (tiny
  layer), U(0, 1) (decode, "uniform-random" routing) or Zipf popularity drawn
  with the Gumbel-top-k trick: logit_e = log p_e + Gumbel(0, 1), with
  p_e proportional to rank(e)^-s over a seeded permutation of the experts.
bf16 values are fp32 draws rounded to nearest-even.
"""
from __future__ import annotations

import numpy as np

from .configs import CONV_REQ_MAX, KV_REQ_MAX, MoEConfig

# Stream ids.
S_X, S_LOGITS, S_WEIGHTS, S_EVENTS, S_UNIFORMS, S_ADJUST, S_POISON, S_GATE = range(8)

# Owner-id ranges for filler requests (expert owners are small integers).
OWNER_KV = 1 << 32
OWNER_SSM = 2 << 32
OWNER_CONV = 3 << 32
FILLER_BASE = {"kv": OWNER_KV, "ssm": OWNER_SSM, "conv": OWNER_CONV}


def rng(cid: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=cid, spawn_key=tuple(key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite draws; NaN handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws -> storage bit patterns (uint32 for f32, uint16 for bf16)."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def x_bits(cfg: MoEConfig, T: int | None = None, seed_key: int = 0) -> np.ndarray:
    """Token activations [T, H] as storage bits."""
    T = cfg.T if T is None else T
    g = rng(cfg.cid, S_X, T, seed_key)
    return encode(g.standard_normal((T, cfg.H), dtype=np.float32), cfg.dtype)


def zipf_probs(cfg: MoEConfig) -> np.ndarray:
    """Expert popularity p_e proportional to rank^-s over a seeded permutation."""
    g = rng(cfg.cid, S_LOGITS, 0xFFFF)
    rank = g.permutation(cfg.E) + 1
    p = rank.astype(np.float64) ** (-cfg.zipf_s)
    return p / p.sum()


def logits(cfg: MoEConfig, T: int | None = None, seed_key: int = 0) -> np.ndarray:
    """Router logits [T, E] fp32."""
    T = cfg.T if T is None else T
    g = rng(cfg.cid, S_LOGITS, T, seed_key)
    if cfg.logits == "normal":
        out = g.standard_normal((T, cfg.E), dtype=np.float32)
    elif cfg.logits == "uniform":
        out = g.random((T, cfg.E), dtype=np.float32)
    elif cfg.logits == "zipf":
        logp = np.log(zipf_probs(cfg))
        u = g.random((T, cfg.E))
        u = np.clip(u, np.finfo(np.float64).tiny, None)
        out = (logp[None, :] - np.log(-np.log(u))).astype(np.float32)
    else:
        raise ValueError(cfg.logits)
    return np.ascontiguousarray(out)


def gate_weight_bits(cfg: MoEConfig) -> np.ndarray:
    """Router weights w_gate [E, H] (a Linear layer's layout) as storage bits,
    N(0, 0.02) like the expert weights."""
    g = rng(cfg.cid, S_GATE)
    return encode(g.normal(0.0, 0.02, size=(cfg.E, cfg.H)).astype(np.float32), cfg.dtype)


def expert_weight_bits(cfg: MoEConfig, e: int) -> np.ndarray:
    """Expert e's projections [3, H*I] as storage bits, in order w1, w3, w2.

    w1 and w3 are [H, I] row-major, w2 is [I, H] row-major; each row is
    flattened, so all three have H*I elements.
    """
    g = rng(cfg.cid, S_WEIGHTS, e)
    w = g.standard_normal((3, cfg.H * cfg.I), dtype=np.float32)
    w *= np.float32(0.02)
    return encode(w, cfg.dtype)


def all_weight_bits(cfg: MoEConfig) -> np.ndarray:
    """All experts' projections [E, 3, H*I] as storage bits."""
    dt = np.uint32 if cfg.dtype == "f32" else np.uint16
    out = np.empty((cfg.E, 3, cfg.H * cfg.I), dtype=dt)
    for e in range(cfg.E):
        out[e] = expert_weight_bits(cfg, e)
    return out


# ----------------------------------------------------------------------------
# Layout event streams. These are lists of requests and random numbers; what
# they do to the pool is decided by whichever allocator runs them.
# ----------------------------------------------------------------------------

def uniforms(cfg: MoEConfig, n: int = 1 << 18, key: int = 0) -> np.ndarray:
    """Uniform [0, 1) draws a layout runner consumes in order (victim picks)."""
    return rng(cfg.cid, S_UNIFORMS, key).random(n)


def scatter_events(cfg: MoEConfig):
    """Tiny-layer recipe: one single-page owner per expert page plus KV blocks,
    in a seeded order. Returns ops ("alloc", view, owner, n_pages)."""
    ops = [("alloc", "expert", (e * 3 + p) * cfg.P + q, 1)
           for e in range(cfg.E) for p in range(3) for q in range(cfg.P)]
    kv_page = cfg.view("kv").page_bytes
    exp_bytes = cfg.E * 3 * cfg.proj_bytes
    n_kv = (cfg.pool_bytes - exp_bytes) // kv_page
    ops += [("alloc", "kv", OWNER_KV + i, 1) for i in range(n_kv)]
    perm = rng(cfg.cid, S_EVENTS).permutation(len(ops))
    return [ops[i] for i in perm]


def filler_requests(cfg: MoEConfig, n: int = 12000):
    """Filler requests (view, owner, n_pages) for the fill-then-place recipe.

    Decode layers: KV requests of U{1..128} blocks. The hybrid layer mixes KV,
    SSM (one 1 MiB state) and conv (U{1..40} states) requests in equal odds.
    """
    g = rng(cfg.cid, S_EVENTS, 1)
    names = [v.name for v in cfg.views if v.name != "expert"]
    kinds = g.integers(0, len(names), n)
    kv_n = g.integers(1, KV_REQ_MAX + 1, n)
    conv_n = g.integers(1, CONV_REQ_MAX + 1, n)
    out = []
    counters = {nm: 0 for nm in names}
    for i in range(n):
        nm = names[kinds[i]]
        cnt = {"kv": int(kv_n[i]), "ssm": 1, "conv": int(conv_n[i])}[nm]
        out.append((nm, FILLER_BASE[nm] + counters[nm], cnt))
        counters[nm] += 1
    return out


def projection_order(cfg: MoEConfig, key: int = 0):
    """Seeded order in which expert projections (owner e*3+p) are placed."""
    return [int(i) for i in rng(cfg.cid, S_EVENTS, 2, key).permutation(cfg.E * 3)]


def churn_events(cfg: MoEConfig):
    """Fragmenting recipe: n_events mixed requests, 70% KV and 30% expert.

    KV: allocate a new request of U{1..128} blocks (odds 0.55) or free one of
    the requests this stream has issued and not yet freed. Expert: allocate a
    projection not yet issued (odds 0.6) or free an issued one; each
    projection is 48 pages. The stream tracks only what it issued, not what
    the allocator granted, so a free may name an owner whose allocation
    failed; runners report that as an error status and carry on.
    """
    g = rng(cfg.cid, S_EVENTS, 3)
    live_kv: list[int] = []
    next_kv = 0
    resident: list[int] = []
    missing = list(range(cfg.E * 3))
    ops = []
    for _ in range(cfg.n_events):
        if g.random() < 0.7:
            if not live_kv or g.random() < 0.55:
                ops.append(("alloc", "kv", OWNER_KV + next_kv, int(g.integers(1, KV_REQ_MAX + 1))))
                live_kv.append(OWNER_KV + next_kv)
                next_kv += 1
            else:
                ops.append(("free", "kv", live_kv.pop(int(g.integers(0, len(live_kv)))), 0))
        else:
            if missing and (not resident or g.random() < 0.6):
                o = missing.pop(int(g.integers(0, len(missing))))
                ops.append(("alloc", "expert", o, cfg.P))
                resident.append(o)
            else:
                o = resident.pop(int(g.integers(0, len(resident))))
                ops.append(("free", "expert", o, 0))
                missing.append(o)
    return ops


def adjuster_plan(cfg: MoEConfig, B: int):
    """Adjuster steps for one batch size: (fraction of pool, direction).

    direction 0 moves capacity from the expert view to the KV view, 1 the
    other way. Fractions are U[0.10, 0.50].
    """
    g = rng(cfg.cid, S_ADJUST, B)
    f = g.uniform(0.10, 0.50, cfg.adjuster_steps)
    d = g.integers(0, 2, cfg.adjuster_steps)
    return [(float(f[i]), int(d[i])) for i in range(cfg.adjuster_steps)]


def adjuster_kv_requests(cfg: MoEConfig, B: int, n: int = 20000):
    """KV request sizes (blocks) that grow the KV view during adjuster steps."""
    g = rng(cfg.cid, S_ADJUST, B, 1)
    return [int(v) for v in g.integers(1, KV_REQ_MAX + 1, n)]


# ---------------------------------------------------------------- serving trace

S_TRACE = 8


def serving_trace(seed: int, steps: int, E: int, k: int, mean_arrivals: float, period: int = 200,
                  prompt_mu: float = 5.5, output_mu: float = 5.0, sigma: float = 0.9,
                  zipf_s: float = 1.1, phase_steps: int = 150, block_tokens: int = 16,
                  max_step_tokens: int | None = None):
    """A synthetic concurrency trace for the adjuster: per forward step, the
    KV blocks the running requests hold plus those arriving need, and how
    many routed slots each expert received.

    Arrivals per step ~ Poisson(mean_arrivals * (1 + 0.8 sin(2 pi s / period)))
    (a request rate that rises and falls over time); prompt and output lengths
    ~ lognormal(mu, sigma), clipped to [16, 8192] and [8, 2048] tokens (a
    chat-like length mix). A running request holds ceil(tokens / block_tokens)
    KV blocks, gains one token per step and leaves after its output length.
    Expert popularity is Zipf(s) over a permutation redrawn every phase_steps
    steps; a step's routed slots (running requests plus the arriving prompts'
    tokens, at most max_step_tokens of them, k each) are one multinomial draw
    over that popularity.
    Returns (blocks int64 [steps], routed int32 [steps, E], concurrency int64 [steps]).
    """
    g = rng(seed, S_TRACE, steps, E)
    running = []                       # [tokens so far, tokens still to generate]
    blocks = np.zeros(steps, dtype=np.int64)
    conc = np.zeros(steps, dtype=np.int64)
    routed = np.zeros((steps, E), dtype=np.int32)
    ranks = np.arange(1, E + 1, dtype=np.float64) ** -zipf_s
    p = None
    for s in range(steps):
        if s % phase_steps == 0:
            p = np.empty(E)
            p[g.permutation(E)] = ranks / ranks.sum()
        lam = mean_arrivals * (1.0 + 0.8 * np.sin(2.0 * np.pi * s / period))
        n_new = int(g.poisson(max(lam, 0.0)))
        prompts = np.clip(np.rint(g.lognormal(prompt_mu, sigma, n_new)), 16, 8192).astype(np.int64)
        outs = np.clip(np.rint(g.lognormal(output_mu, sigma, n_new)), 8, 2048).astype(np.int64)
        tokens = len(running) + int(prompts.sum())
        if max_step_tokens is not None:
            tokens = min(tokens, max_step_tokens)
        for r in running:
            r[0] += 1
            r[1] -= 1
        running = [r for r in running if r[1] > 0]
        running += [[int(a), int(b)] for a, b in zip(prompts, outs)]
        blocks[s] = sum((r[0] + block_tokens - 1) // block_tokens for r in running)
        conc[s] = len(running)
        if tokens:
            routed[s] = g.multinomial(tokens * k, p)
    return blocks, routed, conc
