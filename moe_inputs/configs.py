"""Workload registry for the paged fused-MoE layer.

Shapes come from Table 1 of the Rimuru paper summary (thelatestinai.com,
"Tensor heterogeneity in representative modern LLMs"): per-expert projections
w1/w3 [2048, 768] and w2 [768, 2048] for Qwen3-30B-A3B, [2048, 512] /
[512, 2048] for Qwen3.5-35B-A3B; one token's K and V [2, 4, 128] and
[2, 2, 256]; conv state [3, 8192] and SSM state [32, 128, 128] for
Qwen3.5-35B-A3B only.

Page sizes follow the explainer (learnaivisually.com, "Rimuru unifies
serving memory"), paragraph on moving the fence: KV blocks hold 16 tokens,
each tensor type has its own page size, and huge pages are a common
multiple of the expert and state page sizes.

This module only describes workloads. It holds no arithmetic of the method
and is shared, read-only, by the oracle and by the product.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from math import gcd

KIB = 1 << 10
MIB = 1 << 20
GIB = 1 << 30


def lcm(a: int, b: int) -> int:
    return a // gcd(a, b) * b


@dataclass(frozen=True)
class ViewSpec:
    """One memory view: a tensor type's own page size over the shared pool.

    parent is None when pages are cut straight from huge pages, else the name
    of the view whose page is split into pages of this view.
    """
    name: str
    kind: int          # 0 expert, 1 kv, 2 ssm, 3 conv
    page_bytes: int
    parent: str | None


@dataclass(frozen=True)
class MoEConfig:
    cid: int
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    dtype: str                 # "f32" or "bf16": x, weights, y share it
    page_bytes: int            # expert-view page
    huge_bytes: int
    pool_bytes: int
    logits: str                # "normal", "uniform" or "zipf"
    zipf_s: float = 0.0
    views: tuple = ()
    layout: str = ""           # layout recipe name
    n_events: int = 0          # churn events (fragmented recipe)
    batches: tuple = ()        # decode sweep batch sizes
    adjuster_steps: int = 0
    kv_shape: tuple = ()       # one token's K and V: [2, kv_heads, head_dim] (Table 1)

    @property
    def es(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def proj_bytes(self) -> int:
        return self.H * self.I * self.es

    @property
    def P(self) -> int:
        """Expert-view pages per projection."""
        assert self.proj_bytes % self.page_bytes == 0
        return self.proj_bytes // self.page_bytes

    def view(self, name: str) -> ViewSpec:
        for v in self.views:
            if v.name == name:
                return v
        raise KeyError(name)

    def with_T(self, T: int) -> "MoEConfig":
        from dataclasses import replace
        return replace(self, T=T)


# Per-token KV bytes: K and V tensors of Table 1, 16 tokens per block.
KV_BLOCK_TOKENS = 16


def kv_block_bytes(kv_shape, es):
    n = 1
    for d in kv_shape:
        n *= d
    return KV_BLOCK_TOKENS * n * es


# Tiny fp32 layer: KV block of 16 tokens x [2, 4, 32] fp32 = 16 KiB; expert
# page 4 KiB; huge page = lcm(4 KiB, 16 KiB); 256 pages of 4 KiB in the pool.
_c1_kv = kv_block_bytes((2, 4, 32), 4)
CFG1 = MoEConfig(
    cid=1, name="tiny-fp32", T=16, E=8, k=2, H=128, I=64, dtype="f32",
    page_bytes=4 * KIB, huge_bytes=lcm(4 * KIB, _c1_kv), pool_bytes=256 * 4 * KIB,
    logits="normal",
    views=(ViewSpec("expert", 0, 4 * KIB, None), ViewSpec("kv", 1, _c1_kv, None)),
    layout="scatter", kv_shape=(2, 4, 32),
)

# Qwen3-30B-A3B decode: one 3 MiB page per projection; KV block 16 x [2,4,128]
# bf16 = 32 KiB cut from expert-sized pages; huge = lcm(3 MiB, 32 KiB) = 3 MiB.
_q3_kv = kv_block_bytes((2, 4, 128), 2)
CFG2 = MoEConfig(
    cid=2, name="qwen3-30b-a3b-decode", T=64, E=128, k=8, H=2048, I=768, dtype="bf16",
    page_bytes=3 * MIB, huge_bytes=lcm(3 * MIB, _q3_kv), pool_bytes=4 * GIB,
    logits="uniform",
    views=(ViewSpec("expert", 0, 3 * MIB, None), ViewSpec("kv", 1, _q3_kv, "expert")),
    layout="fill_then_place", kv_shape=(2, 4, 128),
)

# Qwen3.5-35B-A3B prefill: 2 MiB projections; SSM state [32,128,128] bf16 = 1 MiB;
# conv state [3,8192] bf16 = 48 KiB; KV block 16 x [2,2,256] bf16 = 32 KiB.
# huge = lcm(expert page, SSM page) = 2 MiB.
_q35_kv = kv_block_bytes((2, 2, 256), 2)
_q35_ssm = 32 * 128 * 128 * 2
_q35_conv = 3 * 8192 * 2
CFG3 = MoEConfig(
    cid=3, name="qwen3.5-35b-a3b-prefill", T=2048, E=256, k=8, H=2048, I=512, dtype="bf16",
    page_bytes=2 * MIB, huge_bytes=lcm(2 * MIB, _q35_ssm), pool_bytes=4 * GIB,
    logits="zipf", zipf_s=1.1,
    views=(ViewSpec("expert", 0, 2 * MIB, None), ViewSpec("kv", 1, _q35_kv, "expert"),
           ViewSpec("ssm", 2, _q35_ssm, None), ViewSpec("conv", 3, _q35_conv, "expert")),
    layout="fill_then_place", kv_shape=(2, 2, 256),
)

# Large prefill with sub-page fragmentation: 64 KiB expert pages (48 per
# projection), 32 KiB KV blocks cut from 64 KiB pages, 3 MiB huge pages (a
# multiple of lcm(64 KiB, 32 KiB) that one projection fills exactly).
CFG4 = MoEConfig(
    cid=4, name="prefill-fragmented", T=8192, E=128, k=8, H=2048, I=768, dtype="bf16",
    page_bytes=64 * KIB, huge_bytes=3 * MIB, pool_bytes=4 * GIB,
    logits="zipf", zipf_s=1.2,
    views=(ViewSpec("expert", 0, 64 * KIB, None), ViewSpec("kv", 1, _q3_kv, "expert")),
    layout="churn", n_events=10_000, kv_shape=(2, 4, 128),
)

# Decode sweep under a moving KV/expert boundary: the decode layout, then
# seeded adjuster steps between kernel calls.
CFG5 = MoEConfig(
    cid=5, name="decode-sweep", T=64, E=128, k=8, H=2048, I=768, dtype="bf16",
    page_bytes=3 * MIB, huge_bytes=lcm(3 * MIB, _q3_kv), pool_bytes=4 * GIB,
    logits="uniform",
    views=(ViewSpec("expert", 0, 3 * MIB, None), ViewSpec("kv", 1, _q3_kv, "expert")),
    layout="fill_then_place", batches=(1, 4, 16, 64, 256), adjuster_steps=10, kv_shape=(2, 4, 128),
)

CONFIGS = {c.cid: c for c in (CFG1, CFG2, CFG3, CFG4, CFG5)}

# KV request sizes (blocks) drawn U{1..KV_REQ_MAX}; conv requests U{1..CONV_REQ_MAX}.
KV_REQ_MAX = 128
CONV_REQ_MAX = 40
