"""The layer with its router projection (rimuru_fused_moe_paged_router):
logits = x . w_gate^T by the router GEMM kernel in the gating stage, then the
same top-k, sort, GEMMs and combine.

Checks, on the GPU through the C ABI, against the oracle:
  - the fp32 logits (logits_out) against the fp64 oracle logits, within the
    fp32 accumulation bound K * 2^-24 * sum |x w| (plus the fp32 product
    rounding for fp32 inputs);
  - ids and weights: the oracle's routing of the GPU's own logits, exactly
    (ties are decided on the kernel's fp32 logits, as the header states);
  - the layer output: bitwise equal to the plain entry point fed the same
    logits, and within tolerance of the oracle layer on those logits;
  - the same result without logits_out.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from gpu_common import (check_routing, decode_dev, host_pool, paged_pool, record, rel_err, say, to_dev_bits,
                        weights_dev)
from moe_inputs import CONFIGS, gen
from oracle.moe import decode, moe_forward, route, router_logits
from paged_moe_expert_amd import rimuru as R

pytestmark = pytest.mark.gpu

KIB = 1024
TOL = {"bf16": 1e-2, "f32": 1e-4}

CASES = [
    # name, E, k, H, I, T, dtype, page
    ("bf16-router-mid", 16, 4, 256, 128, 100, "bf16", 4 * KIB),
    ("bf16-router-E8-H192", 8, 2, 192, 64, 37, "bf16", 4 * KIB),        # E not a multiple of 16, 2 K slices
    ("bf16-router-E40", 40, 6, 128, 64, 70, "bf16", 4 * KIB),           # partial last expert tile
    ("f32-router", 8, 2, 128, 64, 33, "f32", 4 * KIB),
    ("bf16-router-decode-shape", 128, 8, 2048, 768, 64, "bf16", 3 * 1024 * KIB),
    ("bf16-router-prefill-tiles", 16, 4, 512, 256, 1200, "bf16", 16 * KIB),
    # register-operand router GEMM (fp32 inputs): enough token blocks for
    # its wider expert tiles (32, 64 and 128 experts per workgroup), each
    # with a ragged token tail
    ("f32-router-nt2", 128, 8, 128, 64, 4100, "f32", 8 * KIB),
    ("f32-router-nt4", 128, 8, 128, 64, 8200, "f32", 8 * KIB),
    ("f32-router-nt8-E64", 64, 4, 128, 64, 16400, "f32", 8 * KIB),   # tile wider than E
    # LDS-staged router GEMM (bf16, H a multiple of 64, a workgroup per CU):
    # 128, 64 and 32 experts per workgroup (no K split, 2-way, 4-way), a
    # ragged token tail, an expert tile past E, a one-stage K loop, and the
    # 8192-token prefill's router shape
    ("bf16-router-wide-ne4-E200", 200, 8, 512, 64, 4100, "bf16", 8 * KIB),
    ("bf16-router-wide-ne2", 128, 8, 192, 64, 4100, "bf16", 8 * KIB),
    ("bf16-router-wide-ne1-one-stage", 40, 6, 64, 64, 4100, "bf16", 8 * KIB),
    ("bf16-router-prefill-shape", 128, 8, 2048, 64, 8192, "bf16", 64 * KIB),
]


def _setup(name, E, k, H, I, T, dtype, page, seed):
    cfg = replace(CONFIGS[1], cid=300 + seed, name=name, E=E, k=k, H=H, I=I, T=T, dtype=dtype,
                  page_bytes=page, logits="normal")
    es = cfg.es
    P = -(-H * I * es // page)
    n_pages = E * 3 * P + 3
    r = np.random.default_rng(2000 + seed)
    pt = r.permutation(n_pages)[:E * 3 * P].astype(np.int32).reshape(E, 3, P)
    wb = gen.all_weight_bits(cfg)
    padded = np.zeros((E, 3, P * page // es), dtype=wb.dtype)
    padded[:, :, :wb.shape[2]] = wb
    pool, ptd = paged_pool(n_pages * page, pt, weights_dev(padded), page)
    xb = gen.x_bits(cfg, T)
    gb = gen.gate_weight_bits(cfg)
    return cfg, pt, pool, ptd, xb, gb, wb, n_pages


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_router_against_oracle(spec):
    name, E, k, H, I, T, dtype, page = spec
    say(f"[router] {name}: E={E} k={k} H={H} I={I} T={T} {dtype}")
    cfg, pt, pool, ptd, xb, gb, wb, n_pages = _setup(*spec, seed=CASES.index(spec))
    x = to_dev_bits(xb, dtype)
    wg = to_dev_bits(gb, dtype)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    b = R.fused_moe_paged(x, None, pool, ptd, page, k, I, w_gate=wg, logits_out=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()

    # fp32 logits vs fp64 oracle logits, within the accumulation bound
    ref_l = router_logits(xb, gb, dtype)
    xd = decode(xb.reshape(-1), dtype).reshape(T, H)
    gd = decode(gb.reshape(-1), dtype).reshape(E, H)
    mag = np.abs(xd) @ np.abs(gd).T
    bound = (H + 2) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(lg.astype(np.float64) - ref_l)
    say(f"[router] {name}: max logit error {err.max():.3e}, max bound ratio {(err / bound).max():.3f}")
    assert np.all(err <= bound)

    # routing: exactly the oracle's routing of these fp32 logits
    ids_ref, w_ref = route(lg, k)
    assert np.array_equal(b.topk_ids.cpu().numpy(), ids_ref)

    # layer: bitwise equal to the plain entry point on the same logits ...
    b2 = R.fused_moe_paged(x, logits, pool, ptd, page, k, I)
    torch.cuda.synchronize()
    assert torch.equal(b.y, b2.y)
    assert torch.equal(b.topk_w, b2.topk_w)
    # ... and the oracle layer on them, every token, its pool built on the
    # host from the generator's weights and the page table
    ref = moe_forward(xb, lg, host_pool(n_pages * page, page, pt, wb), pt, page, E=E, k=k, H=H, I=I,
                      dtype=dtype)
    check_routing(b, ref, T, k, E, b.block_m)
    e2 = rel_err(decode_dev(b.y), ref["y"])
    say(f"[router] {name}: block_m={b.block_m} rel_err={e2:.3e} over all {T} tokens")
    record(f"router {name} (block_m {b.block_m})", e2, TOL[dtype])
    record(f"router {name} logits", float((err / bound).max()), 1.0, "err/fp32 bound")
    assert e2 <= TOL[dtype]

    # without logits_out: same result
    b3 = R.fused_moe_paged(x, None, pool, ptd, page, k, I, w_gate=wg)
    torch.cuda.synchronize()
    assert torch.equal(b3.y, b.y)
