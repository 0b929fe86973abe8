"""rimuru_fused_moe_paged_noalloc: the layer with the library's fixed device
scratch as its workspace, for callers that cannot allocate. Checked on the
GPU through the C ABI against rimuru_fused_moe_paged (the same kernels with a
caller workspace): routing outputs and y bitwise equal, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents), and y within the 1e-2 bar of the oracle; a shape whose workspace
exceeds the scratch is refused with ENOMEM before anything is enqueued."""
import numpy as np
import pytest
import torch

from gpu_common import host_pool, paged_pool, record, rel_err, decode_dev, say, to_dev_bits, weights_dev
from moe_inputs import gen
from moe_inputs.configs import CFG1
from oracle.moe import moe_forward
from paged_moe_expert_amd import rimuru as R

pytestmark = pytest.mark.gpu

KIB = 1024


def _setup(E, k, H, I, page, seed):
    from dataclasses import replace
    cfg = replace(CFG1, cid=500 + seed, name=f"noalloc-{seed}", E=E, k=k, H=H, I=I, T=1, dtype="bf16",
                  page_bytes=page, logits="normal")
    P = -(-H * I * 2 // page)
    n_pages = E * 3 * P + 5
    pt = np.random.default_rng(3000 + seed).permutation(n_pages)[:E * 3 * P].astype(np.int32).reshape(E, 3, P)
    wb = gen.all_weight_bits(cfg)
    padded = np.zeros((E, 3, P * page // 2), dtype=wb.dtype)
    padded[:, :, :wb.shape[2]] = wb
    pool, ptd = paged_pool(n_pages * page, pt, weights_dev(padded), page)
    return cfg, pt, wb, pool, ptd, n_pages


@pytest.mark.parametrize("E,k,H,I,page,tokens", [
    (128, 8, 2048, 768, 3 * 1024 * KIB, (64, 5)),      # decode layer shape: 64 tokens, then 5
    (16, 4, 512, 256, 16 * KIB, (3000, 500)),          # tiled plans: 128-row, then 64-row tiles
])
def test_noalloc_matches_workspace_entry_point(E, k, H, I, page, tokens):
    cfg, pt, wb, pool, ptd, n_pages = _setup(E, k, H, I, page, seed=E)
    href = host_pool(n_pages * page, page, pt, wb)
    for call, T in enumerate(tokens):
        say(f"[noalloc] E={E} k={k} H={H} I={I} call {call}: T={T}")
        c2 = cfg.with_T(T)
        xb, lg = gen.x_bits(c2, T, seed_key=call), gen.logits(c2, T, seed_key=call)
        x, lgd = to_dev_bits(xb, "bf16"), torch.from_numpy(lg).cuda()
        ref = R.fused_moe_paged(x, lgd, pool, ptd, page, k, I)
        got = R.fused_moe_paged_noalloc(x, lgd, pool, ptd, page, k, I)
        torch.cuda.synchronize()
        for name in ("topk_ids", "topk_w", "expert_off", "y"):
            assert torch.equal(getattr(got, name), getattr(ref, name)), f"call {call}: {name} differs"
        n = int(ref.expert_off[-1].item())
        assert torch.equal(got.sorted_ids[:n], ref.sorted_ids[:n]), f"call {call}: sorted_ids differ"
        o = moe_forward(xb, lg, href, pt, page, E=E, k=k, H=H, I=I, dtype="bf16")
        err = rel_err(decode_dev(got.y), o["y"])
        say(f"[noalloc] call {call}: block_m={got.block_m} rel_err={err:.3e}")
        record(f"no-allocation layer E={E} T={T} (block_m {got.block_m})", err, 1e-2)
        assert err <= 1e-2


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    E, k, H, I, page = 16, 4, 512, 256, 16 * KIB
    T = 40000                                           # workspace far above 64 MiB
    _, ws, _ = R.moe_sizes(T, E, k, H, I, -(-H * I * 2 // page), R.BF16)
    assert ws > R.NOALLOC_SCRATCH_BYTES
    cfg, pt, wb, pool, ptd, n_pages = _setup(E, k, H, I, page, seed=7)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    lgd = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    with pytest.raises(R.RimuruError) as ei:
        R.fused_moe_paged_noalloc(x, lgd, pool, ptd, page, k, I)
    assert ei.value.status == R.ENOMEM
