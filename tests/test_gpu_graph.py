"""The fused MoE layer captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed. The layer allocates nothing, synchronises nothing and issues no
memset, so it can be captured as it is; a decode step at small batches is
then one graph launch instead of several kernel launches from the host.

Each replay gets new inputs written into the captured x and logits buffers,
with eager work and synchronisations between replays, and its outputs must
equal those of an eager call on the same inputs bitwise. Cases: 3 tokens
(the gate/up stream routes the batch itself), 8 tokens (one-workgroup
routing, weight streaming), 40 tokens (gating + sort, weight streaming) and
300 tokens (64-row tiled GEMMs).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from moe_inputs import gen
from moe_inputs.configs import CFG1, KIB

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_common import paged_pool, say, to_dev_bits, weights_dev
    from paged_moe_expert_amd import rimuru as R


@pytest.mark.parametrize("T", [3, 8, 40, 300])
def test_graph_replay_equals_eager(T):
    E, k, H, I, page = 16, 4, 256, 128, 4 * KIB
    cfg = replace(CFG1, cid=400 + T, name=f"bf16-graph-T{T}", E=E, k=k, H=H, I=I, T=T, dtype="bf16",
                  page_bytes=page, logits="normal")
    P = H * I * 2 // page
    n_pages = E * 3 * P + 5
    pt = np.random.default_rng(500 + T).permutation(n_pages)[:E * 3 * P].astype(np.int32).reshape(E, 3, P)
    pool, ptd = paged_pool(n_pages * page, pt, weights_dev(gen.all_weight_bits(cfg)), page)
    xs = [to_dev_bits(gen.x_bits(cfg, T, s), "bf16") for s in range(3)]
    lgs = [torch.from_numpy(gen.logits(cfg, T, s)).cuda() for s in range(3)]

    bufs = R.MoeBuffers(T, E, k, H, I, P, R.BF16)
    say(f"[graph] T={T} E={E} k={k} block_m={bufs.block_m}")
    ref = []
    for s in range(3):
        R.fused_moe_paged(xs[s], lgs[s], pool, ptd, page, k, I, bufs=bufs)
        torch.cuda.synchronize()
        ref.append((bufs.y.clone(), bufs.topk_ids.clone(), bufs.sorted_ids.clone(), bufs.expert_off.clone()))
    assert not torch.equal(ref[0][0], ref[1][0])

    x = xs[0].clone()
    lg = lgs[0].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        R.fused_moe_paged(x, lg, pool, ptd, page, k, I, bufs=bufs)     # warm-up on the capture side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        R.fused_moe_paged(x, lg, pool, ptd, page, k, I, bufs=bufs)

    other = R.MoeBuffers(T, E, k, H, I, P, R.BF16)
    for rep in range(7):
        s = (rep * 2 + 1) % 3
        x.copy_(xs[s])
        lg.copy_(lgs[s])
        g.replay()
        torch.cuda.synchronize()
        y, ids, srt, off = ref[s]
        assert torch.equal(bufs.y, y), f"replay {rep} (input {s}): y differs from the eager call"
        assert torch.equal(bufs.topk_ids, ids) and torch.equal(bufs.expert_off, off)
        n = int(off[-1].item())
        assert torch.equal(bufs.sorted_ids[:n], srt[:n])
        # eager work between replays: another layer call and a torch reduction
        R.fused_moe_paged(xs[rep % 3], lgs[rep % 3], pool, ptd, page, k, I, bufs=other)
        float(other.y.float().abs().sum())
        torch.cuda.synchronize()
