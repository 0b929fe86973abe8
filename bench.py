"""Benchmark of the paged fused-MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 4] [--nested 2,3] [--no-cpu]

Headline workload (default): the large prefill with sub-page fragmentation --
8192 tokens, 128 experts, top-8, hidden 2048, inter 768, bf16 weights split
into 64 KiB pages placed by 10,000 seeded allocator events on a 4 GiB pool
shared with KV blocks, Zipf(1.2) routing. It is the largest single-GPU
configuration and the MFMA-bound one. The Qwen3-30B-A3B-shaped decode layer
(64 tokens, one 3 MiB page per projection) and the Qwen3.5-35B-A3B-shaped
prefill (2048 tokens, 256 experts) are measured in the same run and nested in
the line under "other_workloads", each with its own roofline.

Inputs are synthetic and resident in HBM before timing starts. One step is
one call of the whole layer (gating, count, sort, gate/up GEMM, down GEMM,
combine). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # dense bf16 MFMA
CSRC = os.path.join(ROOT, "paged_moe_expert_amd", "csrc")
# sources each GEMM kernel is compiled from: a traffic measurement stays valid
# while these are unchanged
KERNEL_SOURCES = {"stream": ("moe_common.h", "moe_gemm_stream.hip"),
                  "tiled": ("moe_common.h", "moe_gemm_tiled.hip"),
                  "prefill": ("moe_common.h", "moe_gemm_prefill.hip")}
# GEMM kernel family (gate/up, down) of each tile height
KIND_OF_BLOCK_M = {16: ("stream", "stream"), 32: ("stream", "stream"), 64: ("tiled", "prefill"),
                   128: ("prefill", "prefill")}
STAGES = ["gating", "count", "sort", "gemm_up", "gemm_down", "combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def traffic_from_profiles(workload: str, kernel: str, kind: str):
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    measurement was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha256") != kernel_sha(kind):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, xb, lg, wb, n_tokens: int):
    """The oracle, as it stands, on a bounded sample of the same workload:
    routing of every token, the page resolution of every expert the sample
    touches, and the fp64 expert MLPs and combine of the sampled tokens. The
    BLAS thread count is the process's own (OMP_NUM_THREADS where the host
    sets it for this job's CPU share); cores reports the threads the BLAS
    pools actually ran with."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.layout import Layout, build_pool
    from oracle.moe import moe_forward
    lay = Layout(cfg).run()
    pt = lay.page_table()
    pool = build_pool(cfg, pt, wb, poison=False)
    toks = np.arange(n_tokens)
    t0 = time.perf_counter()
    moe_forward(xb, lg, pool, pt, cfg.page_bytes, E=cfg.E, k=cfg.k, H=cfg.H, I=cfg.I,
                dtype=cfg.dtype, tokens=toks)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the first {n_tokens} of {cfg.T} tokens (routing over all {cfg.T}, pages of every "
                      f"expert they touch resolved), fp64 numpy; {dt:.2f} s",
            "host_cpu_count": os.cpu_count(), "host_affinity_cpus": affinity,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"), "cpu_model": cpu_model()}


PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def adjuster_bench(cfg, R, np, gen, upload_gbs):
    """Host-side cost of the adjuster policy on this layer's pool: a seeded
    synthetic serving trace (rising and falling request rate, chat-like
    lengths) drives the native adjuster over the layer's expert and KV views;
    each step's call is timed (ctypes marshalling included), and the experts it
    loads are priced at the measured upload rate."""
    import time as _t
    xs, ks = cfg.view("expert"), cfg.view("kv")
    pool = R.pool_create(cfg.pool_bytes, cfg.huge_bytes)
    xv = R.view_map(pool, xs.kind, xs.page_bytes)
    kv = R.view_map(pool, ks.kind, ks.page_bytes, xv)
    for e in range(cfg.E):
        for p in range(3):
            R.view_alloc(xv, 3 * e + p, cfg.P)
    usable = R.pool_stats(pool)["huge_pages"] * cfg.huge_bytes
    xb = cfg.E * 3 * cfg.P * xs.page_bytes
    R.view_set_budget(xv, xb)
    R.view_set_budget(kv, usable - xb)
    prm = dict(min_resident=96, headroom_blocks=256, return_blocks=2048, shift=3, max_prefetch=4)
    adj = R.adjuster_create(pool, xv, kv, cfg.E, cfg.P, **prm)
    blocks, routed, _ = gen.serving_trace(31, 300, cfg.E, cfg.k, mean_arrivals=30.0, prompt_mu=5.5,
                                          output_mu=4.8, max_step_tokens=8, phase_steps=60, period=100)
    owners, us, ev, ld, met = [], [], 0, 0, 0
    kvb = ks.page_bytes
    for st in range(len(blocks)):
        d = int(blocks[st])
        needed = (routed[st] > 0).astype(np.uint8)
        t0 = _t.perf_counter()
        r = R.adjuster_step(adj, d, routed[st], needed)
        us.append((_t.perf_counter() - t0) * 1e6)
        ev += len(r["evicted"])
        ld += len(r["loaded"])
        for e in r["loaded"]:
            R.adjuster_upload_done(adj, e)
        budget = R.view_usage(kv)[1]
        met += budget >= d * kvb
        target = min(d, budget // kvb)
        held = sum(n for _, n in owners)
        while owners and held > target:
            o, n = owners.pop()
            R.view_free(kv, o)
            held -= n
        if target > held and R.view_alloc_status(kv, (1 << 40) + st, target - held)[0] == R.OK:
            owners.append(((1 << 40) + st, target - held))
    n = len(blocks)
    mb = ld * 3 * cfg.proj_bytes / n / 1e6
    out = {"trace_steps": n, "host_us_per_step_median": round(float(np.median(us)), 1),
           "host_us_per_step_p99": round(float(np.percentile(us, 99)), 1),
           "evictions_per_step": round(ev / n, 2), "loads_per_step": round(ld / n, 2),
           "upload_mb_per_step": round(mb, 2), "demand_met_fraction": round(met / n, 3),
           "params": prm}
    if upload_gbs:
        out["upload_ms_per_step_at_measured_rate"] = round(mb / 1e3 / upload_gbs * 1e3, 3)
    return out


def expert_upload_bench(args, cfg, wb, idt, dev, step, R, torch, np):
    """Upload n experts' weights from pinned host memory into fresh pages of
    their own, first alone, then while the layer runs on the compute stream."""
    n = min(args.upload_experts, cfg.E)
    proj = cfg.proj_bytes
    pages = n * 3 * cfg.P
    dst = torch.empty(pages * cfg.page_bytes, dtype=torch.uint8, device=dev)
    host = torch.from_numpy(np.ascontiguousarray(wb[:n]).view(np.uint8).reshape(n, 3, proj)).pin_memory()
    rows = np.arange(pages, dtype=np.int32).reshape(n, 3, cfg.P)
    side = torch.cuda.Stream(device=dev)
    main = torch.cuda.current_stream(dev)

    # raw entry point with the pointers worked out once: the timed copies are
    # not held back by per-call argument checks on the host
    dptr, dbytes, hptr = dst.data_ptr(), dst.numel(), host.data_ptr()
    rows_c = [np.ascontiguousarray(rows[j]) for j in range(n)]
    sh = side.cuda_stream

    def upload_round():
        for j in range(n):
            R.check(R.expert_upload_raw(dptr, dbytes, rows_c[j], cfg.page_bytes, hptr + j * 3 * proj,
                                        proj, sh), "expert_upload")

    upload_round()                                      # warm
    side.synchronize()
    e0, e1 = R.event_create(), R.event_create()
    R.event_record(e0, side)
    for _ in range(8):
        upload_round()
    R.event_record(e1, side)
    side.synchronize()
    alone_ms = R.event_elapsed_ms(e0, e1) / 8
    bytes_round = n * 3 * proj
    # overlapped: enough rounds to cover the timed layer steps
    torch.cuda.synchronize()
    m0, m1 = R.event_create(), R.event_create()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    layer_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    rounds = max(1, int(round(layer_ms * args.steps / alone_ms)))
    torch.cuda.synchronize()
    R.event_record(e0, side)
    R.event_record(m0, main)
    for _ in range(rounds):
        upload_round()
    for _ in range(args.steps):
        step()
    R.event_record(e1, side)
    R.event_record(m1, main)
    torch.cuda.synchronize()
    up_ms = R.event_elapsed_ms(e0, e1)
    lay_ms = R.event_elapsed_ms(m0, m1) / args.steps
    for e in (e0, e1, m0, m1):
        R.event_destroy(e)
    del dst
    gbs_alone = bytes_round / (alone_ms * 1e-3) / 1e9
    gbs_ovl = rounds * bytes_round / (up_ms * 1e-3) / 1e9
    return {"experts": n, "bytes_per_round": bytes_round, "pages_per_expert": 3 * cfg.P,
            "upload_gbs_alone": round(gbs_alone, 2), "upload_gbs_overlapped": round(gbs_ovl, 2),
            "peak_gbs": PCIE_PEAK_GBS, "frac_alone": round(gbs_alone / PCIE_PEAK_GBS, 4),
            "layer_ms_alone": round(layer_ms, 4), "layer_ms_overlapped": round(lay_ms, 4),
            "rounds_overlapped": rounds}


def attention_bench(args, cfg, lay, pool, dev, R, torch, np):
    """Paged decode attention over the KV view of the layer's own pool: the
    first n live KV requests of the layout (their blocks sit between the
    expert pages), one query token each, K/V filled with N(0, 1) bf16 and
    contexts of (blocks - u) tokens, u ~ U{0..15} seeded. Timed back to back
    (a batch of calls between two events) and cache-cold (a 4 GiB read before
    each call, an event pair around it)."""
    ks = cfg.view("kv")
    bb = ks.page_bytes
    n_kv, D = cfg.kv_shape[1], cfg.kv_shape[2]
    n_q = 8 * n_kv                                   # Qwen3-30B-A3B: 32 query heads over 4 KV heads
    kv = lay.views["kv"]
    reqs = [o for name, o in lay.live if name == "kv"][:args.attn_requests]
    blocks = [R.view_pages(kv, o) // bb for o in reqs]
    B, mb = len(blocks), max(len(b) for b in blocks)
    rng = np.random.default_rng(2024)
    lens = np.array([16 * len(b) - int(rng.integers(0, 16)) for b in blocks], dtype=np.int32)
    table = np.zeros((B, mb), dtype=np.int32)
    for i, b in enumerate(blocks):
        table[i, :len(b)] = b
    R.block_table_check(table, lens, bb, cfg.pool_bytes)
    idx = torch.from_numpy(np.concatenate(blocks).astype(np.int64)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(2025)
    kvv = pool.view(torch.bfloat16).view(-1, bb // 2)
    kvv[idx] = torch.randn((idx.numel(), bb // 2), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((B, n_q, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    bt = torch.from_numpy(table).to(dev)
    lt = torch.from_numpy(lens).to(dev)
    out = torch.empty_like(q)
    ws_bytes, n_split, _ = R.attn_sizes(B, n_q, n_kv, D, mb)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    scale = 1.0 / float(np.sqrt(D))

    def call():
        R.paged_decode_attention(q, pool, bt, lt, n_kv, scale, out=out, workspace=ws)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = R.event_create(), R.event_create()
    R.event_record(e0)
    for _ in range(args.steps):
        call()
    R.event_record(e1)
    torch.cuda.synchronize()
    warm_us = R.event_elapsed_ms(e0, e1) * 1e3 / args.steps
    flush = torch.ones((4096 << 20) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    cold = []
    for _ in range(min(args.steps, 20)):
        torch.sum(flush, dim=0, out=sink)
        R.event_record(e0)
        call()
        R.event_record(e1)
        torch.cuda.synchronize()
        cold.append(R.event_elapsed_ms(e0, e1) * 1e3)
    del flush
    R.event_destroy(e0)
    R.event_destroy(e1)
    kv_bytes = int(lens.sum()) * 2 * n_kv * D * 2
    io_bytes = 2 * B * n_q * D * 2 + B * (mb + 1) * 4
    cold_us = float(np.median(cold))
    return {"requests": B, "n_q": n_q, "n_kv": n_kv, "head_dim": D, "context_tokens": int(lens.sum()),
            "context_min_max": [int(lens.min()), int(lens.max())], "splits": int(n_split),
            "algorithmic_bytes": kv_bytes + io_bytes,
            "us_per_call_back_to_back": round(warm_us, 2),
            "us_per_call_cache_cold_median": round(cold_us, 2),
            "hbm_gbs_cache_cold": round((kv_bytes + io_bytes) / (cold_us * 1e-6) / 1e9, 1),
            "hbm_frac_cache_cold": round((kv_bytes + io_bytes) / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def copy_foil_bench(args, cfg, x, lgd, pool, ptd, pt, bufs, dev, R, torch, np):
    """The copy the paged kernel avoids: each step first gathers every touched
    expert's pages into one contiguous buffer (one device gather of whole
    pages), then runs the same layer on that buffer. The touched set is the
    one this input routes to (the same every step)."""
    # the paged layer on the given logits first: its routing picks the
    # experts to gather and its output is the one the foil must reproduce
    R.fused_moe_paged(x, lgd, pool, ptd, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs)
    torch.cuda.synchronize()
    off = bufs.expert_off.cpu().numpy()
    srt = bufs.sorted_ids.cpu().numpy()
    TK = x.shape[0] * cfg.k
    touched = [e for e in range(cfg.E) if np.any(srt[off[e]:off[e + 1]] < TK)]
    pages = np.ascontiguousarray(pt[touched].reshape(-1)).astype(np.int64)   # [touched][3][P] pool pages
    staged_pt = np.zeros_like(pt)
    staged_pt[touched] = np.arange(pages.size, dtype=np.int32).reshape(len(touched), 3, cfg.P)
    idx = torch.from_numpy(pages).to(dev)
    whole = cfg.pool_bytes // cfg.page_bytes * (cfg.page_bytes // 8)     # the pool's whole pages
    src = pool.view(torch.int64)[:whole].view(-1, cfg.page_bytes // 8)
    staged = torch.empty((pages.size, cfg.page_bytes // 8), dtype=torch.int64, device=dev)
    spt = torch.from_numpy(staged_pt).to(dev)
    sview = staged.view(torch.uint8).view(-1)

    def gather():
        torch.index_select(src, 0, idx, out=staged)

    def fstep():
        gather()
        R.fused_moe_paged(x, lgd, sview, spt, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs)
    ybuf = bufs.y.clone()
    fstep()
    torch.cuda.synchronize()
    same = bool(torch.equal(ybuf.view(torch.uint8), bufs.y.view(torch.uint8)))
    for _ in range(args.warmup):
        fstep()
    e0, e1, e2 = R.event_create(), R.event_create(), R.event_create()
    torch.cuda.synchronize()
    R.event_record(e0)
    for _ in range(args.steps):
        fstep()
    R.event_record(e1)
    for _ in range(args.steps):
        gather()
    R.event_record(e2)
    torch.cuda.synchronize()
    step_ms = R.event_elapsed_ms(e0, e1) / args.steps
    gather_ms = R.event_elapsed_ms(e1, e2) / args.steps
    for e in (e0, e1, e2):
        R.event_destroy(e)
    moved = 2 * pages.size * cfg.page_bytes
    del staged
    return {"experts_gathered": len(touched), "bytes_gathered": int(pages.size * cfg.page_bytes),
            "gather_ms": round(gather_ms, 4), "gather_gbs_read_plus_write": round(moved / (gather_ms * 1e-3) / 1e9, 1),
            "ms_per_step_gather_then_layer": round(step_ms, 4), "bitwise_equal_output": same}


def graph_bench(args, cfg, x, lgd, pool, ptd, bufs, R, torch):
    """The same layer captured once in a HIP graph and replayed: one graph
    launch per step instead of the host enqueueing each kernel."""
    def layer():
        R.fused_moe_paged(x, lgd, pool, ptd, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs)
    layer()
    torch.cuda.synchronize()
    y_eager = bufs.y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(bufs.y, y_eager))
    e0, e1 = R.event_create(), R.event_create()
    R.event_record(e0)
    for _ in range(args.steps):
        g.replay()
    R.event_record(e1)
    torch.cuda.synchronize()
    ms = R.event_elapsed_ms(e0, e1) / args.steps
    R.event_destroy(e0)
    R.event_destroy(e1)
    del g
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(x.shape[0] / (ms * 1e-3), 1),
            "bitwise_equal_output": same}


def read_ceiling(args, dev, R, torch):
    """A plain streaming read on this GPU (rimuru_stream_read: one pass of
    16-byte loads over a 4 GiB buffer), event-timed; the practical bound
    beside the datasheet peak."""
    n = (4096 << 20) // 4
    buf = torch.ones(n, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        R.stream_read(buf, sink)
    e0, e1 = R.event_create(), R.event_create()
    torch.cuda.synchronize()
    R.event_record(e0)
    reps = 5
    for _ in range(reps):
        R.stream_read(buf, sink)
    R.event_record(e1)
    torch.cuda.synchronize()
    ms = R.event_elapsed_ms(e0, e1) / reps
    R.event_destroy(e0)
    R.event_destroy(e1)
    del buf
    return 4 * n / (ms * 1e-3) / 1e9



def setup_layer(cfg, T, dev, R, torch, np, gen):
    """Layout, weights on their pages and device-resident inputs (untimed)."""
    from paged_moe_expert_amd.layouts import DeviceLayout
    t0 = time.perf_counter()
    lay = DeviceLayout(cfg).run()
    pt = lay.page_table()
    wb = gen.all_weight_bits(cfg)
    xb, lg = gen.x_bits(cfg, T), gen.logits(cfg, T)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    idt = np.int16 if cfg.dtype == "bf16" else np.int32
    wdev = torch.from_numpy(wb.view(idt)).to(dev)
    pool = torch.empty(cfg.pool_bytes, dtype=torch.uint8, device=dev)
    pool.view(torch.int32).fill_(0x7FC07FC0)
    ptd = torch.from_numpy(pt).to(dev)
    R.experts_store(pool, ptd, wdev, cfg.page_bytes)
    del wdev
    x = torch.from_numpy(xb.view(idt)).to(dev).view(tdt)
    lgd = torch.from_numpy(lg).to(dev)
    dt_code = R.BF16 if cfg.dtype == "bf16" else R.F32
    bufs = R.MoeBuffers(T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.P, dt_code, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: setup {time.perf_counter() - t0:.1f} s")
    return dict(lay=lay, pt=pt, wb=wb, xb=xb, lg=lg, tdt=tdt, idt=idt, pool=pool, ptd=ptd, x=x, lgd=lgd,
                bufs=bufs)


def measure(args, cfg, T, extras, dev, R, torch, np, gen):
    """Time the layer on one configuration; returns the result object (the
    headline fields plus the extras asked for)."""
    log(f"[bench] {cfg.name}: T={T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} {cfg.dtype} "
        f"page={cfg.page_bytes} pool={cfg.pool_bytes >> 20} MiB")
    L = setup_layer(cfg, T, dev, R, torch, np, gen)
    lay, pt, wb, idt, tdt = L["lay"], L["pt"], L["wb"], L["idt"], L["tdt"]
    pool, ptd, x, lgd, bufs = L["pool"], L["ptd"], L["x"], L["lgd"], L["bufs"]

    def step(events=None):
        R.fused_moe_paged(x, lgd, pool, ptd, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs,
                          stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: warmup done")

    # Timed region 1: the headline. Stage events are left out here because
    # each event record costs the stream a few microseconds.
    flush_buf = None
    if args.flush_mib:
        flush_buf = torch.ones((args.flush_mib << 20) // 4, dtype=torch.float32, device=dev)
        flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def timed(run):
        """Seconds for args.steps calls of run(), and the per-step ms list
        when every step is cache-cold (else None)."""
        pairs = [(R.event_create(), R.event_create()) for _ in range(args.steps)] if flush_buf is not None else []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            if flush_buf is not None:
                torch.sum(flush_buf, dim=0, out=flush_sink)     # a read of the whole buffer
                R.event_record(pairs[s][0])
                run()
                R.event_record(pairs[s][1])
            else:
                run()
        torch.cuda.synchronize()
        secs = time.perf_counter() - t0
        if not pairs:
            return secs, None
        # cache-cold steps: the step time is the event-pair time, not the wall
        ms = [R.event_elapsed_ms(a, b) for a, b in pairs]
        for a, b in pairs:
            R.event_destroy(a)
            R.event_destroy(b)
        return sum(ms) / 1e3, ms

    wall, step_ms = timed(step)
    # Timed region 2: the same steps with an event before and after every
    # stage, on the stream the kernels run on, for per-kernel durations.
    evs = [[R.event_create() for _ in range(R.MOE_STAGES + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t1
    stage_ms = np.zeros((args.steps, R.MOE_STAGES))
    for s in range(args.steps):
        for i in range(R.MOE_STAGES):
            stage_ms[s, i] = R.event_elapsed_ms(evs[s][i], evs[s][i + 1])
    for row in evs:
        for e in row:
            R.event_destroy(e)
    log(f"[bench] {cfg.name}: timed {args.steps} steps in {wall * 1e3:.2f} ms "
        f"({wall_events * 1e3:.2f} ms with stage events)")
    # routing of the given logits, read back before any extra run reuses the buffers
    off = bufs.expert_off.cpu().numpy()
    srt = bufs.sorted_ids.cpu().numpy()
    TK = T * cfg.k
    counts = np.array([int(np.sum(srt[off[e]:off[e + 1]] < TK)) for e in range(cfg.E)])

    # Timed region 3: the same layer on a contiguous layout of the same weights
    # (pages consecutive and in order), for the cost of paging.
    cont = None
    if "contiguous" in extras:
        from paged_moe_expert_amd.layouts import contiguous_page_table
        cpt = torch.from_numpy(contiguous_page_table(cfg)).to(dev)
        cpool = torch.empty(cfg.E * 3 * cfg.P * cfg.page_bytes, dtype=torch.uint8, device=dev)
        wdev = torch.from_numpy(wb.view(idt)).to(dev)
        R.experts_store(cpool, cpt, wdev, cfg.page_bytes)
        del wdev
        ybuf = bufs.y.clone()
        R.fused_moe_paged(x, lgd, cpool, cpt, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs)
        torch.cuda.synchronize()
        same = bool(torch.equal(ybuf.view(torch.uint8), bufs.y.view(torch.uint8)))

        def cstep():
            R.fused_moe_paged(x, lgd, cpool, cpt, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs)
        for _ in range(args.warmup):
            cstep()
        cont_ms = timed(cstep)[0] * 1e3 / args.steps
        del cpool
        cont = {"ms_per_step": round(cont_ms, 4), "bitwise_equal_output": same}

    # Timed region 4: the same layer computing its router logits x . w_gate^T
    # in the gating stage (w_gate [E, H] instead of given logits).
    router = None
    if "router" in extras:
        wg = torch.from_numpy(gen.gate_weight_bits(cfg).view(idt)).to(dev).view(tdt)

        def rstep(events=None):
            R.fused_moe_paged(x, None, pool, ptd, cfg.page_bytes, cfg.k, cfg.I, bufs=bufs, w_gate=wg,
                              stage_events=events)
        for _ in range(args.warmup):
            rstep()
        r_secs, _ = timed(rstep)
        rev = [R.event_create() for _ in range(R.MOE_STAGES + 1)]
        gate_ms = []
        for _ in range(5):
            rstep(rev)
            torch.cuda.synchronize()
            gate_ms.append(R.event_elapsed_ms(rev[0], rev[1]))
        for e_ in rev:
            R.event_destroy(e_)
        router = {"ms_per_step": round(r_secs * 1e3 / args.steps, 4),
                  "gating_with_router_us_median": round(float(np.median(gate_ms)) * 1e3, 2),
                  "router_gflop": round(2.0 * T * cfg.E * cfg.H / 1e9, 4)}

    # Timed region 5: dual-buffer expert upload (host -> fresh expert pages on a
    # copy stream), alone and overlapped with the layer on the compute stream.
    upload = None
    if "upload" in extras and args.upload_experts:
        upload = expert_upload_bench(args, cfg, wb, idt, dev, step, R, torch, np)

    # Timed region 6: the layer captured in a HIP graph, replayed.
    graph = None
    if "graph" in extras and args.flush_mib == 0:
        graph = graph_bench(args, cfg, x, lgd, pool, ptd, bufs, R, torch)

    # Timed region 7: the foil -- gather the touched experts, then the layer.
    foil = None
    if "foil" in extras:
        foil = copy_foil_bench(args, cfg, x, lgd, pool, ptd, pt, bufs, dev, R, torch, np)

    # Timed region 8: paged decode attention over the same pool's KV view.
    attn = None
    if "attention" in extras and args.attn_requests and cfg.dtype == "bf16" \
            and any(v.name == "kv" for v in cfg.views) and any(name == "kv" for name, _ in lay.live):
        attn = attention_bench(args, cfg, lay, pool, dev, R, torch, np)

    # ---- algorithmic work of this input (routing read back after the timed passes)
    touched = int(np.sum(counts > 0))
    es = cfg.es
    HI = cfg.H * cfg.I
    w_bytes = touched * 3 * HI * es
    io_bytes = T * cfg.H * es * 2 + T * cfg.E * 4
    flops = 6.0 * HI * TK
    up_bytes = touched * 2 * HI * es + T * cfg.H * es + TK * cfg.I * es
    up_flops = 4.0 * HI * TK
    dn_bytes = touched * HI * es + TK * cfg.I * es + TK * cfg.H * es
    dn_flops = 2.0 * HI * TK

    ms_step = wall * 1e3 / args.steps
    if step_ms is not None:
        per_step, step_src = np.array(step_ms), "event pair around each cache-cold step"
    else:
        per_step = stage_ms.sum(axis=1)
        step_src = "sum of the stage-event intervals of each step (event records included)"
    med = np.median(stage_ms, axis=0)
    mean = stage_ms.mean(axis=0)
    decode_like = (w_bytes + io_bytes) / HBM_PEAK_GBS > flops / (BF16_PEAK_TFLOPS * 1e3)
    kind_up, kind_dn = KIND_OF_BLOCK_M.get(bufs.block_m, ("tiled", "tiled"))

    def kernel_roof(name, ms, nbytes, nflops, traffic):
        if decode_like:
            a = nbytes / (ms * 1e-3) / 1e9
            return {"bound": "hbm", "kernel": name, "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(ms * 1e3, 2)}
        a = nflops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": name, "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": nflops, "algorithmic_bytes_per_launch": nbytes,
                "avg_launch_us": round(ms * 1e3, 2)}

    roof = kernel_roof("gemm_up", float(mean[3]), up_bytes, up_flops,
                       traffic_from_profiles(cfg.name, "gemm_up", kind_up))
    roof_dn = kernel_roof("gemm_down", float(mean[4]), dn_bytes, dn_flops,
                          traffic_from_profiles(cfg.name, "gemm_down", kind_dn))
    layer_roof_us = max(flops / (BF16_PEAK_TFLOPS * 1e12), (w_bytes + io_bytes) / (HBM_PEAK_GBS * 1e9)) * 1e6
    out = {
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": cfg.name, "T": T, "E": cfg.E, "k": cfg.k, "H": cfg.H, "I": cfg.I,
                   "page_bytes": cfg.page_bytes, "pages_per_projection": cfg.P, "pool_bytes": cfg.pool_bytes,
                   "experts_touched": touched, "block_m": bufs.block_m,
                   "routed_rows_max_min": [int(counts.max()), int(counts.min())],
                   "cache_flush_mib": args.flush_mib},
        "layer": {"tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
                  "mfma_frac": round(flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "hbm_gbs": round((w_bytes + io_bytes) / (ms_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round((w_bytes + io_bytes) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "algorithmic_bytes": w_bytes + io_bytes, "algorithmic_flops": flops,
                  "bound": "hbm" if decode_like else "mfma",
                  "roofline_us": round(layer_roof_us, 2),
                  "roofline_frac": round(layer_roof_us / (ms_step * 1e3), 4)},
        "stages_us_median": {n: round(float(v) * 1e3, 2) for n, v in zip(STAGES, med)},
        "stages_us_mean": {n: round(float(v) * 1e3, 2) for n, v in zip(STAGES, mean)},
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "step_ms_source": step_src,
        "ms_per_step_with_stage_events": round(wall_events * 1e3 / args.steps, 4),
        "roofline": roof,
        "roofline_gemm_down": roof_dn,
    }
    if cont is not None:
        cont["paged_over_contiguous_minus_1"] = round(ms_step / cont["ms_per_step"] - 1.0, 4)
        out["contiguous"] = cont
    if router is not None:
        router["added_ms_vs_given_logits"] = round(router["ms_per_step"] - ms_step, 4)
        out["with_router"] = router
    if upload is not None:
        out["expert_upload"] = upload
    if "adjuster" in extras and any(v.name == "kv" and v.parent == "expert" for v in cfg.views):
        gbs = upload["upload_gbs_alone"] if upload is not None else None
        out["adjuster"] = adjuster_bench(cfg, R, np, gen, gbs)
    if attn is not None:
        out["attention"] = attn
    if graph is not None:
        graph["over_eager"] = round(graph["ms_per_step"] / ms_step, 4)
        out["graph_replay"] = graph
    if foil is not None:
        foil["foil_over_paged"] = round(foil["ms_per_step_gather_then_layer"] / ms_step, 3)
        out["copy_foil"] = foil
    if "cpu" in extras:
        log(f"[bench] {cfg.name}: timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(cfg.with_T(T), L["xb"], L["lg"], wb, min(args.cpu_tokens, T))
    del L, pool, bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


EXTRAS_ALL = ("contiguous", "router", "upload", "graph", "foil", "attention", "adjuster")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, help="headline configuration (default: the 8192-token "
                                                           "fragmented prefill)")
    ap.add_argument("--nested", default="2,3",
                    help="other configurations measured in the same run, nested in the line ('none' or '' = none)")
    ap.add_argument("--tokens", type=int, default=0, help="override T of the headline (decode sweep)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--upload-experts", type=int, default=8,
                    help="experts uploaded host -> fresh pages for the expert-upload measurement (0 = skip)")
    ap.add_argument("--no-adjuster", action="store_true",
                    help="skip the host-side adjuster policy measurement")
    ap.add_argument("--attn-requests", type=int, default=256,
                    help="decode-attention requests taken from the layout's KV view (0: skip)")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the layer")
    ap.add_argument("--no-foil", action="store_true",
                    help="skip the gather-then-contiguous foil (the copy the paged kernel avoids)")
    ap.add_argument("--no-router", action="store_true",
                    help="skip the run that computes the router projection in the gating stage")
    ap.add_argument("--no-contiguous", action="store_true",
                    help="skip the comparison run on a contiguous layout of the same weights")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured streaming-read ceiling")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="before every timed step, read this many MiB of scratch (evicts the "
                         "Infinity Cache with clean lines); steps are then timed by an event pair each")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the paged fused-MoE layer runs on a single "
              "MI355X here and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_inputs import CONFIGS, gen
    from paged_moe_expert_amd import rimuru as R

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    skip = {"contiguous": args.no_contiguous, "router": args.no_router, "graph": args.no_graph,
            "foil": args.no_foil, "adjuster": args.no_adjuster, "upload": args.upload_experts == 0,
            "attention": args.attn_requests == 0}
    extras = {e for e in EXTRAS_ALL if not skip.get(e, False)}

    cfg = CONFIGS[args.config]
    T = args.tokens or cfg.T
    head = measure(args, cfg, T, extras | ({"cpu"} if not args.no_cpu else set()), dev, R, torch, np, gen)

    nested = {}
    for tok in filter(None, (t.strip().strip("'\"") for t in args.nested.split(","))):
        if tok == "none":
            continue
        cid = int(tok)
        if cid == args.config:
            continue
        c2 = CONFIGS[cid]
        # the decode layer carries the serving-side measurements (upload,
        # adjuster, attention, graph); the prefill layers the paging ones
        sub = {"contiguous", "router", "foil"} & extras
        if c2.T * c2.k <= 24 * c2.E:
            sub = set(extras)
        nested[c2.name] = measure(args, c2, c2.T, sub, dev, R, torch, np, gen)

    # the measured streaming-read ceiling
    ceiling = None if args.no_ceiling else read_ceiling(args, dev, R, torch)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")

    out = {
        "metric": "paged fused-MoE tokens/s + TFLOP/s (or HBM GB/s) as % of MI355X roofline",
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": head.pop("config"),
        "roofline": head.pop("roofline"),
    }
    cpu = head.pop("cpu_baseline", None)
    out.update(head)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if ceiling is not None:
        out["measured_read_ceiling"] = {"gbs": round(ceiling, 1),
                                        "method": "rimuru_stream_read over a 4 GiB buffer",
                                        "frac_of_peak": round(ceiling / HBM_PEAK_GBS, 4)}
    if nested:
        out["other_workloads"] = nested
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
