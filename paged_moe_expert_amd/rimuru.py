"""Python binding of librimuru.so, one function per C entry point (the C
name without its ``rimuru_`` prefix). Arguments are marshalled and statuses
turned into RimuruError; all work happens in the library. Device buffers are
torch tensors, streams are torch streams.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from ._lib import (BF16, F32, MOE_STAGES, NO_BUDGET, NOALLOC_SCRATCH_BYTES, EBUSY, EINVAL, ENOMEM, ERANGE,  # noqa: F401
                   AdjusterParams,
                   AttnArgs, MoeArgs, OK, PoolStats, RimuruError, check, lib)


# ----------------------------------------------------------------- pool and views

class Pool:
    """Host state of one shared page pool (owns its views)."""

    def __init__(self, handle: int, pool_bytes: int, huge_bytes: int):
        self.handle = handle
        self.pool_bytes = pool_bytes
        self.huge_bytes = huge_bytes
        self.views = []

    def __del__(self):
        if getattr(self, "handle", None):
            lib().rimuru_pool_destroy(self.handle)
            self.handle = None


class View:
    def __init__(self, pool: Pool, handle: int, kind: int, page_bytes: int):
        self.pool = pool              # keeps the pool (which owns the view) alive
        self.handle = handle
        self.kind = kind
        self.page_bytes = page_bytes


def pool_create(pool_bytes: int, huge_page_bytes: int) -> Pool:
    h = C.c_void_p()
    check(lib().rimuru_pool_create(pool_bytes, huge_page_bytes, C.byref(h)), "pool_create")
    return Pool(h.value, pool_bytes, huge_page_bytes)


def view_map(pool: Pool, kind: int, page_bytes: int, parent: View | None = None) -> View:
    h = C.c_void_p()
    check(lib().rimuru_view_map(pool.handle, kind, page_bytes,
                                parent.handle if parent is not None else None, C.byref(h)),
          "view_map")
    v = View(pool, h.value, kind, page_bytes)
    pool.views.append(v)
    return v


def view_alloc_status(v: View, owner: int, n_pages: int):
    """(status, offsets) without raising: ENOMEM is an ordinary outcome."""
    out = np.zeros(max(n_pages, 1), dtype=np.int64)
    st = lib().rimuru_view_alloc(v.handle, owner, n_pages, out.ctypes.data)
    return st, (out[:n_pages] if st == OK else out[:0])


def view_alloc(v: View, owner: int, n_pages: int) -> np.ndarray:
    st, offs = view_alloc_status(v, owner, n_pages)
    check(st, "view_alloc")
    return offs


def view_free_status(v: View, owner: int) -> int:
    return lib().rimuru_view_free(v.handle, owner)


def view_free(v: View, owner: int) -> None:
    check(view_free_status(v, owner), "view_free")


def view_pages(v: View, owner: int) -> np.ndarray:
    n = C.c_uint64()
    lib().rimuru_view_pages(v.handle, owner, None, 0, C.byref(n))   # count only
    out = np.zeros(max(n.value, 1), dtype=np.int64)
    check(lib().rimuru_view_pages(v.handle, owner, out.ctypes.data, n.value, C.byref(n)), "view_pages")
    return out[:n.value]


def view_set_budget(v: View, nbytes: int | None) -> int:
    return lib().rimuru_view_set_budget(v.handle, NO_BUDGET if nbytes is None else nbytes)


def pool_transfer(pool: Pool, src: View, dst: View, nbytes: int) -> int:
    return lib().rimuru_pool_transfer(pool.handle, src.handle, dst.handle, nbytes)


def view_usage(v: View):
    used, budget = C.c_uint64(), C.c_uint64()
    check(lib().rimuru_view_usage(v.handle, C.byref(used), C.byref(budget)), "view_usage")
    return used.value, (None if budget.value == NO_BUDGET else budget.value)


def view_info(v: View):
    """(kind, page_bytes) as the library records them."""
    kind, page = C.c_int32(), C.c_uint64()
    check(lib().rimuru_view_info(v.handle, None, C.byref(kind), C.byref(page)), "view_info")
    return kind.value, page.value


def pool_stats(pool: Pool) -> dict:
    s = PoolStats()
    check(lib().rimuru_pool_stats(pool.handle, C.byref(s)), "pool_stats")
    return {"huge_pages": s.huge_pages, "huge_free": s.huge_free,
            "bytes_per_kind": list(s.bytes_per_kind), "bytes_free": s.bytes_free,
            "waste_bytes": s.waste_bytes, "split_parents": s.split_parents}


def pool_check(pool: Pool) -> None:
    check(lib().rimuru_pool_check(pool.handle), "pool_check")


def pt_check(pt: np.ndarray, page_bytes: int, pool_bytes: int) -> None:
    pt = np.ascontiguousarray(pt, dtype=np.int32)
    E, three, P = pt.shape
    check(lib().rimuru_pt_check(pt.ctypes.data, E, P, page_bytes, pool_bytes), "pt_check")


# ----------------------------------------------------------------- adjuster policy

class Adjuster:
    """Host state of the workload-aware adjuster (keeps its pool alive)."""

    def __init__(self, handle: int, pool: Pool, E: int):
        self.handle = handle
        self.pool = pool
        self.E = E

    def __del__(self):
        if getattr(self, "handle", None):
            lib().rimuru_adjuster_destroy(self.handle)
            self.handle = None


def adjuster_create(pool: Pool, expert_view: View, kv_view: View, E: int, P: int, min_resident: int = 0,
                    headroom_blocks: int = 0, return_blocks: int = 0, shift: int = 3,
                    max_prefetch: int = 1) -> Adjuster:
    prm = AdjusterParams(E, P, min_resident, headroom_blocks, return_blocks, shift, max_prefetch)
    h = C.c_void_p()
    check(lib().rimuru_adjuster_create(pool.handle, expert_view.handle, kv_view.handle, C.byref(prm),
                                       C.byref(h)), "adjuster_create")
    return Adjuster(h.value, pool, E)


def adjuster_step_status(adj: Adjuster, demand_blocks: int, routed, needed):
    """(status, evicted, loaded, kv_moved) without raising: ENOMEM reports
    what the step did before it ran out of room."""
    routed = np.ascontiguousarray(routed, dtype=np.int32)
    needed = np.ascontiguousarray(needed, dtype=np.uint8)
    if routed.shape != (adj.E,) or needed.shape != (adj.E,):
        raise ValueError("routed and needed must have E entries")
    ev = np.zeros(adj.E, dtype=np.int32)
    ld = np.zeros(adj.E, dtype=np.int32)
    ne, nl, moved = C.c_int32(), C.c_int32(), C.c_int64()
    st = lib().rimuru_adjuster_step(adj.handle, demand_blocks, routed.ctypes.data, needed.ctypes.data,
                                    ev.ctypes.data, C.byref(ne), ld.ctypes.data, C.byref(nl),
                                    C.byref(moved))
    return st, ev[:ne.value].tolist(), ld[:nl.value].tolist(), moved.value


def adjuster_step(adj: Adjuster, demand_blocks: int, routed, needed):
    """{"evicted", "loaded", "kv_moved"} of one policy step."""
    st, ev, ld, moved = adjuster_step_status(adj, demand_blocks, routed, needed)
    check(st, "adjuster_step")
    return {"evicted": ev, "loaded": ld, "kv_moved": moved}


def adjuster_upload_done(adj: Adjuster, e: int) -> None:
    check(lib().rimuru_adjuster_upload_done(adj.handle, e), "adjuster_upload_done")


def adjuster_state(adj: Adjuster):
    """(resident bool [E], in_flight bool [E], score uint64 [E])."""
    r = np.zeros(adj.E, dtype=np.uint8)
    f = np.zeros(adj.E, dtype=np.uint8)
    s = np.zeros(adj.E, dtype=np.uint64)
    check(lib().rimuru_adjuster_state(adj.handle, r.ctypes.data, f.ctypes.data, s.ctypes.data),
          "adjuster_state")
    return r.astype(bool), f.astype(bool), s


# ----------------------------------------------------------------- fused MoE

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise RimuruError(-4, "fused_moe_paged", f"unsupported dtype {t.dtype}")


def moe_sizes(T: int, E: int, k: int, H: int, I: int, P: int, dtype: int):
    """(sorted_len, workspace_bytes, block_m)."""
    sl, ws, bm = C.c_uint64(), C.c_uint64(), C.c_int32()
    check(lib().rimuru_moe_sizes(T, E, k, H, I, P, dtype, C.byref(sl), C.byref(ws), C.byref(bm)),
          "moe_sizes")
    return sl.value, ws.value, bm.value


class MoeBuffers:
    """Outputs and workspace for one shape; reuse them across calls.
    workspace=False leaves the workspace out (the no-allocation entry point
    brings its own)."""

    def __init__(self, T, E, k, H, I, P, dtype, device="cuda", workspace=True):
        import torch
        tdt = torch.bfloat16 if dtype == BF16 else torch.float32
        sl, ws, bm = moe_sizes(T, E, k, H, I, P, dtype)
        self.shape = (T, E, k, H, I, P, dtype)
        self.block_m = bm
        self.y = torch.empty((T, H), dtype=tdt, device=device)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.sorted_ids = torch.empty(max(sl, 1), dtype=torch.int32, device=device)
        self.expert_off = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.workspace_bytes = ws
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device) if workspace else None


def fused_moe_paged(x, logits, pool, pt, page_bytes: int, k: int, I: int,
                    bufs: MoeBuffers | None = None, stream=None, stage_events=None,
                    w_gate=None, logits_out=None) -> MoeBuffers:
    """Enqueue the fused MoE layer on the current (or given) torch stream.

    x [T, H] bf16/fp32, logits [T, E] fp32, pool uint8 device tensor,
    pt int32 [E, 3, P] device tensor, I the intermediate size. Returns the
    buffers holding y, topk_ids, topk_w, sorted_ids and expert_off. Does not
    synchronise.

    With w_gate [E, H] (x's dtype) the router projection runs inside the
    gating stage (rimuru_fused_moe_paged_router): logits is then not read and
    may be None; logits_out [T, E] fp32, if given, receives the logits.
    """
    import torch
    T, H = x.shape
    E = w_gate.shape[0] if w_gate is not None else logits.shape[1]
    P = pt.shape[2]
    dt = _dtype_code(x)
    if bufs is None:
        bufs = MoeBuffers(T, E, k, H, I, P, dt, device=x.device)
    a = MoeArgs()
    a.T, a.E, a.k, a.H, a.I, a.P, a.dtype, a.renormalize = T, E, k, H, I, P, dt, 1
    a.x, a.pool_base, a.pt = x.data_ptr(), pool.data_ptr(), pt.data_ptr()
    a.logits = logits.data_ptr() if logits is not None else None
    a.page_bytes = page_bytes
    a.y, a.topk_ids, a.topk_w = bufs.y.data_ptr(), bufs.topk_ids.data_ptr(), bufs.topk_w.data_ptr()
    a.sorted_ids, a.expert_off = bufs.sorted_ids.data_ptr(), bufs.expert_off.data_ptr()
    if bufs.workspace is None:
        raise ValueError("fused_moe_paged: these buffers have no workspace (made for fused_moe_paged_noalloc)")
    a.workspace, a.workspace_bytes = bufs.workspace.data_ptr(), bufs.workspace.numel()
    ev_arr = None
    if stage_events is not None:
        ev_arr = (C.c_void_p * len(stage_events))(*stage_events)
        a.stage_events = C.cast(ev_arr, C.c_void_p)
        a.n_stage_events = len(stage_events)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    if w_gate is None:
        check(lib().rimuru_fused_moe_paged(C.byref(a), s.cuda_stream), "fused_moe_paged")
    else:
        if w_gate.dtype != x.dtype or tuple(w_gate.shape) != (E, H) or not w_gate.is_contiguous():
            raise ValueError("fused_moe_paged: w_gate must be a contiguous [E, H] tensor of x's dtype")
        out = logits_out.data_ptr() if logits_out is not None else None
        check(lib().rimuru_fused_moe_paged_router(C.byref(a), w_gate.data_ptr(), out, s.cuda_stream),
              "fused_moe_paged_router")
    return bufs


def fused_moe_paged_noalloc(x, logits, pool, pt, page_bytes: int, k: int, I: int,
                            bufs: MoeBuffers | None = None, stream=None) -> MoeBuffers:
    """rimuru_fused_moe_paged_noalloc: the layer with the library's fixed
    device scratch as its workspace (no workspace argument). bufs holds the
    outputs only (MoeBuffers(..., workspace=False))."""
    import torch
    T, H = x.shape
    E = logits.shape[1]
    P = pt.shape[2]
    dt = _dtype_code(x)
    if bufs is None:
        bufs = MoeBuffers(T, E, k, H, I, P, dt, device=x.device, workspace=False)
    a = MoeArgs()
    a.T, a.E, a.k, a.H, a.I, a.P, a.dtype, a.renormalize = T, E, k, H, I, P, dt, 1
    a.x, a.logits, a.pool_base, a.pt = x.data_ptr(), logits.data_ptr(), pool.data_ptr(), pt.data_ptr()
    a.page_bytes = page_bytes
    a.y, a.topk_ids, a.topk_w = bufs.y.data_ptr(), bufs.topk_ids.data_ptr(), bufs.topk_w.data_ptr()
    a.sorted_ids, a.expert_off = bufs.sorted_ids.data_ptr(), bufs.expert_off.data_ptr()
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    check(lib().rimuru_fused_moe_paged_noalloc(C.byref(a), s.cuda_stream), "fused_moe_paged_noalloc")
    return bufs


def fused_moe_paged_raw(args: MoeArgs, stream_handle: int) -> int:
    """Direct entry for callers that fill MoeArgs themselves; returns the status."""
    return lib().rimuru_fused_moe_paged(C.byref(args), stream_handle)


def experts_store(pool, pt, weights, page_bytes: int, stream=None) -> None:
    """Copy contiguous projections weights [E, 3, proj_bytes] (device, uint8 view
    or any dtype) into the pool pages pt names. A host copy of pt is checked
    against the pool first (rimuru_pt_check: ERANGE for a page outside it)."""
    import torch
    E, three, P = pt.shape
    proj_bytes = weights[0, 0].numel() * weights.element_size()
    pool_bytes = pool.numel() * pool.element_size()
    pt_check(pt.cpu().numpy(), page_bytes, pool_bytes)
    s = stream if stream is not None else torch.cuda.current_stream(pool.device)
    check(lib().rimuru_experts_store(pool.data_ptr(), pool_bytes, pt.data_ptr(), E, P, page_bytes,
                                     weights.data_ptr(), proj_bytes, s.cuda_stream), "experts_store")


def expert_upload_raw(pool_ptr: int, pool_bytes: int, pt_rows, page_bytes: int, host_ptr: int,
                      proj_bytes: int, stream_handle: int) -> int:
    """Status of rimuru_expert_upload for raw pointers (validation tests)."""
    rows = np.ascontiguousarray(pt_rows, dtype=np.int32)
    return lib().rimuru_expert_upload(pool_ptr, pool_bytes, rows.ctypes.data_as(C.c_void_p), rows.shape[-1],
                                      page_bytes, host_ptr, proj_bytes, stream_handle)


def expert_upload(pool, pt_rows, page_bytes: int, host, stream=None) -> None:
    """Copy one expert's projections host [3, proj_bytes] (pinned CPU tensor)
    into the pool pages pt_rows [3, P] (host int32) names, asynchronously on
    stream (default: the current stream)."""
    import torch
    if host.device.type != "cpu" or not host.is_pinned():
        raise ValueError("expert_upload: host weights must be a pinned CPU tensor")
    if not host.is_contiguous():
        raise ValueError("expert_upload: host weights must be contiguous")
    proj_bytes = host[0].numel() * host.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(pool.device)
    check(expert_upload_raw(pool.data_ptr(), pool.numel() * pool.element_size(), pt_rows, page_bytes,
                            host.data_ptr(), proj_bytes, s.cuda_stream), "expert_upload")


# ----------------------------------------------------------------- paged decode attention

def attn_sizes(B: int, n_q: int, n_kv: int, head_dim: int, max_blocks: int):
    """(workspace_bytes, n_split, block_bytes)."""
    ws, ns, bb = C.c_uint64(), C.c_int32(), C.c_uint64()
    check(lib().rimuru_attn_sizes(B, n_q, n_kv, head_dim, max_blocks, C.byref(ws), C.byref(ns), C.byref(bb)),
          "attn_sizes")
    return ws.value, ns.value, bb.value


def block_table_check(block_table, context_lens, block_bytes: int, pool_bytes: int) -> None:
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    check(lib().rimuru_block_table_check(bt.ctypes.data, bt.shape[0], bt.shape[1], lens.ctypes.data,
                                         block_bytes, pool_bytes), "block_table_check")


def paged_decode_attention(q, pool, block_table, context_lens, n_kv: int, scale: float, out=None,
                           workspace=None, stream=None):
    """q bf16 [B, n_q, head_dim]; pool uint8 device tensor; block_table int32
    [B, max_blocks] and context_lens int32 [B] on the device. Returns out
    (bf16 [B, n_q, head_dim]); enqueued on stream (default: current)."""
    import torch
    B, n_q, D = q.shape
    max_blocks = block_table.shape[1]
    ws, _, _ = attn_sizes(B, n_q, n_kv, D, max_blocks)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise RimuruError(-4, "paged_decode_attention", "q and out must be bf16")
    for t in (q, block_table, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("paged_decode_attention: tensors must be contiguous")
    a = AttnArgs(B, n_q, n_kv, D, max_blocks, scale, q.data_ptr(), pool.data_ptr(), block_table.data_ptr(),
                 context_lens.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel())
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    check(lib().rimuru_paged_decode_attention(C.byref(a), s.cuda_stream), "paged_decode_attention")
    return out


# ----------------------------------------------------------------- timing helpers

def event_create() -> int:
    h = C.c_void_p()
    check(lib().rimuru_event_create(C.byref(h)), "event_create")
    return h.value


def event_destroy(ev: int) -> None:
    check(lib().rimuru_event_destroy(ev), "event_destroy")


def stream_read(buf, sink, stream=None) -> None:
    """Enqueue one plain streaming read of the device tensor buf (calibration);
    sink is a device int32/uint32 tensor of at least one element."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(buf.device)
    check(lib().rimuru_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                   s.cuda_stream), "stream_read")


def event_record(ev: int, stream=None) -> None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    check(lib().rimuru_event_record(ev, s.cuda_stream), "event_record")


def event_elapsed_ms(a: int, b: int) -> float:
    ms = C.c_float()
    check(lib().rimuru_event_elapsed_ms(a, b, C.byref(ms)), "event_elapsed_ms")
    return ms.value
