"""ctypes declarations of librimuru.so (argument marshalling only).

The library is built in-tree by ``python -m paged_moe_expert_amd.build``.
Loading fails loudly when it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# RIMURU_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("RIMURU_LIB") or os.path.join(HERE, "librimuru.so")

OK, EINVAL, ENOMEM, ERANGE, EDTYPE, EHIP, EBUSY = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
VIEW_EXPERT, VIEW_KV, VIEW_SSM, VIEW_CONV = 0, 1, 2, 3
MOE_STAGES = 6
NOALLOC_SCRATCH_BYTES = 64 << 20     # RIMURU_NOALLOC_SCRATCH_BYTES
STATUS_NAMES = {OK: "OK", EINVAL: "EINVAL", ENOMEM: "ENOMEM", ERANGE: "ERANGE",
                EDTYPE: "EDTYPE", EHIP: "EHIP", EBUSY: "EBUSY"}
NO_BUDGET = (1 << 64) - 1


class RimuruError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PoolStats(C.Structure):
    _fields_ = [("huge_pages", C.c_uint64), ("huge_free", C.c_uint64),
                ("bytes_per_kind", C.c_uint64 * 4), ("bytes_free", C.c_uint64),
                ("waste_bytes", C.c_uint64), ("split_parents", C.c_uint64)]


class AdjusterParams(C.Structure):
    _fields_ = [("E", C.c_int32), ("P", C.c_int32), ("min_resident", C.c_int32),
                ("headroom_blocks", C.c_int32), ("return_blocks", C.c_int32), ("shift", C.c_int32),
                ("max_prefetch", C.c_int32)]


class AttnArgs(C.Structure):
    _fields_ = [("B", C.c_int32), ("n_q", C.c_int32), ("n_kv", C.c_int32), ("head_dim", C.c_int32),
                ("max_blocks", C.c_int32), ("scale", C.c_float), ("q", C.c_void_p), ("pool_base", C.c_void_p),
                ("block_table", C.c_void_p), ("context_lens", C.c_void_p), ("out", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_uint64)]


class MoeArgs(C.Structure):
    _fields_ = [("T", C.c_int32), ("E", C.c_int32), ("k", C.c_int32), ("H", C.c_int32),
                ("I", C.c_int32), ("P", C.c_int32), ("dtype", C.c_int32),
                ("renormalize", C.c_int32),
                ("x", C.c_void_p), ("logits", C.c_void_p), ("pool_base", C.c_void_p),
                ("pt", C.c_void_p), ("page_bytes", C.c_uint64), ("y", C.c_void_p),
                ("topk_ids", C.c_void_p), ("topk_w", C.c_void_p), ("sorted_ids", C.c_void_p),
                ("expert_off", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_uint64), ("stage_events", C.c_void_p),
                ("n_stage_events", C.c_int32)]


_PROTOS = {
    "rimuru_last_error": (C.c_char_p, []),
    "rimuru_abi_version": (C.c_int32, []),
    "rimuru_pool_create": (C.c_int32, [C.c_uint64, C.c_uint64, C.POINTER(C.c_void_p)]),
    "rimuru_pool_destroy": (C.c_int32, [C.c_void_p]),
    "rimuru_view_map": (C.c_int32, [C.c_void_p, C.c_int32, C.c_uint64, C.c_void_p,
                                    C.POINTER(C.c_void_p)]),
    "rimuru_view_alloc": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_uint64, C.c_void_p]),
    "rimuru_view_free": (C.c_int32, [C.c_void_p, C.c_uint64]),
    "rimuru_view_pages": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_uint64,
                                      C.POINTER(C.c_uint64)]),
    "rimuru_view_set_budget": (C.c_int32, [C.c_void_p, C.c_uint64]),
    "rimuru_pool_transfer": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_uint64]),
    "rimuru_view_usage": (C.c_int32, [C.c_void_p, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
    "rimuru_view_info": (C.c_int32, [C.c_void_p, C.POINTER(C.c_void_p), C.POINTER(C.c_int32),
                                     C.POINTER(C.c_uint64)]),
    "rimuru_pool_stats": (C.c_int32, [C.c_void_p, C.POINTER(PoolStats)]),
    "rimuru_adjuster_create": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(AdjusterParams),
                                           C.POINTER(C.c_void_p)]),
    "rimuru_adjuster_destroy": (C.c_int32, [C.c_void_p]),
    "rimuru_adjuster_step": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.POINTER(C.c_int32), C.c_void_p, C.POINTER(C.c_int32),
                                         C.POINTER(C.c_int64)]),
    "rimuru_adjuster_upload_done": (C.c_int32, [C.c_void_p, C.c_int32]),
    "rimuru_adjuster_state": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "rimuru_pool_check": (C.c_int32, [C.c_void_p]),
    "rimuru_moe_sizes": (C.c_int32, [C.c_int32] * 7 + [C.POINTER(C.c_uint64), C.POINTER(C.c_uint64),
                                                      C.POINTER(C.c_int32)]),
    "rimuru_fused_moe_paged": (C.c_int32, [C.POINTER(MoeArgs), C.c_void_p]),
    "rimuru_fused_moe_paged_router": (C.c_int32, [C.POINTER(MoeArgs), C.c_void_p, C.c_void_p, C.c_void_p]),
    "rimuru_fused_moe_paged_noalloc": (C.c_int32, [C.POINTER(MoeArgs), C.c_void_p]),
    "rimuru_pt_check": (C.c_int32, [C.c_void_p, C.c_int32, C.c_int32, C.c_uint64, C.c_uint64]),
    "rimuru_experts_store": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_int32, C.c_int32,
                                         C.c_uint64, C.c_void_p, C.c_uint64, C.c_void_p]),
    "rimuru_expert_upload": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_int32, C.c_uint64,
                                         C.c_void_p, C.c_uint64, C.c_void_p]),
    "rimuru_attn_sizes": (C.c_int32, [C.c_int32] * 5 + [C.POINTER(C.c_uint64), C.POINTER(C.c_int32),
                                                        C.POINTER(C.c_uint64)]),
    "rimuru_paged_decode_attention": (C.c_int32, [C.POINTER(AttnArgs), C.c_void_p]),
    "rimuru_block_table_check": (C.c_int32, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_uint64,
                                             C.c_uint64]),
    "rimuru_event_create": (C.c_int32, [C.POINTER(C.c_void_p)]),
    "rimuru_event_destroy": (C.c_int32, [C.c_void_p]),
    "rimuru_event_record": (C.c_int32, [C.c_void_p, C.c_void_p]),
    "rimuru_event_elapsed_ms": (C.c_int32, [C.c_void_p, C.c_void_p, C.POINTER(C.c_float)]),
    "rimuru_stream_read": (C.c_int32, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m paged_moe_expert_amd.build` (no fallback exists)")
        try:  # share torch's HIP runtime when torch is around (same SONAME)
            import torch  # noqa: F401
        except ImportError:
            pass
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != OK:
        msg = lib().rimuru_last_error().decode(errors="replace")
        raise RimuruError(status, where, msg)
