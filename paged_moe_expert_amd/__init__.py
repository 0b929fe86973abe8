"""Page-table-aware fused MoE for MI355X (gfx950).

The layer and the page allocator live in librimuru.so (C ABI in
include/rimuru.h); ``paged_moe_expert_amd.rimuru`` binds it one function per
entry point, and ``paged_moe_expert_amd.layouts`` produces seeded page
layouts through the library's allocator.
"""
from . import rimuru  # noqa: F401
from ._lib import RimuruError  # noqa: F401
