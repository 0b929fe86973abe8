"""The C-ABI library loads, exports every entry point include/rimuru.h declares,
and validates arguments on the host (no GPU needed for any of these)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from paged_moe_expert_amd import _lib
from paged_moe_expert_amd import rimuru as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rimuru.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rimuru_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 20
    L = _lib.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # and the binding declares a prototype for each
    assert set(names) <= set(_lib._PROTOS), set(names) - set(_lib._PROTOS)


def test_abi_version_and_error_text():
    L = _lib.lib()
    assert L.rimuru_abi_version() == 1
    assert L.rimuru_pool_create(100, 0, C.byref(C.c_void_p())) == _lib.EINVAL
    assert b"huge page" in L.rimuru_last_error()


def test_moe_sizes_and_plans():
    sl, ws, bm = R.moe_sizes(64, 128, 8, 2048, 768, 1, R.BF16)
    assert bm == 16 and sl % bm == 0 and sl >= 64 * 8
    # tiles bound: floor(T*k/bm) + min(E, T*k)
    assert sl == (512 // 16 + 128) * 16
    # the workspace never scales with expert weight bytes: only with tokens
    assert ws < 16 * 2 ** 20
    sl4, ws4, bm4 = R.moe_sizes(8192, 128, 8, 2048, 768, 48, R.BF16)
    assert bm4 == 128
    _, _, bm3 = R.moe_sizes(2048, 256, 8, 2048, 512, 1, R.BF16)
    assert bm3 == 64
    sl1, _, bm1 = R.moe_sizes(1, 128, 8, 2048, 768, 1, R.BF16)
    assert bm1 == 16 and sl1 == 8 * 16
    # too many pages per projection for the streaming plan: the tiled plan takes it
    _, _, bmp = R.moe_sizes(64, 128, 8, 2048, 768, 3000, R.BF16)
    assert bmp == 64
    # streaming tile height by routed rows per expert (T*k/E): 16 up to 8,
    # 32 (bf16) above, up to 24; fp32 streams 16-row tiles throughout
    for T, want in ((128, 16), (129, 32), (256, 32), (384, 32), (385, 64)):
        assert R.moe_sizes(T, 128, 8, 2048, 768, 1, R.BF16)[2] == want, T
    assert R.moe_sizes(256, 128, 8, 2048, 768, 1, R.F32)[2] == 16
    sl32, _, _ = R.moe_sizes(256, 128, 8, 2048, 768, 1, R.BF16)
    assert sl32 == (2048 // 32 + 128) * 32
    with pytest.raises(_lib.RimuruError) as e:
        R.moe_sizes(4, 8, 9, 128, 64, 8, R.F32)
    assert e.value.status == _lib.EINVAL
    with pytest.raises(_lib.RimuruError) as e:
        R.moe_sizes(4, 8, 2, 128, 64, 8, 7)
    assert e.value.status == _lib.EDTYPE
    with pytest.raises(_lib.RimuruError):
        R.moe_sizes(4, 8, 2, 100, 64, 8, R.F32)          # H not a multiple of 64
    with pytest.raises(_lib.RimuruError):
        R.moe_sizes(4, 600, 2, 128, 64, 8, R.F32)        # E above 512


def _args(**over):
    a = _lib.MoeArgs()
    a.T, a.E, a.k, a.H, a.I, a.P, a.dtype, a.renormalize = 16, 8, 2, 128, 64, 8, R.F32, 1
    a.page_bytes = 4096
    for name in ("x", "logits", "pool_base", "pt", "y", "topk_ids", "topk_w", "sorted_ids",
                 "expert_off", "workspace"):
        setattr(a, name, 1 << 20)                       # never dereferenced: validation fails first
    a.workspace_bytes = 1 << 30
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(k=0), _lib.EINVAL), (dict(k=9), _lib.EINVAL), (dict(E=0), _lib.EINVAL),
    (dict(H=96), _lib.EINVAL), (dict(dtype=3), _lib.EDTYPE), (dict(renormalize=0), _lib.EINVAL),
    (dict(page_bytes=100), _lib.EINVAL), (dict(P=7), _lib.EINVAL), (dict(x=0), _lib.EINVAL),
    (dict(pool_base=(1 << 20) + 16), _lib.EINVAL), (dict(workspace_bytes=100), _lib.EINVAL),
    (dict(n_stage_events=3), _lib.EINVAL), (dict(T=-1), _lib.EINVAL),
])
def test_fused_moe_rejects_bad_arguments_without_launching(over, status):
    assert R.fused_moe_paged_raw(_args(**over), 0) == status


def test_zero_tokens_is_a_noop():
    a = _args(T=0, x=0, y=0, logits=0)
    assert R.fused_moe_paged_raw(a, 0) == _lib.OK


def test_pt_check_ranges():
    pt = np.arange(8 * 3 * 4, dtype=np.int32).reshape(8, 3, 4)
    R.pt_check(pt, 4096, 96 * 4096)
    pt[5, 1, 2] = 96
    with pytest.raises(_lib.RimuruError) as e:
        R.pt_check(pt, 4096, 96 * 4096)
    assert e.value.status == _lib.ERANGE and "expert 5, projection 1, page 2" in str(e.value)
    pt[5, 1, 2] = -1
    with pytest.raises(_lib.RimuruError):
        R.pt_check(pt, 4096, 96 * 4096)


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "paged_moe_expert_amd")
    for dp, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dp, f)).read()
                assert "oracle" not in re.sub(r"#.*|//.*", "", txt).lower().replace("oracle/", ""), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            txt = open(os.path.join(ROOT, "oracle", f)).read()
            assert "paged_moe_expert_amd" not in txt and "rimuru" not in txt.replace("Rimuru", ""), f


def test_expert_upload_validates_before_copying():
    rows = np.arange(3 * 4, dtype=np.int32).reshape(3, 4)
    pool, host = 1 << 20, 1 << 21                        # never dereferenced: validation fails first
    ok_args = dict(pool_ptr=pool, pool_bytes=64 * 4096, page_bytes=4096, host_ptr=host, proj_bytes=4 * 4096,
                   stream_handle=0)

    def status(pt_rows=rows, **over):
        a = dict(ok_args, **over)
        return R.expert_upload_raw(a["pool_ptr"], a["pool_bytes"], pt_rows, a["page_bytes"], a["host_ptr"],
                                   a["proj_bytes"], a["stream_handle"])

    assert status(pool_ptr=0) == _lib.EINVAL
    assert status(host_ptr=0) == _lib.EINVAL
    assert status(pool_ptr=pool + 16) == _lib.EINVAL    # pool_base not 256-byte aligned
    assert status(host_ptr=host + 8) == _lib.EINVAL     # host_src not 16-byte aligned
    assert status(page_bytes=100) == _lib.EINVAL
    assert status(proj_bytes=5 * 4096) == _lib.EINVAL   # more than P pages
    assert status(proj_bytes=4096 + 8) == _lib.EINVAL   # not a multiple of 16
    bad = rows.copy()
    bad[2, 3] = 64                                       # one page past the pool's end
    assert status(pt_rows=bad) == _lib.ERANGE
    assert "projection 2, page 3" in _lib.lib().rimuru_last_error().decode()
    bad[2, 3] = -1
    assert status(pt_rows=bad) == _lib.ERANGE


def _attn_args(**over):
    base = dict(B=2, n_q=32, n_kv=4, head_dim=128, max_blocks=4, scale=0.125, q=1 << 20,
                pool_base=1 << 21, block_table=1 << 22, context_lens=1 << 23, out=1 << 24,
                workspace=1 << 25, workspace_bytes=1 << 30)
    base.update(over)
    return _lib.AttnArgs(*[base[f] for f, _ in _lib.AttnArgs._fields_])


@pytest.mark.parametrize("over", [
    dict(head_dim=64), dict(n_q=30), dict(n_q=68), dict(n_kv=0), dict(max_blocks=0), dict(scale=0.0),
    dict(scale=float("inf")), dict(q=0), dict(workspace=0), dict(q=(1 << 20) + 8),
    dict(pool_base=(1 << 21) + 128), dict(workspace_bytes=16), dict(B=-1),
])
def test_attention_rejects_bad_arguments_without_launching(over):
    a = _attn_args(**over)
    assert _lib.lib().rimuru_paged_decode_attention(C.byref(a), None) == _lib.EINVAL


def test_attention_no_requests_is_a_noop_and_split_choice():
    a = _attn_args(B=0, q=0, out=0)
    assert _lib.lib().rimuru_paged_decode_attention(C.byref(a), None) == _lib.OK
    # one split once B * n_kv fills 1024 workgroups; more for few requests;
    # never a split longer than 1024 blocks
    assert R.attn_sizes(256, 32, 4, 128, 127)[1] == 1
    assert R.attn_sizes(1, 32, 4, 128, 256)[1] == 32
    assert R.attn_sizes(300, 32, 4, 128, 1100)[1] == 2
    ws, ns, bb = R.attn_sizes(3, 16, 2, 256, 10)
    assert bb == 2 * 2 * 16 * 256 * 2 and ws == 3 * 16 * ns * (256 + 2) * 4


def test_block_table_check_names_bad_entries():
    table = np.array([[0, 1, 2], [3, 9, 0]], dtype=np.int32)
    R.block_table_check(table, np.array([48, 17], dtype=np.int32), 4096, 10 * 4096)
    with pytest.raises(R.RimuruError, match="ERANGE"):
        R.block_table_check(table, np.array([48, 33], dtype=np.int32), 4096, 9 * 4096)   # block 9 outside
    with pytest.raises(R.RimuruError, match="ERANGE"):
        R.block_table_check(table, np.array([49, 1], dtype=np.int32), 4096, 10 * 4096)   # 4 blocks > 3


def test_bench_is_one_gpu_only():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_layer_and_attention_never_copy_or_clear_memory():
    """The paged kernel reads expert pages where they sit: no translation unit
    of the layer or of the attention copies or clears device memory (the
    only copy in the library is the expert upload from host memory)."""
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "paged_moe_expert_amd", "csrc")
    for f in ("moe_layer.hip", "moe_routing.hip", "moe_gemm_stream.hip", "moe_gemm_tiled.hip", "attention.hip"):
        src = open(os.path.join(csrc, f)).read()
        for call in ("hipMemcpy", "hipMemset", "hipMalloc", "hipFree", "hipStreamSynchronize",
                     "hipDeviceSynchronize"):
            assert call not in src, f"{f} calls {call}"


def test_stream_read_rejects_bad_arguments_without_launching():
    lib = _lib.lib()
    assert lib.rimuru_stream_read(None, 1024, 1 << 20, None) == _lib.EINVAL
    assert lib.rimuru_stream_read(1 << 20, 1024, None, None) == _lib.EINVAL
    assert lib.rimuru_stream_read((1 << 20) + 8, 1024, 1 << 21, None) == _lib.EINVAL
    assert lib.rimuru_stream_read(1 << 20, 1000, 1 << 21, None) == _lib.EINVAL
