"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sparse_li.h, and rejects bad arguments before enqueuing."""
import ctypes
import os
import re

import pytest

import sparse_attention_li_amd as li

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "sparse_li.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|size_t|li_status|void)\s+(\w+)\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(li.EXPORTS)
    L = li.lib()
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.li_version()


def _call_topk(**over):
    L = li.lib()
    P = ctypes.c_void_p(0x10000)
    args = dict(num_seqs=1, q_per_seq=1, seq_lens=P, bt=P, max_pages=32, num_pages=32, q_dtype=0, q=P, q_scales=None,
                w=P, k_dtype=0, k=P, k_scales=None, top_k=256, idx=P, ws=P, ws_bytes=1 << 30, stream=None)
    args.update(over)
    st = L.li_score_topk(*args.values())
    return st, L.li_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(top_k=0), -1), (dict(top_k=2049), -1), (dict(num_seqs=0), -1), (dict(q=None), -1),
    (dict(seq_lens=None), -1), (dict(q_dtype=7, k_dtype=7), -2), (dict(k_dtype=1), -2),
    (dict(q_dtype=1, k_dtype=1), -1), (dict(q_scales=ctypes.c_void_p(0x10000)), -1),
    (dict(q_per_seq=3, q_dtype=1, k_dtype=1, q_scales=ctypes.c_void_p(0x10000),
          k_scales=ctypes.c_void_p(0x10000)), -2),
    (dict(ws_bytes=16), -3), (dict(ws=None), -3), (dict(max_pages=10 ** 6), -2),
    (dict(q=ctypes.c_void_p(0x10004)), -1),
    # MXFP8 keys go with an FP8 query only, need their scales, 4-byte aligned
    (dict(k_dtype=2), -2), (dict(q_dtype=1, k_dtype=2, q_scales=ctypes.c_void_p(0x10000)), -1),
    (dict(q_dtype=1, k_dtype=2, q_scales=ctypes.c_void_p(0x10000), k_scales=ctypes.c_void_p(0x10002)), -1),
    (dict(q_dtype=0, k_dtype=2, k_scales=ctypes.c_void_p(0x10000)), -2),
])
def test_score_topk_argument_errors(over, status):
    st, msg = _call_topk(**over)
    assert st == status and msg


def _call_sfa(fn="sfa_decode", **over):
    L = li.lib()
    P = ctypes.c_void_p(0x10000)
    args = dict(num_seqs=1, q_per_seq=1, seq_lens=P, bt=P, max_pages=32, num_pages=32, q=P, H=128, kv_dtype=0,
                kv=P, kv_scales=None, groups=1, idx=P, top_k=2048, sm=0.1, out=P, lse=None, ws=P,
                ws_bytes=1 << 30, stream=None)
    args.update(over)
    st = getattr(L, fn)(*args.values())
    return st, L.li_last_error().decode()


@pytest.mark.parametrize("fn", ["sfa_decode", "sfa_prefill"])
@pytest.mark.parametrize("over,status", [
    (dict(H=48), -2), (dict(H=256), -2), (dict(top_k=0), -1), (dict(idx=None), -1), (dict(kv_dtype=7), -2),
    (dict(kv_dtype=3), -1), (dict(kv_dtype=3, kv_scales=ctypes.c_void_p(0x10000), groups=5), -2),
    (dict(kv_dtype=1), -1), (dict(kv_dtype=1, kv_scales=ctypes.c_void_p(0x10000), groups=2), -2),
    (dict(kv_scales=ctypes.c_void_p(0x10000)), -1), (dict(sm=float("nan")), -1), (dict(ws_bytes=8), -3),
    (dict(out=ctypes.c_void_p(0x10002)), -1),
])
def test_sfa_argument_errors(fn, over, status):
    st, msg = _call_sfa(fn, **over)
    assert st == status and msg


def test_workspace_sizes():
    assert li.li_score_topk_workspace_size(0, 1, 1, 1) == 0
    a = li.li_score_topk_workspace_size(32, 1, 512, 2048)
    b = li.li_score_topk_workspace_size(32, 2, 512, 2048)
    assert 0 < a < b
    assert li.sfa_workspace_size(32, 128, 2048) > 0


def _call_quant(**over):
    L = li.lib()
    P = ctypes.c_void_p(0x10000)
    args = dict(n_rows=4, row_len=128, x=P, codes=P, scales=P, stream=None)
    args.update(over)
    return L.li_quantize_mxfp8(*args.values()), L.li_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(row_len=100), -1), (dict(row_len=0), -1), (dict(n_rows=-1), -1), (dict(x=None), -1),
    (dict(scales=None), -1), (dict(x=ctypes.c_void_p(0x10008)), -1), (dict(codes=ctypes.c_void_p(0x10004)), -1),
])
def test_quantize_argument_errors(over, status):
    st, msg = _call_quant(**over)
    assert st == status and msg


def test_quantize_zero_rows_is_a_no_op():
    st, _ = _call_quant(n_rows=0, x=None, codes=None, scales=None)
    assert st == 0


def _call_append(**over):
    L = li.lib()
    P = ctypes.c_void_p(0x10000)
    args = dict(num_seqs=2, q_per_seq=1, seq_lens=P, bt=P, max_pages=32, num_pages=64, k_new=P, k_dtype=0, k_cache=P,
                k_scales=None, kv_new=P, kv_dtype=0, kv_cache=P, kv_scales=None, groups=1, stream=None)
    args.update(over)
    return L.li_cache_append(*args.values()), L.li_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(k_new=None, kv_new=None), -1), (dict(num_seqs=0), -1), (dict(seq_lens=None), -1),
    (dict(k_dtype=4), -2), (dict(k_dtype=1), -1), (dict(k_cache=None), -1), (dict(kv_dtype=1), -1),
    (dict(k_dtype=2), -1), (dict(k_dtype=1, k_scales=ctypes.c_void_p(0x10002)), -1),
    (dict(kv_dtype=1, kv_scales=ctypes.c_void_p(0x10000), groups=3), -2), (dict(kv_cache=None), -1),
    (dict(k_new=ctypes.c_void_p(0x10008)), -1), (dict(kv_cache=ctypes.c_void_p(0x10004)), -1),
])
def test_cache_append_argument_errors(over, status):
    st, msg = _call_append(**over)
    assert st == status and msg


def test_noalloc_rejects_geometries_beyond_its_array():
    """The allocation-free indexer serves geometries whose exchange workspace
    fits the library's array and rejects larger ones before touching a device."""
    L = li.lib()
    P = ctypes.c_void_p(0x10000)
    cap = 128 << 20
    assert L.li_score_topk_workspace_size(32, 1, 512, 2048) <= cap       # 32 x 32K decode
    assert L.li_score_topk_workspace_size(128, 2, 2048, 2048) > cap      # 128 x 2 tokens x 128K
    st = L.li_score_topk_noalloc(128, 2, P, P, 2048, 262144, 1, P, P, P, 1, P, P, 2048, P, None)
    assert st == -2 and b"li_score_topk_noalloc" in L.li_last_error()
    st = L.li_score_topk_noalloc(0, 1, P, P, 32, 32, 0, P, None, P, 0, P, None, 256, P, None)
    assert st == -1 and L.li_last_error()


def test_validate_paged_argument_errors():
    L = li.lib()
    P = ctypes.c_void_p(0x10000)
    assert L.li_validate_paged(0, P, P, 4, 8, P, None) == -1
    assert L.li_validate_paged(2, None, P, 4, 8, P, None) == -1
    assert L.li_validate_paged(2, P, P, 4, 0, P, None) == -1
    assert L.li_validate_paged(2, P, P, 4, 8, ctypes.c_void_p(0x10002), None) == -1
    assert L.li_last_error()
