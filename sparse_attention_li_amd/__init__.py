"""Python binding of the MI355X sparse-attention hot path (libsparse_li.so).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI (include/sparse_li.h).  PyTorch supplies device memory and
the current stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

    idx = li_score_topk(q, w, k_cache, seq_lens, block_table, top_k, ...)
    out, lse = sfa_decode(q_mla, kv_cache, idx, seq_lens, block_table, sm_scale, ...)
    out, lse = sfa_prefill(...)            # same arguments, prefill launch shape
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["li_score_topk", "sfa_decode", "sfa_prefill", "lib", "LI_BF16", "LI_FP8", "LI_MXFP8", "LI_FP8_ROPE_BF16", "LiError",
           "li_score_topk_workspace_size", "sfa_workspace_size", "li_workspace_zero", "li_quantize_mxfp8",
           "li_set_exchange_patience", "li_score_topk_noalloc", "li_decode_step", "li_decode_step_workspace_size",
           "li_cache_append", "li_validate_paged"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_li.so")

LI_BF16, LI_FP8, LI_MXFP8, LI_FP8_ROPE_BF16 = 0, 1, 2, 3
LI_OK = 0
_STATUS = {-1: "LI_ERR_INVALID_ARG", -2: "LI_ERR_UNSUPPORTED", -3: "LI_ERR_WORKSPACE", -4: "LI_ERR_HIP"}

EXPORTS = ["li_version", "li_last_error", "li_set_exchange_patience", "li_score_topk_workspace_size",
           "li_score_topk_noalloc", "li_decode_step", "li_decode_step_workspace_size", "li_workspace_zero", "li_score_topk",
           "sfa_workspace_size", "sfa_decode", "sfa_prefill", "li_quantize_mxfp8", "li_cache_append",
           "li_validate_paged"]


class LiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libsparse_li.so (built in place by sparse_attention_li_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m sparse_attention_li_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp, sz, f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        L.li_version.restype = ctypes.c_char_p
        L.li_version.argtypes = []
        L.li_last_error.restype = ctypes.c_char_p
        L.li_last_error.argtypes = []
        L.li_set_exchange_patience.restype = None
        L.li_set_exchange_patience.argtypes = [i32]
        L.li_score_topk_workspace_size.restype = sz
        L.li_score_topk_workspace_size.argtypes = [i32, i32, i32, i32]
        L.li_workspace_zero.restype = i32
        L.li_workspace_zero.argtypes = [vp, sz, vp]
        L.li_validate_paged.restype = i32
        L.li_validate_paged.argtypes = [i32, vp, vp, i32, i32, vp, vp]
        L.li_score_topk.restype = i32
        L.li_score_topk.argtypes = [i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, i32, vp, vp, sz, vp]
        L.li_score_topk_noalloc.restype = i32
        L.li_score_topk_noalloc.argtypes = [i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, i32, vp, vp]
        L.li_decode_step_workspace_size.restype = sz
        L.li_decode_step_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.li_decode_step.restype = i32
        L.li_decode_step.argtypes = [i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, vp, vp, i32,
                                     i32, f32, vp, vp, vp, vp, sz, vp]
        L.sfa_workspace_size.restype = sz
        L.sfa_workspace_size.argtypes = [i32, i32, i32]
        sfa_args = [i32, i32, vp, vp, i32, i32, vp, i32, i32, vp, vp, i32, vp, i32, f32, vp, vp, vp, sz, vp]
        L.sfa_decode.restype = i32
        L.sfa_decode.argtypes = sfa_args
        L.sfa_prefill.restype = i32
        L.sfa_prefill.argtypes = sfa_args
        L.li_quantize_mxfp8.restype = i32
        L.li_quantize_mxfp8.argtypes = [i32, i32, vp, vp, vp, vp]
        L.li_cache_append.restype = i32
        L.li_cache_append.argtypes = [i32, i32, vp, vp, i32, i32, vp, i32, vp, vp, vp, i32, vp, vp, i32, vp]
        _lib = L
    return _lib


def _check(status: int):
    if status != LI_OK:
        raise LiError(status, lib().li_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_of(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return LI_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return LI_FP8
    raise TypeError(f"unsupported cache/query dtype {t.dtype}")


def li_score_topk_workspace_size(num_seqs: int, q_per_seq: int, max_pages: int, top_k: int) -> int:
    return int(lib().li_score_topk_workspace_size(num_seqs, q_per_seq, max_pages, top_k))


def sfa_workspace_size(num_tokens: int, num_heads: int, top_k: int) -> int:
    return int(lib().sfa_workspace_size(num_tokens, num_heads, top_k))


def li_set_exchange_patience(polls: int):
    """Test hook: polls an indexer exchange wait makes before it takes its exact
    fallback (negative = the default)."""
    lib().li_set_exchange_patience(int(polls))


def li_workspace_zero(ws: torch.Tensor, stream=None):
    _check(lib().li_workspace_zero(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def li_validate_paged(seq_lens: torch.Tensor, block_table: torch.Tensor, num_pages: int, stream=None) -> torch.Tensor:
    """Device-side check of the paged-cache metadata: returns a one-element
    int32 device tensor with the number of problems found (requests whose
    length lies outside [0, max_pages*64], used pages whose id lies outside
    [0, num_pages))."""
    B, max_pages = block_table.shape
    bad = torch.empty(1, dtype=torch.int32, device=block_table.device)
    _check(lib().li_validate_paged(B, _ptr(seq_lens), _ptr(block_table), max_pages, num_pages, _ptr(bad),
                                   _stream(stream)))
    return bad


_ws_cache: dict = {}


def _workspace(kind: str, nbytes: int, device) -> torch.Tensor:
    """A cached, zero-initialised byte workspace per (kind, device); grows as needed.
    The indexer leaves its workspace zero after every call."""
    key = (kind, torch.device(device).index)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def li_score_topk(q: torch.Tensor, w: torch.Tensor, k_cache: torch.Tensor, seq_lens: torch.Tensor,
                  block_table: torch.Tensor, top_k: int, q_scales: torch.Tensor | None = None,
                  k_scales: torch.Tensor | None = None, idx_out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fused indexer score + Top-K.  q [T,64,128] (bf16, or uint8 E4M3 codes with
    q_scales [T,64,4] uint8 E8M0), w [T,64] f32, k_cache [NP,64,128] (bf16, or uint8
    codes with k_scales [NP,64] f32 per row, or k_scales [NP,64,4] uint8 E8M0 per
    32 elements = MXFP8 keys).  Returns idx [T,top_k] int32, ascending positions,
    -1 padded."""
    B = seq_lens.shape[0]
    T = q.shape[0]
    if T % B:
        raise ValueError("q.shape[0] must be a multiple of len(seq_lens)")
    n_q = T // B
    max_pages = block_table.shape[1]
    num_pages = k_cache.shape[0]
    if idx_out is None:
        idx_out = torch.empty((T, top_k), dtype=torch.int32, device=q.device)
    if workspace is None:
        need = li_score_topk_workspace_size(B, n_q, max_pages, top_k)
        workspace = _workspace("indexer", need, q.device)
    k_dtype = LI_MXFP8 if k_scales is not None and k_scales.dtype == torch.uint8 else _dtype_of(k_cache)
    st = lib().li_score_topk(B, n_q, _ptr(seq_lens), _ptr(block_table), max_pages, num_pages, _dtype_of(q), _ptr(q),
                             _ptr(q_scales), _ptr(w), k_dtype, _ptr(k_cache), _ptr(k_scales), top_k,
                             _ptr(idx_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check(st)
    return idx_out


def li_score_topk_noalloc(q: torch.Tensor, w: torch.Tensor, k_cache: torch.Tensor, seq_lens: torch.Tensor,
                          block_table: torch.Tensor, top_k: int, idx_out: torch.Tensor,
                          q_scales: torch.Tensor | None = None, k_scales: torch.Tensor | None = None, stream=None):
    """li_score_topk with the library's own exchange workspace (no allocation by
    the library or here): the caller passes idx_out [T,top_k] int32."""
    B = seq_lens.shape[0]
    T = q.shape[0]
    if T % B:
        raise ValueError("q.shape[0] must be a multiple of len(seq_lens)")
    k_dtype = LI_MXFP8 if k_scales is not None and k_scales.dtype == torch.uint8 else _dtype_of(k_cache)
    st = lib().li_score_topk_noalloc(B, T // B, _ptr(seq_lens), _ptr(block_table), block_table.shape[1],
                                     k_cache.shape[0], _dtype_of(q), _ptr(q), _ptr(q_scales), _ptr(w), k_dtype,
                                     _ptr(k_cache), _ptr(k_scales), top_k, _ptr(idx_out), _stream(stream))
    _check(st)
    return idx_out


def _sfa(fn, q, kv_cache, idx, seq_lens, block_table, sm_scale, kv_scales=None, out=None, lse=None,
         want_lse=True, workspace=None, stream=None):
    B = seq_lens.shape[0]
    T, H = q.shape[0], q.shape[1]
    if T % B:
        raise ValueError("q.shape[0] must be a multiple of len(seq_lens)")
    n_q = T // B
    top_k = idx.shape[1]
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    groups = 1 if kv_scales is None else (kv_scales.shape[2] if kv_scales.dim() == 3 else 1)
    kv_dtype = _dtype_of(kv_cache)
    if kv_dtype == LI_FP8 and kv_cache.shape[-1] == 640:
        kv_dtype = LI_FP8_ROPE_BF16  # 512 codes + 64 bf16 rope per row
    if workspace is None:
        workspace = _workspace("attention", sfa_workspace_size(T, H, top_k), q.device)
    st = fn(B, n_q, _ptr(seq_lens), _ptr(block_table), block_table.shape[1], kv_cache.shape[0], _ptr(q), H,
            kv_dtype, _ptr(kv_cache), _ptr(kv_scales), groups, _ptr(idx), top_k, float(sm_scale), _ptr(out),
            _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st)
    return out, lse


def sfa_decode(q, kv_cache, idx, seq_lens, block_table, sm_scale, kv_scales=None, **kw):
    """Sparse MLA attention.  q [T,H,576] bf16, kv_cache [NP,64,576] (bf16, or uint8
    codes with kv_scales [NP,64,G] f32; or uint8 [NP,64,640] = 512 codes + 64 bf16
    rope with G = 1 or 4), idx [T,K] int32.  Returns (out [T,H,512] bf16, lse [T,H] f32)."""
    return _sfa(lib().sfa_decode, q, kv_cache, idx, seq_lens, block_table, sm_scale, kv_scales, **kw)


def sfa_prefill(q, kv_cache, idx, seq_lens, block_table, sm_scale, kv_scales=None, **kw):
    """sfa_decode's operation with the launch shape for a prefill chunk."""
    return _sfa(lib().sfa_prefill, q, kv_cache, idx, seq_lens, block_table, sm_scale, kv_scales, **kw)


def li_decode_step_workspace_size(num_seqs: int, q_per_seq: int, max_pages: int, num_heads: int, top_k: int) -> int:
    return int(lib().li_decode_step_workspace_size(num_seqs, q_per_seq, max_pages, num_heads, top_k))


def li_decode_step(q_idx: torch.Tensor, w: torch.Tensor, k_cache: torch.Tensor, q: torch.Tensor,
                   kv_cache: torch.Tensor, seq_lens: torch.Tensor, block_table: torch.Tensor, top_k: int,
                   sm_scale: float, q_scales=None, k_scales=None, kv_scales=None, idx_out=None, out=None, lse=None,
                   workspace=None, stream=None):
    """The whole decode step (indexer score + Top-K, then sparse MLA attention),
    one launch where the shape allows.  Returns (idx, out, lse)."""
    B = seq_lens.shape[0]
    T, H = q.shape[0], q.shape[1]
    if T % B or q_idx.shape[0] != T:
        raise ValueError("q and q_idx must hold the same multiple of len(seq_lens) tokens")
    n_q = T // B
    max_pages = block_table.shape[1]
    if idx_out is None:
        idx_out = torch.empty((T, top_k), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace("step", li_decode_step_workspace_size(B, n_q, max_pages, H, top_k), q.device)
    k_dtype = LI_MXFP8 if k_scales is not None and k_scales.dtype == torch.uint8 else _dtype_of(k_cache)
    kv_dtype = _dtype_of(kv_cache)
    if kv_dtype == LI_FP8 and kv_cache.shape[-1] == 640:
        kv_dtype = LI_FP8_ROPE_BF16
    groups = 1 if kv_scales is None else (kv_scales.shape[2] if kv_scales.dim() == 3 else 1)
    st = lib().li_decode_step(B, n_q, _ptr(seq_lens), _ptr(block_table), max_pages, k_cache.shape[0], _dtype_of(q_idx),
                              _ptr(q_idx), _ptr(q_scales), _ptr(w), k_dtype, _ptr(k_cache), _ptr(k_scales), _ptr(q), H,
                              kv_dtype, _ptr(kv_cache), _ptr(kv_scales), groups, top_k, float(sm_scale), _ptr(idx_out),
                              _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream))
    _check(st)
    return idx_out, out, lse


def li_quantize_mxfp8(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                      stream=None):
    """MXFP8 quantisation of bf16 x [..., L] (L % 32 == 0): returns (codes uint8
    [..., L] E4M3, scales uint8 [..., L/32] E8M0)."""
    L = x.shape[-1]
    n = x.numel() // L if L else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((*x.shape[:-1], L // 32), dtype=torch.uint8, device=x.device)
    _check(lib().li_quantize_mxfp8(n, L, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def li_cache_append(seq_lens: torch.Tensor, block_table: torch.Tensor, k_new: torch.Tensor | None = None,
                    k_cache: torch.Tensor | None = None, kv_new: torch.Tensor | None = None,
                    kv_cache: torch.Tensor | None = None, k_scales: torch.Tensor | None = None,
                    kv_scales: torch.Tensor | None = None, stream=None):
    """Writes the new tokens' rows into the paged caches.  k_new [T,128] bf16 into
    k_cache [NP,64,128] (bf16, or uint8 codes with k_scales [NP,64] f32, or with
    k_scales [NP,64,4] uint8 E8M0 = MXFP8 keys); kv_new
    [T,576] bf16 into kv_cache [NP,64,576] (bf16, or uint8 codes with kv_scales
    [NP,64,G] f32, G = 1 or 5).  Token t of request b goes to position
    seq_lens[b] - n_q + (t % n_q)."""
    B = seq_lens.shape[0]
    ref = k_new if k_new is not None else kv_new
    T = ref.shape[0]
    if T % B:
        raise ValueError("the number of new rows must be a multiple of len(seq_lens)")
    pool = k_cache if k_cache is not None else kv_cache
    groups = 1 if kv_scales is None else (kv_scales.shape[2] if kv_scales.dim() == 3 else 1)
    st = lib().li_cache_append(B, T // B, _ptr(seq_lens), _ptr(block_table), block_table.shape[1], pool.shape[0],
                               _ptr(k_new), LI_BF16 if k_cache is None else
                               (LI_MXFP8 if k_scales is not None and k_scales.dtype == torch.uint8 else _dtype_of(k_cache)),
                               _ptr(k_cache),
                               _ptr(k_scales), _ptr(kv_new),
                               LI_BF16 if kv_cache is None else
                               (LI_FP8_ROPE_BF16 if kv_cache.shape[-1] == 640 else _dtype_of(kv_cache)),
                               _ptr(kv_cache), _ptr(kv_scales), groups, _stream(stream))
    _check(st)
