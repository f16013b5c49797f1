"""CPU oracle for the sparse-attention hot path (TEST INFRASTRUCTURE ONLY).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never calls it and shares no code
with it; the only thing both sides share is the seeded input generator
(`synth`), which holds none of the method's arithmetic.

Thin ctypes wrapper around oracle.c, which is the plain fp64 definition of the
three steps (indexer score, Top-K, sparse MLA attention); see that file's
header for the passages each step follows and the readings taken where the
pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

FMT = {"bf16": 0, "fp8": 1, "mxfp8": 2, "fp8r": 3}


def build() -> str:
    out = os.path.join(_HERE, "liboracle.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", out,
                           os.path.join(_HERE, "oracle.c"), "-lm"])
    return out


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_bf16.restype = dbl
        L.oracle_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3.restype = dbl
        L.oracle_e8m0.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0.restype = dbl
        L.oracle_index_scores.argtypes = [i32, vp, vp, vp, i32, vp, vp, i64, vp]
        L.oracle_index_scores.restype = None
        L.oracle_topk.argtypes = [vp, i64, i64, vp]
        L.oracle_topk.restype = i64
        L.oracle_sparse_attn.argtypes = [vp, i64, i32, vp, vp, i32, vp, i64, dbl, vp, vp, vp]
        L.oracle_sparse_attn.restype = None
        L.oracle_encode_e4m3.argtypes = [dbl]
        L.oracle_encode_e4m3.restype = ctypes.c_uint8
        L.oracle_quant_mxfp8.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_quant_mxfp8.restype = None
        L.oracle_quant_fp8_rows.argtypes = [vp, i64, i64, i64, vp, vp]
        L.oracle_quant_fp8_rows.restype = None
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def bf16(bits: int) -> float:
    return lib().oracle_bf16(int(bits))


def e4m3(code: int) -> float:
    return lib().oracle_e4m3(int(code))


def e8m0(code: int) -> float:
    return lib().oracle_e8m0(int(code))


def encode_e4m3(v: float) -> int:
    """Nearest E4M3FN code (ties to the even code), saturating at 448."""
    return int(lib().oracle_encode_e4m3(float(v)))


def quant_mxfp8(x):
    """x [n, L] bf16 bits (L % 32 == 0) -> (E4M3 codes [n, L], E8M0 scales [n, L/32])."""
    x = _c(x, np.uint16)
    n, L = x.shape
    codes = np.empty((n, L), dtype=np.uint8)
    scales = np.empty((n, L // 32), dtype=np.uint8)
    lib().oracle_quant_mxfp8(_p(x), n, L, _p(codes), _p(scales))
    return codes, scales


def quant_fp8_rows(x, block: int):
    """x [n, L] bf16 bits -> (E4M3 codes [n, L], f32 scales [n, ceil(L/block)])."""
    x = _c(x, np.uint16)
    n, L = x.shape
    nb = (L + block - 1) // block
    codes = np.empty((n, L), dtype=np.uint8)
    scales = np.empty((n, nb), dtype=np.float32)
    lib().oracle_quant_fp8_rows(_p(x), n, L, block, _p(codes), _p(scales))
    return codes, scales


def index_scores(q, w, k, vis: int, q_fmt="bf16", q_scales=None, k_fmt="bf16", k_scales=None) -> np.ndarray:
    """fp32 scores [vis] of one token; q [64,128], w [64], k [>=vis,128].
    k_fmt "fp8": k_scales [>=vis] f32 per row; "mxfp8": k_scales [>=vis,4] E8M0."""
    q = _c(q, np.uint16 if q_fmt == "bf16" else np.uint8)
    k = _c(k, np.uint16 if k_fmt == "bf16" else np.uint8)
    w = _c(w, np.float32)
    qs = _c(q_scales, np.uint8)
    ks = _c(k_scales, np.uint8 if k_fmt == "mxfp8" else np.float32)
    if k_fmt == "mxfp8":
        assert ks.shape[0] >= vis and ks.shape[1] == 4
    assert q.shape == (64, 128) and w.shape == (64,) and k.shape[1] == 128 and k.shape[0] >= vis
    out = np.empty((vis,), dtype=np.float32)
    lib().oracle_index_scores(FMT[q_fmt], _p(q), _p(qs), _p(w), FMT[k_fmt], _p(k), _p(ks), vis, _p(out))
    return out


def topk(scores, top_k: int):
    """(idx [top_k] int32 in rank order padded with -1, count)."""
    s = _c(scores, np.float32)
    idx = np.empty((top_k,), dtype=np.int32)
    n = lib().oracle_topk(_p(s), s.shape[0], top_k, _p(idx))
    return idx, int(n)


def sparse_attn(q, c, idx, sm_scale: float, c_fmt="bf16", c_scales=None, want_p=False):
    """q [H,576] bf16 bits, c [L,576] logical latent rows (c_fmt "fp8r": [L,640]
    bytes, 512 E4M3 codes + 64 bf16 rope), idx [K].
    Returns (out [H,512] f64, lse [H] f64[, p [H,K]])."""
    q = _c(q, np.uint16)
    c = _c(c, np.uint16 if c_fmt == "bf16" else np.uint8)
    cs = _c(c_scales, np.float32)
    G = 1 if cs is None else (cs.shape[1] if cs.ndim == 2 else 1)
    idx = _c(idx, np.int32)
    H, K = q.shape[0], idx.shape[0]
    assert q.shape[1] == 576 and c.shape[1] == (640 if c_fmt == "fp8r" else 576)
    assert idx.max(initial=-1) < c.shape[0]
    out = np.empty((H, 512), dtype=np.float64)
    lse = np.empty((H,), dtype=np.float64)
    p = np.empty((H, K), dtype=np.float64) if want_p else None
    lib().oracle_sparse_attn(_p(q), H, FMT[c_fmt], _p(c), _p(cs), G, _p(idx), K, float(sm_scale), _p(out),
                             _p(lse), _p(p))
    return (out, lse, p) if want_p else (out, lse)


def run_tokens(case, tokens, with_attn=True):
    """Run the whole path for the given tokens of a synth.Case.

    Returns {t: {"scores", "idx" (rank order), "n", "out", "lse"}}."""
    res = {}
    by_req = {}
    for t in tokens:
        by_req.setdefault(t // case.n_q, []).append(t)
    for b, ts in by_req.items():
        k, ks = case.k_rows(b)
        lat, lats = case.latent_rows(b) if with_attn else (None, None)
        for t in ts:
            q, qs = case.idx_q(t, 1)
            w = case.w(t, 1)
            vis = case.visible(t)
            q_fmt = "bf16" if case.idx_fmt == "bf16" else "fp8"  # the query is MXFP8 in both FP8 layouts
            sc = index_scores(q[0], w[0], k, vis, q_fmt=q_fmt, q_scales=None if qs is None else qs[0],
                              k_fmt=case.idx_fmt, k_scales=ks)
            idx, n = topk(sc, case.top_k)
            r = {"scores": sc, "idx": idx, "n": n}
            if with_attn:
                mq = case.mla_q(t, 1)[0]
                out, lse = sparse_attn(mq, lat, idx, case.sm_scale, c_fmt=case.kv_fmt, c_scales=lats)
                r["out"], r["lse"] = out, lse
            res[t] = r
    return res
