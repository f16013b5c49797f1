"""Moves a synth.Case onto the GPU in the layouts of the C ABI (test and
benchmark helper; no arithmetic of the method)."""
from __future__ import annotations

import numpy as np
import torch


def _t(a: np.ndarray, dev):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class GpuCase:
    def __init__(self, case, dev="cuda", attention=True, latent_requests=None):
        """latent_requests: if given, only those requests' latent rows are
        generated (the pool keeps its full size; other pages hold code 0 with
        scale 1), for full-size launches whose checks sample a few requests."""
        self.case = case
        self.dev = dev
        self.seq_lens = _t(case.seq_lens.astype(np.int32), dev)
        self.block_table = _t(case.block_table(), dev)
        q, qs = case.idx_q()
        self.q = _t(q, dev)
        self.q_scales = None if qs is None else _t(qs, dev)
        self.w = _t(case.w(), dev)
        kp, ks = case.k_pool()
        self.k_pool = _t(kp, dev)
        self.k_scales = None if ks is None else _t(ks, dev)
        del kp, ks
        if attention and latent_requests is None:
            self.mla_q = _t(case.mla_q(), dev)
            lp, ls = case.latent_pool()
            self.kv_pool = _t(lp, dev)
            self.kv_scales = None if ls is None else _t(ls, dev)
            del lp, ls
        elif attention:
            self.mla_q = _t(case.mla_q(), dev)
            NP, fp8 = case.num_pages, case.kv_fmt != "bf16"
            row = 640 if case.kv_fmt == "fp8r" else 576
            self.kv_pool = torch.zeros((NP, 64, row), dtype=torch.uint8 if fp8 else torch.int16, device=dev)
            self.kv_scales = torch.ones((NP, 64, case.kv_groups), dtype=torch.float32, device=dev) if fp8 else None
            bt = case.block_table()
            flat = self.kv_pool.view(NP * 64, row)
            for b in latent_requests:
                L = int(case.seq_lens[b])
                rows, sc = case.latent_rows(b)
                s = np.arange(L)
                phys = torch.from_numpy((bt[b, s // 64].astype(np.int64) * 64 + s % 64)).to(dev)
                flat[phys] = _t(rows.view(np.uint8) if fp8 else rows.view(np.int16), dev)
                if fp8:
                    self.kv_scales.view(NP * 64, case.kv_groups)[phys] = _t(sc, dev)

    def score_topk(self, lib, **kw):
        c = self.case
        return lib.li_score_topk(self.q, self.w, self.k_pool, self.seq_lens, self.block_table, c.top_k,
                                 q_scales=self.q_scales, k_scales=self.k_scales, **kw)

    def attend(self, lib, idx, prefill=False, **kw):
        c = self.case
        fn = lib.sfa_prefill if prefill else lib.sfa_decode
        return fn(self.mla_q, self.kv_pool, idx, self.seq_lens, self.block_table, c.sm_scale,
                  kv_scales=self.kv_scales, **kw)


def rel_err(out_gpu: np.ndarray, out_ref: np.ndarray) -> float:
    """max over (token, head) of max_d |gpu - ref| / max_d |ref|."""
    num = np.abs(out_gpu - out_ref).max(axis=-1)
    den = np.maximum(np.abs(out_ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def encode_indexer_int(case, q_int: np.ndarray, k_ints: list):
    """Integer-valued indexer inputs (values in [-4, 4]) in the case's formats,
    as the generator stores them: q [T,64,128] -> bf16 bits, or MXFP8 codes +
    E8M0 scales; key rows of each request [L_b,128] -> bf16 bits, or E4M3
    codes with scale 1 (f32 per row for "fp8", E8M0 code 127 per 32 elements
    for "mxfp8").  Returns (q, q_scales, [(k_rows, k_scales)] per request)."""
    import ctypes
    import synth
    q_int = np.ascontiguousarray(q_int, dtype=np.int8)
    p = lambda a: ctypes.c_void_p(a.ctypes.data)
    if case.idx_fmt == "bf16":
        q = np.empty(q_int.shape, np.uint16)
        synth.lib().synth_int_to_bf16(p(q_int), q_int.size, p(q))
        qs = None
    else:
        q = np.empty(q_int.shape, np.uint8)
        qs = np.empty(q_int.shape[:2] + (4,), np.uint8)
        synth.lib().synth_mx_encode_int(p(q_int), q_int.size // 32, p(q), p(qs))
    ks = []
    for k in k_ints:
        k = np.ascontiguousarray(k, dtype=np.int8)
        if case.idx_fmt == "bf16":
            rows = np.empty(k.shape, np.uint16)
            synth.lib().synth_int_to_bf16(p(k), k.size, p(rows))
            ks.append((rows, None))
        else:
            rows = torch.from_numpy(k.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            sc = np.ones(k.shape[0], np.float32) if case.idx_fmt == "fp8" else np.full((k.shape[0], 4), 127, np.uint8)
            ks.append((rows, sc))
    return q, qs, ks


def load_indexer(g: "GpuCase", q, q_scales, w, k_rows: list):
    """Replaces g's indexer inputs (logical rows per request, as returned by
    encode_indexer_int) and scatters the key rows into its paged pool."""
    case = g.case
    g.q = _t(q, g.dev)
    g.q_scales = None if q_scales is None else _t(q_scales, g.dev)
    g.w = _t(np.asarray(w, np.float32), g.dev)
    NP = case.num_pages
    bt = case.block_table()
    pool = np.zeros((NP * 64, 128), np.uint16 if case.idx_fmt == "bf16" else np.uint8)
    sc = None
    if case.idx_fmt == "fp8":
        sc = np.zeros((NP * 64,), np.float32)
    elif case.idx_fmt == "mxfp8":
        sc = np.full((NP * 64, 4), 127, np.uint8)
    for b, (rows, rs) in enumerate(k_rows):
        s = np.arange(rows.shape[0])
        phys = bt[b, s // 64].astype(np.int64) * 64 + s % 64
        pool[phys] = rows
        if sc is not None:
            sc[phys] = rs
    g.k_pool = _t(pool.reshape(NP, 64, 128), g.dev)
    g.k_scales = None if sc is None else _t(sc.reshape((NP, 64) + sc.shape[1:]), g.dev)
