"""Seeded synthetic inputs for the sparse-attention hot path.

Test and benchmark infrastructure, shared by the CPU oracle and the HIP path.
It holds value generation and the storage encodings of the caches only; none
of the method's arithmetic (scoring, selection, attention) lives here.

Workloads follow the shapes the pages describe for the hybrid model's sparse
branch: a 64-head x 128-d lightning indexer over a paged key cache, Top-K
selection, and MLA attention over a 512 + 64 latent cache shared by all heads.
Values are drawn so that indexer scores are exact in fp32 under any summation
order: q and k are integers in [-4, 4], head weights lie on the 1/32 grid of
(0, 1] (or of [-1, 1] without 0 for the signed variant), FP8 key block scales
are 1/2 or 1.  MLA queries and latent rows are
N(0, 1) rounded to bf16 (or E4M3 with amax/448 scales for the FP8 cache).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

PAGE = 64
D_IDX = 128
KFMT = {"bf16": 0, "fp8": 1, "mxfp8": 2}  # indexer key row formats of synth_idxk_rows
VFMT = {"bf16": 0, "fp8": 1, "fp8r": 2}   # latent row formats of synth_latent_rows
LAT_ROW_BYTES = {"fp8": 576, "fp8r": 640}  # FP8 latent rows (fp8r: 512 codes + 64 bf16 rope)
H_IDX = 64
D_LAT = 576
D_V = 512


def build() -> str:
    """Compile libsynth.so in place with gcc (plain C, OpenMP)."""
    import subprocess
    out = os.path.join(_HERE, "libsynth.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", out,
                           os.path.join(_HERE, "synth.c"), "-lm"])
    return out


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        sigs = {
            "synth_idxq_int": [u64, i64, i64, vp],
            "synth_w": [u64, i64, i64, vp],
            "synth_w_signed": [u64, i64, i64, vp],
            "synth_int_to_bf16": [vp, i64, vp],
            "synth_mx_encode_int": [vp, i64, vp, vp],
            "synth_idxk_int": [u64, i64, i64, i64, vp],
            "synth_kscale": [u64, i64, i64, i64, vp],
            "synth_idxk_rows": [u64, i32, i64, i64, i64, vp, vp],
            "synth_mlaq_bf16": [u64, i64, i64, i64, vp],
            "synth_latent_rows": [u64, i32, i32, i64, i64, i64, vp, vp],
            "synth_fill_idxk_pool": [u64, i32, i64, vp, i64, vp, vp, vp],
            "synth_fill_latent_pool": [u64, i32, i32, i64, vp, i64, vp, vp, vp],
        }
        for name, argt in sigs.items():
            f = getattr(L, name)
            f.argtypes = argt
            f.restype = None
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


@dataclass
class Case:
    """One synthetic workload.

    B requests with n_q query tokens each; request b holds seq_lens[b] cached
    positions, its n_q new tokens being the last n_q of them.  Token t = b*n_q+j
    sits at absolute position seq_lens[b] - n_q + j and sees positions <= that.

    idx_fmt: "bf16", "fp8" (MXFP8 query, key rows with one f32 scale each) or
    "mxfp8" (MXFP8 query and key rows, one E8M0 scale per 32 elements of both).
    kv_fmt: "bf16", "fp8" (576 E4M3 codes) or "fp8r" (512 E4M3 latent codes +
    64 bf16 rope elements, 640 bytes).  kv_groups: FP8 latent scales per row
    (fp8: 1 = per token, 5 = tiles of 128; fp8r: 1 or 4, over the 512 latent
    elements only).
    """
    seed: int
    B: int
    n_q: int
    seq_lens: np.ndarray
    top_k: int
    H: int
    idx_fmt: str = "bf16"
    kv_fmt: str = "bf16"
    kv_groups: int = 1
    sm_scale: float = 1.0 / 24.0
    extra_pages: int = 0
    permute_pages: bool = True
    signed_w: bool = False
    _bt: np.ndarray | None = field(default=None, repr=False)

    def __post_init__(self):
        self.seq_lens = np.asarray(self.seq_lens, dtype=np.int32)
        assert self.seq_lens.shape == (self.B,)
        assert (self.seq_lens >= 0).all()

    # ---- geometry ----
    @property
    def T(self) -> int:
        return self.B * self.n_q

    @property
    def pages_per_seq(self) -> np.ndarray:
        return (self.seq_lens.astype(np.int64) + PAGE - 1) // PAGE

    @property
    def max_pages(self) -> int:
        return int(self.pages_per_seq.max())

    @property
    def num_pages(self) -> int:
        return int(self.pages_per_seq.sum()) + self.extra_pages

    def token_pos(self, t: int) -> int:
        b, j = divmod(t, self.n_q)
        return int(self.seq_lens[b]) - self.n_q + j

    def visible(self, t: int) -> int:
        return max(0, self.token_pos(t) + 1)

    def block_table(self) -> np.ndarray:
        """[B, max_pages] int32; physical pages are a seeded random permutation
        of the pool (entries past a request's last page are -1)."""
        if self._bt is None:
            rng = np.random.default_rng(self.seed + 7919)
            perm = rng.permutation(self.num_pages) if self.permute_pages else np.arange(self.num_pages)
            bt = np.full((self.B, self.max_pages), -1, dtype=np.int32)
            o = 0
            for b in range(self.B):
                n = int(self.pages_per_seq[b])
                bt[b, :n] = perm[o:o + n]
                o += n
            self._bt = bt
        return self._bt

    # ---- indexer inputs ----
    def idx_q_int(self, t0: int = 0, nt: int | None = None) -> np.ndarray:
        nt = self.T - t0 if nt is None else nt
        out = np.empty((nt, H_IDX, D_IDX), dtype=np.int8)
        lib().synth_idxq_int(self.seed, t0, nt, _p(out))
        return out

    def idx_q(self, t0: int = 0, nt: int | None = None):
        """bf16: (uint16 [nt,64,128], None).  fp8: (uint8 codes [nt,64,128],
        uint8 E8M0 scales [nt,64,4])."""
        qi = self.idx_q_int(t0, nt)
        if self.idx_fmt == "bf16":
            out = np.empty(qi.shape, dtype=np.uint16)
            lib().synth_int_to_bf16(_p(qi), qi.size, _p(out))
            return out, None
        codes = np.empty(qi.shape, dtype=np.uint8)
        scales = np.empty(qi.shape[:2] + (D_IDX // 32,), dtype=np.uint8)
        lib().synth_mx_encode_int(_p(qi), qi.size // 32, _p(codes), _p(scales))
        return codes, scales

    def w(self, t0: int = 0, nt: int | None = None) -> np.ndarray:
        nt = self.T - t0 if nt is None else nt
        out = np.empty((nt, H_IDX), dtype=np.float32)
        (lib().synth_w_signed if self.signed_w else lib().synth_w)(self.seed, t0, nt, _p(out))
        return out

    def k_int(self, b: int, s0: int = 0, s1: int | None = None) -> np.ndarray:
        s1 = int(self.seq_lens[b]) if s1 is None else s1
        out = np.empty((s1 - s0, D_IDX), dtype=np.int8)
        lib().synth_idxk_int(self.seed, b, s0, s1 - s0, _p(out))
        return out

    def k_rows(self, b: int, s0: int = 0, s1: int | None = None):
        """Logical key rows of request b: bf16 (uint16 [n,128], None), fp8
        (uint8 [n,128], f32 [n]) or mxfp8 (uint8 [n,128], uint8 E8M0 [n,4])."""
        s1 = int(self.seq_lens[b]) if s1 is None else s1
        n = s1 - s0
        if self.idx_fmt == "bf16":
            out = np.empty((n, D_IDX), dtype=np.uint16)
            lib().synth_idxk_rows(self.seed, 0, b, s0, n, _p(out), None)
            return out, None
        out = np.empty((n, D_IDX), dtype=np.uint8)
        sc = np.empty((n,), dtype=np.float32) if self.idx_fmt == "fp8" else np.empty((n, 4), dtype=np.uint8)
        lib().synth_idxk_rows(self.seed, KFMT[self.idx_fmt], b, s0, n, _p(out), _p(sc))
        return out, sc

    def k_pool(self):
        """Paged key pool: bf16 uint16 [NP,64,128] (scales None), fp8 uint8
        [NP,64,128] + f32 [NP,64], or mxfp8 uint8 [NP,64,128] + E8M0 [NP,64,4]."""
        NP = self.num_pages
        bt = np.ascontiguousarray(self.block_table())
        if self.idx_fmt == "bf16":
            pool = np.zeros((NP, PAGE, D_IDX), dtype=np.uint16)
            sc = None
        else:
            pool = np.zeros((NP, PAGE, D_IDX), dtype=np.uint8)
            sc = np.zeros((NP, PAGE), dtype=np.float32) if self.idx_fmt == "fp8" else \
                np.full((NP, PAGE, 4), 127, dtype=np.uint8)
        lib().synth_fill_idxk_pool(self.seed, KFMT[self.idx_fmt], self.B, _p(self.seq_lens),
                                   self.max_pages, _p(bt), _p(pool), _p(sc))
        return pool, sc

    # ---- attention inputs ----
    def mla_q(self, t0: int = 0, nt: int | None = None) -> np.ndarray:
        nt = self.T - t0 if nt is None else nt
        out = np.empty((nt, self.H, D_LAT), dtype=np.uint16)
        lib().synth_mlaq_bf16(self.seed, self.H, t0, nt, _p(out))
        return out

    def latent_rows(self, b: int, s0: int = 0, s1: int | None = None):
        s1 = int(self.seq_lens[b]) if s1 is None else s1
        n = s1 - s0
        if self.kv_fmt == "bf16":
            out = np.empty((n, D_LAT), dtype=np.uint16)
            lib().synth_latent_rows(self.seed, 0, 1, b, s0, n, _p(out), None)
            return out, None
        out = np.empty((n, LAT_ROW_BYTES[self.kv_fmt]), dtype=np.uint8)
        sc = np.empty((n, self.kv_groups), dtype=np.float32)
        lib().synth_latent_rows(self.seed, VFMT[self.kv_fmt], self.kv_groups, b, s0, n, _p(out), _p(sc))
        return out, sc

    def latent_pool(self):
        NP = self.num_pages
        bt = np.ascontiguousarray(self.block_table())
        if self.kv_fmt == "bf16":
            pool = np.zeros((NP, PAGE, D_LAT), dtype=np.uint16)
            sc = None
        else:
            pool = np.zeros((NP, PAGE, LAT_ROW_BYTES[self.kv_fmt]), dtype=np.uint8)
            sc = np.ones((NP, PAGE, self.kv_groups), dtype=np.float32)
        lib().synth_fill_latent_pool(self.seed, VFMT[self.kv_fmt], self.kv_groups, self.B,
                                     _p(self.seq_lens), self.max_pages, _p(bt), _p(pool), _p(sc))
        return pool, sc


def workload(name: str) -> Case:
    """The five workloads of the hot path, by name.

    decode_b1_ctx2k      batch 1, context 2048, top-K 256, 16 MLA heads, bf16
    decode_b32_ctx32k    batch 32, context 32768, top-K 2048, 128 heads, bf16
    decode_b64_var_fp8   batch 64, context U[4096,131072], FP8 caches (per-token latent scale)
    prefill_4k_on_64k    4096 causal queries appended to 65536 cached, top-K 2048, bf16
    decode_b128_ctx128k_mtp2  batch 128, context 131072, 2 query tokens, FP8 caches (tile-128 latent)

    and one variant: decode_b64_var_mxfp8 = decode_b64_var_fp8 with MXFP8 indexer
    keys (one E8M0 scale per 32 elements instead of one f32 per row).
    """
    if name == "decode_b1_ctx2k":
        return Case(seed=1001, B=1, n_q=1, seq_lens=[2048], top_k=256, H=16)
    if name == "decode_b32_ctx32k":
        return Case(seed=1002, B=32, n_q=1, seq_lens=[32768] * 32, top_k=2048, H=128)
    if name in ("decode_b64_var_fp8", "decode_b64_var_mxfp8"):
        rng = np.random.default_rng(1003)
        lens = rng.integers(4096, 131072 + 1, size=64)
        return Case(seed=1003, B=64, n_q=1, seq_lens=lens, top_k=2048, H=128,
                    idx_fmt="fp8" if name == "decode_b64_var_fp8" else "mxfp8", kv_fmt="fp8", kv_groups=1)
    if name == "prefill_4k_on_64k":
        return Case(seed=1004, B=1, n_q=4096, seq_lens=[65536 + 4096], top_k=2048, H=128)
    if name == "decode_b128_ctx128k_mtp2":
        return Case(seed=1005, B=128, n_q=2, seq_lens=[131072] * 128, top_k=2048, H=128, idx_fmt="fp8",
                    kv_fmt="fp8", kv_groups=5)
    raise KeyError(name)


WORKLOADS = ["decode_b1_ctx2k", "decode_b32_ctx32k", "decode_b64_var_fp8", "prefill_4k_on_64k",
             "decode_b128_ctx128k_mtp2"]
