"""CPU model of the decode indexer's cross-chunk brackets (li_decode_kernel:
chunk quotas, the per-chunk histogram interval, exchange 1).

The kernel splits a request's positions into chunks; chunk c takes a quota
R_c (K <= sum R_c < K + n) and publishes a key interval [lo_c, hi_c) that
holds its R_c-th largest key.  Then lo = min lo_c and hi = max hi_c bracket
the request's K-th largest key, every key >= hi is selected, and the "band"
[lo, hi) is exchanged and selected exactly.  This model reproduces those
integer steps on the host so that band sizes can be studied without a GPU.

What it shows: when scores rise with position (a recency trend), the chunks'
brackets sit at very different keys and the band holds most positions of the
request -- beyond 65,535 entries at 131,072 positions, so band counts and
offsets must be carried in 32 bits.
"""
import numpy as np
import pytest

import oracle
import synth


def score_key(x: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 image of fp32 scores (-0 folded into +0)."""
    x = np.asarray(x, dtype=np.float32) + np.float32(0.0)
    u = x.view(np.uint32)
    return np.where(u & np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def quota(c: int, vis: int, K: int, chunk: int) -> int:
    """R_c: even split over whole chunks; a partial last chunk takes its share
    of K in proportion to its visible positions."""
    nv = (vis + chunk - 1) // chunk
    v_last = vis - (nv - 1) * chunk
    R = (K + nv - 1) // nv
    if nv > 1 and v_last < chunk:
        r_tail = K * v_last // vis
        R = r_tail if c == nv - 1 else (K - r_tail + nv - 2) // (nv - 1)
    return R


def chunk_interval(keys: np.ndarray, R: int, bins: int = 4096):
    """[lo_c, hi_c) of one chunk's valid keys: the histogram bin (below the
    common prefix of its min and max key) holding its R-th largest key."""
    if len(keys) == 0:
        return 0xFFFFFFFF, 0
    mn, mx = int(keys.min()), int(keys.max())
    if R == 0:
        return 0xFFFFFFFF, min(mx, 0xFFFFFFFE) + 1
    if mn == mx:
        return mn, mn + 1
    top = (mn ^ mx).bit_length() - 1
    shift = max(0, top - (bins.bit_length() - 2))
    base = mn >> shift
    h = np.bincount((keys.astype(np.int64) >> shift) - base, minlength=bins)
    above = np.cumsum(h[::-1])  # keys in bins >= bins-1-i
    i = int(np.searchsorted(above, R))  # first descending bin where the count reaches R
    b = bins - 1 - i + base
    return b << shift, min((b + 1) << shift, 0xFFFFFFFF)


def bracket(scores: np.ndarray, K: int, chunk: int):
    """(lo, hi, keys >= hi, band size) of one token seeing every position."""
    keys = score_key(scores)
    vis = len(keys)
    n = (vis + chunk - 1) // chunk
    ivs = [chunk_interval(keys[c * chunk:(c + 1) * chunk], quota(c, vis, K, chunk)) for c in range(n)]
    lo = max(min(i[0] for i in ivs), 1)
    hi = max(i[1] for i in ivs)
    above = int((keys >= hi).sum())
    band = int(((keys >= lo) & (keys < hi)).sum())
    return lo, hi, above, band


def trend_scores(L: int, noise: int = 0, seed: int = 0) -> np.ndarray:
    """Scores of q = 1, w = 1/2 (64 heads) against key rows with ones in their
    first m(s) = 128 s / L entries (+ optional integer noise): 32 * m(s) + ..."""
    m = (np.arange(L, dtype=np.int64) * 128) // L
    s = 32.0 * m
    if noise:
        s = s + 32.0 * np.random.default_rng(seed).integers(-noise, noise + 1, size=L)
    return np.maximum(s, 0).astype(np.float32)


@pytest.mark.parametrize("chunk", [1024, 2048, 4096])
def test_bracket_holds_kth_key(chunk):
    """lo <= kappa < hi on i.i.d., trend and all-equal scores."""
    K = 2048
    rng = np.random.default_rng(5)
    for sc in (rng.integers(0, 1 << 12, size=40000).astype(np.float32), trend_scores(40000, 3, 1),
               np.zeros(40000, np.float32)):
        lo, hi, above, band = bracket(sc, K, chunk)
        kappa = np.sort(score_key(sc))[::-1][K - 1]
        assert lo <= kappa < hi
        assert above < K <= above + band


@pytest.mark.parametrize("chunk", [1024, 4096])
def test_positional_trend_band_exceeds_16_bits(chunk):
    """131,072 positions whose scores rise with position: the band passes
    65,535 entries (so 16-bit band counts would wrap)."""
    L, K = 131072, 2048
    _, _, above, band = bracket(trend_scores(L), K, chunk)
    assert band > 65535
    assert above < K
    # a mild trend under noise does the same
    _, _, _, band_noisy = bracket(trend_scores(L, noise=8, seed=3), K, chunk)
    assert band_noisy > 65535


def test_all_equal_scores_band_is_every_position():
    """A zero query scores every position alike: each chunk's interval is
    [key, key + 1), and the band is the whole request."""
    L, K = 131072, 2048
    lo, hi, above, band = bracket(np.zeros(L, np.float32), K, 1024)
    assert (above, band) == (0, L)


def test_iid_generator_band_is_small():
    """On the generator's i.i.d. integer data (the benchmark's distribution)
    the band is a few per cent of the positions: it stays in LDS."""
    case = synth.Case(seed=1002, B=1, n_q=1, seq_lens=[32768], top_k=2048, H=16)
    q, _ = case.idx_q(0, 1)
    k, _ = case.k_rows(0)
    sc = oracle.index_scores(q[0], case.w(0, 1)[0], k, 32768)
    _, _, above, band = bracket(sc, 2048, 4096)
    assert above < 2048 and band <= 4096
