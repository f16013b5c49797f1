"""Pins of the CPU oracle against facts fixed outside the oracle itself:
library decoders of the storage formats, exact integer arithmetic, brute force,
closed forms and textbook dense attention.  CPU only."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats
def test_e4m3_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2  # S.1111.111
    assert (got[~nan] == ref[~nan]).all()
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e8m0_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert (got[:255] == ref[:255]).all()


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16(b) for b in bits])
    assert (got == ref).all()


# ---------------------------------------------------------------- generator
def test_generator_bounds_and_mx_exactness():
    c = synth.Case(seed=11, B=2, n_q=2, seq_lens=[300, 130], top_k=32, H=16, idx_fmt="fp8", kv_fmt="fp8",
                   kv_groups=5)
    qi = c.idx_q_int()
    assert qi.min() >= -4 and qi.max() <= 4
    codes, scales = c.idx_q()
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    sc = torch.from_numpy(scales).view(torch.float8_e8m0fnu).double().numpy()
    assert (dec * np.repeat(sc, 32, axis=2) == qi).all()
    w = c.w()
    assert (w * 32 == np.round(w * 32)).all() and w.min() >= 1 / 32 and w.max() <= 1
    k, ks = c.k_rows(0)
    kd = torch.from_numpy(k).view(torch.float8_e4m3fn).double().numpy()
    assert (kd == c.k_int(0)).all() and set(np.unique(ks)) <= {0.5, 1.0}


def test_generator_mxfp8_keys():
    c = synth.Case(seed=14, B=2, n_q=1, seq_lens=[300, 130], top_k=32, H=16, idx_fmt="mxfp8")
    k, ks = c.k_rows(1)
    assert k.shape == (130, 128) and ks.shape == (130, 4) and ks.dtype == np.uint8
    kd = torch.from_numpy(k).view(torch.float8_e4m3fn).double().numpy()
    assert (kd == c.k_int(1)).all()
    sc = torch.from_numpy(ks).view(torch.float8_e8m0fnu).double().numpy()
    assert set(np.unique(sc)) == {0.5, 1.0}  # both values occur, independently per group
    assert (ks[:, 0] != ks[:, 1]).any()
    kp, kps = c.k_pool()
    bt = c.block_table()
    for s in range(130):
        assert (kp[bt[1, s // 64], s % 64] == k[s]).all() and (kps[bt[1, s // 64], s % 64] == ks[s]).all()


def test_generator_page_scatter():
    c = synth.Case(seed=12, B=3, n_q=1, seq_lens=[200, 64, 129], top_k=8, H=16, kv_fmt="fp8", kv_groups=5)
    bt = c.block_table()
    kp, _ = c.k_pool()
    lp, ls = c.latent_pool()
    for b in range(3):
        k, _ = c.k_rows(b)
        lat, lats = c.latent_rows(b)
        for s in range(int(c.seq_lens[b])):
            pg, sl = bt[b, s // 64], s % 64
            assert (kp[pg, sl] == k[s]).all()
            assert (lp[pg, sl] == lat[s]).all() and (ls[pg, sl] == lats[s]).all()
    assert sorted(bt[bt >= 0].tolist()) == list(range(c.num_pages))


# ---------------------------------------------------------------- indexer scores
def _exact_scores_x64(q_int, w, k_int, k_scale=None, k_group_e8m0=None):
    """64 * I[s] as exact integers: w = n/32; optional per-row scale in {1/2, 1},
    or per-32-element E8M0 codes in {126, 127} (scales 1/2, 1)."""
    n = np.round(w * 32).astype(np.int64)
    k2 = 2 * k_int.astype(np.int64)  # 2 x the dequantised key, an integer
    if k_group_e8m0 is not None:
        k2 = k_int.astype(np.int64) * np.repeat(np.where(k_group_e8m0 == 127, 2, 1), 32, axis=1)
    elif k_scale is not None:
        k2 = k_int.astype(np.int64) * np.round(2 * k_scale).astype(np.int64)[:, None]
    dots2 = k2 @ q_int.astype(np.int64).T  # [L, 64], 2 q.k
    return np.maximum(dots2, 0) @ n  # 64 * sum_h w relu(q.k)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
def test_scores_equal_exact_integer_arithmetic(fmt):
    c = synth.Case(seed=21, B=1, n_q=1, seq_lens=[777], top_k=64, H=16, idx_fmt=fmt)
    q, qs = c.idx_q()
    w = c.w()
    k, ks = c.k_rows(0)
    q_fmt = "bf16" if fmt == "bf16" else "fp8"
    sc = oracle.index_scores(q[0], w[0], k, 777, q_fmt=q_fmt, q_scales=None if qs is None else qs[0], k_fmt=fmt,
                             k_scales=ks)
    exact = _exact_scores_x64(c.idx_q_int()[0], w[0], c.k_int(0), ks if fmt == "fp8" else None,
                              ks if fmt == "mxfp8" else None)
    assert (sc.astype(np.float64) * 64 == exact.astype(np.float64)).all()
    assert exact.max() < 2 ** 24 * 2  # the fp32 sum is exact


def test_scores_visibility_prefix():
    c = synth.workload("decode_b1_ctx2k")
    q, _ = c.idx_q()
    k, _ = c.k_rows(0)
    full = oracle.index_scores(q[0], c.w()[0], k, 2048)
    part = oracle.index_scores(q[0], c.w()[0], k, 1000)
    assert (full[:1000] == part).all()


def test_golden_closed_form():
    lines = [l for l in open(os.path.join(GOLDEN, "indexer_closed_form.txt")) if not l.startswith("#")]
    scores = np.array([float(x) for x in lines[0].split()])
    top4 = [int(x) for x in lines[1].split()]
    top7 = [int(x) for x in lines[2].split()]
    q = np.zeros((64, 128), dtype=np.float32)
    q[0, 0], q[0, 1], q[5, 0] = 1, 2, -1
    w = np.ones(64, dtype=np.float32)
    w[0], w[5] = 0.5, 0.25
    k = np.zeros((8, 128), dtype=np.float32)
    k[:, 0] = np.arange(8) - 3
    k[:, 1] = 1
    to_bf16 = lambda a: torch.from_numpy(a).bfloat16().view(torch.int16).numpy().view(np.uint16)
    sc = oracle.index_scores(to_bf16(q), w, to_bf16(k), 8)
    assert (sc == scores).all()
    assert oracle.topk(sc, 4)[0].tolist() == top4
    assert oracle.topk(sc, 7)[0].tolist() == top7


# ---------------------------------------------------------------- top-k
def test_topk_matches_stable_argsort():
    c = synth.workload("decode_b1_ctx2k")
    q, _ = c.idx_q()
    k, _ = c.k_rows(0)
    sc = oracle.index_scores(q[0], c.w()[0], k, 2048)
    idx, n = oracle.topk(sc, 256)
    ref = np.argsort(-sc.astype(np.float64), kind="stable")[:256]
    assert n == 256 and (idx == ref).all()


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(30):
        L = int(rng.integers(1, 65))
        K = int(rng.integers(1, 70))
        q = rng.integers(-1, 2, size=(64, 128)).astype(np.float32)
        k = rng.integers(-1, 2, size=(L, 128)).astype(np.float32)
        w = (rng.integers(0, 2, size=64) + 1).astype(np.float32) / 2
        to_bf16 = lambda a: torch.from_numpy(a).bfloat16().view(torch.int16).numpy().view(np.uint16)
        sc = oracle.index_scores(to_bf16(q), w, to_bf16(k), L)
        idx, n = oracle.topk(sc, K)
        assert n == min(K, L)
        assert (idx[n:] == -1).all()
        sel = set(idx[:n].tolist())
        assert len(sel) == n
        for i in sel:
            for j in range(L):
                if j in sel:
                    continue
                assert sc[i] > sc[j] or (sc[i] == sc[j] and i < j)


def test_topk_closed_forms():
    # all scores equal -> the K lowest positions
    idx, n = oracle.topk(np.zeros(100, np.float32), 10)
    assert idx.tolist() == list(range(10))
    # strictly increasing -> the last K positions, highest first
    idx, n = oracle.topk(np.arange(100, dtype=np.float32), 10)
    assert idx.tolist() == list(range(99, 89, -1))
    # K >= visible -> everything, padded with -1
    idx, n = oracle.topk(np.array([3, 1, 2], np.float32), 5)
    assert n == 3 and idx.tolist() == [0, 2, 1, -1, -1]
    # negative scores are ordered too; -0.0 and +0.0 tie
    idx, _ = oracle.topk(np.array([-1.0, -0.0, 0.0, -2.0], np.float32), 4)
    assert idx.tolist() == [1, 2, 0, 3]


def test_indexer_zero_query_selects_lowest_positions():
    q = np.zeros((64, 128), np.uint16)
    k = np.full((50, 128), 0x3F80, np.uint16)  # 1.0
    sc = oracle.index_scores(q, np.ones(64, np.float32), k, 50)
    assert (sc == 0).all()
    assert oracle.topk(sc, 7)[0].tolist() == list(range(7))


# ---------------------------------------------------------------- attention
def _dense_attention(qd, cd, scale):
    """Textbook softmax attention over all rows, float64."""
    logits = scale * (qd @ cd.T)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ cd[:, :512], (m[:, 0] + np.log(e.sum(axis=1)))


def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def _decode_latent(c, cs):
    d = torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    G = cs.shape[1]
    if G == 1:
        return d * cs.astype(np.float64)
    tile = np.minimum(np.arange(576) // 128, 4)
    return d * cs.astype(np.float64)[:, tile]


def _decode_latent_rope_bf16(c, cs):
    """640-byte rows: 512 E4M3 codes scaled per row (G=1) or per 128-tile (G=4), 64 bf16 rope."""
    lat = torch.from_numpy(np.ascontiguousarray(c[:, :512])).view(torch.float8_e4m3fn).double().numpy()
    tile = np.arange(512) // 128 if cs.shape[1] == 4 else np.zeros(512, int)
    rope = _bf16_to_f64(np.ascontiguousarray(c[:, 512:]).view(np.uint16))
    return np.concatenate([lat * cs.astype(np.float64)[:, tile], rope], axis=1)


@pytest.mark.parametrize("kv", [("bf16", 1), ("fp8", 1), ("fp8", 5), ("fp8r", 1), ("fp8r", 4)])
def test_sparse_with_all_positions_equals_dense(kv):
    fmt, G = kv
    c = synth.Case(seed=31, B=1, n_q=1, seq_lens=[300], top_k=512, H=16, kv_fmt=fmt, kv_groups=G)
    lat, lats = c.latent_rows(0)
    q = c.mla_q()[0]
    rng = np.random.default_rng(1)
    idx = np.concatenate([rng.permutation(300), -np.ones(212, int)]).astype(np.int32)
    out, lse, p = oracle.sparse_attn(q, lat, idx, c.sm_scale, c_fmt=fmt, c_scales=lats, want_p=True)
    cd = (_bf16_to_f64(lat) if fmt == "bf16" else
          _decode_latent(lat, lats) if fmt == "fp8" else _decode_latent_rope_bf16(lat, lats))
    ref_o, ref_lse = _dense_attention(_bf16_to_f64(q), cd, c.sm_scale)
    assert np.abs(out - ref_o).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-12
    assert (p[:, 300:] == 0).all()


def test_generator_rope_bf16_latent_rows():
    """fp8r rows: the rope is the bf16 format's rope, byte for byte; the latent
    codes and scales are the fp8 format's over the first 512 elements (G=1:
    one scale over the 512; G=4: per 128-tile, as fp8 with G=5 for those tiles)."""
    kw = dict(seed=33, B=1, n_q=1, seq_lens=[130], top_k=8, H=4)
    bf, _ = synth.Case(**kw).latent_rows(0)
    r1, s1 = synth.Case(kv_fmt="fp8r", kv_groups=1, **kw).latent_rows(0)
    r4, s4 = synth.Case(kv_fmt="fp8r", kv_groups=4, **kw).latent_rows(0)
    f5, t5 = synth.Case(kv_fmt="fp8", kv_groups=5, **kw).latent_rows(0)
    assert r1.shape == (130, 640) and s1.shape == (130, 1) and s4.shape == (130, 4)
    for r in (r1, r4):
        assert (np.ascontiguousarray(r[:, 512:]).view(np.uint16) == bf[:, 512:]).all()
    assert (r4[:, :512] == f5[:, :512]).all() and (s4 == t5[:, :4]).all()
    amax = np.abs(_bf16_to_f64(bf[:, :512])).max(axis=1)  # the generator quantises the unrounded values:
    assert np.all(np.abs(s1[:, 0] * 448 / amax - 1) < 1e-2)  # scale = amax / 448 up to the bf16 rounding


def test_attention_special_cases():
    c = synth.Case(seed=32, B=1, n_q=1, seq_lens=[64], top_k=8, H=4)
    lat, _ = c.latent_rows(0)
    q = c.mla_q()[0]
    cd = _bf16_to_f64(lat)
    # a single valid index -> that row, lse = its logit
    idx = np.array([-1, 17, -1, -1], np.int32)
    out, lse = oracle.sparse_attn(q, lat, idx, 0.1)
    assert np.abs(out - cd[17, :512]).max() < 1e-15
    assert np.abs(lse - 0.1 * _bf16_to_f64(q) @ cd[17]).max() < 1e-12
    # q = 0 -> mean of the selected rows, lse = log n
    idx = np.array([3, 9, 40, 41, 63], np.int32)
    out, lse = oracle.sparse_attn(np.zeros_like(q), lat, idx, 0.1)
    assert np.abs(out - cd[idx, :512].mean(axis=0)).max() < 1e-12
    assert np.abs(lse - np.log(5)).max() < 1e-12
    # identical rows -> that row
    lat2 = np.repeat(lat[5:6], 64, axis=0)
    out, _ = oracle.sparse_attn(q, lat2, idx, 0.1)
    assert np.abs(out - cd[5, :512]).max() < 1e-12
    # order of idx does not matter
    out1, lse1 = oracle.sparse_attn(q, lat, idx, 0.1)
    out2, lse2 = oracle.sparse_attn(q, lat, idx[::-1].copy(), 0.1)
    assert np.abs(out1 - out2).max() < 1e-12 and np.abs(lse1 - lse2).max() < 1e-12
    # nothing selected -> zeros and -inf
    out, lse = oracle.sparse_attn(q, lat, -np.ones(4, np.int32), 0.1)
    assert (out == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------- quantisers (cache append)
def _all_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = np.array([oracle.e4m3(int(c)) for c in codes])
    ok = ~np.isnan(vals)
    return codes[ok], vals[ok]


def test_encode_e4m3_matches_torch_rounding():
    """Every finite code round-trips; every midpoint between neighbouring
    magnitudes and a spread of random values encode as torch's float8 cast
    (round to nearest even) does."""
    codes, vals = _all_e4m3_values()
    for c, v in zip(codes, vals):
        assert oracle.encode_e4m3(v) == c  # (code 0x80 decodes to -0.0 and encodes back to 0x80)
    mags = np.unique(np.abs(vals))
    mids = (mags[:-1] + mags[1:]) / 2
    rng = np.random.default_rng(5)
    probe = np.concatenate([mids, -mids, rng.uniform(-448, 448, 4000), rng.normal(0, 0.05, 2000),
                            mags * (1 + 2.0 ** -12), mags * (1 - 2.0 ** -12)]).astype(np.float32)
    probe = probe[np.abs(probe) <= 448]
    want = torch.from_numpy(probe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.encode_e4m3(float(v)) for v in probe], dtype=np.uint8)
    assert (got == want).all(), probe[got != want][:5]


def test_encode_e4m3_saturates():
    for v in [448.0, 449.0, 464.0, 1e4, 3.4e38]:
        assert oracle.encode_e4m3(v) == 0x7E and oracle.encode_e4m3(-v) == 0xFE


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).bfloat16().view(torch.int16).numpy().view(np.uint16)


def test_quant_mxfp8_closed_forms():
    # integers in [-4, 4] with amax 4: X = 2^(2 - 8) = 2^-6, codes are exact
    rng = np.random.default_rng(6)
    ints = rng.integers(-4, 5, size=(3, 128)).astype(np.float32)
    ints[:, 0] = 4.0
    ints[2, 32:64] = 0.0  # an all-zero group
    codes, scales = oracle.quant_mxfp8(_bf16_bits(ints))
    assert scales.shape == (3, 4)
    assert (scales[:, 0] == 127 - 6).all()
    assert scales[2, 1] == 127 and (codes[2, 32:64] == 0).all()
    deq = np.array([[oracle.e4m3(int(c)) for c in row] for row in codes]) * \
        np.repeat(np.array([[oracle.e8m0(int(s)) for s in row] for row in scales]), 32, axis=1)
    assert (deq == ints).all()
    # amax = 1.9 * 8: X = 2^(3 - 8), the largest element needs 486.4 > 448 and saturates
    g = np.full((1, 32), 1.0, np.float32)
    g[0, 5] = 15.2
    codes, scales = oracle.quant_mxfp8(_bf16_bits(g))
    assert scales[0, 0] == 127 - 5 and codes[0, 5] == 0x7E
    assert codes[0, 0] == oracle.encode_e4m3(32.0)


def test_quant_mxfp8_is_nearest_code():
    """Brute force: each code is a nearest E4M3 value to x / X (ties to even),
    and X follows the group's amax."""
    _, vals = _all_e4m3_values()
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((4, 64)) * np.exp(rng.uniform(-6, 6, (4, 1)))).astype(np.float32)
    xb = _bf16_bits(x)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    codes, scales = oracle.quant_mxfp8(xb)
    for r in range(4):
        for g in range(2):
            grp = xf[r, 32 * g:32 * g + 32]
            X = oracle.e8m0(int(scales[r, g]))
            assert X == 2.0 ** (np.floor(np.log2(np.abs(grp).max())) - 8)
            for i in range(32):
                t = min(abs(grp[i] / X), 448.0)
                best = np.abs(np.abs(vals) - t).min()
                got = abs(oracle.e4m3(int(codes[r, 32 * g + i])))
                assert abs(got - t) == best


def test_quant_fp8_rows_per_token_and_per_tile():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 576)).astype(np.float32)
    x[3] = 0.0
    xb = _bf16_bits(x)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    _, vals = _all_e4m3_values()
    for block, nb in [(576, 1), (128, 5)]:
        codes, scales = oracle.quant_fp8_rows(xb, block)
        assert scales.shape == (5, nb)
        assert (scales[3] == 1.0).all() and (codes[3] == 0).all()
        for r in [0, 1, 4]:
            for b in range(nb):
                lo, hi = b * block, min(576, b * block + block)
                seg = xf[r, lo:hi]
                amax = np.float32(np.abs(seg).max())
                assert scales[r, b] == np.float32(amax / np.float32(448.0))
                # the block's largest magnitude lands on the largest code
                j = int(np.abs(seg).argmax())
                assert codes[r, lo + j] & 0x7F == 0x7E
                q = (seg / scales[r, b]).astype(np.float32)
                for i in range(0, hi - lo, 7):
                    got = oracle.e4m3(int(codes[r, lo + i]))
                    assert abs(abs(got) - min(abs(q[i]), 448.0)) == np.abs(np.abs(vals) - min(abs(q[i]), 448.0)).min()
                    assert got == 0 or np.sign(got) == np.sign(q[i])


def test_quant_mxfp8_e8m0_clamp_on_tiny_groups():
    """Groups whose largest magnitude is below 2^-119 (bf16 subnormals and the
    smallest normals): floor(log2 amax) - 8 falls below E8M0's least exponent
    -127 (OCP Microscaling v1.0: E8M0 spans 2^-127 .. 2^127), so the scale
    holds at code 0 and the elements are x * 2^127 rounded to E4M3.  Reference
    codes come from torch's float8 cast of the exact products."""
    rng = np.random.default_rng(11)
    groups = []
    # (bf16 bit patterns of one group, expected E8M0 code)
    groups.append((np.full(32, 0x0001, np.uint16), 0))                     # every element 2^-133
    sub = rng.integers(1, 0x80, 32).astype(np.uint16) | (rng.integers(0, 2, 32).astype(np.uint16) << 15)
    groups.append((sub, 0))                                                # mixed subnormals, both signs
    for e_field, code in [(7, 0), (8, 0), (9, 1), (10, 2)]:
        # amax = 2^(e_field - 127) (a normal bf16); floor(log2 amax) - 8 + 127 = e_field - 8
        g = rng.integers(0, 0x80, 32).astype(np.uint16)                    # subnormal fill
        g[int(rng.integers(0, 32))] = np.uint16(e_field << 7)
        groups.append((g, code))
        assert code == max(e_field - 8, 0)
    x = np.stack([g for g, _ in groups])
    codes, scales = oracle.quant_mxfp8(x)
    assert list(scales[:, 0]) == [c for _, c in groups]
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    X = np.array([2.0 ** (c - 127) for _, c in groups])[:, None]
    ref = torch.from_numpy(xf / X).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (codes == ref).all()
    assert (codes[0] == 0x08).all()  # 2^-133 * 2^127 = 2^-6, E4M3's least normal
