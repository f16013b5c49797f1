"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Top-K indices must match exactly (the inputs make every
fp32 score exact); attention outputs to 2e-2 (bf16 cache) / 5e-2 (FP8 cache)
in max relative error per (token, head), lse to 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_inputs import GpuCase, encode_indexer_int, load_indexer, rel_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp8": 5e-2, "fp8r": 5e-2}


@pytest.fixture(scope="module")
def li(gpu_ready):
    import sparse_attention_li_amd as li
    li.lib()
    return li


def _oracle_sorted(r, K):
    n = r["n"]
    ref = np.full(K, -1, dtype=np.int32)
    ref[:n] = np.sort(r["idx"][:n])
    return ref


def _check_indices(case, idx_gpu, tokens, ores):
    for t in tokens:
        ref = _oracle_sorted(ores[t], case.top_k)
        got = idx_gpu[t]
        if not (got == ref).all():
            bad = np.nonzero(got != ref)[0]
            raise AssertionError(f"token {t}: {len(bad)} index mismatches, first at {bad[0]}: "
                                 f"gpu {got[bad[:5]]} oracle {ref[bad[:5]]}")


def _check_attention(case, out, lse, tokens, ores):
    for t in tokens:
        e = rel_err(out[t].astype(np.float64), ores[t]["out"])
        assert e <= TOL[case.kv_fmt], f"token {t}: rel err {e}"
        ref_lse = ores[t]["lse"]
        fin = np.isfinite(ref_lse)
        assert (np.isfinite(lse[t]) == fin).all()
        assert np.abs(lse[t][fin] - ref_lse[fin]).max(initial=0) <= 1e-2


SMALL = {
    "b1_ctx2k": dict(seed=1001, B=1, n_q=1, seq_lens=[2048], top_k=256, H=16),
    "ragged3": dict(seed=7, B=3, n_q=1, seq_lens=[100, 1500, 3000], top_k=256, H=32),
    "short_lt_k": dict(seed=8, B=2, n_q=1, seq_lens=[37, 64], top_k=128, H=16),
    "k1": dict(seed=9, B=2, n_q=1, seq_lens=[777, 1025], top_k=1, H=16),
    "mtp2": dict(seed=10, B=3, n_q=2, seq_lens=[2, 1100, 4097], top_k=512, H=64),
    "k2048": dict(seed=11, B=1, n_q=1, seq_lens=[5000], top_k=2048, H=128),
    "fp8_g1": dict(seed=12, B=2, n_q=1, seq_lens=[1500, 2600], top_k=300, H=32, idx_fmt="fp8", kv_fmt="fp8",
                   kv_groups=1),
    "fp8_g5_mtp2": dict(seed=13, B=2, n_q=2, seq_lens=[3000, 700], top_k=256, H=128, idx_fmt="fp8",
                        kv_fmt="fp8", kv_groups=5),
    # MXFP8 indexer keys (one E8M0 scale per 32 elements), 1024-position chunks and two-token calls
    "mxk_ragged": dict(seed=22, B=3, n_q=1, seq_lens=[700, 2600, 4100], top_k=300, H=32, idx_fmt="mxfp8",
                       kv_fmt="fp8", kv_groups=1),
    "mxk_mtp2": dict(seed=23, B=2, n_q=2, seq_lens=[3000, 129], top_k=256, H=128, idx_fmt="mxfp8", kv_fmt="fp8",
                     kv_groups=5),
    # FP8 latent with the rope in bf16 (640-byte rows), scales per row or per 128-wide latent tile
    "fp8r_g1_h16": dict(seed=25, B=2, n_q=1, seq_lens=[1500, 2600], top_k=300, H=16, idx_fmt="fp8", kv_fmt="fp8r",
                        kv_groups=1),
    "fp8r_g4_mtp2": dict(seed=26, B=2, n_q=2, seq_lens=[3000, 700], top_k=256, H=128, idx_fmt="mxfp8",
                         kv_fmt="fp8r", kv_groups=4),
    # FP8 latent with 64 heads: one workgroup per token slice, both 32-head groups in it
    # FP8 rows with 128 heads: the all-heads kernel (ragged slices, several
    # tiles per split, every scale layout, bf16 rope)
    "fp8_g1_h128_ragged": dict(seed=40, B=3, n_q=1, seq_lens=[900, 2600, 4100], top_k=700, H=128, idx_fmt="fp8",
                               kv_fmt="fp8", kv_groups=1),
    "fp8r_g1_h128_ragged": dict(seed=43, B=3, n_q=1, seq_lens=[900, 2600, 4100], top_k=700, H=128, idx_fmt="fp8",
                                kv_fmt="fp8r", kv_groups=1),
    "fp8_h128_k1": dict(seed=45, B=2, n_q=1, seq_lens=[777, 1025], top_k=1, H=128, idx_fmt="fp8", kv_fmt="fp8",
                        kv_groups=5),
    "fp8r_h128_empty_mtp2": dict(seed=46, B=3, n_q=2, seq_lens=[2100, 0, 700], top_k=300, H=128, idx_fmt="fp8",
                                 kv_fmt="fp8r", kv_groups=4),
    "prefill_fp8_latent_h128": dict(seed=47, B=1, n_q=12, seq_lens=[3000], top_k=256, H=128, kv_fmt="fp8",
                                    kv_groups=5),
    "fp8_g5_h128_mtp2_tiles": dict(seed=41, B=32, n_q=2, seq_lens=[1200 + 97 * i for i in range(32)], top_k=1000,
                                   H=128, idx_fmt="fp8", kv_fmt="fp8", kv_groups=5),
    "fp8_h64_ragged": dict(seed=27, B=3, n_q=1, seq_lens=[900, 2600, 4100], top_k=520, H=64, idx_fmt="fp8",
                           kv_fmt="fp8", kv_groups=1),
    "fp8r_h64_mtp2": dict(seed=28, B=2, n_q=2, seq_lens=[2200, 333], top_k=300, H=64, idx_fmt="fp8",
                          kv_fmt="fp8r", kv_groups=4),
    # more chunks than one round of the chip: the XCD-local block layout
    "xcd_local_ragged": dict(seed=24, B=24, n_q=1, seq_lens=[49152, 20001, 33333, 40960, 47000, 25000, 36000, 44444,
                                                              30001, 49152, 21000, 38000, 41000, 27000, 45000, 32768,
                                                              48000, 23000, 35000, 42000, 29000, 46000, 39000, 31000],
                             top_k=2048, H=16),
    # FP8 keys over more chunks than one round: four-wave workgroups, two per CU
    "xcd_local_fp8": dict(seed=27, B=24, n_q=1, seq_lens=[49152, 20001, 33333, 40960, 47000, 25000, 36000, 44444,
                                                           30001, 49152, 21000, 38000, 41000, 27000, 45000, 32768,
                                                           48000, 23000, 35000, 42000, 29000, 46000, 39000, 31000],
                          top_k=2048, H=16, idx_fmt="mxfp8", kv_fmt="fp8"),
    # FP8 keys, one token, more than three workgroups per CU at 4096 positions: 8192-position chunks
    "fp8_chunk8192": dict(seed=40, B=26, n_q=1, seq_lens=[131000, 90001, 8191, 8193, 16384, 1, 0, 300, 65536, 12345,
                                                          7, 4096, 4097, 20000, 33, 50000, 8192, 100, 2, 24576, 1000,
                                                          8000, 60000, 5, 30000, 129],
                          top_k=2048, H=16, idx_fmt="fp8", kv_fmt="fp8"),
    # head weights of either sign: negative scores, ordered by their keys
    "signed_bf16": dict(seed=30, B=3, n_q=1, seq_lens=[900, 5000, 2049], top_k=512, H=32, signed_w=True),
    "signed_k_deep": dict(seed=31, B=2, n_q=1, seq_lens=[3000, 2500], top_k=2048, H=16, signed_w=True),
    "signed_fp8_mtp2": dict(seed=32, B=2, n_q=2, seq_lens=[4097, 1300], top_k=300, H=64, idx_fmt="fp8",
                            kv_fmt="fp8", kv_groups=5, signed_w=True),
    "signed_mxk": dict(seed=33, B=3, n_q=1, seq_lens=[700, 2600, 4100], top_k=1500, H=32, idx_fmt="mxfp8",
                       kv_fmt="fp8", kv_groups=1, signed_w=True),
    "signed_xcd_local_fp8": dict(seed=34, B=24, n_q=1, seq_lens=[20000 + 1237 * b for b in range(24)], top_k=2048,
                                 H=16, idx_fmt="fp8", kv_fmt="fp8", signed_w=True),
    "signed_prefill": dict(seed=35, B=1, n_q=40, seq_lens=[3000], top_k=256, H=16, signed_w=True),
    "signed_prefill_deep": dict(seed=36, B=1, n_q=12, seq_lens=[2600], top_k=2048, H=32, signed_w=True),
    "signed_prefill_compactions": dict(seed=37, B=1, n_q=12, seq_lens=[9000], top_k=512, H=64, signed_w=True),
    # requests with no cached position: the row is all -1, out 0, lse -inf
    "empty_requests": dict(seed=38, B=3, n_q=1, seq_lens=[0, 1500, 0], top_k=256, H=16),
    "empty_requests_fp8_mtp2": dict(seed=39, B=3, n_q=2, seq_lens=[2100, 0, 700], top_k=300, H=128, idx_fmt="fp8",
                                    kv_fmt="fp8", kv_groups=5),
    # prefill chunks (many causal queries per request)
    "prefill_ragged": dict(seed=19, B=1, n_q=37, seq_lens=[300], top_k=64, H=16),
    "prefill_k_gt_visible": dict(seed=20, B=2, n_q=9, seq_lens=[40, 200], top_k=128, H=32),
    "prefill_compactions": dict(seed=21, B=1, n_q=12, seq_lens=[9000], top_k=512, H=64),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases_full_path(li, name):
    case = synth.Case(**SMALL[name])
    g = GpuCase(case)
    idx = g.score_topk(li)
    out, lse = g.attend(li, idx)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    tokens = list(range(case.T))
    ores = oracle.run_tokens(case, tokens)
    _check_indices(case, idx, tokens, ores)
    _check_attention(case, out, lse, tokens, ores)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_attention_pool_beyond_4gib(li, fmt):
    # the same rows placed past 4.5 GiB of pool: 64-bit row addresses in the
    # all-heads attention kernels give identical results
    case = synth.Case(seed=42, B=2, n_q=1, seq_lens=[3000, 1700], top_k=512, H=128,
                      **({} if fmt == "bf16" else dict(idx_fmt="fp8", kv_fmt="fp8", kv_groups=5)))
    g = GpuCase(case)
    idx = g.score_topk(li)
    out, lse = g.attend(li, idx)
    torch.cuda.synchronize()
    row_bytes = 1152 if fmt == "bf16" else 576
    p0 = -(-(9 << 29) // (64 * row_bytes))  # pages before the case's own
    NP = g.kv_pool.shape[0]
    big = torch.zeros((p0 + NP,) + tuple(g.kv_pool.shape[1:]), dtype=g.kv_pool.dtype, device="cuda")
    big[p0:] = g.kv_pool
    big_sc = None
    if g.kv_scales is not None:
        big_sc = torch.ones((p0 + NP,) + tuple(g.kv_scales.shape[1:]), dtype=torch.float32, device="cuda")
        big_sc[p0:] = g.kv_scales
    out2, lse2 = li.sfa_decode(g.mla_q, big, idx, g.seq_lens, g.block_table + p0, case.sm_scale, kv_scales=big_sc)
    torch.cuda.synchronize()
    assert big.numel() * big.element_size() > (1 << 32)
    assert torch.equal(out2, out) and torch.equal(lse2, lse)
    tokens = list(range(case.T))
    ores = oracle.run_tokens(case, tokens)
    _check_attention(case, out2.float().cpu().numpy(), lse2.cpu().numpy(), tokens, ores)
    del big, big_sc
    torch.cuda.empty_cache()


def test_ties_break_to_lower_position(li):
    # q, k in {-1, 0, 1} and w in {1/2, 1}: many equal scores across chunk boundaries
    rng = np.random.default_rng(3)
    case = synth.Case(seed=14, B=2, n_q=1, seq_lens=[2500, 1300], top_k=700, H=16)
    g = GpuCase(case, attention=False)
    L = 2500
    qv = rng.integers(-1, 2, size=(2, 64, 128)).astype(np.float32)
    wv = ((rng.integers(0, 2, size=(2, 64)) + 1) / 2).astype(np.float32)
    kv = [rng.integers(-1, 2, size=(int(l), 128)).astype(np.float32) for l in case.seq_lens]
    bf = lambda a: torch.from_numpy(a).bfloat16().view(torch.int16)
    g.q = bf(qv).cuda()
    g.w = torch.from_numpy(wv).cuda()
    pool = torch.zeros((case.num_pages, 64, 128), dtype=torch.int16)
    bt = case.block_table()
    for b, kb in enumerate(kv):
        for s0 in range(0, kb.shape[0], 64):
            blk = kb[s0:s0 + 64]
            pool[bt[b, s0 // 64], :blk.shape[0]] = bf(np.ascontiguousarray(blk))
    g.k_pool = pool.cuda()
    idx = g.score_topk(li).cpu().numpy()
    for b in range(2):
        kbits = bf(kv[b]).numpy().view(np.uint16)
        sc = oracle.index_scores(bf(qv[b]).numpy().view(np.uint16), wv[b], kbits, int(case.seq_lens[b]))
        ridx, n = oracle.topk(sc, case.top_k)
        ref = np.full(case.top_k, -1, np.int32)
        ref[:n] = np.sort(ridx[:n])
        assert (idx[b] == ref).all()
        assert len(np.unique(sc)) < len(sc) // 4  # the case really is tie-heavy


def test_all_equal_scores_pick_lowest_positions(li):
    case = synth.Case(seed=15, B=1, n_q=1, seq_lens=[3000], top_k=1000, H=16)
    g = GpuCase(case, attention=False)
    g.q = torch.zeros_like(g.q)
    idx = g.score_topk(li).cpu().numpy()
    assert (idx[0] == np.arange(1000)).all()


def test_deterministic_and_workspace_left_zero(li):
    case = synth.Case(seed=16, B=4, n_q=2, seq_lens=[5000, 3000, 64, 2049], top_k=512, H=128)
    g = GpuCase(case)
    ws = torch.zeros(li.li_score_topk_workspace_size(4, 2, case.max_pages, 512), dtype=torch.uint8, device="cuda")
    a = g.score_topk(li, workspace=ws).clone()
    o1, l1 = g.attend(li, a)
    o1, l1 = o1.clone(), l1.clone()
    b = g.score_topk(li, workspace=ws)
    o2, l2 = g.attend(li, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    counters = ws[: 4 * 128].view(torch.int32).view(4, 32)[:, :2]
    assert int(counters.abs().sum()) == 0


def test_attention_all_positions_equals_dense(li):
    # K >= L: sparse attention over every position is dense softmax attention
    case = synth.Case(seed=17, B=2, n_q=1, seq_lens=[300, 250], top_k=320, H=64)
    g = GpuCase(case)
    idx = torch.full((2, 320), -1, dtype=torch.int32)
    idx[0, :300] = torch.randperm(300, generator=torch.Generator().manual_seed(0)).int()
    idx[1, :250] = torch.arange(250, dtype=torch.int32)
    out, lse = g.attend(li, idx.cuda())
    out = out.float().cpu().numpy()
    for t in range(2):
        lat, _ = case.latent_rows(t)
        cd = torch.from_numpy(lat.view(np.int16)).view(torch.bfloat16).double().numpy()
        qd = torch.from_numpy(case.mla_q(t, 1)[0].view(np.int16)).view(torch.bfloat16).double().numpy()
        logits = case.sm_scale * qd @ cd.T
        p = np.exp(logits - logits.max(1, keepdims=True))
        ref = (p / p.sum(1, keepdims=True)) @ cd[:, :512]
        assert rel_err(out[t], ref) <= 2e-2


def test_decode_b32_ctx32k_sampled(li):
    """Full-size headline workload, same launch as the benchmark; every token
    checked end to end against the oracle."""
    case = synth.workload("decode_b32_ctx32k")
    g = GpuCase(case)
    idx = g.score_topk(li)
    out, lse = g.attend(li, idx)
    torch.cuda.synchronize()
    tokens = list(range(case.T))
    ores = oracle.run_tokens(case, tokens)
    idx = idx.cpu().numpy()
    _check_indices(case, idx, tokens, ores)
    _check_attention(case, out.float().cpu().numpy(), lse.cpu().numpy(), tokens, ores)


def test_repeated_calls_identical_many_chunks(li):
    """Regression test for cross-workgroup publication: candidates written by
    workgroups on other XCDs must be visible to the one that runs the final
    select.  Many requests x many chunks, repeated; every call must equal the
    oracle-checked first call."""
    case = synth.Case(seed=18, B=24, n_q=1, seq_lens=[9000 + 731 * b for b in range(24)], top_k=1, H=16)
    g = GpuCase(case, attention=False)
    first = g.score_topk(li).clone()
    for _ in range(20):
        assert torch.equal(g.score_topk(li), first)
    case2 = synth.Case(seed=18, B=24, n_q=1, seq_lens=case.seq_lens, top_k=1, H=16)
    ores = oracle.run_tokens(case2, [0, 23], with_attn=False)
    fi = first.cpu().numpy()
    _check_indices(case, fi, [0, 23], ores)


@pytest.mark.parametrize("spin", [0, 3])
@pytest.mark.parametrize("name", ["ragged3", "mtp2", "k2048", "fp8_g5_mtp2", "xcd_local_fp8"])
def test_exchange_fallbacks_stay_exact(li, name, spin):
    """The decode indexer's cross-workgroup exchanges with (almost) no patience:
    most waits time out, so workgroups publish every key, give up their share
    and leave the whole request to the last one to arrive.  Indices must still
    equal the oracle's, and the exchange state must be left reset."""
    li.li_set_exchange_patience(spin)
    try:
        _fallback_case(li, name)
    finally:
        li.li_set_exchange_patience(-1)


def _fallback_case(li, name):
    case = synth.Case(**SMALL[name])
    g = GpuCase(case, attention=False)
    ws = torch.zeros(li.li_score_topk_workspace_size(case.B, case.n_q, case.max_pages, case.top_k),
                     dtype=torch.uint8, device="cuda")
    for _ in range(3):
        idx = g.score_topk(li, workspace=ws)
        torch.cuda.synchronize()
        tokens = list(range(case.T))
        _check_indices(case, idx.cpu().numpy(), tokens, oracle.run_tokens(case, tokens, with_attn=False))
    # arrivals, departures and give-up state back at zero (word 4 is the epoch)
    assert int(ws[: case.B * 128].view(torch.int32).view(case.B, 32)[:, :3].abs().sum()) == 0


def test_positional_trend_band_beyond_lds(li):
    """Scores that grow with position (the top K all sit in the last chunks):
    the band between the chunks' bracketing keys then holds most positions,
    more than the select keeps in LDS, and the exact select runs over the
    published lists in global memory."""
    L, K = 6000, 1000
    case = synth.Case(seed=23, B=1, n_q=1, seq_lens=[L], top_k=K, H=16)
    g = GpuCase(case, attention=False)
    qv = np.ones((1, 64, 128), np.float32)
    wv = np.full((1, 64), 0.5, np.float32)
    m = (np.arange(L) * 128) // L  # ones in the first m(s) key entries
    kv = (np.arange(128)[None, :] < m[:, None]).astype(np.float32)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).bfloat16().view(torch.int16)
    g.q = bf(qv).cuda()
    g.w = torch.from_numpy(wv).cuda()
    pool = torch.zeros((case.num_pages, 64, 128), dtype=torch.int16)
    bt = case.block_table()
    for s0 in range(0, L, 64):
        blk = kv[s0:s0 + 64]
        pool[bt[0, s0 // 64], :blk.shape[0]] = bf(blk)
    g.k_pool = pool.cuda()
    idx = g.score_topk(li).cpu().numpy()
    sc = oracle.index_scores(bf(qv[0]).numpy().view(np.uint16), wv[0], bf(kv).numpy().view(np.uint16), L)
    ridx, n = oracle.topk(sc, K)
    assert (idx[0] == np.sort(ridx[:n])).all()
    assert idx[0].min() > L // 2  # the trend really puts the selection in the last chunks


def _trend_keys(L: int, rising: bool, seed: int) -> np.ndarray:
    """Key rows whose score against an all-ones query grows (or falls) with
    position: ones in the first m(s) = 128 s / L entries plus sparse +-1
    noise, all integers in [-4, 4]."""
    rng = np.random.default_rng(seed)
    s = np.arange(L) if rising else np.arange(L)[::-1]
    m = (s * 128) // L
    k = (np.arange(128)[None, :] < m[:, None]).astype(np.int8)
    k += (rng.integers(-1, 2, size=(L, 128)) * (rng.random((L, 128)) < 0.05)).astype(np.int8)
    return k


@pytest.mark.parametrize("kind", ["trend", "zero_query"])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_band_beyond_16_bits(li, fmt, kind):
    """131,072 positions per request whose scores rise (request 0) or fall
    (request 1) with position, or a zero query (every score equal): the band
    between the chunks' bracketing keys holds more than 65,535 entries
    (modelled on the CPU in test_band_model.py), so its counts and offsets
    must be 32-bit.  Indices must equal the oracle's."""
    L, K = 131072, 2048
    case = synth.Case(seed=40, B=2, n_q=1, seq_lens=[L, L], top_k=K, H=16, idx_fmt=fmt,
                      kv_fmt="fp8" if fmt != "bf16" else "bf16")
    g = GpuCase(case, attention=False)
    q_int = np.zeros((2, 64, 128), np.int8) if kind == "zero_query" else np.ones((2, 64, 128), np.int8)
    w = np.full((2, 64), 0.5, np.float32)
    k_int = [_trend_keys(L, True, 1), _trend_keys(L, False, 2)]
    q, qs, ks = encode_indexer_int(case, q_int, k_int)
    load_indexer(g, q, qs, w, ks)
    idx = g.score_topk(li).cpu().numpy()
    q_fmt = "bf16" if fmt == "bf16" else "fp8"
    for b in range(2):
        if kind == "zero_query":
            assert (idx[b] == np.arange(K)).all()
            continue
        sc = oracle.index_scores(q[b], w[b], ks[b][0], L, q_fmt=q_fmt, q_scales=None if qs is None else qs[b],
                                 k_fmt=fmt, k_scales=ks[b][1])
        ridx, n = oracle.topk(sc, K)
        assert (idx[b] == np.sort(ridx[:n])).all(), f"request {b}"
        # the trend really spreads the chunk brackets (far beyond the first / last chunks)
        assert (idx[b].min() > L // 2) if b == 0 else (idx[b].max() < L // 2)


@pytest.mark.parametrize("spin", [0, 3])
def test_band_beyond_16_bits_with_fallbacks(li, spin):
    """The rising-trend request of 131,072 positions with (almost) no patience
    in the exchanges: timed-out workgroups publish every key as band and the
    last to arrive writes the whole request from the lists; still exact."""
    L, K = 131072, 2048
    case = synth.Case(seed=42, B=1, n_q=1, seq_lens=[L], top_k=K, H=16)
    g = GpuCase(case, attention=False)
    q, qs, ks = encode_indexer_int(case, np.ones((1, 64, 128), np.int8), [_trend_keys(L, True, 3)])
    w = np.full((1, 64), 0.5, np.float32)
    load_indexer(g, q, qs, w, ks)
    sc = oracle.index_scores(q[0], w[0], ks[0][0], L)
    ridx, n = oracle.topk(sc, K)
    li.li_set_exchange_patience(spin)
    try:
        for _ in range(2):
            idx = g.score_topk(li).cpu().numpy()
            assert (idx[0] == np.sort(ridx[:n])).all()
    finally:
        li.li_set_exchange_patience(-1)


@pytest.mark.parametrize("kind", ["trend", "zero_query"])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_whole_request_writer_xcd_local(li, fmt, kind):
    """One-token grids of several rounds (24 requests x 12 chunks of 4096
    positions, the XCD-local layout) leave each request to the last chunk to
    publish, which writes the whole index row by merging the keys above the
    band with the band entries it selects.  Scores that rise (even requests)
    or fall (odd ones) with position make the band wider than its LDS copy
    (the selection reads the lists in memory); a zero query makes every score
    equal, so the K lowest positions must be written (ties in position order
    across chunks).  Indices must equal the oracle's."""
    B, L, K = 24, 49152, 1500
    case = synth.Case(seed=43, B=B, n_q=1, seq_lens=[L] * B, top_k=K, H=16, idx_fmt=fmt,
                      kv_fmt="fp8" if fmt != "bf16" else "bf16")
    g = GpuCase(case, attention=False)
    q_int = np.zeros((B, 64, 128), np.int8) if kind == "zero_query" else np.ones((B, 64, 128), np.int8)
    w = np.full((B, 64), 0.5, np.float32)
    k_int = [_trend_keys(L, b % 2 == 0, 100 + b) for b in range(B)]
    q, qs, ks = encode_indexer_int(case, q_int, k_int)
    load_indexer(g, q, qs, w, ks)
    q_fmt = "bf16" if fmt == "bf16" else "fp8"
    refs = []
    for b in range(B):
        if kind == "zero_query":
            refs.append(np.arange(K))
            continue
        sc = oracle.index_scores(q[b], w[b], ks[b][0], L, q_fmt=q_fmt, q_scales=None if qs is None else qs[b],
                                 k_fmt=fmt, k_scales=ks[b][1])
        ridx, n = oracle.topk(sc, K)
        refs.append(np.sort(ridx[:n]))
    for _ in range(2):  # the second call runs on the state the first left
        idx = g.score_topk(li).cpu().numpy()
        for b in range(B):
            assert (idx[b] == refs[b]).all(), f"request {b}"


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_two_token_call_equals_one_token_calls(li, fmt):
    """Token j of a two-token (draft-and-verify) call sees L - 1 + j positions:
    it must select what a one-token call over the same cache with the length
    L - 1 + j selects."""
    case = synth.Case(seed=41, B=3, n_q=2, seq_lens=[5000, 2050, 9001], top_k=700, H=16, idx_fmt=fmt,
                      kv_fmt="fp8" if fmt != "bf16" else "bf16", signed_w=True)
    g = GpuCase(case, attention=False)
    both = g.score_topk(li).cpu().numpy()
    for j in range(2):
        sl = (g.seq_lens - (1 - j)).contiguous()
        one = li.li_score_topk(g.q[j::2].contiguous(), g.w[j::2].contiguous(), g.k_pool, sl, g.block_table,
                               case.top_k, q_scales=None if g.q_scales is None else g.q_scales[j::2].contiguous(),
                               k_scales=g.k_scales).cpu().numpy()
        assert (one == both[j::2]).all(), f"token {j}"


def test_prefill_all_equal_scores(li):
    case = synth.Case(seed=22, B=1, n_q=8, seq_lens=[5000], top_k=700, H=16)
    g = GpuCase(case, attention=False)
    g.q = torch.zeros_like(g.q)
    idx = g.score_topk(li).cpu().numpy()
    assert (idx == np.arange(700)[None, :]).all()


def test_prefill_4k_on_64k_sampled(li):
    """Full-size prefill chunk: 4096 causal queries on a 65536-token cache;
    stratified queries checked against the oracle."""
    case = synth.workload("prefill_4k_on_64k")
    g = GpuCase(case)
    idx = g.score_topk(li)
    out, lse = g.attend(li, idx, prefill=True)
    torch.cuda.synchronize()
    # indices of 258 stratified queries (every 16th, the first and the last),
    # attention of every 64th
    tokens = sorted(set(range(0, case.T, 16)) | {1, case.T - 1})
    ores = oracle.run_tokens(case, tokens, with_attn=False)
    _check_indices(case, idx.cpu().numpy(), tokens, ores)
    atok = sorted(set(range(0, case.T, 64)) | {case.T - 1})
    ores = oracle.run_tokens(case, atok)
    _check_attention(case, out.float().cpu().numpy(), lse.cpu().numpy(), atok, ores)


def test_decode_b64_var_fp8_sampled(li):
    """Full-size FP8 workload (64 requests of 4K..128K positions, MXFP8 indexer
    query, FP8 keys and latent), same launches as a decode step; sampled
    requests (shortest, longest, first, last and every fifth) checked end to end.  Latent rows
    are generated for the sampled requests only."""
    case = synth.workload("decode_b64_var_fp8")
    L = case.seq_lens
    tokens = sorted({0, case.B - 1, int(np.argmin(L)), int(np.argmax(L))} | set(range(3, case.B, 5)))
    assert len(tokens) >= 16
    g = GpuCase(case, latent_requests=tokens)
    idx = g.score_topk(li)
    out, lse = g.attend(li, idx)
    torch.cuda.synchronize()
    ores = oracle.run_tokens(case, tokens)
    _check_indices(case, idx.cpu().numpy(), tokens, ores)
    _check_attention(case, out.float().cpu().numpy(), lse.cpu().numpy(), tokens, ores)


def test_decode_b64_var_mxfp8_keys_sampled(li):
    """The same 64 requests with MXFP8 indexer keys (the 4096-position chunk
    launch of the benchmark's variant figure): indices of the sampled requests
    against the oracle (the latent and its attention are those of the FP8
    workload above)."""
    case = synth.workload("decode_b64_var_mxfp8")
    L = case.seq_lens
    tokens = sorted({0, case.B - 1, int(np.argmin(L)), int(np.argmax(L))} | set(range(2, case.B, 5)))
    g = GpuCase(case, attention=False)
    assert g.k_scales.dtype == torch.uint8 and g.k_scales.shape[-1] == 4
    idx = g.score_topk(li)
    torch.cuda.synchronize()
    ores = oracle.run_tokens(case, tokens, with_attn=False)
    _check_indices(case, idx.cpu().numpy(), tokens, ores)


def test_decode_b128_ctx128k_mtp2_sampled(li):
    """Full-size two-token verification workload: 128 requests x 131072
    positions, FP8 keys, latent FP8 with one scale per 128-wide tile; both
    tokens of eight requests spread over the batch checked end to end."""
    case = synth.workload("decode_b128_ctx128k_mtp2")
    reqs = [0, 17, 38, 55, 64, 90, 111, case.B - 1]
    g = GpuCase(case, latent_requests=reqs)
    idx = g.score_topk(li)
    out, lse = g.attend(li, idx)
    torch.cuda.synchronize()
    tokens = [r * case.n_q + j for r in reqs for j in range(case.n_q)]
    ores = oracle.run_tokens(case, tokens)
    _check_indices(case, idx.cpu().numpy(), tokens, ores)
    _check_attention(case, out.float().cpu().numpy(), lse.cpu().numpy(), tokens, ores)
