"""GPU parity of li_decode_step (the whole decode step, one launch where the
shape allows) through the C ABI: index rows bit-exact against the oracle and
identical to li_score_topk's; attention to 2e-2 (bf16) / 5e-2 (FP8) in max
relative error per (token, head) and lse to 1e-2, as for sfa_decode."""
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


def _step(li, g, **kw):
    c = g.case
    idx, out, lse = li.li_decode_step(g.q, g.w, g.k_pool, g.mla_q, g.kv_pool, g.seq_lens, g.block_table, c.top_k,
                                      c.sm_scale, q_scales=g.q_scales, k_scales=g.k_scales, kv_scales=g.kv_scales,
                                      **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()


def _check(case, idx, out, lse, tokens, ores):
    for t in tokens:
        r = ores[t]
        ref = np.full(case.top_k, -1, np.int32)
        ref[:r["n"]] = np.sort(r["idx"][:r["n"]])
        assert (idx[t] == ref).all(), f"token {t}: index rows differ"
        e = rel_err(out[t].astype(np.float64), r["out"])
        assert e <= TOL[case.kv_fmt], f"token {t}: rel err {e}"
        fin = np.isfinite(r["lse"])
        assert (np.isfinite(lse[t]) == fin).all()
        assert np.abs(lse[t][fin] - r["lse"][fin]).max(initial=0) <= 1e-2


FUSED = {
    # one launch: bf16, one token per request, 128 heads, chunks <= CUs
    "ragged_chunks": dict(seed=60, B=4, n_q=1, seq_lens=[9000, 4096, 20000, 100], top_k=2048, H=128),
    "signed": dict(seed=61, B=3, n_q=1, seq_lens=[12000, 30001, 5000], top_k=1024, H=128, signed_w=True),
    "k_ge_visible": dict(seed=62, B=3, n_q=1, seq_lens=[1500, 2048, 700], top_k=2048, H=128),
    "empty_request": dict(seed=63, B=3, n_q=1, seq_lens=[0, 9000, 1], top_k=512, H=128),
    "one_chunk": dict(seed=64, B=2, n_q=1, seq_lens=[4096, 3000], top_k=256, H=128),
}


@pytest.mark.parametrize("name", list(FUSED))
def test_step_matches_oracle(li, name):
    case = synth.Case(**FUSED[name])
    g = GpuCase(case)
    idx, out, lse = _step(li, g)
    tokens = list(range(case.T))
    _check(case, idx, out, lse, tokens, oracle.run_tokens(case, tokens))
    # the index rows are those of li_score_topk
    assert (g.score_topk(li).cpu().numpy() == idx).all()


@pytest.mark.parametrize("spin", [0, 3])
@pytest.mark.parametrize("name", ["ragged_chunks", "signed"])
def test_step_fallbacks_stay_exact(li, name, spin):
    """Exchanges with (almost) no patience: workgroups give up their share,
    the last to arrive writes and attends the whole request; the merge waits
    end without merging.  Results must still equal the oracle's, every call,
    and the workspace's counters must be left zero."""
    case = synth.Case(**FUSED[name])
    g = GpuCase(case)
    ws = torch.zeros(li.li_decode_step_workspace_size(case.B, 1, case.max_pages, case.H, case.top_k),
                     dtype=torch.uint8, device="cuda")
    tokens = list(range(case.T))
    ores = oracle.run_tokens(case, tokens)
    li.li_set_exchange_patience(spin)
    try:
        for _ in range(3):
            idx, out, lse = _step(li, g, workspace=ws)
            _check(case, idx, out, lse, tokens, ores)
    finally:
        li.li_set_exchange_patience(-1)
    assert int(ws[: case.B * 128].view(torch.int32).view(case.B, 32)[:, :8].abs().sum()) == 0


def test_step_trend_selection_in_few_chunks(li):
    """Scores rising with position: the selection sits in the last chunks, so
    a few workgroups attend many rows and the others none."""
    L, K = 131072, 2048
    case = synth.Case(seed=65, B=1, n_q=1, seq_lens=[L], top_k=K, H=128)
    g = GpuCase(case)
    rng = np.random.default_rng(4)
    m = (np.arange(L) * 128) // L
    k = (np.arange(128)[None, :] < m[:, None]).astype(np.int8)
    k += (rng.integers(-1, 2, size=(L, 128)) * (rng.random((L, 128)) < 0.05)).astype(np.int8)
    q, qs, ks = encode_indexer_int(case, np.ones((1, 64, 128), np.int8), [k])
    w = np.full((1, 64), 0.5, np.float32)
    load_indexer(g, q, qs, w, ks)
    idx, out, lse = _step(li, g)
    sc = oracle.index_scores(q[0], w[0], ks[0][0], L)
    ridx, n = oracle.topk(sc, K)
    assert (idx[0] == np.sort(ridx[:n])).all()
    lat, _ = case.latent_rows(0)
    o_ref, lse_ref = oracle.sparse_attn(case.mla_q(0, 1)[0], lat, ridx, case.sm_scale)
    assert rel_err(out[0].astype(np.float64), o_ref) <= 2e-2
    assert np.abs(lse[0] - lse_ref).max() <= 1e-2


def test_step_headline_every_token(li):
    """The headline decode workload (32 x 32K, 128 heads, K 2048), the launch
    the benchmark times: every token against the oracle."""
    case = synth.workload("decode_b32_ctx32k")
    g = GpuCase(case)
    idx, out, lse = _step(li, g)
    tokens = list(range(case.T))
    _check(case, idx, out, lse, tokens, oracle.run_tokens(case, tokens))


@pytest.mark.parametrize("name", ["fp8_mtp2", "h16", "fp8r"])
def test_step_two_launch_shapes(li, name):
    """Shapes outside the one-launch form (FP8 caches, two tokens, fewer
    heads) run the indexer and the attention back to back: same results."""
    cfg = {"fp8_mtp2": dict(seed=66, B=2, n_q=2, seq_lens=[3000, 700], top_k=256, H=128, idx_fmt="fp8", kv_fmt="fp8",
                            kv_groups=5),
           "h16": dict(seed=67, B=3, n_q=1, seq_lens=[100, 1500, 3000], top_k=256, H=16),
           "fp8r": dict(seed=68, B=2, n_q=1, seq_lens=[1500, 2600], top_k=300, H=16, idx_fmt="mxfp8", kv_fmt="fp8r",
                        kv_groups=4)}[name]
    case = synth.Case(**cfg)
    g = GpuCase(case)
    idx, out, lse = _step(li, g)
    tokens = list(range(case.T))
    _check(case, idx, out, lse, tokens, oracle.run_tokens(case, tokens))


def test_step_pool_beyond_4gib(li):
    # the same pages placed past 4.5 GiB of latent pool (and past 1 GiB of
    # key pool): 64-bit row addresses in the single-launch step give identical
    # results
    case = synth.Case(seed=44, B=4, n_q=1, seq_lens=[3000, 9000, 2000, 5000], top_k=512, H=128)
    g = GpuCase(case)
    idx, out, lse = _step(li, g)
    p0 = -(-(9 << 29) // (64 * 1152))
    NP = g.kv_pool.shape[0]
    big_kv = torch.zeros((p0 + NP,) + tuple(g.kv_pool.shape[1:]), dtype=g.kv_pool.dtype, device="cuda")
    big_kv[p0:] = g.kv_pool
    big_k = torch.zeros((p0 + NP,) + tuple(g.k_pool.shape[1:]), dtype=g.k_pool.dtype, device="cuda")
    big_k[p0:] = g.k_pool
    assert big_kv.numel() * big_kv.element_size() > (1 << 32)
    idx2, out2, lse2 = li.li_decode_step(g.q, g.w, big_k, g.mla_q, big_kv, g.seq_lens, g.block_table + p0,
                                         case.top_k, case.sm_scale)
    torch.cuda.synchronize()
    assert (idx2.cpu().numpy() == idx).all()
    assert np.array_equal(out2.float().cpu().numpy(), out) and np.array_equal(lse2.cpu().numpy(), lse)
    tokens = list(range(case.T))
    _check(case, idx, out, lse, tokens, oracle.run_tokens(case, tokens))
    del big_kv, big_k
    torch.cuda.empty_cache()
