"""li_score_topk_noalloc (the library's own exchange workspace, no allocation)
against li_score_topk (caller workspace) through the C ABI: the indices must
be identical, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_inputs import GpuCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def li(gpu_ready):
    import sparse_attention_li_amd as li
    li.lib()
    return li


def _both(li, case):
    g = GpuCase(case, attention=False)
    ref = g.score_topk(li).clone()
    out = torch.full_like(ref, -7)
    li.li_score_topk_noalloc(g.q, g.w, g.k_pool, g.seq_lens, g.block_table, case.top_k, out,
                             q_scales=g.q_scales, k_scales=g.k_scales)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_noalloc_equals_workspace_entry_point(li, fmt):
    kw = dict(idx_fmt=fmt, kv_fmt="fp8" if fmt != "bf16" else "bf16", signed_w=True)
    big = synth.Case(seed=50, B=12, n_q=1, seq_lens=[32768 - 999 * b for b in range(12)], top_k=2048, H=16, **kw)
    small = synth.Case(seed=51, B=3, n_q=2, seq_lens=[5000, 1300, 64], top_k=512, H=16, **kw)
    for case in (big, small):
        ref, out = _both(li, case)
        assert (ref == out).all()
    # and the smaller call is right, not merely equal
    ores = oracle.run_tokens(small, list(range(small.T)), with_attn=False)
    for t in range(small.T):
        r = ores[t]
        exp = np.full(small.top_k, -1, np.int32)
        exp[:r["n"]] = np.sort(r["idx"][:r["n"]])
        assert (out[t] == exp).all()
