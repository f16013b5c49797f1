"""GPU parity of the cache append and the quantisers (through the C ABI)
against the CPU oracle on the same seeded inputs: codes, scales and the
written cache bytes must match bit for bit, and rows of other positions must
be left untouched."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def li(gpu_ready):
    import sparse_attention_li_amd as li
    li.lib()
    return li


def _bf16(a):
    """float32 array -> (bf16 bits as uint16, the same bits as a device int16 tensor)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).bfloat16()
    return t.view(torch.int16).numpy().view(np.uint16), t.view(torch.int16).cuda()


def test_mxfp8_matches_oracle(li):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((7 * 64, 128)).astype(np.float32) * np.exp(rng.uniform(-8, 8, (7 * 64, 1)))
    x[3, 32:64] = 0.0                      # an all-zero group
    x[5, 0:32] = rng.integers(-4, 5, 32)   # integers, amax <= 4
    x[9, 64:96] = 1.0
    x[9, 70] = 15.2                        # largest element saturates at 448
    bits, xt = _bf16(x)
    codes, scales = li.li_quantize_mxfp8(xt.view(torch.bfloat16))
    torch.cuda.synchronize()
    rc, rs = oracle.quant_mxfp8(bits)
    assert (scales.cpu().numpy() == rs).all()
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[:3]}: gpu {got[tuple(bad[0])]} oracle {rc[tuple(bad[0])]}"


def test_mxfp8_tiny_groups_hold_least_scale(li):
    """Groups with subnormal or tiny maxima (below 2^-119): the E8M0 scale
    holds at code 0 (2^-127) and codes are x * 2^127, bit-exact against the
    oracle."""
    rng = np.random.default_rng(41)
    n = 64
    bits = rng.integers(0, 0x80, (n, 32)).astype(np.uint16)              # subnormal magnitudes
    bits |= rng.integers(0, 2, (n, 32)).astype(np.uint16) << 15          # both signs
    e_field = rng.integers(1, 12, n).astype(np.uint16)                   # amax 2^-126 .. 2^-116
    pos = rng.integers(0, 32, n)
    bits[np.arange(n) // 2 * 2, pos[np.arange(n) // 2 * 2]] = e_field[np.arange(n) // 2 * 2] << 7
    bits[7] = 0x0001                                                     # 2^-133 everywhere
    xt = torch.from_numpy(bits.view(np.int16)).cuda()
    codes, scales = li.li_quantize_mxfp8(xt.view(torch.bfloat16))
    torch.cuda.synchronize()
    rc, rs = oracle.quant_mxfp8(bits)
    assert (rs <= 3).all() and (rs == 0).sum() > n // 4  # the clamp is reached
    assert (scales.cpu().numpy() == rs).all()
    assert (codes.cpu().numpy() == rc).all()


def _pools(rng, num_pages, fp8_k, fp8_kv, groups):
    k = torch.from_numpy(rng.integers(0, 256, (num_pages, 64, 256), dtype=np.uint8)).cuda()
    kv = torch.from_numpy(rng.integers(0, 256, (num_pages, 64, 1152), dtype=np.uint8)).cuda()
    k_pool = k[:, :, :128].contiguous() if fp8_k else k.view(torch.int16)
    kv_pool = kv[:, :, :(640 if fp8_kv == "rope16" else 576)].contiguous() if fp8_kv else kv.view(torch.int16)
    if fp8_k == "mx":
        ks = torch.from_numpy(rng.integers(0, 255, (num_pages, 64, 4), dtype=np.uint8)).cuda()
    else:
        ks = torch.from_numpy(rng.uniform(1, 2, (num_pages, 64)).astype(np.float32)).cuda() if fp8_k else None
    kvs = torch.from_numpy(rng.uniform(1, 2, (num_pages, 64, groups)).astype(np.float32)).cuda() if fp8_kv else None
    return k_pool, kv_pool, ks, kvs


@pytest.mark.parametrize("fp8_k,fp8_kv,groups,n_q", [
    (False, False, 1, 1), (True, True, 1, 1), (True, True, 5, 2), (False, True, 5, 1), (True, False, 1, 2),
    ("mx", True, 1, 1), ("mx", False, 5, 2),   # MXFP8 key rows (E8M0 per 32 elements)
    (True, "rope16", 1, 1), ("mx", "rope16", 4, 2),  # FP8 latent with the rope in bf16 (640-byte rows)
])
def test_cache_append_matches_oracle(li, fp8_k, fp8_kv, groups, n_q):
    rng = np.random.default_rng(40 + 2 * groups + n_q + 4 * (fp8_k is True) + 8 * (fp8_k == "mx") + 16 * (fp8_kv == "rope16"))
    B, max_pages, num_pages = 5, 6, 40
    seq_lens = np.array([1, 64, 65, 200, 384][:B], dtype=np.int32)   # (L = 1 with two new tokens: one has no slot)
    bt = np.stack([rng.permutation(num_pages)[:max_pages] for _ in range(B)]).astype(np.int32)
    T = B * n_q
    k_new = rng.standard_normal((T, 128)).astype(np.float32) * np.exp(rng.uniform(-3, 3, (T, 1)))
    kv_new = rng.standard_normal((T, 576)).astype(np.float32) * np.exp(rng.uniform(-3, 3, (T, 1)))
    kv_new[min(2, T - 1), 128:256] = 0.0  # an all-zero tile
    kb, kt = _bf16(k_new)
    vb, vt = _bf16(kv_new)
    k_pool, kv_pool, ks, kvs = _pools(rng, num_pages, fp8_k, fp8_kv, groups)
    before = [t.clone() if t is not None else None for t in (k_pool, kv_pool, ks, kvs)]
    li.li_cache_append(torch.from_numpy(seq_lens).cuda(), torch.from_numpy(bt).cuda(), k_new=kt.view(torch.bfloat16),
                       k_cache=k_pool, kv_new=vt.view(torch.bfloat16), kv_cache=kv_pool, k_scales=ks, kv_scales=kvs)
    torch.cuda.synchronize()
    # expected: the pools before, with each token's row replaced
    exp = [t.cpu().numpy().copy() if t is not None else None for t in before]
    if fp8_k == "mx":
        kc, ksc = oracle.quant_mxfp8(kb)
    elif fp8_k:
        kc, ksc = oracle.quant_fp8_rows(kb, 128)
    if fp8_kv == "rope16":
        lc, vsc = oracle.quant_fp8_rows(np.ascontiguousarray(vb[:, :512]), 128 if groups == 4 else 512)
        vc = np.concatenate([lc, np.ascontiguousarray(vb[:, 512:]).view(np.uint8)], axis=1)  # rope bytes as is
    elif fp8_kv:
        vc, vsc = oracle.quant_fp8_rows(vb, 128 if groups == 5 else 576)
    for t in range(T):
        b, j = divmod(t, n_q)
        pos = int(seq_lens[b]) - n_q + j
        if pos < 0:
            continue
        pg, sl = bt[b, pos // 64], pos % 64
        if fp8_k == "mx":
            exp[0][pg, sl] = kc[t]
            exp[2][pg, sl] = ksc[t]
        elif fp8_k:
            exp[0][pg, sl] = kc[t]
            exp[2][pg, sl] = ksc[t, 0]
        else:
            exp[0][pg, sl] = kb[t].view(np.int16)
        if fp8_kv:
            exp[1][pg, sl] = vc[t]
            exp[3][pg, sl] = vsc[t]
        else:
            exp[1][pg, sl] = vb[t].view(np.int16)
    for got, want, name in zip((k_pool, kv_pool, ks, kvs), exp, ("k_cache", "kv_cache", "k_scales", "kv_scales")):
        if got is None:
            continue
        g = got.cpu().numpy()
        assert np.array_equal(g.view(np.uint8), want.view(np.uint8)), f"{name}: {int((g != want).sum())} mismatches"


def _bad_metadata_count(seq_lens, bt, num_pages):
    """Host count of what li_validate_paged reports, from its documented rule."""
    B, max_pages = bt.shape
    cap = max_pages * 64
    bad = 0
    for b in range(B):
        L = int(seq_lens[b])
        bad += int(L < 0 or L > cap)
        used = (min(max(L, 0), cap) + 63) // 64
        bad += int(((bt[b, :used] < 0) | (bt[b, :used] >= num_pages)).sum())
    return bad


def test_validate_paged_counts_bad_metadata(li):
    """The device check of the paged-cache metadata: a valid table gives 0; a
    table with planted bad lengths and page ids (some on unused pages, which
    do not count) gives the host count."""
    rng = np.random.default_rng(71)
    B, max_pages, num_pages = 6, 10, 40
    lens = np.array([0, 64, 65, 640, 641, -3], np.int32)
    bt = rng.integers(0, num_pages, (B, max_pages)).astype(np.int32)
    dev = lambda x: torch.from_numpy(x).cuda()
    ok_lens = np.clip(lens, 0, 640).astype(np.int32)
    assert int(li.li_validate_paged(dev(ok_lens), dev(bt), num_pages).item()) == 0
    bt[0, 0] = -5           # request of length 0: page unused
    bt[1, 0] = -1           # used
    bt[2, 1] = num_pages    # used (65 positions: pages 0 and 1)
    bt[2, 5] = -1           # unused
    bt[3, 9] = 1000         # used (640 positions: all ten pages)
    bt[4, 2] = -2           # used (641 is held to 640)
    want = _bad_metadata_count(lens, bt, num_pages)
    assert want == 6
    assert int(li.li_validate_paged(dev(lens), dev(bt), num_pages).item()) == want
    # a second call on the same output clears it first
    assert int(li.li_validate_paged(dev(ok_lens), dev(bt), num_pages).item()) == _bad_metadata_count(ok_lens, bt, num_pages)
