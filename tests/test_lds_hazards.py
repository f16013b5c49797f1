"""The build's scan for early uses of in-flight LDS reads (CPU only): it must
flag a read, copy or spill of a register before the wait that covers it, and
accept uses after it."""
from sparse_attention_li_amd import lds_hazards


def _scan(text):
    return lds_hazards.scan_function(text.strip().splitlines())


def test_use_after_wait_is_clean():
    assert _scan("""
        ds_read_b128 v[10:13], v1
        ds_read_b64_tr_b16 v[14:15], v2 offset:1024
        s_waitcnt lgkmcnt(0)
        v_mfma_f32_32x32x16_bf16 a[0:15], v[10:13], v[20:23], a[0:15]
        v_mov_b32_e32 v30, v15
    """) == []


def test_copy_and_spill_before_wait_are_flagged():
    found = _scan("""
        ds_read_b128 v[10:13], v1
        v_mov_b32_e32 v30, v11
        scratch_store_dwordx4 off, v[10:13], off offset:16
        s_waitcnt lgkmcnt(0)
    """)
    assert {r for _, r in found} == {("v", 10), ("v", 11), ("v", 12), ("v", 13)}
    assert any("v_mov_b32" in t for t, _ in found)


def test_partial_wait_completes_oldest_reads_only():
    found = _scan("""
        ds_read_b128 v[10:13], v1
        ds_read_b128 v[14:17], v1 offset:64
        s_waitcnt lgkmcnt(1)
        v_add_f32_e32 v30, v10, v31
        v_add_f32_e32 v32, v14, v31
    """)
    assert [r for _, r in found] == [("v", 14)]


def test_scalar_load_sharing_the_counter_does_not_complete_lds_reads():
    found = _scan("""
        s_load_dwordx2 s[4:5], s[0:1], 0x10
        ds_read_b128 v[10:13], v1
        ds_read_b128 v[14:17], v1 offset:64
        s_waitcnt lgkmcnt(1)
        v_add_f32_e32 v30, v10, v31
        v_add_f32_e32 v32, v14, v31
    """)
    assert [r for _, r in found] == [("v", 14)]


def test_overwrite_of_pending_destination_is_flagged():
    found = _scan("""
        ds_read_b64_tr_b16 v[4:5], v2
        v_mov_b32_e32 v5, 0
        s_waitcnt lgkmcnt(0)
    """)
    assert [r for _, r in found] == [("v", 5)]


def test_lds_writes_count_without_destination():
    found = _scan("""
        ds_read_b128 v[10:13], v1
        ds_write_b32 v2, v40
        s_waitcnt lgkmcnt(1)
        v_add_f32_e32 v30, v10, v31
    """)
    assert found == []


def test_loop_carried_read_is_checked_at_the_loop_head():
    """A read issued at the end of a loop body and used at the loop head of
    the next iteration, before any wait."""
    found = _scan("""
        s_mov_b32 s0, 0
    .LBB0_1:
        v_add_f32_e32 v30, v10, v31
        s_waitcnt lgkmcnt(0)
        ds_read_b32 v10, v1
        s_add_u32 s0, s0, 1
        s_cbranch_scc1 .LBB0_1
        s_waitcnt lgkmcnt(0)
        s_endpgm
    """)
    assert [r for _, r in found] == [("v", 10)]


def test_wait_on_a_skipped_branch_clears_nothing_after_the_join():
    found = _scan("""
        ds_read_b128 v[10:13], v1
        s_cbranch_vccz .LBB0_2
        s_waitcnt lgkmcnt(0)
    .LBB0_2:
        v_mov_b32_e32 v30, v12
        s_waitcnt lgkmcnt(0)
        v_mov_b32_e32 v31, v13
        s_endpgm
    """)
    assert [r for _, r in found] == [("v", 12)]


def test_code_after_the_first_endpgm_is_scanned():
    from sparse_attention_li_amd import lds_hazards as lh
    asm = """_ZN3sli1kEv:
    s_cbranch_vccz .LBB0_3
    s_endpgm
.LBB0_3:
    ds_read_b32 v10, v1
    v_mov_b32_e32 v30, v10
    s_waitcnt lgkmcnt(0)
    s_endpgm
.Lfunc_end0:
"""
    found = lh.check_asm(asm, ("_ZN3sli1kEv",))
    assert [r for _, _, r in found] == ["v10"]
