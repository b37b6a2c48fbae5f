"""No kernel rewrites a register that a DS write has yet to store (see
tests/isa_scan.py).  Scans the gfx950 code of the objects built in this tree;
skipped when they or the LLVM tools are absent."""

import os

import pytest

import isa_scan as S


def test_scanner_finds_the_pattern():
    # A store followed by a rewrite of its first data register: flagged.
    bad = ["ds_write_b128 v32, v[12:15]", "v_bfe_u32 v12, v197, 16, 1", "s_waitcnt lgkmcnt(0)"]
    assert [h[0] for h in S.violations(bad)] == [0]
    # The wait comes first, or the rewritten register is not a data register,
    # or the write's own address register is reused: not flagged.
    assert not S.violations(["ds_write_b128 v32, v[12:15]", "s_waitcnt lgkmcnt(0)", "v_mov_b32 v12, 0"])
    assert not S.violations(["ds_write_b128 v32, v[12:15]", "v_mov_b32 v16, 0", "v_mov_b32 v32, 1"])
    assert [h[0] for h in S.violations(["ds_write2st64_b32 v61, v60, v62 offset1:1", "v_fma_f32 v62, s9, v7, v57"])] == [0]
    assert not S.violations(["ds_write_b32 v1, v2", "s_waitcnt lgkmcnt(0)", "v_add_u32 v2, v2, v3"])


def test_store_scanner_finds_the_pattern():
    # A 128-bit buffer store whose first data register is rewritten before a
    # vmcnt wait: flagged; likewise the data pair of a global store.
    bad = ["buffer_store_dwordx4 v[52:55], v83, s[12:15], 0 offen", "v_bfe_u32 v53, v126, 16, 1"]
    assert [h[0] for h in S.store_reuse(bad)] == [0]
    bad_g = ["global_store_dwordx4 v[2:3], v[4:7], off", "v_lshrrev_b32_e32 v7, 28, v13"]
    assert [h[0] for h in S.store_reuse(bad_g)] == [0]
    # The wait first, a rewrite of the address register only, or a load
    # into another register: not flagged.
    assert not S.store_reuse(["buffer_store_dwordx4 v[52:55], v83, s[12:15], 0 offen", "s_waitcnt vmcnt(0)",
                              "v_mov_b32 v52, 0"])
    assert not S.store_reuse(["global_store_dwordx4 v[2:3], v[4:7], off", "v_mov_b32 v2, 0"])
    assert not S.store_reuse(["buffer_store_dword v9, v1, s[0:3], 0 offen", "ds_read_b32 v10, v2"])


@pytest.mark.parametrize("name", S.KERNEL_OBJECTS)
def test_no_lds_write_register_reuse(name):
    obj = os.path.join(S.BUILD, f"{name}.o")
    if not os.path.exists(obj) or not os.path.exists(f"{S.LLVM}/llvm-objdump"):
        pytest.skip("built objects or LLVM tools not present (run __graft_entry__.build())")
    funcs = S.disassemble(obj)
    assert funcs, "no device functions found"
    bad = {f: S.violations(lines)[:2] for f, lines in funcs.items() if S.violations(lines)}
    assert not bad, bad
