"""The kernels' MFMAs are issued as inline asm, which the compiler does not pad
for data hazards: scan the gfx950 assembly hipcc produces for every kernel
source and require the hazard distances (VALU write -> MFMA read, MFMA write
-> any other access) to be met. Runs on the CPU (hipcc cross-compiles)."""
import concurrent.futures as cf
import os
import shutil

import pytest

from head_dim_attention_flash_amd import build as B
from head_dim_attention_flash_amd import check_hazards as H

SRCS = [s for s in B.sources() if os.path.basename(s) != "api.hip"]


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
def test_no_mfma_hazards_in_kernels():
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        reports = list(ex.map(H.check_file, SRCS))
    bad = [line for r in reports for line in r]
    assert not bad, "\n".join(bad[:20])


def test_checker_flags_a_planted_hazard():
    lines = ["v_mov_b32 v45, 0", "s_and_b64 vcc, exec, s[2:3]",
             "v_mfma_f32_32x32x16_f16 v[2:17], v[46:49], v[42:45], v[2:17]",
             "v_add_f32 v3, v3, v3"]
    issues = H.check_kernel(lines)
    assert len(issues) == 2  # VALU -> MFMA operand, MFMA result -> VALU


def test_checker_follows_loop_back_edges():
    # the MFMA at the end of the loop body reaches the VALU at the loop top
    lines = [".LBB0_1:", "v_add_f32 v3, v3, v3", "s_nop 7",
             "v_mfma_f32_32x32x16_f16 v[2:17], v[46:49], v[42:45], v[2:17]",
             "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    issues = H.check_kernel(lines)
    assert any("touches MFMA result" in m for _, m in issues)


def test_checker_skips_code_after_an_unconditional_branch():
    # the instruction after s_branch is reached only from .LBB0_9 (no MFMA there)
    lines = ["v_mfma_f32_32x32x16_f16 v[2:17], v[46:49], v[42:45], v[2:17]",
             "s_nop 7", "s_nop 7", "s_nop 4", "s_branch .LBB0_9",
             "v_mov_b32 v3, 0", ".LBB0_9:", "v_add_f32 v3, v3, v3", "s_endpgm"]
    assert H.check_kernel(lines) == []


def test_checker_merges_predecessors_at_a_join():
    # one predecessor pads, the other does not: the join must be flagged
    lines = ["v_mfma_f32_32x32x16_f16 v[2:17], v[46:49], v[42:45], v[2:17]",
             "s_cbranch_scc1 .LBB0_5", "s_nop 7", "s_nop 7", "s_nop 4",
             ".LBB0_5:", "v_add_f32 v3, v3, v3", "s_endpgm"]
    issues = H.check_kernel(lines)
    assert any("touches MFMA result" in m for _, m in issues)


def test_checker_flags_scratch_use():
    meta = ("  - .agpr_count:     256\n    .name:           _ZN4ffpa3fooEv\n"
            "    .private_segment_fixed_size: 104\n    .vgpr_spill_count: 25\n"
            "  - .agpr_count:     0\n    .name:           _ZN4ffpa3barEv\n"
            "    .private_segment_fixed_size: 0\n    .vgpr_spill_count: 0\n")
    found = H.scratch_users(meta)
    assert len(found) == 1 and "foo" in found[0]


def test_checker_flags_valu_sgpr_write_before_vector_memory():
    # a spilled SGPR restored by v_readlane right before a copy that reads it
    bad = ["v_readlane_b32 s1, v82, 3", "s_nop 0",
           "buffer_load_dwordx4 v2, s[36:39], s1 offen lds", "s_endpgm"]
    assert any("SGPR s1" in m for _, m in H.check_kernel(bad))
    ok = ["v_readlane_b32 s1, v82, 3", "s_nop 4",
          "buffer_load_dwordx4 v2, s[36:39], s1 offen lds", "s_endpgm"]
    assert H.check_kernel(ok) == []


def test_scratch_is_rejected_but_agpr_parking_is_not():
    meta = ("  - .agpr_count: 12\n    .name: kern_a\n    .private_segment_fixed_size: 16\n"
            "    .vgpr_spill_count: 3\n"
            "  - .agpr_count: 250\n    .name: kern_b\n    .private_segment_fixed_size: 0\n"
            "    .vgpr_spill_count: 2\n")
    out = H.scratch_users(meta)
    assert len(out) == 1 and out[0].startswith("kern_a")
