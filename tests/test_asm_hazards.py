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
