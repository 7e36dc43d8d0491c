"""Static check of MFMA data hazards in the library's own gfx950 assembly.

The attention kernels issue their MFMAs as inline asm so that operands can
sit in AGPRs; the compiler then cannot pad the hazards around them. This
scans the assembly hipcc generates for each kernel (straight-line order, each
instruction counted as one wait state, ``s_nop N`` as N + 1) and reports:

* a VALU/accvgpr write of a register that an MFMA reads (A, B or C) fewer
  than ``VALU_TO_MFMA`` wait states later;
* a VALU/accvgpr/LDS/VMEM instruction that reads or overwrites an MFMA
  result fewer than ``MFMA_TO_VALU`` wait states after that MFMA.

Branches are ignored (the scan follows the text), which is conservative for
fall-through code. Usage: ``python -m head_dim_attention_flash_amd.check_hazards``.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

from . import build as B

VALU_TO_MFMA = 4   # wait states required between a VALU write and an MFMA read
MFMA_TO_VALU = 19  # wait states required between an MFMA write and any other read

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def regs(text: str) -> set[tuple[str, int]]:
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((kind, r))
    return out


def kernels(asm: str):
    """Yield (name, [instruction lines]) for every kernel in an assembly file."""
    name, body = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            if "s_endpgm" in t:
                yield name, body
                name = None
            continue
        body.append(t)
        if t.startswith("s_endpgm"):
            yield name, body
            name = None


def check_kernel(lines):
    issues = []
    clock = 0
    last_valu_write = {}   # reg -> clock
    last_mfma_write = {}   # reg -> (clock, index)
    for i, ins in enumerate(lines):
        op = ins.split()[0]
        if op == "s_nop":
            clock += int(ins.split()[1], 0) + 1
            continue
        clock += 1
        operands = ins[len(op):]
        parts = [p.strip() for p in operands.split(",")]
        if op.startswith("v_mfma"):
            dst, srcs = regs(parts[0]), regs(",".join(parts[1:4]))
            for r in srcs:
                t = last_valu_write.get(r)
                if t is not None and clock - t < VALU_TO_MFMA:
                    issues.append((i, f"VALU write of {r} read by MFMA after {clock - t} wait states: {ins}"))
            for r in dst:
                last_mfma_write[r] = (clock, i)
            continue
        if not (op.startswith("v_") or op.startswith("ds_") or op.startswith("buffer_")
                or op.startswith("global_") or op.startswith("scratch_")):
            continue
        touched = regs(operands)
        for r in touched:
            w = last_mfma_write.get(r)
            if w is not None and clock - w[0] < MFMA_TO_VALU:
                issues.append((i, f"{op} touches MFMA result {r} after {clock - w[0]} wait states: {ins}"))
        if op.startswith("v_") and parts and parts[0]:
            for r in regs(parts[0]):
                last_valu_write[r] = clock
    return issues


def check_file(src: str) -> list[str]:
    cmd = [B.HIPCC, *B.FLAGS, "-S", "--cuda-device-only", src, "-o", "-"]
    asm = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout
    report = []
    for name, lines in kernels(asm):
        for i, msg in check_kernel(lines):
            report.append(f"{os.path.basename(src)} {name[:60]} #{i}: {msg}")
    return report


def main(argv=None) -> int:
    srcs = argv or [s for s in B.sources() if os.path.basename(s).startswith(("fwd_d", "bwd_d"))]
    bad = []
    for s in srcs:
        bad += check_file(s)
    for line in bad[:200]:
        print(line)
    print(f"{len(bad)} hazard(s) in {len(srcs)} file(s)")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
