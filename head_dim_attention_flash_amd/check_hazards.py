"""Static check of MFMA data hazards in the library's own gfx950 assembly.

The attention kernels issue their MFMAs as inline asm so that operands can
sit in AGPRs; the compiler then cannot pad the hazards around them. This
scans the assembly hipcc generates for each kernel (straight-line order, each
instruction counted as one wait state, ``s_nop N`` as N + 1) and reports:

* a VALU/accvgpr write of a register that an MFMA reads (A, B or C) fewer
  than ``VALU_TO_MFMA`` wait states later;
* a VALU/accvgpr/LDS/VMEM instruction that reads or overwrites an MFMA
  result fewer than ``MFMA_TO_VALU`` wait states after that MFMA;
* an SGPR written by a VALU instruction (v_readlane, v_readfirstlane, ...)
  and read by a vector-memory instruction fewer than ``VALU_SGPR_TO_VMEM``
  wait states later;
* any kernel that uses scratch memory (registers spilled to memory). A
  register the compiler parks in a free AGPR ("Reload Reuse") is allowed: the
  move is a v_accvgpr_read/write, which the hazard scan above checks like any
  other VALU instruction.

The scan follows the control flow: basic blocks split at labels and
branches, and the pending distances (registers still inside a hazard window)
flow along every edge, loop back-edges included, taking at each block entry
the worst case over its predecessors until nothing changes.
Usage: ``python -m head_dim_attention_flash_amd.check_hazards``.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

from . import build as B

VALU_TO_MFMA = 4   # wait states required between a VALU write and an MFMA read
MFMA_TO_VALU = 19  # wait states required between an MFMA write and any other read
VALU_SGPR_TO_VMEM = 5  # VALU write of an SGPR -> vector-memory instruction reading it

SREG = re.compile(r"\bs(?:\[(\d+):(\d+)\]|(\d+)\b)")


def sregs(text: str) -> set[int]:
    out = set()
    for m in SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out

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
    """Yield (name, [instruction or 'label:' lines]) for every kernel in an assembly file."""
    name, body = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            if t.startswith(".L") and t.endswith(":"):
                body.append(t)  # a local label (branch target)
            continue
        if t.endswith(":"):
            body.append(t)
            continue
        body.append(t)
        if t.startswith("s_endpgm"):
            yield name, body
            name = None


def _effects(ins):
    """(wait states, kind, written regs, read regs, SGPRs written by VALU,
    SGPRs read by vector memory) of one instruction."""
    op = ins.split()[0]
    if op == "s_nop":
        return int(ins.split()[1], 0) + 1, "nop", set(), set(), set(), set()
    operands = ins[len(op):]
    parts = [p.strip() for p in operands.split(",")]
    if op.startswith("v_mfma"):
        return 1, "mfma", regs(parts[0]), regs(",".join(parts[1:4])), set(), set()
    if op.startswith(("v_", "ds_", "buffer_", "global_", "scratch_")):
        written = regs(parts[0]) if op.startswith("v_") and parts and parts[0] else set()
        s_written = sregs(parts[0]) if op.startswith("v_") and parts and parts[0] else set()
        s_read = sregs(operands) if op.startswith(("buffer_", "global_", "scratch_")) else set()
        return 1, "vec", written, regs(operands), s_written, s_read
    return 1, "other", set(), set(), set(), set()


def _blocks(lines):
    """Basic blocks: list of (label or None, [instruction indices]) and the successor map."""
    blocks, cur, label = [], [], None
    for i, ins in enumerate(lines):
        if ins.endswith(":"):
            if cur or label is not None:
                blocks.append((label, cur))
            label, cur = ins[:-1], []
            continue
        cur.append(i)
        op = ins.split()[0]
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op == "s_endpgm" or op.startswith("s_setpc"):
            blocks.append((label, cur))
            label, cur = None, []
    if cur or label is not None:
        blocks.append((label, cur))
    index = {lab: k for k, (lab, _) in enumerate(blocks) if lab is not None}
    succ = []
    for k, (_, idx) in enumerate(blocks):
        last = lines[idx[-1]].split() if idx else [""]
        op = last[0]
        nxt = [k + 1] if k + 1 < len(blocks) else []
        if op == "s_branch":
            succ.append([index[last[1]]] if last[1] in index else [])
        elif op.startswith("s_cbranch"):
            tgt = [index[last[1]]] if len(last) > 1 and last[1] in index else []
            succ.append(tgt + nxt)
        elif op == "s_endpgm" or op.startswith("s_setpc"):
            succ.append([])
        else:
            succ.append(nxt)
    return blocks, succ


def check_kernel(lines):
    """Hazards in one kernel's instruction list (labels as 'name:' lines)."""
    blocks, succ = _blocks(lines)
    # state: (mfma_pending, valu_pending, sgpr_pending): reg -> wait states still required
    entry = {0: ({}, {}, {})} if blocks else {}
    issues = {}
    work = [0] if blocks else []
    while work:
        k = work.pop()
        mp, vp, sp = (dict(d) for d in entry[k])
        for i in blocks[k][1]:
            w, kind, written, read, s_written, s_read = _effects(lines[i])
            mp = {r: c - w for r, c in mp.items() if c - w > 0}
            vp = {r: c - w for r, c in vp.items() if c - w > 0}
            sp = {r: c - w for r, c in sp.items() if c - w > 0}
            for r in s_read:
                if r in sp:
                    issues.setdefault(i, f"SGPR s{r} written by VALU read by vector memory "
                                         f"{VALU_SGPR_TO_VMEM - sp[r]} wait states later: {lines[i]}")
            for r in s_written:
                sp[r] = VALU_SGPR_TO_VMEM
            if kind == "mfma":
                for r in read:
                    if r in vp:
                        issues.setdefault(i, f"VALU write of {r} read by MFMA {VALU_TO_MFMA - vp[r]} wait states later: {lines[i]}")
                for r in written:
                    mp[r] = MFMA_TO_VALU
            elif kind == "vec":
                for r in read | written:
                    if r in mp:
                        issues.setdefault(i, f"{lines[i].split()[0]} touches MFMA result {r} "
                                             f"{MFMA_TO_VALU - mp[r]} wait states after it: {lines[i]}")
                for r in written:
                    vp[r] = VALU_TO_MFMA
        for n in succ[k]:
            old = entry.get(n)
            if old is None:
                entry[n] = (dict(mp), dict(vp), dict(sp))
                work.append(n)
                continue
            changed = False
            for o, x in ((old[0], mp), (old[1], vp), (old[2], sp)):
                for r, c in x.items():
                    if o.get(r, 0) < c:
                        o[r] = c
                        changed = True
            if changed:
                work.append(n)
    return sorted(issues.items())


def scratch_users(asm: str) -> list[str]:
    """Kernels that use scratch memory at all.

    A spill to scratch reloads MFMA operands and accumulators from memory
    around the inline-asm MFMAs, out of sight of the wait counts the kernels
    manage by hand; besides the cost, such a kernel gave wrong results once.
    The kernels are written to fit their registers, so any scratch use is
    reported as an error. VGPRs spilled into AGPRs stay in registers and are
    covered by the hazard scan."""
    out = []
    for block in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        vsp = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        if name and priv and int(priv.group(1)):
            out.append(f"{name.group(1)[:60]}: scratch {priv.group(1)} bytes, "
                       f"{vsp.group(1) if vsp else '?'} VGPRs spilled")
    return out


def check_file(src: str) -> list[str]:
    cmd = [B.HIPCC, *B.FLAGS, "-S", "--cuda-device-only", src, "-o", "-"]
    asm = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout
    report = []
    for name, lines in kernels(asm):
        for i, msg in check_kernel(lines):
            report.append(f"{os.path.basename(src)} {name[:60]} #{i}: {msg}")
    for msg in scratch_users(asm):
        report.append(f"{os.path.basename(src)} {msg}")
    return report


def main(argv=None) -> int:
    srcs = argv or [s for s in B.sources()
                    if os.path.basename(s).startswith(("fwd_d", "fwd_w", "fwd_x", "bwd_d"))]
    bad = []
    for s in srcs:
        bad += check_file(s)
    for line in bad[:200]:
        print(line)
    print(f"{len(bad)} hazard(s) in {len(srcs)} file(s)")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
