"""Wait states around the inline-asm MFMAs of the attention kernels.

The decode and prefill attention kernels write their 32x32x16 bf16 MFMAs as
inline asm (to fix the accumulators' register class), so the compiler inserts
none of the wait states the matrix core needs around them.  This test compiles
those sources to gfx950 assembly with the library's own flags and checks, in
the linear order of each kernel, that:

  - no VALU instruction writes a register that an asm MFMA reads (A, B or C)
    fewer than 2 wait states before it (the compiler may materialise an
    operand by a VALU copy, e.g. an AGPR read-back, right before the asm);
  - no VALU, LDS or memory instruction touches an asm MFMA's result fewer
    than 19 wait states after it (the longest result latency of these
    MFMAs), unless an MFMA accumulating into the same registers comes first;
  - no VALU instruction overwrites an asm MFMA's accumulator input fewer than
    15 wait states after it while the MFMA may still be reading it.

A wait state is one issued instruction; s_nop k counts k + 1.  Branches are
not followed (the kernels pad their MFMA results before any branch that
leaves a loop).  Runs on the CPU; skipped when hipcc is missing.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from mla_latent_kv_14_amd import build as B

RAW_IN, RAW_OUT, WAR_C = 2, 19, 15
_REG = re.compile(r"(?<![\w])([va])(?:\[(\d+):(\d+)\]|(\d+))(?![\w])")


def _regs(tok: str) -> set:
    out = set()
    for m in _REG.finditer(tok):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _wait_states(op: str, ops: list) -> int:
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def _valu_defs(op: str, ops: list) -> set:
    if not ops or op.startswith(("v_cmp", "v_readfirstlane", "v_readlane")):
        return set()  # these write scalar registers
    d = _regs(ops[0])
    if op.startswith("v_permlane") and "swap" in op:
        d |= _regs(ops[1])  # swaps write both operands
    return d


def _kernels(asm: str):
    """Yield (name, [(op, operands, in_asm)]) for every function in the file."""
    name, insts, in_asm = None, [], False
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name, insts = m.group(1), []
            continue
        if line.startswith(".Lfunc_end") and name:
            yield name, insts
            name = None
            continue
        if name is None:
            continue
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        s = line.split(";")[0].strip()
        if not s or s.endswith(":") or s.startswith("."):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        insts.append((parts[0], ops, in_asm))


def hazards(asm: str) -> list:
    found = []
    for name, insts in _kernels(asm):
        for i, (op, ops, in_asm) in enumerate(insts):
            if not (in_asm and op.startswith("v_mfma")):
                continue
            dst, srcab = _regs(ops[0]), _regs(ops[1]) | _regs(ops[2])
            srcc = _regs(ops[3]) if len(ops) > 3 else set()
            w = 0
            for j in range(i - 1, -1, -1):
                if w >= RAW_IN:
                    break
                oj, osj, _ = insts[j]
                if oj.startswith("v_") and not oj.startswith("v_mfma") and _valu_defs(oj, osj) & (srcab | srcc):
                    found.append((name, "VALU write then MFMA read", i, j, w))
                w += _wait_states(oj, osj)
            w = 0
            for j in range(i + 1, len(insts)):
                if w >= RAW_OUT:
                    break
                oj, osj, _ = insts[j]
                if oj.startswith("v_mfma"):
                    if _regs(osj[0]) == dst:
                        break  # same accumulator: the matrix core forwards it
                    w += 1
                    continue
                if oj.startswith(("v_", "ds_", "global_", "buffer_", "flat_")):
                    touched = set().union(*[_regs(o) for o in osj]) if osj else set()
                    if touched & dst:
                        found.append((name, "MFMA result used early", i, j, w))
                    if oj.startswith("v_") and w < WAR_C and _valu_defs(oj, osj) & (srcc - dst):
                        found.append((name, "accumulator input overwritten", i, j, w))
                w += _wait_states(oj, osj)
    return found


def _device_asm(src: str, tmp_path) -> str:
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [cc, "-S", "--cuda-device-only", os.path.join(B.CSRC, src), "-o", out] + \
        [f for f in B.COMMON if f != "-fPIC"] + B.DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.parametrize("src", ["decode_mfma.hip", "prefill.hip"])
def test_no_mfma_hazards(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    n_mfma = sum(1 for _, insts in _kernels(asm) for op, _, a in insts if a and op.startswith("v_mfma"))
    assert n_mfma > 0, "no inline-asm MFMA found: the check would prove nothing"
    found = hazards(asm)
    assert not found, f"{len(found)} hazards, first: {found[:5]}"


def test_checker_sees_a_planted_hazard():
    """The checker flags a VALU write one wait state before an asm MFMA."""
    asm = "\n".join([
        "_Zk:", "\tv_accvgpr_read_b32 v43, a85", "\ts_waitcnt lgkmcnt(3)", "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[82:85], v[40:43], 0", "\t;;#ASMEND", ".Lfunc_end0:"])
    assert [h[1] for h in hazards(asm)] == ["VALU write then MFMA read"]
    padded = asm.replace("\t;;#ASMSTART", "\t;;#ASMSTART\n\ts_nop 1")
    assert hazards(padded) == []
    early = "\n".join([
        "_Zk:", "\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[82:85], v[40:43], 0",
        "\t;;#ASMEND", "\tv_max3_f32 v40, v1, v2, v3", ".Lfunc_end0:"])
    assert [h[1] for h in hazards(early)] == ["MFMA result used early"]
