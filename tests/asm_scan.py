"""Scans of the gfx950 assembly of the main kernel for invariants the C++
source relies on but cannot express.

The kernel issues its MFMAs, its staged global loads and its transposing LDS
reads through inline assembly.  The compiler neither pads hazards around
inline assembly nor knows that an inline-assembly load completes later, so:

* a VALU write of a VGPR must be at least 2 wait states before an MFMA that
  reads it, and an MFMA result must not be touched by a non-MFMA instruction
  within 19 wait states (the longest MFMA used here);
* a register that a staged load targets must not be copied anywhere in a
  loop that issues staged loads, nor between a prologue's loads and its loop
  (the copy would read it before the data arrives);
* the tile loop must not move MFMA accumulators or operands between register
  files (v_accvgpr_*), which is what keeps the loop short;
* a transcendental result (v_exp_f32 and the like) must not be read by the
  very next instruction (one wait state), a hazard the compiler pads only in
  front of its own instructions;
* in the fp8 kernel, whose MFMA accumulators live in AGPRs named by its
  inline assembly, the compiler must not place anything in an AGPR.
"""
from __future__ import annotations

import re

MAIN_KERNEL = re.compile(r"^(_Z\S*mla_decode_main\S*):", re.M)
MERGE_KERNEL = re.compile(r"^(_Z\S*mla_(?:decode_reduce|merge_shards)\S*):", re.M)
FP8_KERNEL = re.compile(r"^(_Z\S*mla_decode_fp8\S*):", re.M)
TRANS_OP = re.compile(r"^v_(exp|log|rcp|rcp_iflag|rsq|sqrt|sin|cos)(_legacy)?_f(16|32)")
STAGED_LOAD = re.compile(r"buffer_load_dwordx[24] (v\S+?),? v\d+, s\[\d+:\d+\], s\d+ offen")


def kernels(asm: str, pattern=MAIN_KERNEL) -> dict:
    """Kernel name -> list of its assembly lines (the body and the compiler's
    resource summary comments that follow it), for the kernels whose symbol
    matches `pattern`."""
    out = {}
    for m in pattern.finditer(asm):
        end = asm.find(".Lfunc_end", m.end())
        stats = asm.find("; Occupancy:", end)
        out[m.group(1)] = asm[m.end():stats if stats >= 0 else end].split("\n")
    return out


def scratch_bytes(lines) -> int:
    """ScratchSize of the kernel's resource summary (private memory per lane)."""
    for line in lines:
        m = re.match(r"; ScratchSize: (\d+)", line.strip())
        if m:
            return int(m.group(1))
    raise AssertionError("no ScratchSize line")


def regs(tok: str) -> set:
    """{('v'|'a', index)} named by an operand such as v[4:7], a3."""
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", tok):
        if m.group(1):
            out |= {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _instructions(lines):
    """[(opcode, [operands])]; block labels become ('LABEL', [])."""
    out = []
    for line in lines:
        t = line.strip()
        if re.match(r"^\.LBB\S+:", t):
            out.append(("LABEL", []))
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        op, _, rest = t.partition(" ")
        ops = [o.strip() for o in rest.split(";")[0].split(",")] if rest else []
        out.append((op, ops))
    return out


def _wait_states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def mfma_hazards(lines) -> list:
    """Unpadded VALU->MFMA and MFMA->non-MFMA register dependences inside a block."""
    ins = _instructions(lines)
    found = []
    for i, (op, ops) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        srcs = set().union(*[regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
        ws = 0
        for k in range(i - 1, -1, -1):
            pop, pops = ins[k]
            if pop == "LABEL" or ws >= 2:
                break
            if pop.startswith("v_") and not pop.startswith("v_mfma") and pops and regs(pops[0]) & srcs:
                found.append(f"VALU {pop} {pops[0]} -> {op} {','.join(ops)} after {ws} wait states")
            ws += _wait_states(pop, pops)
        dst = regs(ops[0])
        ws = 0
        for k in range(i + 1, len(ins)):
            pop, pops = ins[k]
            if pop == "LABEL" or ws >= 19:
                break
            if not pop.startswith("v_mfma") and pops and set().union(*[regs(o) for o in pops]) & dst:
                found.append(f"{op} {ops[0]} -> {pop} {','.join(pops)} after {ws} wait states")
            ws += _wait_states(pop, pops)
    return found


def _loops(lines):
    """{header label: [line indices]} from the compiler's block annotations
    ("Loop Header" / "in Loop: Header=..."); layout order does not matter."""
    out = {}
    cur = None
    for n, line in enumerate(lines):
        t = line.strip()
        if re.match(r"^(\.LBB\S+:|; %bb\.\d+:)", t):
            m = re.match(r"^(\.LBB\S+):.*Loop Header: Depth=1", t)
            if m:
                cur = m.group(1)[1:]  # "LBBx_y"; members say "Header=BBx_y"
            else:
                m = re.search(r"in Loop: Header=(BB\S+) Depth=1", t)
                cur = "L" + m.group(1) if m else None
        if cur is not None:
            out.setdefault(cur, []).append(n)
    return out


def tile_loops(lines):
    """{label: line indices} of the loops that contain MFMAs (the KV tile loops)."""
    return {lab: idx for lab, idx in _loops(lines).items()
            if any("v_mfma" in lines[k] for k in idx)}


def staging_loops(lines):
    """{label: line indices} of the loops that issue staged loads."""
    return {lab: idx for lab, idx in _loops(lines).items()
            if any(STAGED_LOAD.search(lines[k]) for k in idx)}


def _written(line):
    """Registers an instruction line writes (first operand; both operands of a
    lane swap); stores and scalar instructions write none we track."""
    t = line.strip()
    if not t or t.startswith(";") or t.startswith("."):
        return set()
    op, _, rest = t.partition(" ")
    ops = [o.strip() for o in rest.split(";")[0].split(",")] if rest else []
    if not ops or "store" in op or "write" in op or op.startswith("s_"):
        return set()
    if op.startswith("v_permlane") and "swap" in op:
        return regs(ops[0]) | regs(ops[1])
    return regs(ops[0])


def _copy_of_staged(lines, order, pos, src):
    """Walking back from order[pos] (wrapping around the loop), is the last
    write of any register in src a staged load?"""
    n = len(order)
    for step in range(1, n):
        line = lines[order[(pos - step) % n]]
        w = _written(line)
        if w & src:
            return bool(STAGED_LOAD.search(line))
    return False


def staged_copies_in_loops(lines) -> list:
    """Register copies that read a staged-load destination before anything
    else has redefined it, i.e. copies of data that may still be in flight."""
    found = []
    for lab, idx in staging_loops(lines).items():
        order = sorted(idx)
        for pos, k in enumerate(order):
            m = re.search(r"v_mov_b(?:32|64)_e32 (v\S+), (v\S+)", lines[k])
            if m and _copy_of_staged(lines, order, pos, regs(m.group(2))):
                found.append(f"{lab}: {lines[k].strip()}")
    return found


def staged_copies_in_prologues(lines) -> list:
    """Copies of staged-load destinations between a prologue's loads and the
    start of its loop (layout order) before anything redefined them."""
    loop_lines = set(k for idx in staging_loops(lines).values() for k in idx)
    found = []
    staged = set()
    for n, line in enumerate(lines):
        if n in loop_lines:
            staged = set()
            continue
        m = STAGED_LOAD.search(line)
        if m:
            staged |= regs(m.group(1))
            continue
        m = re.search(r"v_mov_b(?:32|64)_e32 (v\S+), (v\S+)", line)
        if m and regs(m.group(2)) & staged:
            found.append(f"line {n}: {line.strip()}")
        staged -= _written(line)
    return found


DMA_LOAD = re.compile(r"buffer_load_dword\S* .*\blds\s*$")


def dma_loads_in_loops(lines) -> int:
    """LDS DMA loads (buffer_load ... lds) inside the KV tile loops."""
    return sum(1 for idx in tile_loops(lines).values() for k in idx if DMA_LOAD.search(lines[k]))


def staged_loads_in_loops(lines) -> int:
    return sum(1 for idx in staging_loops(lines).values() for k in idx
               if STAGED_LOAD.search(lines[k]))


def accvgpr_moves_in_loops(lines) -> list:
    return [f"{lab}: {lines[k].strip()}" for lab, idx in tile_loops(lines).items()
            for k in idx if "v_accvgpr_" in lines[k]]


def trans_hazards(lines) -> list:
    """Transcendental results read by the instruction right after them."""
    ins = _instructions(lines)
    found = []
    for i in range(len(ins) - 1):
        op, ops = ins[i]
        if not TRANS_OP.match(op) or not ops:
            continue
        nop, nops = ins[i + 1]
        if nop == "LABEL" or not nop.startswith("v_") or len(nops) < 2:
            continue
        if set().union(*[regs(o) for o in nops[1:]]) & regs(ops[0]):
            found.append(f"{op} {ops[0]} -> {nop} {','.join(nops)}")
    return found


def compiler_agprs(lines) -> list:
    """AGPRs named outside inline-assembly blocks (the compiler's own use)."""
    found = []
    inasm = False
    for line in lines:
        t = line.strip()
        if ";;#ASMSTART" in t:
            inasm = True
            continue
        if ";;#ASMEND" in t:
            inasm = False
            continue
        if inasm or not t or t.startswith(";") or t.startswith("."):
            continue
        if any(kind == "a" for kind, _ in regs(t.split(";")[0])):
            found.append(t)
    return found
