"""Static check of the decode kernels' machine code (CPU only: hipcc cross-compiles).

The cache stream is staged by inline-assembly DMAs (global_load_lds_dwordx4) whose base
address sits in scalar registers.  On this GPU family a vector-memory instruction that
reads an SGPR written by a VALU instruction (v_readfirstlane, a compare, the carry-out
of a 64-bit multiply-add, ...) needs 5 wait states in between.  The compiler inserts them
for its own instructions but cannot see into inline assembly, so a base moved into SGPRs
right before the statement could be read stale, that is as the registers' previous
contents: an arbitrary address.  This test compiles the decode sources to assembly with
the library's own flags and checks every inline-assembly vector-memory instruction
against the VALU writes of its base registers that precede it, counting s_nop wait
states, and every inline-assembly LDS DMA against a scalar write of M0 (the DMA's LDS
address) right before it, which needs 1 wait state.

The prologue loads of the decode kernels are inline assembly too (the compiler's own
waits would also stall on the DMAs it cannot see), so the compiler takes their
destination registers as written the moment the load issues.  A copy, spill or any other
use of such a register before the explicit `s_waitcnt vmcnt` that the kernel places
after it would read whatever the register held before the data arrived.  The scan also
checks that no instruction touches an inline-assembly load's destination registers
between the load and the next inline-assembly vmcnt wait."""
import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from looped_transformer_decode_amd import build as B

SOURCES = list(B.SOURCES)          # every source of the library
NEEDED = 5


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _valu_sgpr_defs(line):
    parts = line.split(None, 1)
    if len(parts) < 2 or not parts[0].startswith("v_"):
        return set()
    op, ops = parts[0], [o.strip() for o in parts[1].split(",")]
    out = set()
    if op.startswith(("v_readfirstlane", "v_readlane", "v_cmp")):
        out |= _sgprs(ops[0])
    if re.match(r"v_(mad_u64_u32|mad_i64_i32|add_co|sub_co|subrev_co|addc_co|subb_co|div_scale)", op) and len(ops) > 1:
        out |= _sgprs(ops[1])
    return out


def _vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vgprs_in(line):
    out = set()
    for tok in re.findall(r"v\[\d+:\d+\]|\bv\d+\b", line):
        out |= _vgprs(tok)
    return out


def _writes_m0(line):
    parts = line.split(None, 1)
    return len(parts) == 2 and parts[0].startswith("s_") and parts[1].split(",")[0].strip() == "m0"


def scan_load_uses(asm_text):
    """(kernel, load line, offending line) for every instruction that reads or writes a
    destination register of an inline-assembly load (a load into VGPRs, not an LDS DMA)
    after the load and before the next inline-assembly vmcnt wait, in program order."""
    bad, kern, inasm, pending = [], None, False, []
    for raw in asm_text.splitlines():
        line = raw.strip()
        if re.match(r"^_Z\S+:", line):
            kern, pending = line.split(":")[0], []
            continue
        if line.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if line.startswith(";;#ASMEND"):
            inasm = False
            continue
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        if inasm and re.match(r"s_waitcnt\b.*vmcnt", line):
            pending = []
            continue
        used = _vgprs_in(line)
        for regs, load in pending:
            if regs & used:
                bad.append((kern, load, line))
        m = re.match(r"(global_load_dword\S*|global_atomic\S*|buffer_load_dword\S*)\s+(v\[\d+:\d+\]|v\d+)", line)
        if inasm and m and "_lds_" not in line:
            pending.append((_vgprs(m.group(2)), line))
    return bad


def scan(asm_text):
    """(kernel, wait states, writer line, memory line) for every short gap, in straight-line order:
    a VALU write of an inline-assembly memory instruction's SGPR base fewer than 5 wait states
    before it, or a scalar write of M0 directly before an inline-assembly LDS DMA."""
    bad, hist, kern, inasm = [], [], None, False
    for raw in asm_text.splitlines():
        line = raw.strip()
        if re.match(r"^_Z\S+:", line):
            kern, hist = line.split(":")[0], []
            continue
        if line.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if line.startswith(";;#ASMEND"):
            inasm = False
            continue
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        nop = re.match(r"s_nop\s+(\d+)", line)
        if inasm and not nop:
            m = re.match(r"(global_load\S*|buffer_load\S*|global_store\S*)\s+.*?(s\[\d+:\d+\])", line)
            if m:
                base, ws = _sgprs(m.group(2)), 0
                for kind, val, text in reversed(hist):
                    if kind == "nop":
                        ws += val
                        continue
                    if val & base:
                        if ws < NEEDED:
                            bad.append((kern, ws, text, line))
                        break
                    ws += 1
                    if ws >= NEEDED:
                        break
            if "_lds_" in line:
                ws = 0
                for kind, val, text in reversed(hist):
                    if kind == "nop":
                        ws += val
                        continue
                    if _writes_m0(text):
                        if ws < 1:
                            bad.append((kern, ws, text, line))
                        break
                    ws += 1
                    if ws >= 1:
                        break
        hist.append(("nop", int(nop.group(1)) + 1, line) if nop else ("i", _valu_sgpr_defs(line), line))
        hist = hist[-16:]
    return bad


def test_scanner_flags_a_short_gap_and_counts_nops():
    text = "\n".join([
        "_Zk:",
        "v_mad_u64_u32 v[0:1], s[10:11], s4, v2, v[4:5]",
        "v_readfirstlane_b32 s11, v1",
        "v_readfirstlane_b32 s10, v0",
        ";;#ASMSTART",
        "global_load_lds_dwordx4 v8, s[10:11]",
        ";;#ASMEND",
        "v_readfirstlane_b32 s12, v0",
        ";;#ASMSTART",
        "s_nop 4",
        "global_load_lds_dwordx4 v8, s[12:13]",
        ";;#ASMEND",
        "s_add_i32 m0, s5, 0x400",
        ";;#ASMSTART",
        "global_load_lds_dwordx4 v8, s[12:13]",
        ";;#ASMEND",
        "s_mov_b32 m0, s6",
        ";;#ASMSTART",
        "s_nop 0",
        "global_load_lds_dwordx4 v8, s[12:13]",
        ";;#ASMEND",
    ])
    bad = scan(text)
    assert len(bad) == 2, bad
    assert bad[0][1] == 0 and "s10" in bad[0][2]
    assert bad[1][1] == 0 and "m0" in bad[1][2]


def test_load_use_scanner_flags_a_touch_before_the_wait():
    text = "\n".join([
        "_Zk:",
        ";;#ASMSTART",
        "global_load_dwordx4 v[20:23], v4, s[2:3]",
        ";;#ASMEND",
        "v_mov_b32 v30, v5",                       # other registers: fine
        "v_accvgpr_write_b32 a0, v21",             # a copy of a register still in flight
        ";;#ASMSTART",
        "s_waitcnt vmcnt(8)",
        ";;#ASMEND",
        "v_add_f32 v31, v20, v22",                 # after the wait: fine
        ";;#ASMSTART",
        "global_load_dwordx2 v[40:41], v4, s[2:3]",
        ";;#ASMEND",
        "s_waitcnt lgkmcnt(0)",                    # the compiler's wait does not count
        "v_mov_b32 v41, 0",
    ])
    bad = scan_load_uses(text)
    assert [b[2] for b in bad] == ["v_accvgpr_write_b32 a0, v21", "v_mov_b32 v41, 0"], bad


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_decode_kernels_wait_before_dma_bases():
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            with open(out) as f:
                return src, f.read()
        with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
            texts = list(ex.map(compile_one, SOURCES))
    for src, text in texts:
        if src in ("rq_decode.hip", "rq_decode_gqa.hip"):
            assert "global_load_lds_dwordx4" in text
        bad = scan(text)
        assert not bad, f"{src}: {len(bad)} DMA(s) too close to the VALU write of their base, e.g. {bad[0]}"
        bad = scan_load_uses(text)
        assert not bad, f"{src}: {len(bad)} use(s) of an inline-assembly load's registers before its wait, e.g. {bad[0]}"
