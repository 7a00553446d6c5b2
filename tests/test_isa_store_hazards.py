"""The generated gfx950 code has no store-data race of the kind found in the split-slice pieces,
and no matrix instruction reads an operand written right before it without wait states.

A vector store of more than 64 bits reads its data registers after it issues.  When the next
instruction (across a basic-block boundary the compiler did not pad) wrote one of those
registers, the store now and then sent the new value: element 0 of row block 7 of a 128-row
piece went out as zero.  The kernels now keep wait states there; this test compiles every
kernel source to gfx950 assembly with the library's own flags and checks that no store of
three or four dwords has a data register written by a VALU or matrix instruction (one register
or a register range) within the next two instructions without an s_nop or s_waitcnt in
between.  It also checks that every matrix instruction whose A or B operand register was
written by a VALU instruction has at least two wait states after that write (the compiler
inserts them for the instructions it knows; an inline-asm write feeding a matrix operand had
none, and the instruction read stale values now and then).  Host-only: it needs hipcc, no GPU.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from mixed_precision_w4a16_amd import build

pytestmark = pytest.mark.timeout(600)

STORE = re.compile(r"(buffer|global)_store_dwordx[34] ")


def device_asm(src: str, out: str) -> str:
    cmd = [c for c in build.command(out) if c not in ("-fPIC", "-shared") and c not in build.SOURCES]
    i = cmd.index("-o")
    cmd = cmd[:i] + ["-S", "--offload-device-only", "-I", os.path.dirname(src), src] + cmd[i:]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def unpadded_store_data_writes(asm: str):
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    lines = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    found = []
    for k, l in enumerate(lines):
        if not STORE.match(l):
            continue
        m = (re.match(r"\S+ v\[(\d+):(\d+)\]", l) if l.startswith("buffer")
             else re.search(r", v\[(\d+):(\d+)\]", l))
        if not m:
            continue
        lo, hi = int(m[1]), int(m[2])
        for nxt in lines[k + 1:k + 3]:
            if nxt.startswith("s_nop") or nxt.startswith("s_waitcnt"):
                break
            d = vector_dest(nxt)
            if d and d[0] <= hi and lo <= d[1]:
                found.append((l, nxt))
                break
    return found


def vector_dest(line: str):
    """The VGPR range (first, last) a VALU or matrix instruction writes, or None: a single
    register (v_mov_b32 v2, ...), a range (v_mov_b64 v[2:3], ..., v_mfma_... v[0:3], ...)."""
    w = re.match(r"v_\S+\s+v\[(\d+):(\d+)\]", line)
    if w:
        return int(w[1]), int(w[2])
    w = re.match(r"v_\S+\s+v(\d+)\b", line)
    if w:
        return int(w[1]), int(w[1])
    return None


MFMA = re.compile(r"v_s?mfmac?_\S+\s+(.*)$")


def _regs(op: str):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return int(m[1]), int(m[2])
    m = re.fullmatch(r"v(\d+)", op)
    if m:
        return int(m[1]), int(m[1])
    return None


def unpadded_mfma_operand_writes(asm: str, need: int = 2):
    """Matrix instructions whose A or B operand was written by a VALU instruction fewer than
    `need` wait states earlier (each instruction in between is one, s_nop n is n + 1),
    within straight-line code.  The compiler pads such reads for the instructions it knows;
    an inline-asm write right before the read is what this catches."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    lines = [l for l in lines if l and not l.startswith(".")]
    found = []
    for k, l in enumerate(lines):
        m = MFMA.match(l)
        if not m or l.endswith(":"):
            continue
        ops = [o.strip() for o in m[1].split(",")]
        srcs = [r for r in (_regs(o) for o in ops[1:3]) if r]
        slots = 0
        for prev in reversed(lines[max(0, k - need):k]):
            if prev.endswith(":") or prev.startswith("s_cbranch") or prev.startswith("s_branch"):
                break
            if not MFMA.match(prev) and not prev.startswith("s_"):
                d = vector_dest(prev)
                if d and any(lo <= d[1] and d[0] <= hi for lo, hi in srcs):
                    found.append((prev, l))
                    break
            n = re.match(r"s_nop\s+(\d+)", prev)
            slots += int(n[1]) + 1 if n else 1
            if slots >= need:
                break
    return found


def smfmac_accumulator_hazards(asm: str, before: int = 4, after: int = 10):
    """Sparse matrix instructions (v_smfmac) whose accumulator -- their destination register,
    read and written by the instruction -- was written by a VALU instruction within `before`
    instructions before them, or is read by a non-matrix instruction within `after`
    instructions behind them, in straight-line code.  Per-tile sums started from a zero moved
    into the accumulator right before the instruction and read right behind it gave wrong
    results on gfx950 with the compiler's own wait states; the kernels keep the sparse
    instruction's accumulators loop-carried and read them only after the last tile."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    lines = [l for l in lines if l and not l.startswith(".")]
    found = []
    for k, l in enumerate(lines):
        if not l.startswith("v_smfmac"):
            continue
        d = _regs(l.split(None, 1)[1].split(",")[0].strip())
        for prev in reversed(lines[max(0, k - before):k]):
            if prev.endswith(":"):
                break
            w = vector_dest(prev)
            if w and not MFMA.match(prev) and w[0] <= d[1] and d[0] <= w[1]:
                found.append((prev, l))
                break
        for nxt in lines[k + 1:k + 1 + after]:
            if nxt.endswith(":"):
                break
            if MFMA.match(nxt) or " " not in nxt:
                continue
            ops = [o.strip() for o in nxt.split(None, 1)[1].split(",")]
            srcs = [r for r in (_regs(o) for o in (ops[1:] if nxt.startswith("v_") else ops)) if r]
            if any(lo <= d[1] and d[0] <= hi for lo, hi in srcs):
                found.append((l, nxt))
                break
    return found


def test_smfmac_scanner_flags_fresh_and_early_read_accumulators():
    sm = "v_smfmac_f32_16x16x64_f16 v[70:73], v[58:61], v[2:9], v40\n"
    assert len(smfmac_accumulator_hazards("v_mov_b64_e32 v[70:71], s[28:29]\nv_lshrrev_b32 v1, 8, v2\n" + sm)) == 1
    assert len(smfmac_accumulator_hazards(sm + "s_nop 7\nv_sub_f32_e32 v3, v73, v65\n")) == 1
    assert smfmac_accumulator_hazards(sm + "v_smfmac_f32_16x16x64_f16 v[70:73], v[62:65], v[10:17], v38\n") == []
    assert smfmac_accumulator_hazards("v_mov_b64_e32 v[80:81], 0\n" + sm + "v_add_f32 v3, v74, v65\n") == []


def test_mfma_scanner_flags_an_unpadded_operand_write():
    mf = "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
    assert len(unpadded_mfma_operand_writes("v_and_or_b32 v9, v1, v2, v3\n" + mf)) == 1
    assert len(unpadded_mfma_operand_writes("v_and_or_b32 v5, v1, v2, v3\ns_waitcnt vmcnt(0)\n" + mf)) == 1
    assert unpadded_mfma_operand_writes("v_and_or_b32 v9, v1, v2, v3\ns_nop 1\n" + mf) == []
    assert unpadded_mfma_operand_writes("v_and_or_b32 v9, v1, v2, v3\ns_waitcnt vmcnt(0)\ns_nop 0\n" + mf) == []
    assert unpadded_mfma_operand_writes("v_and_or_b32 v12, v1, v2, v3\n" + mf) == []
    assert len(unpadded_mfma_operand_writes("v_mov_b64 v[6:7], 0\n" + mf)) == 1


def test_scanner_flags_the_pattern_and_passes_padded_code():
    bad = "buffer_store_dwordx4 v[2:5], v254, s[28:31], s1 offen sc1\n.LBB0_1:\nv_mov_b32_e32 v2, 0\n"
    ok = "buffer_store_dwordx4 v[2:5], v254, s[28:31], s1 offen sc1\ns_nop 7\nv_mov_b32_e32 v2, 0\n"
    other = "buffer_store_dwordx4 v[2:5], v254, s[28:31], s1 offen sc1\nv_mov_b32_e32 v6, 0\n"
    assert len(unpadded_store_data_writes(bad)) == 1
    assert unpadded_store_data_writes(ok) == []
    assert unpadded_store_data_writes(other) == []
    # writes of register ranges: a 64-bit move and a matrix instruction's destination
    st = "buffer_store_dwordx4 v[2:5], v254, s[28:31], s1 offen sc1\n"
    assert len(unpadded_store_data_writes(st + "v_mov_b64 v[4:5], 0\n")) == 1
    assert len(unpadded_store_data_writes(st + "v_mov_b64 v[0:1], 0\n")) == 0
    assert len(unpadded_store_data_writes(st + "v_mov_b64 v[0:1], 0\nv_mov_b64 v[0:1], 0\n")) == 0
    assert len(unpadded_store_data_writes(
        st + "s_add_u32 s0, s0, 4\nv_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[14:17], v[0:3]\n")) == 1
    assert len(unpadded_store_data_writes(
        st + "v_mfma_f32_16x16x32_f16 v[6:9], v[10:13], v[14:17], v[6:9]\n")) == 0
    assert len(unpadded_store_data_writes(
        "global_store_dwordx3 v0, v[2:4], s[0:1]\nv_mov_b64 v[3:4], 0\n")) == 1


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                    reason="hipcc not available")
def test_no_store_data_written_right_behind_a_wide_store():
    srcs = [s for s in build.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
            asms = list(ex.map(lambda s: device_asm(s, os.path.join(d, os.path.basename(s) + ".s")),
                               srcs))
    assert sum(len(STORE.findall(asm)) for asm in asms) > 1000     # the pieces' stores are there
    assert sum(len(re.findall(r"v_mfma_", asm)) for asm in asms) > 10000
    for src, asm in zip(srcs, asms):
        found = unpadded_store_data_writes(asm)
        assert not found, (os.path.basename(src), found[:3])
        found = unpadded_mfma_operand_writes(asm)
        assert not found, (os.path.basename(src), found[:3])
        found = smfmac_accumulator_hazards(asm)
        assert not found, (os.path.basename(src), found[:3])
