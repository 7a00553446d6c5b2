"""The generated gfx950 code has no store-data race of the kind found in the split-slice pieces.

A vector store of more than 64 bits reads its data registers after it issues.  When the next
instruction (across a basic-block boundary the compiler did not pad) wrote one of those
registers, the store now and then sent the new value: element 0 of row block 7 of a 128-row
piece went out as zero.  The kernels now keep wait states there; this test compiles every
kernel source to gfx950 assembly with the library's own flags and checks that no store of
three or four dwords has a data register written by a VALU or matrix instruction (one register
or a register range) within the next two instructions without an s_nop or s_waitcnt in
between.  Host-only: it needs hipcc, no GPU.
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
    for src, asm in zip(srcs, asms):
        found = unpadded_store_data_writes(asm)
        assert not found, (os.path.basename(src), found[:3])
