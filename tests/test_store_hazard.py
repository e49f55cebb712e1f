"""The kernels' gfx950 assembly has no VALU write of a wide store's data
registers in the instruction right after the store.

A buffer store of 96 or 128 bits whose soffset operand is a register is
taken by the compiler as free of the store-data hazard, so it may overwrite
the data registers with the very next VALU instruction; on gfx950 that has
corrupted stored dwords now and then (the dequantizing lookup streams, a few
rows per run).  The kernels keep soffset a constant, which makes the compiler
insert the wait state; this test compiles every kernel source to assembly
(no GPU needed) and checks the pattern is absent everywhere.
"""
import concurrent.futures
import os
import re
import subprocess

import pytest

from layer_embedding_lookup_amd import build as B

WIDE_STORES = ("buffer_store_dwordx3", "buffer_store_dwordx4", "global_store_dwordx3", "global_store_dwordx4",
               "flat_store_dwordx3", "flat_store_dwordx4")


def _regs(op):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", op)
    if m:
        return m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = re.match(r"([va])(\d+)$", op)
    return (m.group(1), {int(m.group(2))}) if m else (None, set())


def store_data_overwrites(asm: str):
    """(kernel, store, next instruction) for each wide store followed directly by a VALU write of its data."""
    found, kernel, prev = [], None, None
    for line in asm.splitlines():
        if re.match(r"^[A-Za-z_]\w*:", line):
            kernel, prev = line.split(":")[0], None
            continue
        text = line.split(";")[0].strip()
        if not text or text.startswith(".") or text.endswith(":"):
            continue
        parts = text.replace(",", " ").split()
        if prev is not None and parts[0].startswith("v_") and len(parts) > 1:
            f, dst = _regs(parts[1])
            if f == prev[0] and dst & prev[1]:
                found.append((kernel, prev[2], text))
        prev = None
        if parts[0] in WIDE_STORES:
            data = parts[1] if parts[0].startswith("buffer") else parts[2]
            f, regs = _regs(data)
            prev = (f, regs, text)
    return found


def test_scanner_finds_the_pattern():
    asm = ("k:\n\tbuffer_store_dwordx4 v[0:3], v4, s[0:3], s5 offen\n\tv_mov_b32_e32 v2, 0\n"
           "\tglobal_store_dwordx4 v[8:9], v[10:13], off\n\tv_mov_b32_e32 v0, 0\n"
           "\tbuffer_store_dwordx4 v[20:23], v4, s[0:3], 0 offen\n\ts_nop 0\n\tv_mov_b32_e32 v20, 0\n")
    hits = store_data_overwrites(asm)
    assert len(hits) == 1 and hits[0][1].startswith("buffer_store_dwordx4 v[0:3]")


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc is needed to compile the kernels")
def test_no_store_data_overwrite_in_any_kernel(tmp_path):
    srcs = [s for s in B.SOURCES if s.endswith(".hip")]

    def asm_of(src):
        out = tmp_path / (src + ".s")
        cmd = [B.hipcc(), *B.common_flags(), "--cuda-device-only", "-S", "-o", str(out), os.path.join(B.CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        return src, out.read_text()

    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        listings = list(ex.map(asm_of, srcs))
    bad = [(src, hit) for src, text in listings for hit in store_data_overwrites(text)]
    assert not bad, bad[:5]
