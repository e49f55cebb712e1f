"""Two register hazards, checked in the kernels' gfx950 assembly (compiled
here, no GPU needed).

1. No VALU write of a wide store's data registers in the instruction right
   after the store.  A buffer store of 96 or 128 bits whose soffset operand is
   a register is taken by the compiler as free of the store-data hazard, so it
   may overwrite the data registers with the very next VALU instruction; on
   gfx950 that has corrupted stored dwords now and then (the dequantizing
   lookup streams, a few rows per run).  The kernels keep soffset a constant,
   which makes the compiler insert the wait state.
2. No instruction touches the destination registers of an LDS read written
   in inline asm before an lgkmcnt(0) wait.  The compiler takes such a read's
   registers as written when the asm ends; the kv_proj pipelines keep them
   reserved by naming them in the wait that follows, including the wait after
   the last slice, whose look-ahead reads are never used.
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


def _all_regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.add((m.group(1), int(m.group(2))))
    return out


def _blocks(asm: str):
    """{kernel: [[label, [(in_asm, instruction)], [branch targets], falls_through]]}: each kernel's basic
    blocks in text order, split at labels and after branches and s_endpgm."""
    out, blocks, in_asm = {}, None, False
    for line in asm.splitlines():
        if re.match(r"^[A-Za-z_]\w*:", line):
            name = line.split(":")[0]
            blocks = out.setdefault(name, [])
            blocks.append([name, [], [], True])
            continue
        if blocks is None:
            continue
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        text = line.split(";")[0].strip()
        if not text:
            continue
        if re.match(r"^\.L\w+:$", text):
            blocks.append([text[:-1], [], [], True])
            continue
        if text.startswith("."):
            continue
        op = text.split()[0]
        blocks[-1][1].append((in_asm, text))
        if op.startswith("s_cbranch") or op == "s_branch":
            blocks[-1][2].append(text.split()[1])
            blocks[-1][3] = op != "s_branch"
            blocks.append([None, [], [], True])
        elif op in ("s_endpgm", "s_setpc_b64"):
            blocks[-1][3] = False
            blocks.append([None, [], [], True])
    return out


def inline_lds_read_reuses(asm: str):
    """(kernel, pending read, instruction) for each instruction that names a register an inline-asm
    LDS read may still be loading: one that no lgkmcnt(0) wait separates from the read on some path
    through the kernel's branches (a forward data-flow over its basic blocks)."""
    found = []
    for kernel, blocks in _blocks(asm).items():
        index = {b[0]: i for i, b in enumerate(blocks) if b[0]}
        succ = []
        for i, b in enumerate(blocks):
            s = [index[t] for t in b[2] if t in index]
            if b[3] and i + 1 < len(blocks):
                s.append(i + 1)
            succ.append(s)
        entry = [{} for _ in blocks]

        def walk(i, hits):
            pending = dict(entry[i])
            for in_asm, text in blocks[i][1]:
                op = text.split()[0]
                if op == "s_waitcnt" and "lgkmcnt(0)" in text:
                    pending = {}
                    continue
                hit = _all_regs(text) & set(pending)
                if hit and hits is not None:
                    hits.append((kernel, pending[next(iter(hit))], text))
                if in_asm and op.startswith("ds_read"):
                    for r in _all_regs(text.split()[1].rstrip(",")):
                        pending[r] = text
            return pending

        work = list(range(len(blocks)))
        while work:  # the pending sets only grow, so this ends
            i = work.pop()
            for j in succ[i]:
                grown = False
                for r, t in walk(i, None).items():
                    if r not in entry[j]:
                        entry[j][r] = t
                        grown = True
                if grown:
                    work.append(j)
        for i in range(len(blocks)):
            walk(i, found)
    return found


def test_scanners_find_the_patterns():
    asm = ("k:\n\tbuffer_store_dwordx4 v[0:3], v4, s[0:3], s5 offen\n\tv_mov_b32_e32 v2, 0\n"
           "\tglobal_store_dwordx4 v[8:9], v[10:13], off\n\tv_mov_b32_e32 v0, 0\n"
           "\tbuffer_store_dwordx4 v[20:23], v4, s[0:3], 0 offen\n\ts_nop 0\n\tv_mov_b32_e32 v20, 0\n")
    hits = store_data_overwrites(asm)
    assert len(hits) == 1 and hits[0][1].startswith("buffer_store_dwordx4 v[0:3]")
    asm = ("k:\n\t;;#ASMSTART\n\tds_read_b128 v[8:11], v1\n\t;;#ASMEND\n\tv_mfma_f32_16x16x32_bf16 v[0:3], "
           "v[20:23], v[24:27], v[0:3]\n\tv_add_u32_e32 v9, 1, v2\n\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32_e32 v8, 0\n"
           "\tds_read_b128 v[30:33], v1\n\tv_mov_b32_e32 v30, 0\n")
    hits = inline_lds_read_reuses(asm)
    assert len(hits) == 1 and hits[0][2].startswith("v_add_u32_e32 v9")
    # a loop body laid out before its header: the prologue's reads reach the body only through the
    # header's wait, so reusing their registers there is fine
    asm = ("k:\n\t;;#ASMSTART\n\tds_read_b128 v[8:11], v1\n\t;;#ASMEND\n\ts_branch .LBB0_2\n"
           ".LBB0_1:\n\tv_mov_b32_e32 v8, 0\n.LBB0_2:\n\ts_waitcnt lgkmcnt(0)\n\ts_cbranch_scc1 .LBB0_1\n"
           "\ts_endpgm\n")
    assert inline_lds_read_reuses(asm) == []
    # a read issued at the end of a loop body reaches the top of the body again over the back edge
    asm = ("k:\n.LBB0_1:\n\tv_mov_b32_e32 v21, 0\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMSTART\n\tds_read_b128 "
           "v[20:23], v1\n\t;;#ASMEND\n\ts_cbranch_scc1 .LBB0_1\n\ts_waitcnt lgkmcnt(0)\n\ts_endpgm\n")
    hits = inline_lds_read_reuses(asm)
    assert len(hits) == 1 and hits[0][2] == "v_mov_b32_e32 v21, 0", hits
    # and one taken branch skipping the wait is enough
    asm = ("j:\n\t;;#ASMSTART\n\tds_read_b128 v[8:11], v1\n\t;;#ASMEND\n\ts_cbranch_scc1 .LBB1_1\n"
           "\ts_waitcnt lgkmcnt(0)\n.LBB1_1:\n\tv_mov_b32_e32 v9, 0\n\ts_endpgm\n")
    hits = inline_lds_read_reuses(asm)
    assert len(hits) == 1 and hits[0][2] == "v_mov_b32_e32 v9, 0", hits


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    if not os.path.exists(B.hipcc()):
        pytest.skip("hipcc is needed to compile the kernels")
    tmp = tmp_path_factory.mktemp("asm")
    srcs = [s for s in B.SOURCES if s.endswith(".hip")]

    def asm_of(src):
        out = tmp / (src + ".s")
        cmd = [B.hipcc(), *B.common_flags(), "--cuda-device-only", "-S", "-o", str(out), os.path.join(B.CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        return src, out.read_text()

    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        return list(ex.map(asm_of, srcs))


def test_no_store_data_overwrite_in_any_kernel(listings):
    bad = [(src, hit) for src, text in listings for hit in store_data_overwrites(text)]
    assert not bad, bad[:5]


def test_no_early_reuse_of_inline_lds_read_targets(listings):
    assert sum(text.count("ds_read_b128") for src, text in listings if src == "ple_kv_proj.hip") > 0
    bad = [(src, hit) for src, text in listings for hit in inline_lds_read_reuses(text)]
    assert not bad, bad[:5]
