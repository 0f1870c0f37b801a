"""The LDS-DMA loads are inline asm (`dma16` / `dma4`), and the compiler inserts no wait states
in front of inline asm. On gfx9-family parts a vector-memory instruction that reads an SGPR
written by a VALU instruction less than five wait states earlier reads the old value; an SGPR
operand of a DMA (buffer resource, soffset) reloaded from a spill with `v_readlane_b32` right
before the asm would send the load to the wrong address. This test compiles the kernels that use
the DMAs to device assembly with the library's flags and checks that no such pair occurs.

The check walks each function's instructions in order (fall-through paths): for every inline-asm
memory instruction it looks back over the previous five wait states and reports the most recent
writer of each SGPR the instruction reads if that writer is a VALU instruction.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_scaled_precision_row_amd import build

DMA_SOURCES = ["gemm_fp8.hip", "gemm_w4a4.hip", "gemm_a16.hip", "gemm_skinny.hip"]
WAIT_STATES = 5


def _sgprs(tok):
    tok = tok.strip()
    m = re.match(r"^s\[(\d+):(\d+)\]$", tok)
    if m:
        return {"s%d" % i for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.match(r"^s\d+$", tok) or tok in ("m0", "vcc_lo", "vcc_hi"):
        return {tok}
    if tok == "vcc":
        return {"vcc_lo", "vcc_hi"}
    return set()


def find_hazards(asm_text):
    """(function, VALU instruction, inline-asm instruction) for each hazard in `asm_text`."""
    found = []
    func = None
    hist = []  # (text, SGPRs written, is VALU, wait states)
    in_asm = False
    for line in asm_text.split("\n"):
        t = line.strip()
        if re.match(r"^_Z\w+:", line):
            func, hist = line.split(":")[0], []
            continue
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        args = [a.strip() for a in t[len(op):].split(",")] if len(t) > len(op) else []
        if in_asm and (op.startswith("buffer_") or op.startswith("global_")):
            pending = {"m0"}
            for a in args[1:]:
                if a:
                    pending |= _sgprs(a.split()[0])
            ws = 0
            for ht, written, valu, n in reversed(hist):
                hit = written & pending
                if hit and valu:
                    found.append((func, ht, t))
                    break
                pending -= hit
                ws += n
                if ws >= WAIT_STATES or not pending:
                    break
        written = _sgprs(args[0].split()[0]) if args and args[0] else set()
        if op.startswith("v_cmp"):
            written |= {"vcc_lo", "vcc_hi"}
        m = re.match(r"s_nop\s+(\d+)", t)
        hist.append((t, written, op.startswith("v_"), int(m.group(1)) + 1 if m else 1))
        hist = hist[-16:]
    return found


def test_detector_flags_a_reloaded_soffset():
    # a spilled soffset reloaded by v_readlane right before the DMA (the pattern that was seen
    # to fetch the wrong rows), the same with enough wait states, and with an SALU rewrite
    bad = """_Zk:
	v_readlane_b32 s7, v250, 13
	;;#ASMSTART
	buffer_load_dwordx4 v68, s[24:27], s7 offen lds
	;;#ASMEND
"""
    waited = bad.replace("\t;;#ASMSTART", "\ts_nop 4\n\t;;#ASMSTART")
    rewritten = bad.replace("\t;;#ASMSTART", "\ts_mov_b32 s7, s9\n\t;;#ASMSTART")
    rsrc = bad.replace("v_readlane_b32 s7", "v_readfirstlane_b32 s26").replace("v250, 13", "v3")
    assert len(find_hazards(bad)) == 1
    assert find_hazards(waited) == []
    assert find_hazards(rewritten) == []
    assert len(find_hazards(rsrc)) == 1


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")
def test_no_valu_written_sgpr_read_by_inline_dma():
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            out = os.path.join(tmp, src + ".s")
            subprocess.run([build.HIPCC, "--cuda-device-only", "-S"] + flags + [os.path.join(build.CSRC, src), "-o", out],
                           check=True, capture_output=True)
            text = open(out).read()
            return src, text.count(";;#ASMSTART"), find_hazards(text)

        with ThreadPoolExecutor(max_workers=len(DMA_SOURCES)) as ex:
            results = list(ex.map(compile_one, DMA_SOURCES))
    for src, n_asm, hazards in results:
        assert n_asm > 0, src
        assert hazards == [], "%s: %s" % (src, hazards[:3])
