"""CPU audit of the GEMM kernels' LDS-DMA addressing (no GPU).

tests/dma_audit.hip calls the address functions the kernels use (csrc/gemm_tiles.hpp) for
every load of every launched tile configuration and checks each lane's LDS destination and
buffer offsets; see its header. This test builds it with hipcc (host code only), runs it, and
checks that planted addressing mistakes (in a copy of the header, on the CPU) make it fail.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_row_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _build_and_run(tmp_path, include_dir):
    exe = str(tmp_path / "dma_audit")
    cmd = [HIPCC, "-std=c++17", "-O1", "-x", "hip", "--cuda-host-only", "-I" + include_dir, "-I" + CSRC,
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "dma_audit.hip"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    return subprocess.run([exe], capture_output=True, text=True, timeout=600)


def test_every_lds_dma_load_is_in_bounds(tmp_path):
    r = _build_and_run(tmp_path, CSRC)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "all LDS-DMA loads in bounds" in r.stdout
    # every kernel family was enumerated
    for family in ("fp8 256x192", "fp8 128x128 ring 2", "fp8 256x256", "fp8 scales 256x192", "fp8 scales 64x64",
                   "fp8 adapter rows 256x192", "fp8 adapter rows late 256x192", "w4a4 256x256", "a16 nvfp4",
                   "a16 e4m3", "skinny w8a8", "skinny w8a16"):
        assert re.search(r"^ok %s" % family, r.stdout, re.M), family


@pytest.mark.parametrize("old,new,what", [
    # an out-of-range mark that lands inside the records of large tiles
    ("constexpr int kOutOfRange = 0x40000000;", "constexpr int kOutOfRange = 0x00100000;", "out-of-range mark"),
    # the K check forgotten: a partial last stage reads the next row's bytes
    ("const int voff = (kb + c * Rg::VPC < K) ? lrow * stride + (c << 4) : kOutOfRange;",
     "const int voff = lrow * stride + (c << 4);", "past K"),
    # lanes written one chunk too far in LDS
    ("return DmaAddr{ld * 1024 + 16 * lane, voff, ld * Rg::RPL * stride + kbyte};",
     "return DmaAddr{ld * 1024 + 16 * lane + 16, voff, ld * Rg::RPL * stride + kbyte};", "LDS destination"),
    # dword scale loads written 8 bytes apart in LDS instead of 4
    ("return DmaAddr{ld * 256 + 4 * lane, voff, ld * 32 * ks + (kb >> 4)};",
     "return DmaAddr{ld * 256 + 8 * lane, voff, ld * 32 * ks + (kb >> 4)};", "scale LDS destination"),
    # a few-token activation load whose row offset ignores the row pitch
    ("const int voff = kv + c * vpc < K ? row * pitch + kbyte + 16 * c : kOutOfRange;",
     "const int voff = kv + c * vpc < K ? row * (pitch + 16) + kbyte + 16 * c : kOutOfRange;", "row pitch"),
])
def test_planted_addressing_mistakes_are_caught(tmp_path, old, new, what):
    mdir = tmp_path / "mutant"
    mdir.mkdir()
    text = open(os.path.join(CSRC, "gemm_tiles.hpp")).read()
    assert old in text
    (mdir / "gemm_tiles.hpp").write_text(text.replace(old, new))
    r = _build_and_run(tmp_path, str(mdir))
    assert r.returncode != 0 and "VIOLATION" in r.stdout, (what, r.stdout[-500:])
