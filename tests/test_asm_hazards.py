"""Static check of the gfx950 code (CPU only; needs hipcc, no GPU).

The KV-major kernels read LDS operands with hand-written asm blocks that
issue several reads from one address register.  If the register allocator
gave a read's destination the address register, the next read of the same
block would use the overwritten value.  The asm outputs are declared
early-clobber to forbid that; this test compiles the kernels to assembly and
checks every asm block of every instantiation: no LDS read may take its
address from a register written earlier in the same block.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from block_sparse_long_msa_amd import build as B

READ = re.compile(r"^(ds_read\w*)\s+v\[(\d+):(\d+)\],\s*v(\d+)\b")


def clobbered_address_reads(asm_text: str):
    """(line, instruction) of LDS reads inside one asm block whose address
    register an earlier read of the same block wrote."""
    bad = []
    written = None
    for n, line in enumerate(asm_text.splitlines(), 1):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            written = set()
            continue
        if t.startswith(";;#ASMEND"):
            written = None
            continue
        if written is None:
            continue
        m = READ.match(t)
        if m:
            lo, hi, addr = int(m.group(2)), int(m.group(3)), int(m.group(4))
            if addr in written:
                bad.append((n, t))
            written.update(range(lo, hi + 1))
    return bad


def test_scanner_flags_a_clobbered_address():
    """The scanner itself: a block whose first read overwrites the address."""
    bad_block = (";;#ASMSTART\nds_read_b64_tr_b16 v[2:3], v2 offset:0\n"
                 "ds_read_b64_tr_b16 v[4:5], v2 offset:0x800\n;;#ASMEND\n")
    good_block = (";;#ASMSTART\nds_read_b64_tr_b16 v[2:3], v6 offset:0\n"
                  "ds_read_b64_tr_b16 v[4:5], v6 offset:0x800\n;;#ASMEND\n")
    assert len(clobbered_address_reads(bad_block)) == 1
    assert clobbered_address_reads(good_block) == []


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("variant", ["release", "debug"])
def test_kv_major_asm_blocks_keep_their_address(variant):
    src = os.path.join(B.CSRC, "attn_kvmajor.hip")
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "attn_kvmajor.s")
        cmd = ["hipcc", "--cuda-device-only", "-S", *[a for a in B.COMMON if a != "-fPIC"],
               *(["-DMSA_DEBUG"] if variant == "debug" else []), src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    assert ";;#ASMSTART" in text
    n_reads = sum(1 for line in text.splitlines() if READ.match(line.strip()))
    assert n_reads > 0
    assert clobbered_address_reads(text) == []


def test_multi_read_asm_outputs_are_early_clobber():
    """Asm blocks that issue several reads before their outputs are dead
    must declare the outputs early-clobber (=&v), whatever the allocator
    happens to choose today."""
    text = open(os.path.join(B.CSRC, "attn_kvmajor.hip")).read()
    for fn in ("vt_tile_read", "k_step_read4"):
        start = text.index(f"void {fn}(")
        body = text[start:text.index("\n}\n", start)]
        assert "asm volatile" in body
        assert '"=v"(' not in body, fn
        assert '"=&v"(' in body, fn
