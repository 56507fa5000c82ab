"""Checks on the gfx950 assembly of the library's own kernels (CPU: hipcc cross-compiles).

* Inline assembly that issues several LDS or memory loads from one address register
  must not let the compiler give that register to the destination of an earlier load of
  the same block: the load's data may land before a later load of the block reads the
  address.  The helpers declare their outputs early-clobber; this scans every inline-asm
  block of the compiled kernels for a source register written earlier in the block.
* The device code is compiled without the packed-fp32 VALU forms.
"""

import os
import re
import shutil

import pytest

from mla_split_kv_decode_amd import build as mbuild

CSRC = mbuild.CSRC


def _hipcc_available():
    exe = mbuild.hipcc()
    return os.path.exists(exe) or shutil.which(exe) is not None


def _sources_with_asm():
    out = []
    for name in mbuild.SOURCES:
        with open(os.path.join(CSRC, name)) as f:
            if "asm volatile(\"" in f.read():
                out.append(name)
    return out


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not _hipcc_available():
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    texts = {}
    for name in mbuild.SOURCES:
        path = mbuild.device_asm(name, str(d / (name + ".s")))
        with open(path) as f:
            texts[name] = f.read()
    return texts


_REG = re.compile(r"v\[(\d+):(\d+)\]|\bv(\d+)\b")
_NO_DEST = ("ds_write", "ds_store", "global_store", "buffer_store", "global_load_lds", "buffer_load_lds",
            "global_atomic", "buffer_atomic", "flat_store")


def _vregs(text):
    regs = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def asm_block_hazards(asm_text):
    """(line, instruction, registers) for every instruction inside an inline-asm block
    that reads a VGPR written by an earlier load or instruction of the same block."""
    hazards = []
    lines = asm_text.splitlines()
    i = 0
    while i < len(lines):
        if "ASMSTART" not in lines[i]:
            i += 1
            continue
        written = set()
        i += 1
        while i < len(lines) and "ASMEND" not in lines[i]:
            ins = lines[i].split(";")[0].strip()
            i += 1
            if not ins or ins.startswith("s_"):
                continue
            op, _, rest = ins.partition(" ")
            operands = [o.strip() for o in rest.split(",") if o.strip()]
            if not operands:
                continue
            if op.startswith(_NO_DEST):
                dest, sources = set(), operands
            else:
                dest, sources = _vregs(operands[0]), operands[1:]
            read = set()
            for o in sources:
                read |= _vregs(o)
            if read & written:
                hazards.append((i, ins, sorted(read & written)))
            written |= dest
        i += 1
    return hazards


def test_scanner_flags_a_reused_address():
    # the pattern the compiler produced before the outputs were early-clobber
    bad = "\t;;#ASMSTART\n\tds_read_b32 v3, v3\n\tds_read_b32 v4, v3 offset:64\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n"
    good = "\t;;#ASMSTART\n\tds_read_b32 v4, v3\n\tds_read_b32 v5, v3 offset:64\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n"
    assert asm_block_hazards(bad) == [(3, "ds_read_b32 v4, v3 offset:64", [3])]
    assert asm_block_hazards(good) == []
    # an LDS-DMA copy has no destination register: its address operand is only read
    dma = "\t;;#ASMSTART\n\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v[2:3], off\n\t;;#ASMEND\n"
    assert asm_block_hazards(dma) == []


def test_inline_asm_blocks_keep_their_addresses(device_asm):
    assert _sources_with_asm(), "no inline assembly found in the sources"
    found = {name: asm_block_hazards(text) for name, text in device_asm.items()}
    assert sum(text.count("ASMSTART") for text in device_asm.values()) > 0
    bad = {k: v[:5] for k, v in found.items() if v}
    assert not bad, f"inline-asm blocks read registers they overwrote: {bad}"


def test_no_packed_fp32_forms(device_asm):
    pat = re.compile(r"^\s*v_pk_(add|mul|fma)_f32\b", re.M)
    hits = {name: len(pat.findall(text)) for name, text in device_asm.items()}
    assert not any(hits.values()), hits
