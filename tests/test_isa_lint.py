"""Checks on the gfx950 machine code built into libfr.so (CPU only).

A buffer store of more than 8 bytes reads its data registers over several
cycles after it issues, and a VALU write to those registers right behind it
has to wait one cycle. The compiler inserts that wait only when the store's
scalar offset is not a register. With an SGPR there it let the next
instruction rewrite the first data register, and on MI355X the store then
wrote the new value from lane 12 on (LayerNorm rows with a run of wrong
outputs from that lane on, changing from run to run). Every wide buffer
store in the kernels therefore keeps its scalar offset at the constant 0
(``store16`` in fr_device.h). This test disassembles the library's gfx950
code objects, which were built here, and checks that none has a register
there.
"""
import os
import re
import shutil
import struct
import subprocess

import pytest

import pointwise_reduction_amd as fr

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


def gfx950_code_objects(lib, workdir):
    """The gfx950 entries of every offload bundle in the library's
    .hip_fatbin section (one bundle per translation unit)."""
    fat = os.path.join(workdir, "fatbin")
    subprocess.run([tool("llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", lib, os.path.join(workdir, "x")],
                   check=True, capture_output=True)
    data = open(fat, "rb").read()
    out, pos = [], 0
    while (i := data.find(MAGIC, pos)) >= 0:
        count = struct.unpack_from("<Q", data, i + len(MAGIC))[0]
        p = i + len(MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if triple.endswith("gfx950"):
                out.append(data[i + off:i + off + size])
        pos = i + 1
    return out


@pytest.mark.skipif(not (tool("llvm-objcopy") and tool("llvm-objdump")), reason="LLVM binutils not found")
def test_no_wide_buffer_store_takes_a_register_scalar_offset(tmp_path):
    objs = gfx950_code_objects(fr.LIB_PATH, str(tmp_path))
    assert objs, "no gfx950 code object in libfr.so"
    wide = re.compile(r"^\s*buffer_store_dwordx[34]\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)")
    stores, bad = 0, []
    for n, blob in enumerate(objs):
        path = tmp_path / f"co{n}.o"
        path.write_bytes(blob)
        dis = subprocess.run([tool("llvm-objdump"), "-d", "--mcpu=gfx950", str(path)], check=True,
                             capture_output=True, text=True).stdout
        for line in dis.splitlines():
            m = wide.match(line)
            if m:
                stores += 1
                if m.group(4) not in ("0", "off"):
                    bad.append(line.strip())
    assert stores > 100, stores
    assert not bad, f"{len(bad)} wide buffer stores with a register scalar offset, e.g. {bad[:3]}"
