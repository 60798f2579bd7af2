"""Resource checks of the built library's gfx950 code object (CPU only: reads the kernel
metadata that the compiler writes into the code object, runs nothing).

Every kernel runs without a private (scratch) segment and without register spills to
memory, and the fused kernels' shared arrays leave room for three workgroups per compute
unit outside the verify launches (which use larger arrays at head dim 128)."""
import os
import re
import shutil
import struct
import subprocess

import pytest

from gated_deltanet_linear_decode_amd import abi

READELF = "/opt/rocm/llvm/bin/llvm-readelf"
LDS_PER_CU = 160 * 1024


def _code_object(tmp_path):
    data = open(abi.LIB_PATH, "rb").read()
    base = data.find(b"__CLANG_OFFLOAD_BUNDLE__")
    assert base >= 0, "no offload bundle in the library"
    (count,) = struct.unpack_from("<Q", data, base + 24)
    pos = base + 32
    for _ in range(count):
        off, size, tlen = struct.unpack_from("<QQQ", data, pos)
        pos += 24
        triple = data[pos:pos + tlen].decode()
        pos += tlen
        if triple.endswith("gfx950"):
            out = tmp_path / "gfx950.co"
            out.write_bytes(data[base + off:base + off + size])
            return out
    raise AssertionError("no gfx950 code object in the library")


def _kernels(tmp_path):
    if not os.path.exists(abi.LIB_PATH):
        pytest.skip("the library is not built")
    if shutil.which(READELF) is None:
        pytest.skip("llvm-readelf is not installed")
    notes = subprocess.run([READELF, "--notes", str(_code_object(tmp_path))], check=True,
                           capture_output=True, text=True).stdout
    # one list entry per kernel at two spaces; its own keys at four (the argument list's
    # entries sit deeper)
    listing = re.split(r"\namdhsa\.", notes.split("amdhsa.kernels:", 1)[1])[0]
    entries = re.split(r"\n  - ", listing)[1:]
    kernels = {}
    for e in entries:
        fields = dict(re.findall(r"^ {4}\.(\w+):\s+(\S+)", "    " + e, re.M))
        kernels[fields["name"]] = fields
    assert kernels, "no kernel metadata found"
    return kernels


def test_no_kernel_has_scratch_or_spills_to_memory(tmp_path):
    kernels = _kernels(tmp_path)
    # weight layouts (2) x formats (3) x head dims (3) x state types (2) x {decode, decode with
    # the fold, verify}, and the one-token verify at head dim 128 (2 x 3 x 2)
    assert sum("decode_kernel" in n for n in kernels) == 2 * 3 * 3 * 2 * 3 + 2 * 3 * 2
    bad = {n: (k["private_segment_fixed_size"], k["vgpr_spill_count"]) for n, k in kernels.items()
           if int(k["private_segment_fixed_size"]) or int(k["vgpr_spill_count"])}
    assert not bad, bad


def test_shared_arrays_fit_three_workgroups_per_cu_outside_chunked_verify(tmp_path):
    kernels = _kernels(tmp_path)
    for name, k in kernels.items():
        lds = int(k["group_segment_fixed_size"])
        # decode_kernel<PACKED, FMT, DK, ST, FOLD, MULTI, DST>: MULTI at DK 128 is the chunked verify
        chunked = re.search(r"decode_kernelILb\dELi\dELi128E\wLb\dELb1E", name) is not None
        assert lds <= (LDS_PER_CU // 2 if chunked else LDS_PER_CU // 3), (name, lds)
