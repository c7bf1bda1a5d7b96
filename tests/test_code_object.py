"""The gfx950 code object inside the built library: no kernel may use scratch
memory (a private segment, i.e. spilled vector registers that would turn into
global-memory traffic in the hot loops), and every kernel fits the CU's
register file and LDS.  Reads the library built in this checkout (no GPU); the
per-kernel registers and LDS are printed with -s."""
import os
import re
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_prefill_amd", "libkda.so")
READELF = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-readelf")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
LDS_BYTES = 160 * 1024          # per workgroup on gfx950
VGPRS = 512                     # per lane; .vgpr_count includes the accumulation registers


def _gfx950_objects(lib_bytes: bytes):
    """The gfx950 entries of the library's (uncompressed) offload bundles, one
    bundle per linked object: magic, entry count, then per entry offset,
    size, triple length and triple."""
    objs = []
    base = lib_bytes.find(BUNDLE_MAGIC)
    while base >= 0:
        (count,) = struct.unpack_from("<Q", lib_bytes, base + len(BUNDLE_MAGIC))
        pos = base + len(BUNDLE_MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", lib_bytes, pos)
            pos += 24
            triple = lib_bytes[pos:pos + tlen].decode()
            pos += tlen
            if triple.endswith("gfx950"):
                objs.append(lib_bytes[base + off:base + off + size])
        base = lib_bytes.find(BUNDLE_MAGIC, pos)
    if not objs:
        pytest.skip("no uncompressed gfx950 code object in the library")
    return objs


def _kernels():
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    if not os.path.exists(READELF):
        pytest.skip("llvm-readelf not found")
    with open(LIB, "rb") as fh:
        objs = _gfx950_objects(fh.read())
    notes = ""
    for co in objs:
        with tempfile.NamedTemporaryFile(suffix=".co") as tmp:
            tmp.write(co)
            tmp.flush()
            notes += subprocess.run([READELF, "--notes", tmp.name], capture_output=True, text=True,
                                    check=True).stdout
    kernels, cur = [], None
    for line in notes.splitlines():
        if re.match(r"^  - \.", line):          # a new entry of amdhsa.kernels
            cur = {}
            kernels.append(cur)
            line = "    " + line[4:]
        m = re.match(r"^    \.(\w+):\s+(\S+)", line)
        if cur is not None and m:
            cur[m.group(1)] = m.group(2)
    kernels = [k for k in kernels if "name" in k]
    assert kernels, "no kernel metadata found"
    return kernels


def test_every_kernel_is_present():
    names = " ".join(k["name"] for k in _kernels())
    for kern in ("kda_intra_kernel", "kda_fused_prefill_kernel", "kda_scan_kernel", "kda_decode_kernel",
                 "kda_decode_tokens_kernel", "kda_decode_conv_kernel", "kda_conv_kernel",
                 "kda_conv_window_kernel"):
        assert kern in names, kern
    # the scan with one and with two 16-column slices per workgroup (bf16)
    assert "kda_scan_kernelIDF16bLi128ELi128ELi1E" in names
    assert "kda_scan_kernelIDF16bLi128ELi128ELi2E" in names


def test_no_kernel_uses_scratch():
    bad = []
    for k in _kernels():
        print("%-70s vgpr %3s agpr %3s sgpr-spill %3s lds %6s" % (
            k["name"][:70], k.get("vgpr_count"), k.get("agpr_count"), k.get("sgpr_spill_count"),
            k.get("group_segment_fixed_size")))
        if int(k.get("private_segment_fixed_size", 0)) or int(k.get("vgpr_spill_count", 0)):
            bad.append((k["name"], k.get("private_segment_fixed_size"), k.get("vgpr_spill_count")))
    assert not bad, bad


def test_resources_fit_the_cu():
    for k in _kernels():
        assert int(k["group_segment_fixed_size"]) <= LDS_BYTES, k["name"]
        assert int(k["vgpr_count"]) <= VGPRS, k["name"]
