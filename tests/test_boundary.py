"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/kda.h declares, and rejects bad arguments before any launch.

Only error paths are exercised here (they return before any HIP call), so no
GPU is needed.  Fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from linear_attention_prefill_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from linear_attention_prefill_amd import build
        build.build()
    return K.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_library_matches_sources():
    """libkda.so was built from the sources in the tree (the build records a
    hash of csrc/ and include/ next to it); a stale library would make every
    other test check old code."""
    from linear_attention_prefill_amd import build
    if not os.path.exists(build.HASH_FILE):
        build.build()
    with open(build.HASH_FILE) as fh:
        built = fh.read().strip()
    assert built == build.source_hash(), "libkda.so is stale: run python -m linear_attention_prefill_amd.build"


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("kda_chunk_prefill", "kda_decode_step", "kda_prefill_workspace_size",
              "kda_status_string", "kda_version", "kda_chunk_prefill_timed",
              "kda_decode_step_lines", "kda_decode_tokens", "kda_chunk_prefill_conv",
              "kda_decode_step_conv", "kda_prefill_check", "kda_chunk_prefill_static",
              "kda_prefill_windows", "kda_prefill_fuse_chunks", "kda_phase_clocks",
              "kda_stream_probe", "kda_mfma_probe"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_version() == 109
    for code in range(9):
        s = lib.kda_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.kda_status_string(99).decode() == "unknown status"


def test_phase_clocks_need_the_instrumented_build(lib):
    """libkda.so records no phase clocks: kda_phase_clocks says so before any
    HIP call (an unknown kernel is a shape error first)."""
    import numpy as np
    buf = np.full(16, 7, dtype=np.uint64)
    assert lib.kda_phase_clocks(K.KDA_CLOCK_INTRA, buf.ctypes.data, buf.size, 1) == 6
    assert lib.kda_phase_clocks(K.KDA_CLOCK_FUSED, None, 0, 0) == 6
    assert lib.kda_phase_clocks(K.KDA_CLOCK_SCAN, None, 0, 1) == 6
    assert lib.kda_phase_clocks(3, buf.ctypes.data, buf.size, 0) == 2
    assert np.all(buf == 7)


def test_phase_clock_build_records_the_phases():
    """The instrumented build differs only by the records: its kernels read
    the core clock counter (s_memtime) at every mark, libkda.so's never."""
    import subprocess
    import tempfile
    from linear_attention_prefill_amd import build
    src = os.path.join(build.CSRC, "kda_prefill.hip")
    outs = {}
    for tag, extra in (("plain", []), ("clocks", ["-DKDA_PHASE_CLOCKS"])):
        with tempfile.TemporaryDirectory() as td:
            asm = os.path.join(td, "p.s")
            subprocess.check_call([build._hipcc(), "-x", "hip", "--offload-arch=" + build.ARCH,
                                   *build.COMMON, *build.DEVICE_FLAGS,
                                   *build.PER_SOURCE_FLAGS["kda_prefill.hip"], *extra,
                                   "--cuda-device-only", "-S", src, "-o", asm],
                                  stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
            outs[tag] = open(asm).read()
    assert "s_memtime" not in outs["plain"]
    assert outs["clocks"].count("s_memtime") >= 2 * 13 + 5


def test_stream_probe_rejects_bad_arguments(lib):
    """Host checks of kda_stream_probe, all before any launch (bytes = 0 with
    valid arguments launches nothing)."""
    A16, B16 = 0x1000, 0x2000
    assert lib.kda_stream_probe(3, A16, B16, 1 << 20, 1024, None) == 2       # mode
    assert lib.kda_stream_probe(-1, A16, B16, 1 << 20, 1024, None) == 2
    assert lib.kda_stream_probe(1, A16, B16, (1 << 20) + 8, 1024, None) == 2  # not 16-byte units
    assert lib.kda_stream_probe(1, A16, B16, 1 << 20, 0, None) == 2          # grid
    assert lib.kda_stream_probe(1, None, B16, 1 << 20, 1024, None) == 1      # copy needs src
    assert lib.kda_stream_probe(0, A16, None, 1 << 20, 1024, None) == 1      # read needs a sink
    assert lib.kda_stream_probe(1, A16 + 8, B16, 1 << 20, 1024, None) == 4
    assert lib.kda_stream_probe(2, None, B16 + 4, 1 << 20, 1024, None) == 4
    assert lib.kda_stream_probe(2, None, B16, 0, 1024, None) == 0


def test_mfma_probe_rejects_bad_arguments(lib):
    """Host checks of kda_mfma_probe, all before any launch."""
    A8 = 0x1000
    for chains in (0, 3, 5, 16, -1):
        assert lib.kda_mfma_probe(chains, 64, A8, None) == 2
    assert lib.kda_mfma_probe(8, 0, A8, None) == 2                            # iters
    assert lib.kda_mfma_probe(8, (1 << 20) + 1, A8, None) == 2
    assert lib.kda_mfma_probe(8, 64, None, None) == 1
    assert lib.kda_mfma_probe(8, 64, A8 + 4, None) == 4


def _desc(**kw):
    d = dict(T=8192, N=16, H=32, dk=128, dv=128, slots=64, io=K.KDA_BF16, scale=1.0, ss=0, hs=0,
             conv=0)
    d.update(kw)
    return K.make_desc(d["T"], d["N"], d["H"], d["dk"], d["dv"], d["slots"], d["io"], d["scale"],
                       d["ss"], d["hs"], d["conv"])


def test_fuse_chunks_policy(lib):
    """kda_prefill_fuse_chunks: a positive request is taken as is for bf16, a
    negative one fuses nothing, fp32 never fuses, an invalid desc gives -1."""
    def f(fc, io=K.KDA_BF16, **kw):
        d = dict(T=8192, N=16, H=32, dk=128, dv=128, slots=64)
        d.update(kw)
        desc = K.make_desc(d["T"], d["N"], d["H"], d["dk"], d["dv"], d["slots"], io,
                           fuse_chunks=fc)
        return lib.kda_prefill_fuse_chunks(ctypes.byref(desc))
    assert f(5) == 5 and f(64) == 64
    assert f(-1) == -1 and f(-7) == -1
    assert f(5, io=K.KDA_F32) == -1 and f(0, io=K.KDA_F32) == -1
    assert f(3, dk=96) == -1
    assert lib.kda_prefill_fuse_chunks(None) == -1
    # the library's choice: by the average sequence length
    assert f(0) == -1                                  # 16 sequences in 8192 rows
    assert f(0, N=1) == -1
    assert f(0, N=31) == -1                            # more than four chunks on average
    assert f(0, N=32) == 8 and f(0, N=40) == 8         # at most four
    assert f(0, N=64) == 6 and f(0, N=100) == 6        # at most two
    assert f(0, N=128) == 8 and f(0, N=300) == 8       # at most one
    # windows: none when every sequence is fused (F * 64 >= T)
    d = K.make_desc(8192, 16, 32, 128, 128, 64, K.KDA_BF16, fuse_chunks=128)
    assert lib.kda_prefill_windows(ctypes.byref(d)) == 0
    d = K.make_desc(8192, 16, 32, 128, 128, 64, K.KDA_BF16, fuse_chunks=127)
    assert lib.kda_prefill_windows(ctypes.byref(d)) == 1


def _ws_formula(T, N, H, dk, dv, es):
    rec = (64 * (3 * dk + dv) + 6 * 512) * es + dk * 4
    ids = (T - 1) // 64 + N if T > 0 else N     # the last chunk's id is below this
    return ids * H * rec


def test_static_scratch_holds_the_packed_chunk(lib):
    """The allocation-free entry point's array holds an 8192-row chunk of up
    to 18 sequences at H = 32, d = 128, bf16, and no more."""
    size = lambda n: lib.kda_prefill_workspace_size(ctypes.byref(
        K.make_desc(8192, n, 32, 128, 128, 64, K.KDA_BF16, 1.0)))
    assert size(16) == 330350592                      # 315.05 MiB
    assert size(18) <= K.STATIC_SCRATCH_BYTES < size(19)


def test_workspace_size(lib):
    for T, N, H, dk, dv, io, es in [(8192, 16, 32, 128, 128, K.KDA_BF16, 2),
                                    (256, 1, 2, 64, 64, K.KDA_F32, 4),
                                    (0, 3, 1, 64, 128, K.KDA_BF16, 2),
                                    (77, 5, 3, 128, 64, K.KDA_F32, 4)]:
        d = K.make_desc(T, N, H, dk, dv, N, io, 1.0)
        assert lib.kda_prefill_workspace_size(ctypes.byref(d)) == _ws_formula(T, N, H, dk, dv, es)
    assert lib.kda_prefill_workspace_size(None) == 0
    d = _desc(dk=96)
    assert lib.kda_prefill_workspace_size(ctypes.byref(d)) == 0


A = 0x10000  # a 16-byte aligned fake address, never dereferenced


def _prefill(lib, desc, q=A, k=A, v=A, g=A, beta=A, cu=A, sin=None, sout=None, o=A, slots=None,
             ws=A, ws_bytes=1 << 40):
    return lib.kda_chunk_prefill(q, k, v, g, beta, cu, sin, sout, o, slots,
                                 ctypes.byref(desc) if desc is not None else None, ws, ws_bytes, None)


def test_prefill_rejects_bad_arguments(lib):
    assert _prefill(lib, None) == 1                                   # NULL desc
    assert _prefill(lib, _desc(io=7)) == 3                            # dtype
    assert _prefill(lib, _desc(dk=96)) == 6                           # unsupported d_k
    assert _prefill(lib, _desc(dv=256)) == 6                          # unsupported d_v
    assert _prefill(lib, _desc(T=-1)) == 2
    assert _prefill(lib, _desc(N=0)) == 2
    assert _prefill(lib, _desc(H=0)) == 2
    assert _prefill(lib, _desc(slots=-1)) == 2
    assert _prefill(lib, _desc(H=70000)) == 2
    # identity slots with a pool smaller than N
    assert _prefill(lib, _desc(N=16, slots=8), sin=A) == 2
    for key in ("q", "k", "v", "g", "beta", "cu"):
        assert _prefill(lib, _desc(), **{key: None}) == 1, key
    assert _prefill(lib, _desc(), o=None) == 1
    assert _prefill(lib, _desc(T=0), cu=None) == 1                    # cu_seqlens even with no rows
    assert _prefill(lib, _desc(), ws=None) == 1
    assert _prefill(lib, _desc(), q=A + 8) == 4                       # misaligned
    assert _prefill(lib, _desc(), sin=A + 4) == 4
    assert _prefill(lib, _desc(), slots=A + 2) == 4
    d = _desc()
    need = lib.kda_prefill_workspace_size(ctypes.byref(d))
    assert _prefill(lib, d, ws_bytes=need - 1) == 5


def test_prefill_rejects_bad_line_strides(lib):
    blk = 128 * 128
    assert _prefill(lib, _desc(hs=blk - 4)) == 2                      # heads would overlap
    assert _prefill(lib, _desc(hs=blk + 2)) == 2                      # not a multiple of 4
    assert _prefill(lib, _desc(ss=31 * blk + blk - 4)) == 2           # lines would overlap
    assert _prefill(lib, _desc(ss=32 * blk + 2)) == 2                 # not a multiple of 4
    assert _prefill(lib, _desc(hs=blk + 576, ss=31 * (blk + 576) + blk - 4)) == 2
    assert _prefill(lib, _desc(ss=-32 * blk)) == 2


def _decode(lib, q=A, k=A, v=A, g=A, beta=A, pool=A, slots=A, o=A, N=64, H=32, dk=128, dv=128,
            ns=64, io=K.KDA_BF16):
    return lib.kda_decode_step(q, k, v, g, beta, pool, slots, o, N, H, dk, dv, ns, io, 1.0, None)


def _decode_lines(lib, ss, hs, N=64, H=32, dk=128, dv=128, ns=64):
    return lib.kda_decode_step_lines(A, A, A, A, A, A, A, A, N, H, dk, dv, ns, K.KDA_BF16, 1.0,
                                     ss, hs, None)


def test_decode_lines_rejects_bad_strides(lib):
    blk = 128 * 128
    assert _decode_lines(lib, 0, blk - 4) == 2
    assert _decode_lines(lib, 0, blk + 2) == 2
    assert _decode_lines(lib, 31 * blk + blk - 4, 0) == 2
    assert _decode_lines(lib, 32 * blk + 6, 0) == 2


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, io=5) == 3
    assert _decode(lib, dk=32) == 6
    assert _decode(lib, N=0) == 2
    assert _decode(lib, H=0) == 2
    assert _decode(lib, ns=0) == 2
    for key in ("q", "k", "v", "g", "beta", "pool", "slots", "o"):
        assert _decode(lib, **{key: None}) == 1, key
    assert _decode(lib, pool=A + 4) == 4
    assert _decode(lib, o=A + 2) == 4


def _tokens(lib, q=A, o=A, acc=None, T=4, commit=1, N=64, H=32, dk=128, dv=128, ns=64, ss=0, hs=0,
            pool=A, slots=A):
    return lib.kda_decode_tokens(q, A, A, A, A, pool, slots, o, acc, N, T, H, dk, dv, ns,
                                 K.KDA_BF16, 1.0, commit, ss, hs, None)


def test_decode_tokens_rejects_bad_arguments(lib):
    assert _tokens(lib, T=0) == 2
    assert _tokens(lib, T=17) == 2
    assert _tokens(lib, N=0) == 2
    assert _tokens(lib, ns=0) == 2
    assert _tokens(lib, dk=96) == 6
    assert _tokens(lib, o=None, commit=0) == 1          # nothing to do
    assert _tokens(lib, q=None) == 1                    # outputs need q
    assert _tokens(lib, pool=None) == 1
    assert _tokens(lib, slots=None) == 1
    assert _tokens(lib, acc=A + 4) == 4
    assert _tokens(lib, o=A + 2) == 4
    assert _tokens(lib, hs=128 * 128 - 4) == 2


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of kda_prefill_desc_t and kda_conv_t have the C
    sizes and field offsets (checked with gcc against include/kda.h)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "layout.c"
    fields = [("kda_prefill_desc_t", n) for n, _ in K.PrefillDesc._fields_] + \
             [("kda_conv_t", n) for n, _ in K.ConvDesc._fields_]
    body = "".join('printf("%%s.%%s %%zu\\n", "%s", "%s", offsetof(%s, %s));\n' % (t, f, t, f)
                   for t, f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kda.h"\nint main(void){\n'
                   + body + 'printf("size.desc %zu\\nsize.conv %zu\\n", sizeof(kda_prefill_desc_t),'
                   ' sizeof(kda_conv_t));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(line.rsplit(" ", 1) for line in subprocess.check_output([str(exe)]).decode().split("\n")
               if line)
    for t, cls in (("kda_prefill_desc_t", K.PrefillDesc), ("kda_conv_t", K.ConvDesc)):
        for n, _ in cls._fields_:
            assert int(got["%s.%s" % (t, n)]) == getattr(cls, n).offset, (t, n)
    assert int(got["size.desc"]) == ctypes.sizeof(K.PrefillDesc)
    assert int(got["size.conv"]) == ctypes.sizeof(K.ConvDesc)


def _conv(w=A, win=A, ss=0, hs=0, rs=0, ps=0):
    return K.ConvDesc(w, win, ss, hs, rs, ps)


def _prefill_conv(lib, desc, conv, ws_bytes=1 << 40):
    return lib.kda_chunk_prefill_conv(A, A, A, A, A, A, None, None, A, None, ctypes.byref(desc),
                                      ctypes.byref(conv) if conv is not None else None, A,
                                      ws_bytes, None, None, 0)


def test_prefill_conv_rejects_bad_arguments(lib):
    assert _prefill(lib, _desc(conv=1)) == 1                          # conv mode without conv
    assert _prefill_conv(lib, _desc(conv=0), _conv()) == 2            # conv entry, no mode
    assert _prefill_conv(lib, _desc(conv=3), _conv()) == 2
    assert _prefill_conv(lib, _desc(conv=1), None) == 1
    assert _prefill_conv(lib, _desc(conv=1), _conv(w=None)) == 1
    assert _prefill_conv(lib, _desc(conv=2), _conv(win=None)) == 1
    assert _prefill_conv(lib, _desc(conv=1), _conv(win=A + 8)) == 4
    assert _prefill_conv(lib, _desc(conv=1), _conv(ps=64)) == 2       # part stride < d_k
    assert _prefill_conv(lib, _desc(conv=1), _conv(rs=386)) == 2      # not a multiple of 4
    assert _prefill_conv(lib, _desc(conv=1), _conv(ss=-4)) == 2
    d = _desc(conv=2)
    need = lib.kda_prefill_workspace_size(ctypes.byref(d))
    assert _prefill_conv(lib, d, _conv(), ws_bytes=need - 1) == 5


def test_conv_workspace_size(lib):
    """The convolved q, k, v take workspace only when the conv runs as a pass
    of its own: fp32, d_k != d_v, or a call that fuses sequences (bf16 with
    d_k = d_v and nothing fused folds the conv into the intra-chunk loads)."""
    up = lambda x: (x + 255) // 256 * 256
    cases = [(8192, 2, 32, 128, 128, K.KDA_BF16, 2, 0, False),
             (8192, 2, 32, 128, 128, K.KDA_BF16, 2, 1, True),      # fuse one-chunk sequences
             (8192, 128, 32, 128, 128, K.KDA_BF16, 2, 0, True),    # short: fused by default
             (8192, 128, 32, 64, 64, K.KDA_BF16, 2, -1, False),
             (77, 2, 3, 128, 64, K.KDA_BF16, 2, 0, True),
             (77, 2, 3, 128, 64, K.KDA_F32, 4, 0, True)]
    for T, N, H, dk, dv, io, es, fuse, pass_of_own in cases:
        d0 = K.make_desc(T, N, H, dk, dv, N, io, 1.0, fuse_chunks=fuse)
        d1 = K.make_desc(T, N, H, dk, dv, N, io, 1.0, conv_mode=1, fuse_chunks=fuse)
        extra = 256 + 2 * up(T * H * dk * es) + up(T * H * dv * es) if pass_of_own else 0
        assert (lib.kda_prefill_workspace_size(ctypes.byref(d1))
                == lib.kda_prefill_workspace_size(ctypes.byref(d0)) + extra), (T, N, H, dk, dv, io, fuse)


def _decode_conv(lib, mode=1, conv="ok", **kw):
    c = _conv(**kw) if conv == "ok" else conv
    return lib.kda_decode_step_conv(A, A, A, A, A, A, A, A, 64, 32, 128, 128, 64, K.KDA_BF16, 1.0,
                                    0, 0, mode, ctypes.byref(c) if c is not None else None, None)


def test_decode_conv_rejects_bad_arguments(lib):
    assert _decode_conv(lib, mode=0) == 2
    assert _decode_conv(lib, mode=3) == 2
    assert _decode_conv(lib, conv=None) == 1
    assert _decode_conv(lib, w=None) == 1
    assert _decode_conv(lib, win=A + 4) == 4
    assert _decode_conv(lib, ps=100) == 2
    assert _decode_conv(lib, hs=6) == 2


def test_conv_extent_matches_the_layouts():
    """Dense, tap-major and hybrid-page windows need exactly the elements
    their tensors hold (the binding refuses smaller ones)."""
    for S, H, dk, dv in [(6, 4, 128, 128), (3, 2, 64, 128), (1, 32, 128, 64)]:
        C = 2 * dk + dv
        assert K.conv_extent(S, H, dk, dv, (0, 0, 0, 0)) == S * H * 3 * C
    S, H, d = 5, 4, 128
    C = 3 * d
    assert K.conv_extent(S, H, d, d, (3 * H * C, d, H * C, H * d)) == S * 3 * H * C
    # a window right after each head's 64 KiB state in 884,736-byte pages
    ss, hs = 2 * (884736 // 4), 2 * (67840 // 4)
    assert K.conv_extent(4, 12, d, d, (ss, hs, C, d)) == 3 * ss + 11 * hs + 3 * C


def test_prefill_check_rejects_before_launch(lib):
    """kda_prefill_check validates its host arguments before anything runs."""
    fake = ctypes.c_void_p(0x10000)
    flags = ctypes.c_void_p(0x20000)
    d = _desc()
    assert lib.kda_prefill_check(None, fake, None, ctypes.byref(d), flags, None) == 1   # g NULL, T > 0
    assert lib.kda_prefill_check(fake, None, None, ctypes.byref(d), flags, None) == 1   # cu NULL
    assert lib.kda_prefill_check(fake, fake, None, ctypes.byref(d), None, None) == 1    # flags NULL
    assert lib.kda_prefill_check(fake, fake, None, None, flags, None) == 1              # desc NULL
    assert lib.kda_prefill_check(ctypes.c_void_p(0x10004), fake, None, ctypes.byref(d), flags,
                                 None) == 4                                             # misaligned
    bad = _desc(dk=96)
    assert lib.kda_prefill_check(fake, fake, None, ctypes.byref(bad), flags, None) == 6
    bad = _desc(N=0)
    assert lib.kda_prefill_check(fake, fake, None, ctypes.byref(bad), flags, None) == 2


def test_static_prefill_rejects_before_launch(lib):
    """kda_chunk_prefill_static checks its arguments, and that the call fits
    the static scratch, before it looks anything up on a device."""
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 6 + [None, None, fake, None]
    big = _desc(T=16384, N=16, H=32, slots=16)
    assert lib.kda_prefill_workspace_size(ctypes.byref(big)) > K.STATIC_SCRATCH_BYTES
    assert lib.kda_chunk_prefill_static(*args, ctypes.byref(big), None) == 8
    d = _desc()
    bad = list(args)
    bad[0] = None
    assert lib.kda_chunk_prefill_static(*bad, ctypes.byref(d), None) == 1
    assert lib.kda_chunk_prefill_static(*args, None, None) == 1
    conv = _desc(conv=1)
    assert lib.kda_chunk_prefill_static(*args, ctypes.byref(conv), None) == 1
    assert lib.kda_prefill_workspace_size(ctypes.byref(d)) <= K.STATIC_SCRATCH_BYTES
