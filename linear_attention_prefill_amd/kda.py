"""Python binding of libkda.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(``include/kda.h``).  PyTorch supplies device memory and the current stream;
nothing here computes.  If the library is missing the calls raise: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
# The same kernels with phase clocks recorded (``build --phase-clocks``).
CLOCKS_LIB_PATH = os.path.join(_PKG, "libkda_clocks.so")

KDA_F32 = 0
KDA_BF16 = 1

STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
          4: "KDA_ERR_ALIGN", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_UNSUPPORTED", 7: "KDA_ERR_HIP",
          8: "KDA_ERR_TOO_LARGE"}

# Bytes of the static scratch behind kda_chunk_prefill_static (kda.h).
STATIC_SCRATCH_BYTES = 320 << 20


class PrefillDesc(ctypes.Structure):
    _fields_ = [("total_rows", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("state_slot_stride", ctypes.c_int64),
                ("state_head_stride", ctypes.c_int64), ("conv_mode", ctypes.c_int32),
                ("window_chunks", ctypes.c_int32), ("fuse_chunks", ctypes.c_int32)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("window", ctypes.c_void_p),
                ("slot_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("part_stride", ctypes.c_int64)]


CONV_MODES = {"none": 1, "silu": 2}     # activation after the conv -> kda_conv_mode_t


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libkda.so (built by ``python -m linear_attention_prefill_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libkda.so is not built (%s); run "
                           "`python -m linear_attention_prefill_amd.build`" % p)
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kda_prefill_workspace_size.restype = sz
    lib.kda_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc)]
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_chunk_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.POINTER(PrefillDesc), vp, sz, vp]
    lib.kda_chunk_prefill_timed.restype = ctypes.c_int
    lib.kda_chunk_prefill_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.POINTER(PrefillDesc), vp, sz, vp,
                                            ctypes.POINTER(ctypes.c_void_p), i32]
    lib.kda_chunk_prefill_conv.restype = ctypes.c_int
    lib.kda_chunk_prefill_conv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.POINTER(PrefillDesc), ctypes.POINTER(ConvDesc),
                                           vp, sz, vp, ctypes.POINTER(ctypes.c_void_p), i32]
    lib.kda_prefill_windows.restype = i32
    lib.kda_prefill_windows.argtypes = [ctypes.POINTER(PrefillDesc)]
    lib.kda_prefill_fuse_chunks.restype = i32
    lib.kda_prefill_fuse_chunks.argtypes = [ctypes.POINTER(PrefillDesc)]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                    i32, i32, i32, i32, i32, i32, f32, vp]
    i64 = ctypes.c_int64
    lib.kda_decode_step_lines.restype = ctypes.c_int
    lib.kda_decode_step_lines.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                          i32, i32, i32, i32, i32, i32, f32, i64, i64, vp]
    lib.kda_decode_step_conv.restype = ctypes.c_int
    lib.kda_decode_step_conv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                         i32, i32, i32, i32, i32, i32, f32, i64, i64, i32,
                                         ctypes.POINTER(ConvDesc), vp]
    lib.kda_decode_tokens.restype = ctypes.c_int
    lib.kda_decode_tokens.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      i32, i32, i32, i32, i32, i32, i32, f32, i32, i64, i64, vp]
    lib.kda_chunk_prefill_static.restype = ctypes.c_int
    lib.kda_chunk_prefill_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.POINTER(PrefillDesc), vp]
    lib.kda_prefill_check.restype = ctypes.c_int
    lib.kda_prefill_check.argtypes = [vp, vp, vp, ctypes.POINTER(PrefillDesc), vp, vp]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_version.restype = i32
    lib.kda_version.argtypes = []
    lib.kda_phase_clocks.restype = ctypes.c_int
    lib.kda_phase_clocks.argtypes = [i32, vp, sz, i32]
    lib.kda_stream_probe.restype = ctypes.c_int
    lib.kda_stream_probe.argtypes = [i32, vp, vp, sz, i32, vp]
    lib.kda_mfma_probe.restype = ctypes.c_int
    lib.kda_mfma_probe.argtypes = [i32, i32, vp, vp]
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise KdaError(status, load_library().kda_status_string(status).decode())


def _io_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise ValueError("q, k, v must be bfloat16 or float32, got %s" % dt)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_obj(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(_stream_obj(stream).cuda_stream)


# kda_prefill_check flag bits (kda.h) and what each says.
CHECK_BITS = {1: "cu_seqlens must start at 0, end at T and never decrease",
              2: "g must be <= 0 (and not NaN)",
              4: "two live sequences name the same slot"}


def check_prefill_inputs(g, cu_seqlens, slots=None, num_slots=None, stream=None) -> int:
    """Opt-in check of the device-side preconditions of chunk_prefill
    (``kda_prefill_check``): returns the KDA_CHECK_* bits of the violated
    ones, 0 when all hold.  Reads the flag back, so it synchronises with the
    launch stream."""
    lib = load_library()
    _dev(g, "g", torch.float32)
    T, H, dk = g.shape
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.shape[0] - 1
    _dev(slots, "slots", torch.int32, (N,) if slots is not None else None)
    if num_slots is None:
        num_slots = N
    desc = make_desc(T, N, H, dk, dk, num_slots, KDA_F32)
    s = _stream_obj(stream)
    with torch.cuda.stream(s):
        flags = torch.empty(4, dtype=torch.int32, device=g.device)
    _check(lib.kda_prefill_check(_ptr(g) if T > 0 else None, _ptr(cu_seqlens), _ptr(slots),
                                 ctypes.byref(desc), _ptr(flags), _stream(stream)))
    s.synchronize()
    return int(flags[0].item())


def make_desc(T, N, H, d_k, d_v, num_slots, io_dtype, scale=1.0, slot_stride=0,
              head_stride=0, conv_mode=0, window_chunks=0, fuse_chunks=0) -> PrefillDesc:
    return PrefillDesc(int(T), int(N), int(H), int(d_k), int(d_v), int(num_slots),
                       int(io_dtype), float(scale), int(slot_stride), int(head_stride),
                       int(conv_mode), int(window_chunks), int(fuse_chunks))


def conv_extent(num_slots, H, d_k, d_v, strides) -> int:
    """Elements a conv window pool must hold for the given (slot, head, row,
    part) strides, zeros meaning the dense layout (kda.h, kda_conv_t)."""
    C = 2 * d_k + d_v
    ss, hs, rs, ps = (int(x) for x in strides)
    ps = ps or d_k
    rs = rs or C
    hs = hs or 3 * C
    ss = ss or H * hs
    return (num_slots - 1) * ss + (H - 1) * hs + 2 * rs + max(ps + d_k, 2 * ps + d_v)


def _conv_desc(weight, window, H, dk, dv, dtype, strides, num_slots):
    """Checks the conv taps and window tensors and packs a kda_conv_t."""
    C = 2 * dk + dv
    _dev(weight, "conv_weight", torch.float32, (H, 4, C))
    if window is None:
        raise ValueError("conv_window is required with conv_weight")
    _dev(window, "conv_window", dtype)
    ss, hs, rs, ps = (int(x) for x in strides)
    if not any((ss, hs, rs, ps)):
        if window.dim() != 4 or tuple(window.shape[1:]) != (H, 3, C) or window.shape[0] < num_slots:
            raise ValueError("a dense conv_window must be [>= %d, %d, 3, %d], got %s"
                             % (num_slots, H, C, tuple(window.shape)))
    elif window.numel() < conv_extent(num_slots, H, dk, dv, strides):
        raise ValueError("conv_window holds %d elements, the strides need %d"
                         % (window.numel(), conv_extent(num_slots, H, dk, dv, strides)))
    return ConvDesc(weight.data_ptr(), window.data_ptr(), ss, hs, rs, ps)


def _conv_mode(activation):
    if activation not in CONV_MODES:
        raise ValueError("conv_activation must be 'none' or 'silu'")
    return CONV_MODES[activation]


def line_extent(num_slots, H, d_k, d_v, slot_stride, head_stride) -> int:
    """fp32 elements a pool addressed by lines must hold (kda.h, "State
    addressing by lines")."""
    hs = head_stride or d_k * d_v
    ss = slot_stride or H * hs
    return (num_slots - 1) * ss + (H - 1) * hs + d_k * d_v


def _check_pool(p, name, num_slots, H, dk, dv, slot_stride, head_stride):
    """Dense pools are [num_slots, H, d_v, d_k]; pools addressed by lines are
    any contiguous fp32 tensor holding line_extent(...) elements."""
    if p is None:
        return
    if slot_stride or head_stride:
        _dev(p, name, torch.float32)
        need = line_extent(num_slots, H, dk, dv, slot_stride, head_stride)
        if p.numel() < need:
            raise ValueError("%s holds %d fp32 elements, the lines need %d" % (name, p.numel(), need))
    else:
        _dev(p, name, torch.float32, (num_slots, H, dv, dk))


def prefill_windows(T, N, H, d_k, d_v, dtype=torch.bfloat16, window_chunks=0,
                    fuse_chunks=0) -> int:
    """Windows of chunk ids a prefill call of these sizes runs as
    (``kda_prefill_windows``): its kernels are an intra-chunk kernel and a
    state scan per window, in that order (none when every sequence runs in
    the fused prefill)."""
    d = make_desc(T, N, H, d_k, d_v, N, _io_code(dtype), window_chunks=window_chunks,
                  fuse_chunks=fuse_chunks)
    return int(load_library().kda_prefill_windows(ctypes.byref(d)))


def prefill_fuse_chunks(T, N, H, d_k, d_v, dtype=torch.bfloat16, fuse_chunks=0) -> int:
    """Most chunks of a sequence that a prefill call of these sizes runs in
    the fused prefill (``kda_prefill_fuse_chunks``; -1: none).  When it is
    not negative the fused kernel runs after the windows."""
    d = make_desc(T, N, H, d_k, d_v, N, _io_code(dtype), fuse_chunks=fuse_chunks)
    return int(load_library().kda_prefill_fuse_chunks(ctypes.byref(d)))


def prefill_workspace_size(T, N, H, d_k, d_v, dtype=torch.bfloat16, conv=False,
                           window_chunks=0, fuse_chunks=0) -> int:
    d = make_desc(T, N, H, d_k, d_v, N, _io_code(dtype), conv_mode=1 if conv else 0,
                  window_chunks=window_chunks, fuse_chunks=fuse_chunks)
    return int(load_library().kda_prefill_workspace_size(ctypes.byref(d)))


def chunk_prefill(q, k, v, g, beta, cu_seqlens, state_in=None, state_out=None, o=None,
                  slots=None, num_slots=None, scale=1.0, workspace=None, stream=None,
                  events=None, state_slot_stride=0, state_head_stride=0, conv_weight=None,
                  conv_window=None, conv_activation="none", conv_strides=(0, 0, 0, 0),
                  check_inputs=False, window_chunks=0, fuse_chunks=0):
    """KDA chunked prefill over packed sequences (see ``kda_chunk_prefill``).

    q, k: [T, H, d_k]; v: [T, H, d_v] (bf16 or fp32, same dtype); g: [T, H, d_k]
    fp32; beta: [T, H] fp32; cu_seqlens: [N+1] int32 (device); state_in /
    state_out: [num_slots, H, d_v, d_k] fp32 pools or None (may be the same
    tensor); slots: [N] int32 or None.  With state_slot_stride /
    state_head_stride (fp32 elements, kda.h "State addressing by lines") the
    pools are flat fp32 buffers and num_slots must be given.  With conv_weight
    [H, 4, 2 d_k + d_v] fp32 and conv_window (io dtype; dense
    [num_slots, H, 3, 2 d_k + d_v] or any tensor the conv_strides (slot,
    head, row, part) address) q, k, v are raw inputs to the short conv front
    end (``kda_chunk_prefill_conv``); the window is updated in place.
    events: optional list of recorded torch.cuda.Event(enable_timing=True)
    objects: the first is recorded before the first kernel and the i-th after
    the i-th kernel launch (intra and scan of each window in turn, then the
    fused prefill when prefill_fuse_chunks(...) >= 0; 2 W + 1 or 2 W + 2
    events for W = prefill_windows(...) windows; ``kda_chunk_prefill_timed``).
    check_inputs: first run the opt-in check
    of the device data (``kda_prefill_check``, which synchronises) and raise
    ValueError if it fails.  Tensors the call allocates (o when None, the
    workspace when None) come from the launch stream's memory pool.
    window_chunks: chunk ids per window (kda.h, kda_prefill_windows); 0 lets
    the library choose.  fuse_chunks: bf16 sequences of at most this many
    chunks run in the fused prefill (kda.h, kda_prefill_fuse_chunks); 0 lets
    the library choose, a negative value fuses none.  Returns o [T, H, d_v].
    """
    lib = load_library()
    _dev(q, "q")
    T, H, dk = q.shape
    dv = v.shape[2]
    io = _io_code(q.dtype)
    _dev(k, "k", q.dtype, (T, H, dk))
    _dev(v, "v", q.dtype, (T, H, dv))
    _dev(g, "g", torch.float32, (T, H, dk))
    _dev(beta, "beta", torch.float32, (T, H))
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.shape[0] - 1
    pools = [p for p in (state_in, state_out) if p is not None]
    lines = bool(state_slot_stride or state_head_stride)
    if num_slots is None:
        if lines and pools:
            raise ValueError("num_slots is required for pools addressed by lines")
        num_slots = pools[0].shape[0] if pools else N
    for name, p in (("state_in", state_in), ("state_out", state_out)):
        _check_pool(p, name, num_slots, H, dk, dv, state_slot_stride, state_head_stride)
    _dev(slots, "slots", torch.int32, (N,) if slots is not None else None)
    if check_inputs:
        bad = check_prefill_inputs(g, cu_seqlens, slots, num_slots=num_slots, stream=stream)
        if bad:
            raise ValueError("prefill inputs break the preconditions of kda.h: "
                             + "; ".join(m for b, m in CHECK_BITS.items() if bad & b))
    s = _stream_obj(stream)
    if o is None:
        with torch.cuda.stream(s):   # owned by the launch stream's memory pool
            o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    _dev(o, "o", q.dtype, (T, H, dv))
    conv = None
    if conv_weight is not None:
        conv = _conv_desc(conv_weight, conv_window, H, dk, dv, q.dtype, conv_strides, num_slots)
    desc = make_desc(T, N, H, dk, dv, num_slots, io, scale, state_slot_stride, state_head_stride,
                     _conv_mode(conv_activation) if conv is not None else 0, window_chunks,
                     fuse_chunks)
    need = int(lib.kda_prefill_workspace_size(ctypes.byref(desc)))
    if workspace is None:
        # Allocated from the launch stream's pool: when it is freed on return
        # the caching allocator hands its blocks out again only to work on
        # that stream, which runs after this call's kernels.
        with torch.cuda.stream(s):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(state_in),
            _ptr(state_out), _ptr(o), _ptr(slots), ctypes.byref(desc), _ptr(workspace),
            workspace.numel(), _stream(stream))
    handles, n_ev = None, 0
    if events is not None:
        n_ev = len(events)
        handles = (ctypes.c_void_p * max(n_ev, 1))(*[_event_handle(e) for e in events])
    if conv is not None:
        _check(lib.kda_chunk_prefill_conv(*args[:11], ctypes.byref(conv), *args[11:], handles,
                                          n_ev))
    elif handles is None:
        _check(lib.kda_chunk_prefill(*args))
    else:
        _check(lib.kda_chunk_prefill_timed(*args, handles, n_ev))
    return o


def chunk_prefill_no_alloc(q, k, v, g, beta, cu_seqlens, o, state_in=None, state_out=None,
                           slots=None, num_slots=None, scale=1.0, stream=None,
                           state_slot_stride=0, state_head_stride=0, window_chunks=0,
                           fuse_chunks=0):
    """chunk_prefill through ``kda_chunk_prefill_static``, for callers that
    cannot allocate: o is required, no workspace is passed and nothing is
    allocated, here or in the library (its workspace is a static device array
    of STATIC_SCRATCH_BYTES per GPU).  Calls that overlap on one GPU race.
    Same arguments and results as chunk_prefill otherwise; no conv front end.
    Returns o."""
    lib = load_library()
    _dev(q, "q")
    T, H, dk = q.shape
    dv = v.shape[2]
    io = _io_code(q.dtype)
    _dev(k, "k", q.dtype, (T, H, dk))
    _dev(v, "v", q.dtype, (T, H, dv))
    _dev(g, "g", torch.float32, (T, H, dk))
    _dev(beta, "beta", torch.float32, (T, H))
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.shape[0] - 1
    pools = [p for p in (state_in, state_out) if p is not None]
    lines = bool(state_slot_stride or state_head_stride)
    if num_slots is None:
        if lines and pools:
            raise ValueError("num_slots is required for pools addressed by lines")
        num_slots = pools[0].shape[0] if pools else N
    for name, p in (("state_in", state_in), ("state_out", state_out)):
        _check_pool(p, name, num_slots, H, dk, dv, state_slot_stride, state_head_stride)
    _dev(slots, "slots", torch.int32, (N,) if slots is not None else None)
    if o is None:
        raise ValueError("o is required: this entry point allocates nothing")
    _dev(o, "o", q.dtype, (T, H, dv))
    desc = make_desc(T, N, H, dk, dv, num_slots, io, scale, state_slot_stride, state_head_stride,
                     window_chunks=window_chunks, fuse_chunks=fuse_chunks)
    _check(lib.kda_chunk_prefill_static(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(cu_seqlens), _ptr(state_in), _ptr(state_out),
                                        _ptr(o), _ptr(slots), ctypes.byref(desc),
                                        _stream(stream)))
    return o


def _event_handle(ev) -> int:
    """The hipEvent_t behind a torch.cuda.Event (created on first record)."""
    h = ev.cuda_event
    if not h:
        raise ValueError("record each event once before passing it (torch creates it lazily)")
    return h


def decode_step(q, k, v, g, beta, state_pool, slots, o=None, scale=1.0, stream=None,
                num_slots=None, state_slot_stride=0, state_head_stride=0, conv_weight=None,
                conv_window=None, conv_activation="none", conv_strides=(0, 0, 0, 0)):
    """One token per sequence; state_pool [num_slots, H, d_v, d_k] updated in
    place (see ``kda_decode_step``).  q, k, g: [N, H, d_k]; v: [N, H, d_v];
    beta: [N, H]; slots: [N] int32.  With state_slot_stride /
    state_head_stride the pool is a flat fp32 buffer addressed by lines
    (``kda_decode_step_lines``) and num_slots must be given.  With
    conv_weight and conv_window (as for chunk_prefill) the short conv runs
    fused into the step (``kda_decode_step_conv``).  Returns o [N, H, d_v]."""
    lib = load_library()
    _dev(q, "q")
    N, H, dk = q.shape
    dv = v.shape[2]
    io = _io_code(q.dtype)
    _dev(k, "k", q.dtype, (N, H, dk))
    _dev(v, "v", q.dtype, (N, H, dv))
    _dev(g, "g", torch.float32, (N, H, dk))
    _dev(beta, "beta", torch.float32, (N, H))
    _dev(state_pool, "state_pool", torch.float32)
    lines = bool(state_slot_stride or state_head_stride)
    if num_slots is None:
        if lines:
            raise ValueError("num_slots is required for a pool addressed by lines")
        num_slots = state_pool.shape[0]
    _check_pool(state_pool, "state_pool", num_slots, H, dk, dv, state_slot_stride, state_head_stride)
    _dev(slots, "slots", torch.int32, (N,))
    if o is None:
        with torch.cuda.stream(_stream_obj(stream)):
            o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _dev(o, "o", q.dtype, (N, H, dv))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(slots),
            _ptr(o), N, H, dk, dv, num_slots, io, float(scale), int(state_slot_stride),
            int(state_head_stride))
    if conv_weight is not None:
        conv = _conv_desc(conv_weight, conv_window, H, dk, dv, q.dtype, conv_strides, num_slots)
        _check(lib.kda_decode_step_conv(*args, _conv_mode(conv_activation), ctypes.byref(conv),
                                        _stream(stream)))
    else:
        _check(lib.kda_decode_step_lines(*args, _stream(stream)))
    return o


def decode_tokens(q, k, v, g, beta, state_pool, slots, o=None, num_accepted=None, commit=True,
                  outputs=True, scale=1.0, stream=None, num_slots=None, state_slot_stride=0,
                  state_head_stride=0):
    """T tokens per sequence against one state (see ``kda_decode_tokens``).

    k, g: [N, T, H, d_k]; v: [N, T, H, d_v]; beta: [N, T, H]; q: [N, T, H, d_k]
    (may be None when outputs is False); slots: [N] int32; num_accepted: [N]
    int32 or None.  commit=False only reads the state (verify); commit=True
    writes back the state after num_accepted[n] tokens (all T when None).
    outputs=False skips the outputs (a commit of a verified window).  Returns
    o [N, T, H, d_v], or None when outputs is False."""
    lib = load_library()
    _dev(k, "k")
    N, T, H, dk = k.shape
    dv = v.shape[3]
    io = _io_code(k.dtype)
    _dev(v, "v", k.dtype, (N, T, H, dv))
    _dev(g, "g", torch.float32, (N, T, H, dk))
    _dev(beta, "beta", torch.float32, (N, T, H))
    if outputs:
        _dev(q, "q", k.dtype, (N, T, H, dk))
        if o is None:
            with torch.cuda.stream(_stream_obj(stream)):
                o = torch.empty((N, T, H, dv), dtype=k.dtype, device=k.device)
        _dev(o, "o", k.dtype, (N, T, H, dv))
    else:
        if q is not None:
            _dev(q, "q", k.dtype, (N, T, H, dk))
        o = None
    _dev(state_pool, "state_pool", torch.float32)
    lines = bool(state_slot_stride or state_head_stride)
    if num_slots is None:
        if lines:
            raise ValueError("num_slots is required for a pool addressed by lines")
        num_slots = state_pool.shape[0]
    _check_pool(state_pool, "state_pool", num_slots, H, dk, dv, state_slot_stride, state_head_stride)
    _dev(slots, "slots", torch.int32, (N,))
    _dev(num_accepted, "num_accepted", torch.int32, (N,) if num_accepted is not None else None)
    _check(lib.kda_decode_tokens(_ptr(q) if outputs else None, _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state_pool), _ptr(slots), _ptr(o), _ptr(num_accepted), N, T,
                                 H, dk, dv, num_slots, io, float(scale), 1 if commit else 0,
                                 int(state_slot_stride), int(state_head_stride), _stream(stream)))
    return o


# kda.h: KDA_CLOCK_* (the layout of kda_phase_clocks)
KDA_CLOCK_INTRA, KDA_CLOCK_FUSED, KDA_CLOCK_SCAN = 0, 1, 2
CLOCK_WAVES, CLOCK_ITEMS, CLOCK_MARKS = 8, 64, 16


def phase_clocks(kernel: int, clear: bool = False):
    """Phase clocks of workgroup 0 of the intra-chunk kernel (KDA_CLOCK_INTRA),
    the fused prefill (KDA_CLOCK_FUSED) or the state scan (KDA_CLOCK_SCAN)
    (``kda_phase_clocks``): an int64 array [wave][item][mark] of core clock
    counts, 0 where not reached.
    Needs the library built with phase clocks (``load_library(CLOCKS_LIB_PATH)``
    first); raises KdaError (KDA_ERR_UNSUPPORTED) otherwise."""
    import numpy as np
    buf = np.zeros(CLOCK_WAVES * CLOCK_ITEMS * CLOCK_MARKS, dtype=np.uint64)
    _check(load_library().kda_phase_clocks(int(kernel), buf.ctypes.data, buf.size, 1 if clear else 0))
    return buf.astype(np.int64).reshape(CLOCK_WAVES, CLOCK_ITEMS, CLOCK_MARKS)


# kda.h: KDA_STREAM_*
KDA_STREAM_READ, KDA_STREAM_COPY, KDA_STREAM_UPDATE = 0, 1, 2


def stream_probe(mode: int, src, dst, grid: int = 1024, stream=None):
    """One plain streaming kernel (``kda_stream_probe``) over dst's bytes
    (src's for a read): read src, copy src to dst, or update dst in place.
    src, dst: contiguous CUDA tensors; for a read dst is the sink (at least
    4 grid bytes).  Enqueued on `stream` (default: the current stream)."""
    nbytes = (src if mode != KDA_STREAM_UPDATE else dst).numel() * \
        (src if mode != KDA_STREAM_UPDATE else dst).element_size()
    _check(load_library().kda_stream_probe(int(mode), _ptr(src) if src is not None else None,
                                           _ptr(dst), nbytes, int(grid), _stream(stream)))


def mfma_probe(chains: int, iters: int = 4096) -> dict:
    """Core clocks per bf16 16x16x32 product that one wave per SIMD reaches
    with `chains` independent accumulators (``kda_mfma_probe``), and the core
    clock over the loop in MHz.  Runs on the current stream and waits."""
    out = torch.zeros(12, dtype=torch.int64, device="cuda")
    _check(load_library().kda_mfma_probe(int(chains), int(iters), _ptr(out), _stream(None)))
    w = out.cpu().numpy()
    clocks, ticks = int(w[0]), int(w[1])
    return {"chains": int(chains), "clocks_per_product": clocks / (iters * chains),
            "core_MHz": 100.0 * clocks / ticks if ticks else float("nan")}
