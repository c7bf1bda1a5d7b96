"""KDA oracle: fp64 CPU reference for the chunked prefill and the decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP path: the recurrence lives in ``kda_oracle.c`` (plain C, fp64),
built with gcc, and this module only marshals numpy arrays and applies the
state-pool bookkeeping that the boundary documents.

The recurrence (see ``kda_oracle.c``) is the gated delta rule with a
per-key-channel decay, run token by token:

    S <- Diag(exp(g_t)) S;  S <- S + beta_t k_t (v_t - S^T k_t)^T;  o_t = scale S^T q_t

State pools follow the kern-k3-pp-prefill page, section "D inside SGLang":
``[slot][head][v][k]`` fp32, so pool entry ``(j, i)`` holds ``S[i][j]``.
Sequence bookkeeping follows the same page, section "P: the packed prefill":
sequences packed back to back, split by ``cu_seqlens``.

Slot semantics (mirroring the boundary): sequence ``n`` uses slot
``slots[n]`` (or ``n`` when ``slots`` is None).  When ``slots`` is given and
``slots[n]`` lies outside ``[0, num_slots)``, the sequence is a padded row:
its output rows are left untouched and no state is read or written, as the
"D inside SGLang" section describes for slot -1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
# The same source in fp32 working precision, for the noise-floor measurement
# only (see kda_oracle.c, "Working precision").
_LIB_PATH_F32 = os.path.join(_HERE, "libkda_oracle_f32.so")
_libs = {}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libkda_oracle.so`` (fp64)
    and ``oracle/libkda_oracle_f32.so`` (the fp32 noise-floor build)."""
    for path, extra in ((_LIB_PATH, []), (_LIB_PATH_F32, ["-DKDA_REAL=float"])):
        if force or not os.path.exists(path):
            tmp = path + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                                   *extra, _SRC, "-o", tmp, "-lm"])
            os.replace(tmp, path)
    return _LIB_PATH


def _load(precision="f64"):
    if precision not in ("f64", "f32"):
        raise ValueError("precision must be 'f64' or 'f32'")
    if precision not in _libs:
        path = _LIB_PATH if precision == "f64" else _LIB_PATH_F32
        if not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, dp, dp, dp,
                                           ctypes.c_double, ctypes.c_int32]
        _libs[precision] = lib
    return _libs[precision]


MAX_THREADS = 16   # the host CPU share one GPU job may use


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(MAX_THREADS, n))


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def recurrence(q, k, v, g, beta, cu_seqlens, s0=None, scale=1.0, threads=None,
               precision="f64"):
    """Run the token-by-token fp64 recurrence (precision="f32": the same loop
    in fp32, only for noise-floor measurements).

    q, k, g: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H]; cu_seqlens: [N+1];
    s0: per-sequence initial states [N, H, d_v, d_k] or None (zeros).
    Returns (o [T, H, d_v] fp64, s_final [N, H, d_v, d_k] fp64).
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch")
    if N < 0 or (N > 0 and (cu[0] != 0 or cu[-1] > T)):
        raise ValueError("bad cu_seqlens")
    o = np.zeros((T, H, dv), dtype=np.float64)
    s_out = np.zeros((max(N, 0), H, dv, dk), dtype=np.float64)
    if s0 is not None:
        s0 = _f64(s0)
        if s0.shape != (N, H, dv, dk):
            raise ValueError("s0 must be [N, H, d_v, d_k]")
    if N == 0:
        return o, s_out
    nt = threads if threads is not None else default_threads()
    dp = ctypes.c_double
    rc = _load(precision).kda_oracle_prefill(
        _ptr(q, dp), _ptr(k, dp), _ptr(v, dp), _ptr(g, dp), _ptr(beta, dp),
        _ptr(cu, ctypes.c_int32), N, H, dk, dv,
        _ptr(s0, dp) if s0 is not None else None, _ptr(s_out, dp), _ptr(o, dp),
        float(scale), int(nt))
    if rc != 0:
        raise RuntimeError("kda_oracle_prefill failed with %d" % rc)
    return o, s_out


def chunk_prefill(q, k, v, g, beta, cu_seqlens, state_pool=None, slots=None, scale=1.0,
                  o_init=None, threads=None, num_slots=None):
    """The boundary's prefill semantics on top of the recurrence.

    state_pool: [num_slots, H, d_v, d_k] or None (zero initial states, final
    states not kept).  slots: [N] or None (identity).  num_slots: the slot
    index space (default: the pool's rows, or N without a pool); with slots
    given, a slot outside [0, num_slots) is a padded sequence.  o_init: the contents of
    the output buffer before the call (rows of skipped sequences keep them);
    zeros when None.
    Returns (o [T,H,d_v] fp64, pool_out [num_slots,H,d_v,d_k] fp64 or None,
    s_final [N,H,d_v,d_k] fp64 with zeros for skipped sequences).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    T, H, dk = np.shape(q)
    dv = np.shape(v)[2]
    if num_slots is None:
        num_slots = N if state_pool is None else np.shape(state_pool)[0]
    if slots is None:
        sl = np.arange(N, dtype=np.int64)
        live = np.ones(N, dtype=bool)
    else:
        sl = np.asarray(slots, dtype=np.int64)
        live = (sl >= 0) & (sl < num_slots)
    if state_pool is not None:
        pool = _f64(state_pool)
        s0 = np.zeros((N, H, dv, dk), dtype=np.float64)
        s0[live] = pool[sl[live]]
    else:
        pool = None
        s0 = None
    o, s_fin = recurrence(q, k, v, g, beta, cu.astype(np.int32), s0=s0, scale=scale, threads=threads)
    o_out = np.zeros((T, H, dv), dtype=np.float64) if o_init is None else _f64(o_init).copy()
    for n in range(N):
        if live[n]:
            o_out[cu[n]:cu[n + 1]] = o[cu[n]:cu[n + 1]]
    s_fin[~live] = 0.0
    pool_out = None
    if pool is not None:
        pool_out = pool.copy()
        pool_out[sl[live]] = s_fin[live]
    return o_out, pool_out, s_fin


def decode_step(q, k, v, g, beta, state_pool, slots, scale=1.0, o_init=None, threads=None):
    """One token per sequence, state updated in place in the pool.

    q, k, g: [N, H, d_k]; v: [N, H, d_v]; beta: [N, H]; state_pool:
    [num_slots, H, d_v, d_k]; slots [N] (entries outside [0, num_slots) are
    padded rows: o untouched, no state touched).
    Returns (o [N,H,d_v] fp64, pool_out fp64).
    """
    N = np.shape(q)[0]
    cu = np.arange(N + 1, dtype=np.int32)
    o, pool_out, _ = chunk_prefill(q, k, v, g, beta, cu, state_pool=state_pool, slots=slots,
                                   scale=scale, o_init=o_init, threads=threads)
    return o, pool_out


def decode_tokens(q, k, v, g, beta, state_pool, slots, num_accepted=None, commit=True, scale=1.0,
                  o_init=None, threads=None):
    """T tokens per sequence against one state: multi-token decode, and the
    verify and commit of speculative tokens (the prhub report on SGLang PR
    #32890, section "关键文件": the conv-MTP decode kernel's multi-token
    verify, and ReplaySSM's exact fold of the accepted tokens at commit).

    q, k, g: [N, T, H, d_k]; v: [N, T, H, d_v]; beta: [N, T, H]; state_pool
    [num_slots, H, d_v, d_k]; slots [N] (padded rows as in decode_step).
    Every token's output is the recurrence's output over the sequence's
    tokens 0..t from its slot's state, i.e. what t + 1 decode steps give.
    With commit, the slot's state becomes the state after the first c_n
    tokens, c_n = num_accepted[n] clamped to [0, T] (T when None); c_n = 0
    and commit=False leave it unchanged.
    Returns (o [N,T,H,d_v] fp64, pool_out fp64).
    """
    N, T, H, dk = np.shape(k)
    dv = np.shape(v)[3]

    def rows(x, d=None):
        x = np.asarray(x)
        return x.reshape((N * T, H) if d is None else (N * T, H, d))

    cu = np.arange(0, N * T + 1, T, dtype=np.int32)
    oi = None if o_init is None else rows(o_init, dv)
    o, _, _ = chunk_prefill(rows(q, dk), rows(k, dk), rows(v, dv), rows(g, dk), rows(beta), cu,
                            state_pool=state_pool, slots=slots, scale=scale, o_init=oi,
                            threads=threads)
    pool_out = _f64(state_pool).copy()
    if commit:
        c = np.full(N, T, dtype=np.int64) if num_accepted is None else \
            np.clip(np.asarray(num_accepted, dtype=np.int64), 0, T)
        keep = np.concatenate([n * T + np.arange(c[n]) for n in range(N)]).astype(np.int64)
        cu_c = np.concatenate([[0], np.cumsum(c)]).astype(np.int32)
        _, pool_out, _ = chunk_prefill(rows(q, dk)[keep], rows(k, dk)[keep], rows(v, dv)[keep],
                                       rows(g, dk)[keep], rows(beta)[keep], cu_c,
                                       state_pool=state_pool, slots=slots, scale=scale,
                                       threads=threads)
    return o.reshape(N, T, H, dv), pool_out


# ---------------------------------------------------------------------------
# Short conv front end.  On the prefill side of the kern-k3-pp-prefill page
# every sequence carries a conv window next to its recurrent state (section
# "P: the packed prefill"), its decode build fuses the conv into the step
# (section "D: TP8 / EP8 / DCP8"), and SGLang keeps the window as
# [slot][tap][q|k|v] bf16 (section "D inside SGLang").  The page's state size (the "kern" page,
# section "The manifest": 19,537,920 bytes a sequence, 288 blocks of a
# 64 KiB state plus 3 x 3 x 128 bf16) gives a window of 3 rows.  Reading: the
# window holds a sequence's 3 most recent raw inputs, so the conv is causal,
# per channel, of width 4; an optional SiLU follows it.

CONV_WINDOW = 3
CONV_WIDTH = CONV_WINDOW + 1


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def conv_front(q, k, v, cu_seqlens, weight, window=None, slots=None, num_slots=None,
               activation="none"):
    """Causal per-channel conv of width 4 over the channels [q | k | v] of each
    head, run per sequence from the sequence's conv window.

    q, k: [T, H, d_k]; v: [T, H, d_v]; weight: [H, 4, 2 d_k + d_v], tap j
    multiplying input x_{t-3+j}; window: [num_slots, H, 3, 2 d_k + d_v] raw
    inputs, row i holding x_{start-3+i}, or None for zeros.  slots and
    num_slots as in chunk_prefill; a padded sequence convolves from a zero
    window and leaves every window untouched.  activation: "none" or "silu".
    Returns (qc, kc, vc) in fp64 and the window pool after the call (fp64, or
    None without a window pool): each live sequence's slot then holds its
    last 3 raw inputs, older window rows filling in for short sequences.
    """
    q, k, v, w = _f64(q), _f64(k), _f64(v), _f64(weight)
    T, H, dk = q.shape
    dv = v.shape[2]
    C = 2 * dk + dv
    if w.shape != (H, CONV_WIDTH, C):
        raise ValueError("weight must be [H, 4, 2 d_k + d_v]")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    if num_slots is None:
        num_slots = N if window is None else np.shape(window)[0]
    sl = np.arange(N) if slots is None else np.asarray(slots, dtype=np.int64)
    live = (sl >= 0) & (sl < num_slots)
    x = np.concatenate([q, k, v], axis=2)                      # [T, H, C]
    y = np.zeros_like(x)
    win = None if window is None else _f64(window).copy()
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        w0 = win[sl[n]] if (win is not None and live[n]) else np.zeros((H, CONV_WINDOW, C))
        ext = np.concatenate([w0.transpose(1, 0, 2), x[a:b]], axis=0)   # [L + 3, H, C]
        for t in range(b - a):
            acc = np.zeros((H, C))
            for j in range(CONV_WIDTH):
                acc += w[:, j, :] * ext[t + j]
            y[a + t] = acc
        if win is not None and live[n]:
            win[sl[n]] = ext[-CONV_WINDOW:].transpose(1, 0, 2)
    if activation == "silu":
        y = silu(y)
    elif activation != "none":
        raise ValueError("activation must be 'none' or 'silu'")
    return y[:, :, :dk], y[:, :, dk:2 * dk], y[:, :, 2 * dk:], win


def chunk_prefill_conv(q, k, v, g, beta, cu_seqlens, weight, window=None, state_pool=None,
                       slots=None, scale=1.0, o_init=None, num_slots=None, activation="none",
                       threads=None):
    """chunk_prefill on the conv front end's outputs (q, k, v are the raw
    inputs).  Returns (o, pool_out, s_final, window_out)."""
    if num_slots is None:
        if state_pool is not None:
            num_slots = np.shape(state_pool)[0]
        elif window is not None:
            num_slots = np.shape(window)[0]
    qc, kc, vc, win = conv_front(q, k, v, cu_seqlens, weight, window, slots, num_slots,
                                 activation)
    o, pool_out, s_fin = chunk_prefill(qc, kc, vc, g, beta, cu_seqlens, state_pool=state_pool,
                                       slots=slots, scale=scale, o_init=o_init,
                                       threads=threads, num_slots=num_slots)
    return o, pool_out, s_fin, win


def decode_step_conv(q, k, v, g, beta, state_pool, slots, weight, window, scale=1.0,
                     o_init=None, activation="none", threads=None):
    """decode_step with the conv front end: one token per sequence, state and
    window pools updated.  Returns (o, pool_out, window_out)."""
    N = np.shape(q)[0]
    cu = np.arange(N + 1, dtype=np.int32)
    qc, kc, vc, win = conv_front(q, k, v, cu, weight, window, slots, np.shape(state_pool)[0],
                                 activation)
    o, pool_out = decode_step(qc, kc, vc, g, beta, state_pool, slots, scale=scale,
                              o_init=o_init, threads=threads)
    return o, pool_out, win
