"""Seeded synthetic inputs for the KDA prefill and decode paths.

This module holds only random draws, input normalisation and dtype casting:
none of the method's arithmetic.  Both the HIP path's tests and the oracle take
their inputs from here; neither side imports the other.

Shapes and distributions follow the workloads the pages run KDA under (the
kern-k3-pp-prefill page, sections "P: the packed prefill" and "Deploy": up to
16 sequences packed back to back in an 8192-row chunk, 262144-token context,
decode batches of at most 64 sequences; the kern page, section "The manifest":
one state slot per sequence):

* q, k ~ N(0, 1), L2-normalised over d_k per (token, head), in fp64, then
  cast to fp32 and, for bf16 inputs, rounded to bf16 (round to nearest even);
* v ~ N(0, 1), cast the same way;
* g = -softplus(N(mu_g, 1)) per key channel, fp32 (natural-log decay <= 0);
* beta = sigmoid(N(0, 1)) per (token, head), fp32;
* state pools ~ N(0, 0.02^2) fp32, layout [slot][head][d_v][d_k].

Streams per case: numpy SeedSequence(seed) spawns four children, for the
tokens (q, k, v, g, beta in that order, each drawn in 256-row blocks from
child streams of its own), the pool (one child per slot), the lengths and the
slots.
Every array is returned as float32 (bf16 cases hold exactly bf16-representable
values) so that both sides see identical numbers.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest bf16 (ties to even); returns fp32."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _cast(x64: np.ndarray, io_dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return round_to_bf16(x32) if io_dtype == "bf16" else x32


def _l2norm(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


# Row blocks drawn from their own child streams, so generation is
# deterministic for a seed whatever the number of worker threads.
_BLOCK_ROWS = 256
_WORKERS = max(1, min(16, (len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                            else (os.cpu_count() or 1))))


def _blocked(ss: np.random.SeedSequence, T: int, fn) -> np.ndarray:
    """Concatenate fn(rng, rows) over row blocks, block b using child b of ss."""
    nb = max(1, (T + _BLOCK_ROWS - 1) // _BLOCK_ROWS)
    kids = ss.spawn(nb)
    sizes = [min(_BLOCK_ROWS, T - b * _BLOCK_ROWS) for b in range(nb)]
    if T == 0:
        sizes = [0]

    def run(b):
        return fn(np.random.default_rng(kids[b]), sizes[b])

    if nb == 1 or _WORKERS == 1:
        parts = [run(b) for b in range(nb)]
    else:
        with ThreadPoolExecutor(_WORKERS) as ex:
            parts = list(ex.map(run, range(nb)))
    return np.concatenate(parts, axis=0)


@dataclass
class Case:
    """One call's inputs.  ``io_dtype`` is the dtype of q, k, v and o."""
    name: str
    q: np.ndarray            # [T, H, d_k] f32
    k: np.ndarray            # [T, H, d_k] f32
    v: np.ndarray            # [T, H, d_v] f32
    g: np.ndarray            # [T, H, d_k] f32
    beta: np.ndarray         # [T, H] f32
    cu_seqlens: np.ndarray   # [N+1] int32
    io_dtype: str            # "bf16" or "f32"
    state_pool: Optional[np.ndarray] = None   # [num_slots, H, d_v, d_k] f32
    slots: Optional[np.ndarray] = None        # [N] int32
    scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def d_k(self):
        return self.q.shape[2]

    @property
    def d_v(self):
        return self.v.shape[2]

    @property
    def N(self):
        return self.cu_seqlens.shape[0] - 1


def draw_tokens(ss: np.random.SeedSequence, T, H, dk, dv, io_dtype, mu_g=0.0):
    """q, k, v, g, beta for T rows; child streams 0..4 of ss, in that order."""
    cq, ck, cv, cg, cb = ss.spawn(5)
    unit = lambda d: (lambda r, n: _cast(_l2norm(r.standard_normal((n, H, d))), io_dtype))
    q = _blocked(cq, T, unit(dk))
    k = _blocked(ck, T, unit(dk))
    v = _blocked(cv, T, lambda r, n: _cast(r.standard_normal((n, H, dv)), io_dtype))
    g = _blocked(cg, T, lambda r, n: (-np.logaddexp(0.0, r.normal(mu_g, 1.0, (n, H, dk))))
                 .astype(np.float32))
    beta = _blocked(cb, T, lambda r, n: (1.0 / (1.0 + np.exp(-r.standard_normal((n, H)))))
                    .astype(np.float32))
    return q, k, v, g, beta


def draw_pool(ss: np.random.SeedSequence, num_slots, H, dv, dk, std=0.02):
    """State pool [num_slots, H, d_v, d_k] ~ N(0, std^2), one child stream per slot."""
    return _blocked_slots(ss, num_slots, lambda r: r.normal(0.0, std, (H, dv, dk)).astype(np.float32))


def _blocked_slots(ss, n, fn):
    kids = ss.spawn(n)
    if n == 0:
        return np.zeros((0,) + fn(np.random.default_rng(0)).shape, dtype=np.float32)
    with ThreadPoolExecutor(_WORKERS) as ex:
        return np.stack(list(ex.map(lambda c: fn(np.random.default_rng(c)), kids)))


def _streams(seed):
    """Child streams of a case: [tokens, pool, lengths, slots]."""
    return np.random.SeedSequence(seed).spawn(4)


def dirichlet_lengths(rng, total=8192, n=16, min_unaligned=9, chunk=64):
    """Sequence lengths for a packed chunk: a seeded Dirichlet(1) partition of
    ``total`` rows into ``n`` sequences, every length >= 1, the smallest forced
    to 1, redrawn until at least ``min_unaligned`` lengths are not multiples of
    ``chunk``."""
    while True:
        p = rng.dirichlet(np.ones(n))
        spare = total - n
        raw = p * spare
        L = 1 + np.floor(raw).astype(np.int64)
        rem = total - int(L.sum())
        frac = raw - np.floor(raw)
        for i in np.argsort(-frac, kind="stable")[:rem]:
            L[i] += 1
        i_min = int(np.argmin(L))
        i_max = int(np.argmax(L))
        excess = int(L[i_min]) - 1
        L[i_min] = 1
        L[i_max] += excess
        assert int(L.sum()) == total and L.min() >= 1
        if int(np.sum(L % chunk != 0)) >= min_unaligned:
            return L


def cu_from_lengths(L) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(L, dtype=np.int64))]).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

def tiny_prefill(seed=1) -> Case:
    """1 sequence, T=256, H=2, d_k=d_v=64, fp32 throughout, zero initial state."""
    st = _streams(seed)
    q, k, v, g, beta = draw_tokens(st[0], 256, 2, 64, 64, "f32")
    return Case("tiny_prefill_T256_H2_d64_f32", q, k, v, g, beta,
                cu_from_lengths([256]), "f32")


def single_seq_prefill(seed=2, T=8192, H=32, d=128) -> Case:
    """1 sequence of T rows, bf16 q/k/v/o, fp32 g/beta/state, zero initial state."""
    st = _streams(seed)
    q, k, v, g, beta = draw_tokens(st[0], T, H, d, d, "bf16")
    return Case("single_seq_prefill_T%d_H%d_d%d_bf16" % (T, H, d), q, k, v, g, beta,
                cu_from_lengths([T]), "bf16")


def packed_varlen_prefill(seed=3, T=8192, H=32, d=128, n=16, num_slots=64) -> Case:
    """n sequences packed in T rows (Dirichlet lengths), states gathered from a
    num_slots pool by an int32 slot index and scattered back."""
    st = _streams(seed)
    q, k, v, g, beta = draw_tokens(st[0], T, H, d, d, "bf16")
    pool = draw_pool(st[1], num_slots, H, d, d)
    L = dirichlet_lengths(np.random.default_rng(st[2]), T, n)
    slots = np.random.default_rng(st[3]).permutation(num_slots)[:n].astype(np.int32)
    return Case("packed_varlen_prefill_N%d_T%d_H%d_d%d_bf16" % (n, T, H, d), q, k, v, g, beta,
                cu_from_lengths(L), "bf16", state_pool=pool, slots=slots,
                meta={"lengths": L.tolist()})


LONG_CONTEXT_CALLS = 32


def long_context_call(c, T=8192, H=32, d=128, mu_g=-4.0) -> Case:
    """Call c (0-based) of a 262144-token sequence fed as 32 consecutive
    8192-row calls; slow decay g = -softplus(N(-4, 1)).  Seed (4, c).  The
    state is carried by the caller through a one-slot pool that starts at
    zero."""
    st = _streams([4, c])
    q, k, v, g, beta = draw_tokens(st[0], T, H, d, d, "bf16", mu_g=mu_g)
    return Case("long_context_call%d_T%d_H%d_d%d_bf16" % (c, T, H, d), q, k, v, g, beta,
                cu_from_lengths([T]), "bf16", slots=np.zeros(1, dtype=np.int32),
                meta={"call": c})


def decode_case(seed=5, n=64, H=32, d=128, num_slots=64) -> Case:
    """n sequences x 1 token, states from a num_slots pool updated in place."""
    st = _streams(seed)
    q, k, v, g, beta = draw_tokens(st[0], n, H, d, d, "bf16")
    pool = draw_pool(st[1], num_slots, H, d, d)
    slots = np.random.default_rng(st[3]).permutation(num_slots)[:n].astype(np.int32)
    return Case("decode_N%d_H%d_d%d_bf16" % (n, H, d), q, k, v, g, beta,
                np.arange(n + 1, dtype=np.int32), "bf16", state_pool=pool, slots=slots)


def decode_tokens_case(seed=7, n=64, tokens=4, H=32, d=128, num_slots=64) -> Case:
    """n sequences x `tokens` draft tokens (rows n * tokens + t), states from a
    num_slots pool: the multi-token decode / speculative-verify shape."""
    st = _streams(seed)
    q, k, v, g, beta = draw_tokens(st[0], n * tokens, H, d, d, "bf16")
    pool = draw_pool(st[1], num_slots, H, d, d)
    slots = np.random.default_rng(st[3]).permutation(num_slots)[:n].astype(np.int32)
    return Case("decode_tokens_N%d_T%d_H%d_d%d_bf16" % (n, tokens, H, d), q, k, v, g, beta,
                np.arange(0, n * tokens + 1, tokens, dtype=np.int32), "bf16", state_pool=pool,
                slots=slots, meta={"tokens": tokens})


CONV_TAP_SCALE = (0.1, 0.15, 0.25, 0.5)   # bound on |tap j|; the bounds sum to 1


def draw_conv(seed, num_slots, H, d_k, d_v, io_dtype="bf16"):
    """Synthetic short-conv parameters: taps [H, 4, 2 d_k + d_v] fp32, tap j
    uniform in +-CONV_TAP_SCALE[j] (so a conv of unit-norm rows stays within
    unit norm), and a window pool [num_slots, H, 3, 2 d_k + d_v] of raw
    inputs drawn like tokens (unit-norm q and k rows, N(0, 1) v), rounded to
    the io dtype."""
    ss = np.random.SeedSequence([seed, 0xC0])
    cw, cq, ck, cv = ss.spawn(4)
    C = 2 * d_k + d_v
    rng = np.random.default_rng(cw)
    weight = (rng.uniform(-1.0, 1.0, (H, 4, C)) *
              np.asarray(CONV_TAP_SCALE)[None, :, None]).astype(np.float32)
    n = num_slots * 3
    wq = _l2norm(np.random.default_rng(cq).standard_normal((n, H, d_k)))
    wk = _l2norm(np.random.default_rng(ck).standard_normal((n, H, d_k)))
    wv = np.random.default_rng(cv).standard_normal((n, H, d_v))
    win = np.concatenate([_cast(wq, io_dtype), _cast(wk, io_dtype), _cast(wv, io_dtype)], axis=2)
    window = win.reshape(num_slots, 3, H, C).transpose(0, 2, 1, 3).copy()
    return weight, window


def random_case(seed, lengths, H=2, d_k=64, d_v=64, io_dtype="bf16", num_slots=None,
                with_state=True, mu_g=0.0, scale=1.0, slots=None, pool_std=0.1) -> Case:
    """A small packed case for sweeps: given per-sequence lengths (zero allowed)."""
    st = _streams(seed)
    L = np.asarray(lengths, dtype=np.int64)
    T = int(L.sum())
    q, k, v, g, beta = draw_tokens(st[0], T, H, d_k, d_v, io_dtype, mu_g=mu_g)
    n = len(L)
    pool = None
    if with_state:
        ns = num_slots if num_slots is not None else n + 3
        pool = draw_pool(st[1], ns, H, d_v, d_k, std=pool_std)
        if slots is None:
            slots = np.random.default_rng(st[3]).permutation(ns)[:n].astype(np.int32)
    return Case("random_seed%d_N%d_T%d_H%d_dk%d_dv%d_%s" % (seed, n, T, H, d_k, d_v, io_dtype),
                q, k, v, g, beta, cu_from_lengths(L), io_dtype, state_pool=pool,
                slots=None if slots is None else np.asarray(slots, dtype=np.int32), scale=scale,
                meta={"lengths": L.tolist()})
