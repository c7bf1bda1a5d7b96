"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes one part of the recurrence so that a plausible slip (a dropped
decay, decay after the write, output before the update, a wrong sign, a
transposed state, exp2 for exp, a wrong head or sequence index) fails at least
one of them:

* hand-worked d=2 example (tests/golden/hand_worked_d2_t2.txt): order of decay
  and write, sign, inclusive output, [v][k] state layout, natural exp;
* literal matrix products (I - beta k k^T) Diag(exp g) S + beta k v^T on T <= 4
  with random S0 over several heads and sequences: the whole algebra;
* beta = 0: pure decay closed form; g = 0 and beta = 0: identity;
* beta = 1, |k| = 1, q = k: o_t = v_t exactly, for any decay;
* orthonormal keys e_i, beta = 1, g = 0: row i of S replaced by v_t;
* split continuity, linearity in (v, S0), value-column independence;
* varlen independence and permutation of the pack;
* the chunk (WY) form in ``oracle/chunked.py`` against the recurrence.
"""
import os

import numpy as np
import pytest

from oracle import chunked, oracle
from linear_attention_prefill_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, H, dk, dv, unit_k=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def _literal(q, k, v, g, beta, cu, s0):
    """(I - beta k k^T) Diag(exp g) S + beta k v^T, o = S^T q, as explicit
    matrix products per token (written independently of the oracle)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dv, dk))
    for n in range(N):
        for h in range(H):
            S = s0[n, h].T.copy()
            for t in range(cu[n], cu[n + 1]):
                kt = k[t, h][:, None]
                M = np.eye(dk) - beta[t, h] * (kt @ kt.T)
                S = M @ np.diag(np.exp(g[t, h])) @ S + beta[t, h] * kt @ v[t, h][None, :]
                o[t, h] = S.T @ q[t, h]
            sf[n, h] = S.T
    return o, sf


def test_hand_worked_example():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_worked_d2_t2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = np.array([float(x) for x in nums])
    T, H, d = 2, 1, 2
    q = np.stack([vals["t1_q"], vals["t2_q"]])[:, None, :]
    k = np.stack([vals["t1_k"], vals["t2_k"]])[:, None, :]
    v = np.stack([vals["t1_v"], vals["t2_v"]])[:, None, :]
    g = np.log(np.stack([vals["t1_expg"], vals["t2_expg"]]))[:, None, :]
    beta = np.array([vals["t1_beta"][0], vals["t2_beta"][0]])[:, None]
    s0 = vals["s0_pool"].reshape(1, 1, d, d)
    o, sf = oracle.recurrence(q, k, v, g, beta, [0, 2], s0=s0)
    np.testing.assert_allclose(o[0, 0], vals["o1"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[1, 0], vals["o2"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sf[0, 0].ravel(), vals["s2_pool"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_brute_force_literal_products(T):
    rng = np.random.default_rng(100 + T)
    H, dk, dv = 3, 5, 4
    # two sequences of length T, plus random initial states
    q, k, v, g, beta = _rand_inputs(rng, 2 * T, H, dk, dv, unit_k=False)
    cu = [0, T, 2 * T]
    s0 = rng.standard_normal((2, H, dv, dk))
    o_ref, s_ref = _literal(q, k, v, g, beta, cu, s0)
    o, sf = oracle.recurrence(q, k, v, g, beta, cu, s0=s0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sf, s_ref, rtol=1e-12, atol=1e-12)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(7)
    T, H, dk, dv = 37, 2, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    beta[:] = 0.0
    s0 = rng.standard_normal((1, H, dv, dk))
    o, sf = oracle.recurrence(q, k, v, g, beta, [0, T], s0=s0)
    gam = np.cumsum(g, axis=0)  # inclusive [T, H, dk]
    for h in range(H):
        S0 = s0[0, h].T
        np.testing.assert_allclose(sf[0, h].T, np.exp(gam[-1, h])[:, None] * S0, rtol=1e-12, atol=1e-14)
        o_cf = (q[:, h] * np.exp(gam[:, h])) @ S0
        np.testing.assert_allclose(o[:, h], o_cf, rtol=1e-11, atol=1e-14)


def test_identity_when_no_decay_no_write():
    rng = np.random.default_rng(8)
    T, H, dk, dv = 20, 2, 6, 7
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    g[:] = 0.0
    beta[:] = 0.0
    s0 = rng.standard_normal((1, H, dv, dk))
    o, sf = oracle.recurrence(q, k, v, g, beta, [0, T], s0=s0)
    np.testing.assert_array_equal(sf, s0)
    for h in range(H):
        np.testing.assert_allclose(o[:, h], q[:, h] @ s0[0, h].T, rtol=1e-13, atol=1e-14)


def test_unit_key_full_write_returns_value():
    """beta = 1, |k| = 1 and q = k give S_t^T k_t = v_t for any decay."""
    rng = np.random.default_rng(9)
    T, H, dk, dv = 50, 3, 16, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    beta[:] = 1.0
    q = k.copy()
    s0 = rng.standard_normal((1, H, dv, dk))
    o, _ = oracle.recurrence(q, k, v, g, beta, [0, T], s0=s0)
    np.testing.assert_allclose(o, v, rtol=1e-11, atol=1e-11)


def test_orthonormal_keys_replace_rows():
    rng = np.random.default_rng(10)
    T, H, dk, dv = 12, 1, 4, 3
    q, _, v, _, _ = _rand_inputs(rng, T, H, dk, dv)
    idx = rng.integers(0, dk, T)
    k = np.zeros((T, H, dk))
    k[np.arange(T), 0, idx] = 1.0
    g = np.zeros((T, H, dk))
    beta = np.ones((T, H))
    S = rng.standard_normal((dk, dv))
    s0 = S.T[None, None].copy()
    o, sf = oracle.recurrence(q, k, v, g, beta, [0, T], s0=s0)
    for t in range(T):
        S[idx[t]] = v[t, 0]
        np.testing.assert_allclose(o[t, 0], S.T @ q[t, 0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sf[0, 0], S.T, rtol=0, atol=1e-14)


def test_split_continuity():
    rng = np.random.default_rng(11)
    T1, T2, H, dk, dv = 70, 45, 2, 16, 16
    q, k, v, g, beta = _rand_inputs(rng, T1 + T2, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk)) * 0.1
    o_all, s_all = oracle.recurrence(q, k, v, g, beta, [0, T1 + T2], s0=s0)
    o1, s1 = oracle.recurrence(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], [0, T1], s0=s0)
    o2, s2 = oracle.recurrence(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], [0, T2], s0=s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, s_all, rtol=1e-12, atol=1e-13)


def test_linearity_in_values_and_state():
    rng = np.random.default_rng(12)
    T, H, dk, dv = 40, 2, 8, 8
    q, k, v1, g, beta = _rand_inputs(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, dv, dk))
    s2 = rng.standard_normal((1, H, dv, dk))
    a, b = 0.7, -1.3
    oa, sa = oracle.recurrence(q, k, v1, g, beta, [0, T], s0=s1)
    ob, sb = oracle.recurrence(q, k, v2, g, beta, [0, T], s0=s2)
    oc, sc = oracle.recurrence(q, k, a * v1 + b * v2, g, beta, [0, T], s0=a * s1 + b * s2)
    np.testing.assert_allclose(oc, a * oa + b * ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sc, a * sa + b * sb, rtol=1e-11, atol=1e-12)


def test_value_columns_are_independent():
    """Column j of S depends only on column j of v and of S0: running on a
    subset of value columns returns exactly those columns."""
    rng = np.random.default_rng(13)
    T, H, dk, dv = 60, 2, 8, 10
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    cols = np.array([1, 4, 9])
    o, sf = oracle.recurrence(q, k, v, g, beta, [0, T], s0=s0)
    o_s, sf_s = oracle.recurrence(q, k, v[:, :, cols], g, beta, [0, T], s0=s0[:, :, cols])
    np.testing.assert_array_equal(o_s, o[:, :, cols])
    np.testing.assert_array_equal(sf_s, sf[:, :, cols])


def test_scale_multiplies_output_only():
    rng = np.random.default_rng(14)
    T, H, dk, dv = 30, 1, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    o1, s1 = oracle.recurrence(q, k, v, g, beta, [0, T])
    o2, s2 = oracle.recurrence(q, k, v, g, beta, [0, T], scale=0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(s1, s2)


def test_varlen_independence_and_permutation():
    rng = np.random.default_rng(15)
    L = [5, 0, 64, 1, 77, 13]
    H, dk, dv = 2, 8, 8
    cu = W.cu_from_lengths(L)
    T = int(cu[-1])
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((len(L), H, dv, dk))
    o, sf = oracle.recurrence(q, k, v, g, beta, cu, s0=s0)
    for n in range(len(L)):
        a, b = cu[n], cu[n + 1]
        on, sn = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a], s0=s0[n:n + 1])
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(sf[n], sn[0])
    # permuting the pack permutes the outputs
    perm = rng.permutation(len(L))
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in perm])
    cu_p = W.cu_from_lengths([L[n] for n in perm])
    op, sp = oracle.recurrence(q[rows], k[rows], v[rows], g[rows], beta[rows], cu_p, s0=s0[perm])
    np.testing.assert_array_equal(op, o[rows])
    np.testing.assert_array_equal(sp, sf[perm])


def test_zero_length_sequence_copies_state():
    rng = np.random.default_rng(16)
    H, dk, dv = 2, 4, 4
    q, k, v, g, beta = _rand_inputs(rng, 3, H, dk, dv)
    s0 = rng.standard_normal((2, H, dv, dk))
    _, sf = oracle.recurrence(q, k, v, g, beta, [0, 0, 3], s0=s0)
    np.testing.assert_array_equal(sf[0], s0[0])


@pytest.mark.parametrize("chunk", [1, 16, 64])
@pytest.mark.parametrize("T", [1, 65, 77, 130, 200, 256])
def test_chunk_form_matches_recurrence(chunk, T):
    rng = np.random.default_rng(1000 + T + chunk)
    H, dk, dv = 2, 16, 12
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk)) * 0.1
    o_ref, s_ref = oracle.recurrence(q, k, v, g, beta, [0, T], s0=s0, scale=0.5)
    o_c, s_c = chunked.chunk_prefill(q, k, v, g, beta, [0, T], s0=s0, chunk=chunk, scale=0.5)
    np.testing.assert_allclose(o_c, o_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s_c, s_ref, rtol=1e-10, atol=1e-11)


def test_chunk_form_packed_varlen():
    rng = np.random.default_rng(17)
    L = [1, 63, 64, 65, 0, 130]
    cu = W.cu_from_lengths(L)
    T = int(cu[-1])
    H, dk, dv = 2, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((len(L), H, dv, dk)) * 0.1
    o_ref, s_ref = oracle.recurrence(q, k, v, g, beta, cu, s0=s0)
    o_c, s_c = chunked.chunk_prefill(q, k, v, g, beta, cu, s0=s0, chunk=64)
    np.testing.assert_allclose(o_c, o_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s_c, s_ref, rtol=1e-10, atol=1e-11)


def test_pool_semantics_gather_scatter_and_padding():
    """Slots gather the initial states and scatter the final ones; a slot
    outside the pool marks a padded sequence that touches nothing."""
    c = W.random_case(21, [3, 0, 9, 4], H=2, d_k=8, d_v=8, io_dtype="f32", num_slots=7)
    slots = np.array([5, 2, -1, 0], dtype=np.int32)
    o_init = np.full((c.T, c.H, c.d_v), 7.0)
    o, pool_out, _ = oracle.chunk_prefill(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens,
                                          state_pool=c.state_pool, slots=slots, o_init=o_init)
    cu = c.cu_seqlens
    # padded sequence 2: output rows untouched
    np.testing.assert_array_equal(o[cu[2]:cu[3]], o_init[cu[2]:cu[3]])
    # untouched slots keep their bytes
    for s in (1, 3, 4, 6):
        np.testing.assert_array_equal(pool_out[s], c.state_pool[s])
    # zero-length sequence 1 copies slot 2 through
    np.testing.assert_array_equal(pool_out[2], c.state_pool[2].astype(np.float64))
    # sequence 0 equals running it alone from slot 5
    o0, s0 = oracle.recurrence(c.q[:3], c.k[:3], c.v[:3], c.g[:3], c.beta[:3], [0, 3],
                               s0=c.state_pool[5:6])
    np.testing.assert_array_equal(o[:3], o0)
    np.testing.assert_array_equal(pool_out[5], s0[0])


def test_decode_is_one_recurrence_step():
    c = W.random_case(22, [1] * 6, H=2, d_k=8, d_v=8, io_dtype="f32", num_slots=9)
    o, pool_out = oracle.decode_step(c.q, c.k, c.v, c.g, c.beta, c.state_pool, c.slots)
    for n in range(6):
        S = c.state_pool[c.slots[n]].astype(np.float64)  # [H, dv, dk]
        for h in range(2):
            St = S[h].T * np.exp(c.g[n, h].astype(np.float64))[:, None]
            kk = c.k[n, h].astype(np.float64)
            d = c.beta[n, h] * (c.v[n, h] - St.T @ kk)
            St = St + np.outer(kk, d)
            np.testing.assert_allclose(o[n, h], St.T @ c.q[n, h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(pool_out[c.slots[n], h], St.T, rtol=1e-12, atol=1e-13)


def test_decode_tokens_against_literal_products():
    """Multi-token decode: each token's output, and the state committed after
    the first c_n accepted tokens, against explicit matrix products; padded
    rows and unnamed slots stay untouched; a verify (no commit) leaves the
    pool as it was."""
    rng = np.random.default_rng(23)
    N, T, H, dk, dv, S = 5, 4, 2, 6, 5, 8
    q, k, v, g, beta = _rand_inputs(rng, N * T, H, dk, dv)
    pool = 0.3 * rng.standard_normal((S, H, dv, dk))
    slots = np.array([6, -1, 0, 3, 8], dtype=np.int32)     # -1 and 8 are padded rows
    acc = np.array([4, 2, 0, 1, 3], dtype=np.int32)
    shape4 = lambda x: x.reshape((N, T) + x.shape[1:])
    o_init = np.full((N, T, H, dv), 9.0)
    args = [shape4(x) for x in (q, k, v, g, beta)]
    o, pool_out = oracle.decode_tokens(*args, pool, slots, num_accepted=acc, o_init=o_init)
    for n in range(N):
        s = int(slots[n])
        if not 0 <= s < S:
            np.testing.assert_array_equal(o[n], o_init[n])
            continue
        r = slice(n * T, (n + 1) * T)
        o_l, _ = _literal(q[r], k[r], v[r], g[r], beta[r], [0, T], pool[s][None])
        np.testing.assert_allclose(o[n], o_l, rtol=1e-11, atol=1e-12)
        c = slice(n * T, n * T + int(acc[n]))
        _, s_l = _literal(q[c], k[c], v[c], g[c], beta[c], [0, int(acc[n])], pool[s][None])
        np.testing.assert_allclose(pool_out[s], s_l[0], rtol=1e-11, atol=1e-12)
    for s in (1, 2, 4, 5, 7):
        np.testing.assert_array_equal(pool_out[s], pool[s])
    o2, pool2 = oracle.decode_tokens(*args, pool, slots, commit=False, o_init=o_init)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(pool2, pool)
    # all tokens committed when no counts are given
    _, pool3 = oracle.decode_tokens(*args, pool, slots)
    _, s_all = _literal(q[:T], k[:T], v[:T], g[:T], beta[:T], [0, T], pool[6][None])
    np.testing.assert_allclose(pool3[6], s_all[0], rtol=1e-11, atol=1e-12)


def test_decode_tokens_single_token_is_decode_step():
    c = W.random_case(24, [1] * 5, H=3, d_k=8, d_v=4, io_dtype="f32", num_slots=7)
    o1, p1 = oracle.decode_step(c.q, c.k, c.v, c.g, c.beta, c.state_pool, c.slots)
    o2, p2 = oracle.decode_tokens(c.q[:, None], c.k[:, None], c.v[:, None], c.g[:, None],
                                  c.beta[:, None], c.state_pool, c.slots)
    np.testing.assert_array_equal(o2[:, 0], o1)
    np.testing.assert_array_equal(p2, p1)


def _conv_inputs(rng, lengths, H, dk, dv, S):
    T = int(sum(lengths))
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    C = 2 * dk + dv
    weight = rng.uniform(-1, 1, (H, 4, C)) * np.array([0.1, 0.15, 0.25, 0.5])[None, :, None]
    window = rng.standard_normal((S, H, 3, C)) * 0.3
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, g, beta, weight, window, cu


def test_conv_front_against_numpy_convolve():
    """Each (sequence, head, channel) is np.convolve of [window; inputs] with
    the reversed taps ('valid' part); SiLU is x * expit(x)."""
    from scipy.special import expit
    rng = np.random.default_rng(31)
    lengths = [5, 1, 0, 2, 9]
    H, dk, dv, S = 2, 3, 4, 7
    q, k, v, g, beta, w, win, cu = _conv_inputs(rng, lengths, H, dk, dv, S)
    slots = np.array([3, 0, 5, -1, 6], dtype=np.int32)
    for act in ("none", "silu"):
        qc, kc, vc, wout = oracle.conv_front(q, k, v, cu, w, win, slots, S, activation=act)
        y = np.concatenate([qc, kc, vc], axis=2)
        x = np.concatenate([q, k, v], axis=2)
        for n in range(len(lengths)):
            a, b = cu[n], cu[n + 1]
            s = slots[n]
            w0 = win[s] if 0 <= s < S else np.zeros((H, 3, 2 * dk + dv))
            for h in range(H):
                for c in range(2 * dk + dv):
                    ext = np.concatenate([w0[h, :, c], x[a:b, h, c]])
                    ref = np.convolve(ext, w[h, ::-1, c], mode="valid")[:b - a]
                    if act == "silu":
                        ref = ref * expit(ref)
                    np.testing.assert_allclose(y[a:b, h, c], ref, rtol=1e-12, atol=1e-14)
                    if 0 <= s < S:
                        np.testing.assert_allclose(wout[s, h, :, c], ext[-3:], rtol=0, atol=0)
        for s in (1, 2, 4):
            np.testing.assert_array_equal(wout[s], win[s])


def test_conv_identity_taps_reduce_to_plain_prefill():
    """Taps (0, 0, 0, 1) with no activation: the conv passes inputs through,
    so prefill with the conv equals prefill without it."""
    rng = np.random.default_rng(32)
    lengths = [6, 2, 11]
    H, dk, dv, S = 2, 4, 3, 5
    q, k, v, g, beta, _, win, cu = _conv_inputs(rng, lengths, H, dk, dv, S)
    w = np.zeros((H, 4, 2 * dk + dv))
    w[:, 3, :] = 1.0
    pool = 0.2 * rng.standard_normal((S, H, dv, dk))
    slots = np.array([4, 1, 2], dtype=np.int32)
    o1, p1, _, wout = oracle.chunk_prefill_conv(q, k, v, g, beta, cu, w, win, pool, slots)
    o2, p2, _ = oracle.chunk_prefill(q, k, v, g, beta, cu, state_pool=pool, slots=slots)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)
    # sequence 1 has 2 rows: the window keeps its newest old row, then the 2 inputs
    x = np.concatenate([q, k, v], axis=2)
    np.testing.assert_array_equal(wout[1][:, 0], win[1][:, 2])
    np.testing.assert_array_equal(wout[1][:, 1:].transpose(1, 0, 2), x[6:8])


def test_conv_prefill_split_and_decode_continuity():
    """One prefill over 13 rows equals 8 rows then 5 rows (state and window
    carried in the pools), and equals 8 rows then 5 decode steps."""
    rng = np.random.default_rng(33)
    H, dk, dv, S = 2, 4, 4, 3
    q, k, v, g, beta, w, win, _ = _conv_inputs(rng, [13], H, dk, dv, S)
    pool = 0.2 * rng.standard_normal((S, H, dv, dk))
    sl = np.array([2], dtype=np.int32)
    full = oracle.chunk_prefill_conv(q, k, v, g, beta, [0, 13], w, win, pool, sl,
                                     activation="silu")
    r1 = slice(0, 8)
    a = oracle.chunk_prefill_conv(q[r1], k[r1], v[r1], g[r1], beta[r1], [0, 8], w, win, pool, sl,
                                  activation="silu")
    r2 = slice(8, 13)
    b = oracle.chunk_prefill_conv(q[r2], k[r2], v[r2], g[r2], beta[r2], [0, 5], w, a[3], a[1],
                                  sl, activation="silu")
    np.testing.assert_allclose(np.concatenate([a[0], b[0]]), full[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b[1], full[1], rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(b[3], full[3])
    pool_d, win_d = a[1], a[3]
    for t in range(8, 13):
        r = slice(t, t + 1)
        o, pool_d, win_d = oracle.decode_step_conv(q[r], k[r], v[r], g[r], beta[r], pool_d, sl, w,
                                                   win_d, activation="silu")
        np.testing.assert_allclose(o[0], full[0][t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(pool_d, full[1], rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(win_d, full[3])
