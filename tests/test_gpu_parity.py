"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: normwise max|x - ref| / max|ref| per sequence, <= 2e-2 with bf16
q/k/v/o and <= 1e-4 with fp32 throughout, for o and for the final states.
Small cases span several 64-row chunks with ragged tails; the five full-size
workloads run in the configuration bench.py times.
"""
import numpy as np
import pytest
import torch

from linear_attention_prefill_amd import workloads as W
from oracle import oracle
from kda_testlib import (TOL, announce, dev, gpu_prefill, oracle_prefill, per_head_error,
                         per_sequence_errors, rel_err, torch_dtype)
import linear_attention_prefill_amd as lap

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _check_case(case, tol=None, **kw):
    tol = TOL[case.io_dtype] if tol is None else tol
    o_init = np.full((case.T, case.H, case.d_v), 3.0, dtype=np.float32)
    announce("prefill %s" % case.name)
    o_g, pool_g = gpu_prefill(case, o_init=o_init, **kw)
    o_r, pool_r, _ = oracle_prefill(case, o_init=o_init, num_slots=kw.get("num_slots"))
    live = None
    if case.slots is not None:
        ns = kw.get("num_slots") or (case.state_pool.shape[0] if case.state_pool is not None
                                     else case.N)
        live = (case.slots >= 0) & (case.slots < ns)
    eo, es = per_sequence_errors(case, o_g, o_r, pool_g, pool_r, live=live)
    announce("  max relative error: o %.3g, state %.3g (tolerance %.3g)" % (eo, es, tol))
    assert eo <= tol, "o error %.3g > %.3g" % (eo, tol)
    assert es <= tol, "state error %.3g > %.3g" % (es, tol)
    return o_g, pool_g, o_r, pool_r, live


def test_tiny_prefill_fp32():
    """1 x 256 rows, H=2, d=64, fp32 throughout, zero initial state."""
    c = W.tiny_prefill()
    announce("prefill %s" % c.name)
    pool = np.zeros((1, c.H, c.d_v, c.d_k), dtype=np.float32)
    o_g, pool_g = gpu_prefill(c, pool=pool, state_in_null=True)
    o_r, s_r = oracle.recurrence(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens)
    eo = per_head_error(o_g, o_r)
    es = max(rel_err(pool_g[0, h], s_r[0, h]) for h in range(c.H))
    announce("  max relative error per head: o %.3g, state %.3g (tolerance 1e-4)" % (eo, es))
    assert eo <= 1e-4 and es <= 1e-4


SWEEP = [
    # (seed, lengths, H, d_k, d_v, io)
    (1, [1], 1, 64, 64, "bf16"),
    (2, [63], 2, 128, 128, "bf16"),
    (3, [64], 2, 128, 128, "bf16"),
    (4, [65], 2, 128, 128, "bf16"),
    (5, [200, 1, 0, 129, 64, 7], 2, 128, 128, "bf16"),
    (6, [130, 77, 1, 63], 3, 64, 64, "bf16"),
    (7, [191, 5], 2, 64, 128, "bf16"),
    (8, [100, 64, 0, 3], 2, 128, 64, "bf16"),
    (9, [1, 63, 64, 65, 2, 127, 128, 129, 0, 31, 33, 96, 250, 1, 17, 60], 2, 128, 128, "bf16"),
    (10, [200, 1, 0, 129, 64, 7], 2, 128, 128, "f32"),
    (11, [130, 77, 1, 63], 3, 64, 64, "f32"),
    (12, [191, 5], 2, 64, 128, "f32"),
    (13, [100, 64, 0, 3], 2, 128, 64, "f32"),
]


@pytest.mark.parametrize("seed,lengths,H,dk,dv,io", SWEEP)
def test_random_sweep(seed, lengths, H, dk, dv, io):
    c = W.random_case(seed, lengths, H=H, d_k=dk, d_v=dv, io_dtype=io)
    o_g, pool_g, o_r, pool_r, live = _check_case(c)
    # slots not named by the call keep their bytes
    used = set(int(s) for s in c.slots)
    for s in range(c.state_pool.shape[0]):
        if s not in used:
            np.testing.assert_array_equal(pool_g[s], c.state_pool[s])


def test_state_in_and_out_separate_buffers():
    c = W.random_case(21, [70, 3, 129], H=2, d_k=128, d_v=128, io_dtype="bf16")
    _check_case(c, in_place=False)


def test_null_state_in_and_null_state_out():
    c = W.random_case(22, [70, 3, 129], H=2, d_k=64, d_v=64, io_dtype="f32")
    announce("prefill %s state_in=NULL" % c.name)
    o_g, pool_g = gpu_prefill(c, state_in_null=True, in_place=False)
    zero_pool = np.zeros_like(c.state_pool)
    o_r, pool_r, _ = oracle_prefill(c, pool=zero_pool)
    eo, es = per_sequence_errors(c, o_g, o_r, pool_g, pool_r)
    assert eo <= 1e-4 and es <= 1e-4
    announce("prefill %s state_out=NULL" % c.name)
    o_g2, _ = gpu_prefill(c, state_out_null=True)
    o_r2, _, _ = oracle_prefill(c)
    assert per_sequence_errors(c, o_g2, o_r2)[0] <= 1e-4


def test_padded_sequences_touch_nothing():
    c = W.random_case(23, [40, 65, 9, 0, 77], H=2, d_k=128, d_v=128, io_dtype="bf16",
                      num_slots=8, slots=[3, -1, 5, 9, 0])
    o_g, pool_g, o_r, pool_r, live = _check_case(c)
    cu = c.cu_seqlens
    # padded sequences 1 (slot -1) and 3 (slot 9 >= 8): o rows keep the sentinel
    assert np.all(o_g[cu[1]:cu[2]] == 3.0)
    for s in (1, 2, 4, 6, 7):
        np.testing.assert_array_equal(pool_g[s], c.state_pool[s])


def test_zero_rows_pass_states_through():
    """T = 0 with three sequences, all empty: no rows and no outputs; each
    sequence's final state is its initial state (the recurrence over no
    tokens), copied to its slot of a separate output pool bit for bit, and the
    slots no sequence names keep their contents.  With the conv front end the
    windows, which hold the last three inputs, stay as they were."""
    H, d, num_slots = 2, 64, 5
    for io in ("bf16", "f32"):
        announce("prefill T=0 N=3 H=%d d=%d %s" % (H, d, io))
        dt = torch_dtype(io)
        # zero-row views of one-row buffers: non-null, aligned pointers
        q, k, v = (torch.zeros((1, H, d), dtype=dt, device="cuda")[:0] for _ in range(3))
        g = torch.zeros((1, H, d), dtype=torch.float32, device="cuda")[:0]
        beta = torch.zeros((1, H), dtype=torch.float32, device="cuda")[:0]
        cu = torch.zeros(4, dtype=torch.int32, device="cuda")
        rng = np.random.default_rng(31)
        s_in = dev((0.02 * rng.standard_normal((num_slots, H, d, d))).astype(np.float32))
        s_out = torch.full_like(s_in, 7.0)
        slots = torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda")
        o = lap.chunk_prefill(q, k, v, g, beta, cu, state_in=s_in, state_out=s_out, slots=slots,
                              num_slots=num_slots)
        torch.cuda.synchronize()
        assert o.shape[0] == 0
        for s in (4, 0, 2):
            assert torch.equal(s_out[s], s_in[s])
        for s in (1, 3):
            assert torch.all(s_out[s] == 7.0)
        # the conv front end over no rows leaves every window as it was
        announce("prefill+conv T=0 N=3 H=%d d=%d %s" % (H, d, io))
        C = 3 * d
        weight = dev(rng.standard_normal((H, 4, C)).astype(np.float32))
        window = dev(rng.standard_normal((num_slots, H, 3, C)).astype(np.float32)).to(dt)
        win0 = window.clone()
        s_out.fill_(7.0)
        lap.chunk_prefill(q, k, v, g, beta, cu, state_in=s_in, state_out=s_out, slots=slots,
                          num_slots=num_slots, conv_weight=weight, conv_window=window,
                          conv_activation="silu")
        torch.cuda.synchronize()
        assert torch.equal(window, win0)
        for s in (4, 0, 2):
            assert torch.equal(s_out[s], s_in[s])


def test_identity_slots():
    c = W.random_case(24, [33, 100], H=2, d_k=64, d_v=64, io_dtype="bf16", num_slots=2)
    c.slots = None
    _check_case(c)


def test_scale_applies_to_output_only():
    c = W.random_case(25, [90, 14], H=2, d_k=128, d_v=128, io_dtype="f32", scale=0.088)
    _check_case(c)


def test_deterministic_reruns():
    c = W.random_case(26, [300, 1, 70], H=4, d_k=128, d_v=128, io_dtype="bf16")
    announce("prefill %s twice" % c.name)
    o1, p1 = gpu_prefill(c)
    o2, p2 = gpu_prefill(c)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2)


def test_split_continuity_across_calls():
    """Feeding a sequence as two calls equals one call (state carried)."""
    c = W.random_case(27, [150, 90], H=2, d_k=128, d_v=128, io_dtype="f32", num_slots=1,
                      slots=[0, 0])
    whole = W.Case("whole", c.q, c.k, c.v, c.g, c.beta, W.cu_from_lengths([240]), "f32",
                   state_pool=c.state_pool, slots=np.zeros(1, np.int32))
    announce("prefill split-continuity whole")
    o_w, p_w = gpu_prefill(whole)
    first = W.Case("first", c.q[:150], c.k[:150], c.v[:150], c.g[:150], c.beta[:150],
                   W.cu_from_lengths([150]), "f32", state_pool=c.state_pool,
                   slots=np.zeros(1, np.int32))
    announce("prefill split-continuity first")
    o_1, p_1 = gpu_prefill(first)
    second = W.Case("second", c.q[150:], c.k[150:], c.v[150:], c.g[150:], c.beta[150:],
                    W.cu_from_lengths([90]), "f32", state_pool=p_1, slots=np.zeros(1, np.int32))
    announce("prefill split-continuity second")
    o_2, p_2 = gpu_prefill(second)
    assert rel_err(np.concatenate([o_1, o_2]), o_w) <= 1e-5
    assert rel_err(p_2, p_w) <= 1e-5


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def test_single_sequence_prefill_full():
    """1 x 8192 rows, H=32, d=128, bf16; whole o and final state vs the oracle."""
    c = W.single_seq_prefill()
    pool = np.zeros((1, c.H, c.d_v, c.d_k), dtype=np.float32)
    announce("prefill %s" % c.name)
    o_g, pool_g = gpu_prefill(c, pool=pool, state_in_null=True)
    o_r, s_r = oracle.recurrence(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens)
    eo = per_head_error(o_g, o_r)
    es = max(rel_err(pool_g[0, h], s_r[0, h]) for h in range(c.H))
    announce("  max relative error per head: o %.3e  state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_packed_varlen_prefill_full():
    """16 Dirichlet-length sequences in 8192 rows, 64-slot pool gathered and
    scattered; untouched slots keep their bytes."""
    c = W.packed_varlen_prefill()
    o_g, pool_g, o_r, pool_r, live = _check_case(c)
    used = set(int(s) for s in c.slots)
    for s in range(c.state_pool.shape[0]):
        if s not in used:
            np.testing.assert_array_equal(pool_g[s], c.state_pool[s])


@pytest.mark.parametrize("H,fuse", [(12, 0), (12, 2)])
def test_packed_prefill_twelve_heads(H, fuse):
    """The packed chunk's sequences at 12 heads, the per-GPU head count of the
    pages' tensor-parallel decode groups (kern-k3-pp-prefill, "D: TP8 / EP8 /
    DCP8"): fewer items than the 32-head call, another slice grouping in the
    scan; fuse = 2 also runs the fused prefill on the sequences of at most
    two chunks beside the two kernels."""
    c = W.packed_varlen_prefill(H=H)
    _check_case(c, fuse_chunks=fuse)


@pytest.mark.timeout(900)
def test_long_context_continuation():
    """262144 tokens, run twice: as 32 consecutive 8192-row calls with the
    state carried in a one-slot pool, and as one 262144-row call (4096 chunks
    in one scan chain, element offsets past 2^31).  Slow decay.  The oracle
    runs the same 32 calls one after another, carrying its fp64 state, over
    every head and value column: the final state and the whole o of the last
    call are checked per head against it."""
    H, d, n_calls = 32, 128, W.LONG_CONTEXT_CALLS
    L = 8192
    T = n_calls * L
    Q = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    K = torch.empty_like(Q)
    V = torch.empty_like(Q)
    G = torch.empty((T, H, d), dtype=torch.float32, device="cuda")
    B = torch.empty((T, H), dtype=torch.float32, device="cuda")
    cu_call = np.array([0, L], dtype=np.int32)
    s_ref = None
    o_ref_last = None
    for c_idx in range(n_calls):
        c = W.long_context_call(c_idx)
        rows = slice(c_idx * L, (c_idx + 1) * L)
        Q[rows] = dev(c.q, torch.bfloat16)
        K[rows] = dev(c.k, torch.bfloat16)
        V[rows] = dev(c.v, torch.bfloat16)
        G[rows] = dev(c.g)
        B[rows] = dev(c.beta)
        o_r, s_ref = oracle.recurrence(c.q, c.k, c.v, c.g, c.beta, cu_call, s0=s_ref)
        if c_idx == n_calls - 1:
            o_ref_last = o_r
    announce("oracle ran %d calls of %d rows, all %d heads, state carried" % (n_calls, L, H))
    cu_dev = dev(cu_call)
    slot0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = torch.zeros((1, H, d, d), dtype=torch.float32, device="cuda")
    o_chain = None
    for c_idx in range(n_calls):
        rows = slice(c_idx * L, (c_idx + 1) * L)
        announce("prefill long_context call %d (carried state)" % c_idx)
        o_chain = lap.chunk_prefill(Q[rows], K[rows], V[rows], G[rows], B[rows], cu_dev,
                                    state_in=pool, state_out=pool, slots=slot0)
        torch.cuda.synchronize()
    announce("prefill long_context as one %d-row call" % T)
    pool1 = torch.full((1, H, d, d), 7.0, dtype=torch.float32, device="cuda")
    o_one = lap.chunk_prefill(Q, K, V, G, B, torch.tensor([0, T], dtype=torch.int32, device="cuda"),
                              state_out=pool1)
    torch.cuda.synchronize()
    o_chain = o_chain.float().cpu().numpy()
    o_one = o_one[-L:].float().cpu().numpy()
    # Chunks fall on the same rows either way and the pool carries the fp32
    # state unchanged, so the two runs agree bit for bit.
    np.testing.assert_array_equal(o_chain, o_one)
    np.testing.assert_array_equal(pool.cpu().numpy(), pool1.cpu().numpy())
    s_g = pool.cpu().numpy()[0]
    es = max(rel_err(s_g[h], s_ref[0, h]) for h in range(H))
    eo = per_head_error(o_chain, o_ref_last)
    announce("  per head: final-state err %.3e  last-call o err %.3e (tolerance %.3g)"
             % (es, eo, TOL["bf16"]))
    assert es <= TOL["bf16"] and eo <= TOL["bf16"]


def _check_decode(c, tol):
    dt = torch_dtype(c.io_dtype)
    pool = dev(c.state_pool)
    o = torch.full((c.N, c.H, c.d_v), 5.0, dtype=dt, device="cuda")
    announce("decode %s" % c.name)
    lap.decode_step(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta), pool,
                    dev(c.slots), o=o, scale=c.scale)
    torch.cuda.synchronize()
    o_g, pool_g = o.float().cpu().numpy(), pool.cpu().numpy()
    o_init = np.full((c.N, c.H, c.d_v), 5.0)
    o_r, pool_r = oracle.decode_step(c.q, c.k, c.v, c.g, c.beta, c.state_pool, c.slots,
                                     scale=c.scale, o_init=o_init)
    ns = c.state_pool.shape[0]
    eo = es = 0.0
    for n in range(c.N):
        s = int(c.slots[n])
        if 0 <= s < ns:
            for h in range(c.H):
                eo = max(eo, rel_err(o_g[n, h], o_r[n, h]))
                es = max(es, rel_err(pool_g[s, h], pool_r[s, h]))
        else:
            assert np.all(o_g[n] == 5.0)
    announce("  max relative error per (sequence, head): o %.3g, state %.3g (tolerance %.3g)"
             % (eo, es, tol))
    assert eo <= tol and es <= tol
    used = set(int(s) for s in c.slots)
    for s in range(ns):
        if s not in used:
            np.testing.assert_array_equal(pool_g[s], c.state_pool[s])


def test_decode_full():
    """64 sequences x 1 token, H=32, d=128, bf16, 64-slot pool in place."""
    _check_decode(W.decode_case(), TOL["bf16"])


def test_decode_many_sequences():
    """1000 sequences x 1 token in a 1024-slot pool (2 GiB of state, slot
    offsets past 2^31 bytes), every 40th padded: 256,000 workgroups."""
    c = W.decode_case(seed=56, n=1000, num_slots=1024)
    c.slots[::40] = -1
    _check_decode(c, TOL["bf16"])


@pytest.mark.parametrize("dk,dv,io", [(64, 64, "f32"), (128, 64, "f32"), (64, 128, "bf16"),
                                      (128, 128, "f32")])
def test_decode_small_with_padding(dk, dv, io):
    c = W.random_case(30 + dk + dv, [1] * 9, H=3, d_k=dk, d_v=dv, io_dtype=io, num_slots=12,
                      slots=[4, -1, 0, 11, 7, 12, 2, 9, 5], scale=0.7)
    _check_decode(c, TOL[io])


@pytest.mark.parametrize("mu_g,io", [(5.0, "bf16"), (5.0, "f32"), (2.0, "bf16"), (-4.0, "f32")])
def test_decay_range_paths(mu_g, io):
    """Fast decay pushes diagonal 16-row blocks onto the exact path (mu_g = 5:
    about 100 log2 units of decay per block), mu_g = 2 mixes both paths
    across channels and blocks, slow decay (mu_g = -4) keeps the state large."""
    c = W.random_case(40 + int(mu_g), [150, 64, 37], H=3, d_k=128, d_v=128, io_dtype=io,
                      mu_g=mu_g)
    _check_case(c)


def _scan_slices_per_workgroup(n_slices, dv, cus=256):
    """The number of 16-column slices a bf16 scan workgroup takes: the largest
    of 4 and 2 that divides d_v / 16 and still leaves every CU ns
    workgroups' worth of slices, else 1."""
    for ns in (4, 2):
        if (dv // 16) % ns == 0 and n_slices >= ns * cus:
            return ns
    return 1


@pytest.mark.parametrize("dk,dv,H,ns", [(128, 128, 4, 4), (128, 128, 2, 2), (64, 64, 4, 2),
                                        (128, 64, 4, 2), (64, 128, 4, 4), (128, 128, 5, 4),
                                        (64, 128, 5, 4)])
def test_many_pairs_multi_slice_scan(dk, dv, H, ns):
    """Enough (sequence, head, 16-column slice) triples for bf16 calls to take
    the scan whose workgroups apply each chunk's operands to ns = 2 or 4
    slices (at least ns slices per CU on a 256-CU part); ragged and empty
    sequences, padded slots and in-place pools included."""
    rng = np.random.default_rng(17 + dk + dv + H)
    lengths = [int(x) for x in rng.choice([0, 1, 2, 63, 64, 65, 129, 200], size=48)]
    slots = [int(s) for s in rng.permutation(60)[:48]]
    slots[5] = -1
    c = W.random_case(400 + dk + dv + H, lengths, H=H, d_k=dk, d_v=dv, io_dtype="bf16",
                      num_slots=60, slots=slots)
    n_slices = c.N * c.H * (dv // 16)
    assert _scan_slices_per_workgroup(n_slices, dv) == ns
    announce("%d-slice scan %s" % (ns, c.name))
    o_g, _, _, _, _ = _check_case(c)
    cu = c.cu_seqlens
    assert np.all(o_g[cu[5]:cu[6]] == 3.0)           # the padded sequence keeps its rows


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_many_pairs_ragged(dk, dv):
    """280 (sequence, head) pairs of ragged, empty and one-row sequences of
    1..6 chunks, a padded slot and a pool updated in place, at every d_k, d_v:
    bf16 calls that take the scan with the most slices per workgroup their
    d_v allows."""
    rng = np.random.default_rng(23 + dk + dv)
    lengths = [int(x) for x in rng.choice([0, 1, 2, 63, 64, 65, 128, 129, 200, 321, 384], size=70)]
    slots = [int(s) for s in rng.permutation(80)[:70]]
    slots[9] = -1
    c = W.random_case(430 + dk + dv, lengths, H=4, d_k=dk, d_v=dv, io_dtype="bf16",
                      num_slots=80, slots=slots)
    assert _scan_slices_per_workgroup(c.N * c.H * (dv // 16), dv) == 4
    announce("many pairs %s" % c.name)
    o_g, _, _, _, _ = _check_case(c)
    cu = c.cu_seqlens
    assert np.all(o_g[cu[9]:cu[10]] == 3.0)           # the padded sequence keeps its rows


def test_many_pairs_windows_match_one_window():
    """A four-slice scan run as windows of 3 chunk ids (fp32 states carried
    between windows) gives the bits of one window, and the oracle's
    results."""
    rng = np.random.default_rng(29)
    lengths = [int(x) for x in rng.choice([0, 1, 64, 65, 200, 450], size=70)]
    c = W.random_case(439, lengths, H=4, d_k=128, d_v=128, io_dtype="bf16", num_slots=70)
    assert _scan_slices_per_workgroup(c.N * c.H * (c.d_v // 16), c.d_v) == 4
    dt = torch.bfloat16
    outs = []
    for wc in (0, 3):
        pool = dev(c.state_pool)
        o = torch.full((c.T, c.H, c.d_v), 3.0, dtype=dt, device="cuda")
        announce("prefill %s window_chunks=%d" % (c.name, wc))
        lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta),
                          dev(c.cu_seqlens), state_in=pool, state_out=pool, o=o,
                          slots=dev(c.slots), window_chunks=wc)
        torch.cuda.synchronize()
        outs.append((o, pool))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    o_r, pool_r, _ = oracle_prefill(c, o_init=np.full((c.T, c.H, c.d_v), 3.0))
    eo, es = per_sequence_errors(c, outs[1][0].float().cpu().numpy(), o_r,
                                 outs[1][1].cpu().numpy(), pool_r)
    announce("  max relative error: o %.3g, state %.3g (tolerance %.3g)" % (eo, es, TOL["bf16"]))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_malformed_device_data_stays_in_bounds():
    """Non-monotone cu_seqlens and duplicate slots give unspecified results
    (kda.h), but the kernels clamp them: nothing outside the buffers is
    touched.  o and the pool sit inside guard regions that must come back
    unchanged, and slots no sequence names keep their bytes."""
    T, H, d, S = 500, 2, 64, 5
    c = W.random_case(501, [T], H=H, d_k=d, d_v=d, io_dtype="bf16", num_slots=S)
    cu = np.array([0, 300, 100, 500, 480], dtype=np.int32)       # not monotone
    slots = np.array([1, 1, 7, 2], dtype=np.int32)                # duplicate and out of range
    dt = torch.bfloat16
    guard = 4096
    o_buf = torch.full((guard + T * H * d + guard,), 9.0, dtype=dt, device="cuda")
    p_buf = torch.full((guard + S * H * d * d + guard,), -3.0, dtype=torch.float32, device="cuda")
    o = o_buf[guard:guard + T * H * d].view(T, H, d)
    pool = p_buf[guard:guard + S * H * d * d].view(S, H, d, d)
    pool.copy_(dev(c.state_pool))
    weight, window = W.draw_conv(502, S, H, d, d, "bf16")
    w_buf = torch.full((guard + window.size + guard,), 5.0, dtype=dt, device="cuda")
    win = w_buf[guard:guard + window.size].view(window.shape)
    win.copy_(dev(window, dt))
    announce("malformed cu_seqlens and slots")
    for conv in (False, True):
        kw = dict(conv_weight=dev(weight), conv_window=win, conv_activation="silu") if conv else {}
        lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta),
                          dev(cu), state_in=pool, state_out=pool, o=o, slots=dev(slots),
                          num_slots=S, **kw)
        torch.cuda.synchronize()
    for buf, val in ((o_buf, 9.0), (p_buf, -3.0), (w_buf, 5.0)):
        assert torch.all(buf[:guard] == val) and torch.all(buf[-guard:] == val)
    p = pool.cpu().numpy()
    for s in (0, 3, 4):                                            # named by no sequence
        np.testing.assert_array_equal(p[s], c.state_pool[s])
    wn = win.float().cpu().numpy()
    for s in (0, 3, 4):
        np.testing.assert_array_equal(wn[s], window[s])


@pytest.mark.parametrize("n,io", [(100, "bf16"), (300, "f32"), (300, "bf16")])
def test_many_sequences(n, io):
    """Sequence bounds beyond the register path of the intra kernel: 100
    sequences (bounds in LDS) and 300 (scalar loads), short and ragged, with
    empty ones and padded slots."""
    rng = np.random.default_rng(600 + n)
    lengths = [int(x) for x in rng.integers(0, 41, size=n)]
    slots = [int(s) for s in rng.permutation(n + 10)[:n]]
    slots[3] = -1
    c = W.random_case(610 + n, lengths, H=2, d_k=64, d_v=64, io_dtype=io, num_slots=n + 10,
                      slots=slots)
    announce("many sequences %s" % c.name)
    o_g, _, _, _, _ = _check_case(c)
    cu = c.cu_seqlens
    assert np.all(o_g[cu[3]:cu[4]] == 3.0)


def test_fp32_scan_steady_state():
    """fp32 throughout at d = 128 over 4,100 + 30 rows: the long sequence is
    65 chunks, so the fp32 scan's three register stages and its L2 warm-up
    run for many rotations, not just their start-up."""
    c = W.random_case(701, [4100, 30], H=2, d_k=128, d_v=128, io_dtype="f32")
    _check_case(c)


def test_two_slice_scan_long_sequences():
    """Two sequences of 4,096 rows at H = 32, d = 128, bf16: 512 slices of 16
    columns, two per CU on a 256-CU part, so the scan takes two slices per
    workgroup with three register stages through 64 chunks per chain."""
    c = W.random_case(702, [4096, 4096], H=32, d_k=128, d_v=128, io_dtype="bf16", num_slots=4,
                      pool_std=0.02)
    n_slices = c.N * c.H * (c.d_v // 16)
    assert _scan_slices_per_workgroup(n_slices, c.d_v) == 2
    _check_case(c)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_mildly_positive_decay(io):
    """g > 0 breaks the documented precondition g <= 0 (kda.h): the split
    decay factors then exceed 1.  For a mild growth, g uniform in
    [0, 0.02] (at most e^1.28 a chunk per channel), the same path still meets
    the usual tolerance, which is what the header states."""
    c = W.random_case(703 if io == "bf16" else 704, [150, 64, 37], H=3, d_k=128, d_v=128,
                      io_dtype=io)
    rng = np.random.default_rng(705)
    c.g = rng.uniform(0.0, 0.02, c.g.shape).astype(np.float32)
    _check_case(c)


def test_check_inputs_flags_each_violation():
    """kda_prefill_check sets one bit per violated precondition and nothing on
    clean inputs; chunk_prefill(check_inputs=True) raises on a bad call."""
    c = W.random_case(706, [70, 3, 129], H=2, d_k=128, d_v=128, io_dtype="bf16", num_slots=6)
    g = dev(c.g)
    cu = dev(c.cu_seqlens)
    slots = dev(c.slots)
    announce("prefill input check")
    assert lap.check_prefill_inputs(g, cu, slots, num_slots=6) == 0
    bad_cu = c.cu_seqlens.copy()
    bad_cu[1], bad_cu[2] = bad_cu[2], bad_cu[1]
    assert lap.check_prefill_inputs(g, dev(bad_cu), slots, num_slots=6) == 1
    bad_end = c.cu_seqlens.copy()
    bad_end[-1] -= 1
    assert lap.check_prefill_inputs(g, dev(bad_end), slots, num_slots=6) == 1
    g_pos = c.g.copy()
    g_pos[77, 1, 5] = 0.5
    assert lap.check_prefill_inputs(dev(g_pos), cu, slots, num_slots=6) == 2
    g_nan = c.g.copy()
    g_nan[3, 0, 127] = np.nan
    assert lap.check_prefill_inputs(dev(g_nan), cu, slots, num_slots=6) == 2
    dup = c.slots.copy()
    dup[2] = dup[0]
    assert lap.check_prefill_inputs(g, cu, dev(dup), num_slots=6) == 4
    padded = c.slots.copy()
    padded[0] = padded[2] = -1                    # two padded rows may share -1
    assert lap.check_prefill_inputs(g, cu, dev(padded), num_slots=6) == 0
    assert lap.check_prefill_inputs(dev(g_pos), dev(bad_cu), dev(dup), num_slots=6) == 7
    dt = torch.bfloat16
    with pytest.raises(ValueError):
        lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(g_pos), dev(c.beta), cu,
                          state_in=dev(c.state_pool), state_out=None, slots=slots,
                          check_inputs=True)
    o = lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), g, dev(c.beta), cu,
                          state_in=dev(c.state_pool), slots=slots, check_inputs=True)
    torch.cuda.synchronize()
    o_r, _, _ = oracle_prefill(c)
    assert per_sequence_errors(c, o.float().cpu().numpy(), o_r)[0] <= TOL["bf16"]


WINDOW_LENGTHS = [1, 63, 64, 65, 2, 127, 128, 129, 0, 31, 33, 96, 250, 1, 17, 60]


@pytest.mark.parametrize("window_chunks,io", [(1, "bf16"), (2, "bf16"), (5, "bf16"), (3, "f32")])
def test_windows_match_one_window(window_chunks, io):
    """A call run as windows of chunk ids (intra kernel and scan per window,
    states carried between windows in fp32) gives the same bits as one
    window: the records, their use and the carried states are the same
    numbers.  Window edges fall inside sequences, between them and on empty
    ones; checked against the oracle too."""
    c = W.random_case(711 + window_chunks, WINDOW_LENGTHS, H=2, d_k=128, d_v=128, io_dtype=io)
    dt = torch_dtype(io)
    nw = lap.prefill_windows(c.T, c.N, c.H, c.d_k, c.d_v, dt, window_chunks=window_chunks)
    assert nw == -(-((c.T - 1) // 64 + c.N) // window_chunks)
    outs = []
    for wc in (0, window_chunks):
        pool = dev(c.state_pool)
        o = torch.full((c.T, c.H, c.d_v), 3.0, dtype=dt, device="cuda")
        announce("prefill %s window_chunks=%d" % (c.name, wc))
        lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta),
                          dev(c.cu_seqlens), state_in=pool, state_out=pool, o=o,
                          slots=dev(c.slots), window_chunks=wc)
        torch.cuda.synchronize()
        outs.append((o, pool))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    o_r, pool_r, _ = oracle_prefill(c, o_init=np.full((c.T, c.H, c.d_v), 3.0))
    eo, es = per_sequence_errors(c, outs[1][0].float().cpu().numpy(), o_r,
                                 outs[1][1].cpu().numpy(), pool_r)
    announce("  max relative error: o %.3g, state %.3g (tolerance %.3g)" % (eo, es, TOL[io]))
    assert eo <= TOL[io] and es <= TOL[io]


@pytest.mark.parametrize("workload,window_chunks", [("packed", 37), ("single", 33)])
def test_windows_full_size(workload, window_chunks):
    """The full packed chunk and the full single sequence run as 4 windows,
    bit for bit against one window, with the state carried in place (packed)
    and out of a null state_in (single)."""
    c = W.packed_varlen_prefill() if workload == "packed" else W.single_seq_prefill()
    dt = torch.bfloat16
    q, k, v, g, beta = dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta)
    cu = dev(c.cu_seqlens)
    outs = []
    for wc in (0, window_chunks):
        if c.state_pool is not None:
            pool, pin, slots = dev(c.state_pool), None, dev(c.slots)
            pin = pool
        else:
            pool = torch.zeros((1, c.H, c.d_v, c.d_k), dtype=torch.float32, device="cuda")
            pin, slots = None, None
        announce("prefill %s window_chunks=%d" % (c.name, wc))
        o = lap.chunk_prefill(q, k, v, g, beta, cu, state_in=pin, state_out=pool, slots=slots,
                              window_chunks=wc)
        torch.cuda.synchronize()
        outs.append((o, pool))
    assert lap.prefill_windows(c.T, c.N, c.H, c.d_k, c.d_v, dt, window_chunks=window_chunks) == 4
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------------------
# The fused prefill: whole (sequence, head) chains in one workgroup
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,dk,dv", [(20, 128, 128), (70, 128, 128), (20, 64, 64), (70, 64, 128),
                                     (20, 128, 64)])
def test_fused_and_windowed_chains_in_one_call(n, dk, dv):
    """fuse_chunks = 3: sequences of at most three chunks run in the fused
    prefill, longer ones in the intra-chunk kernel and scan, in the same
    call.  Fewer than 64 sequences take the ranked chain order, more the
    natural one; empty and one-row sequences, a padded slot and a pool
    updated in place included."""
    rng = np.random.default_rng(800 + n + dk + dv)
    lengths = [int(x) for x in rng.choice([0, 1, 5, 64, 65, 130, 192, 193, 300, 700], size=n)]
    slots = [int(s) for s in rng.permutation(n + 10)[:n]]
    slots[3] = -1
    c = W.random_case(810 + n + dk + dv, lengths, H=3, d_k=dk, d_v=dv, io_dtype="bf16",
                      num_slots=n + 10, slots=slots)
    assert lap.prefill_fuse_chunks(c.T, c.N, c.H, dk, dv, torch.bfloat16, fuse_chunks=3) == 3
    o_g, _, _, _, _ = _check_case(c, fuse_chunks=3)
    cu = c.cu_seqlens
    assert np.all(o_g[cu[3]:cu[4]] == 3.0)             # the padded sequence keeps its rows


@pytest.mark.parametrize("state", ["in_place", "null_in", "null_out"])
def test_fused_state_handling(state):
    """Every chain fused: states read from and written to the pool (in
    place), started from zero (state_in NULL, empty sequences then write
    zeros), or not written (state_out NULL)."""
    c = W.random_case(830, [0, 1, 64, 65, 100, 0, 129, 17], H=4, d_k=128, d_v=128,
                      io_dtype="bf16", num_slots=12)
    kw = {"state_in_null": state == "null_in", "state_out_null": state == "null_out"}
    o_init = np.full((c.T, c.H, c.d_v), 3.0, dtype=np.float32)
    announce("fused prefill %s (%s)" % (c.name, state))
    o_g, pool_g = gpu_prefill(c, o_init=o_init, fuse_chunks=64, **kw)
    pool = c.state_pool if state != "null_in" else np.zeros_like(c.state_pool)
    o_r, pool_r, _ = oracle_prefill(c, pool=pool, o_init=o_init)
    if state == "null_out":
        pool_g = pool_r = None
    eo, es = per_sequence_errors(c, o_g, o_r, pool_g, pool_r)
    announce("  max relative error: o %.3g, state %.3g" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_fused_full_packed_chunk():
    """The full packed chunk (16 sequences in 8192 rows, H = 32, d = 128)
    with every chain fused, against the oracle, and the same call with none
    fused."""
    c = W.packed_varlen_prefill()
    assert lap.prefill_fuse_chunks(c.T, c.N, c.H, 128, 128, torch.bfloat16, fuse_chunks=64) == 64
    _check_case(c, fuse_chunks=64)
    _check_case(c, fuse_chunks=-1)


def test_fused_with_windows_matches_one_window():
    """Windows apply to the chains that are not fused: a call with fused short
    chains and windows of two chunk ids gives the bits of the same call in
    one window."""
    lengths = [3, 700, 64, 0, 500, 129, 1, 900]
    c = W.random_case(840, lengths, H=2, d_k=128, d_v=128, io_dtype="bf16", num_slots=8)
    dt = torch.bfloat16
    outs = []
    for wc in (0, 2):
        pool = dev(c.state_pool)
        o = torch.full((c.T, c.H, c.d_v), 3.0, dtype=dt, device="cuda")
        announce("prefill %s window_chunks=%d fuse_chunks=3" % (c.name, wc))
        lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta),
                          dev(c.cu_seqlens), state_in=pool, state_out=pool, o=o,
                          slots=dev(c.slots), window_chunks=wc, fuse_chunks=3)
        torch.cuda.synchronize()
        outs.append((o, pool))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    o_r, pool_r, _ = oracle_prefill(c, o_init=np.full((c.T, c.H, c.d_v), 3.0))
    eo, es = per_sequence_errors(c, outs[1][0].float().cpu().numpy(), o_r,
                                 outs[1][1].cpu().numpy(), pool_r)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_fused_is_bf16_only():
    """fp32 calls never fuse: the fused kernel keeps bf16 operands."""
    assert lap.prefill_fuse_chunks(1000, 10, 2, 64, 64, torch.float32, fuse_chunks=5) == -1
    c = W.random_case(850, [10, 70, 0, 130], H=2, d_k=64, d_v=64, io_dtype="f32")
    _check_case(c, fuse_chunks=5)


def test_fused_by_default_for_short_sequences():
    """The library's choice: 96 sequences of at most one chunk average one
    chunk, so every sequence runs in the fused prefill (the window of
    intra-chunk kernel and scan finds nothing to do).  With fuse_chunks
    covering all T rows that window is not launched at all."""
    rng = np.random.default_rng(860)
    lengths = [int(x) for x in rng.integers(1, 65, size=96)]
    lengths[7] = 0
    c = W.random_case(861, lengths, H=4, d_k=128, d_v=128, io_dtype="bf16", num_slots=100)
    assert lap.prefill_fuse_chunks(c.T, c.N, c.H, 128, 128, torch.bfloat16) == 8
    assert lap.prefill_windows(c.T, c.N, c.H, 128, 128, torch.bfloat16) == 1
    _check_case(c)
    every = -(-c.T // 64)
    assert lap.prefill_windows(c.T, c.N, c.H, 128, 128, torch.bfloat16, fuse_chunks=every) == 0
    _check_case(c, fuse_chunks=every)


@pytest.mark.parametrize("n_long", [40, 290])
def test_fused_with_many_unfused_sequences(n_long):
    """fuse_chunks = 1 with 300 sequences: the intra-chunk kernel lists the
    unfused ones (n_long of them, two or three chunks each) and walks their
    chunks only, or, past 256 of them, walks the chunk ids and passes over the
    fused ones."""
    rng = np.random.default_rng(870 + n_long)
    lengths = [int(x) for x in rng.integers(65, 190, size=n_long)] + \
              [int(x) for x in rng.integers(0, 65, size=300 - n_long)]
    lengths = [lengths[i] for i in rng.permutation(300)]
    c = W.random_case(871 + n_long, lengths, H=2, d_k=64, d_v=64, io_dtype="bf16",
                      num_slots=310)
    _check_case(c, fuse_chunks=1)
