"""The short conv front end on the GPU (``kda_chunk_prefill_conv``,
``kda_decode_step_conv``) against the oracle's conv_front + recurrence.

Windows hold raw inputs, so the windows a call leaves behind must equal the
oracle's bit for bit; o and the states meet the usual tolerance.  The window
layouts are the dense head-major one, SGLang's tap-major [slot][tap][q|k|v]
(the kern-k3-pp-prefill page, section "D inside SGLang"), and the window
placed inside each head's block of a hybrid page right after the state (the
same page, section "D inside vLLM"); every layout must give the same results.
"""
import numpy as np
import pytest
import torch

from linear_attention_prefill_amd import workloads as W
from oracle import oracle
from kda_testlib import (TOL, announce, block_error, dev, per_head_error, per_sequence_errors,
                         rel_err, torch_dtype)
import linear_attention_prefill_amd as lap

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_prefill_conv(c, weight, window_dev, dt, act, strides=(0, 0, 0, 0), o_init=None,
                     pool=None, fuse_chunks=0, window_chunks=0):
    q, k, v = dev(c.q, dt), dev(c.k, dt), dev(c.v, dt)
    o = dev(o_init, dt) if o_init is not None else torch.zeros((c.T, c.H, c.d_v), dtype=dt,
                                                                device="cuda")
    p = dev(c.state_pool if pool is None else pool)
    lap.chunk_prefill(q, k, v, dev(c.g), dev(c.beta), dev(c.cu_seqlens), state_in=p, state_out=p,
                      o=o, slots=dev(c.slots), num_slots=c.state_pool.shape[0], scale=c.scale,
                      conv_weight=dev(weight), conv_window=window_dev, conv_activation=act,
                      conv_strides=strides, fuse_chunks=fuse_chunks, window_chunks=window_chunks)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), p.cpu().numpy()


@pytest.mark.parametrize("dk,dv,io,act,fuse", [(128, 128, "bf16", "silu", -1),
                                               (64, 64, "f32", "none", -1),
                                               (64, 128, "bf16", "none", -1),
                                               (128, 64, "f32", "silu", -1),
                                               (128, 128, "bf16", "silu", 1),
                                               (64, 64, "bf16", "none", 64),
                                               (64, 64, "bf16", "silu", -1)])
def test_prefill_conv_parity(dk, dv, io, act, fuse):
    """fuse: bf16 sequences of at most this many chunks run in the fused
    prefill on the convolved inputs (1: the short ones; 64: all).  bf16 with
    d_k = d_v and fuse = -1 folds the conv into the intra-chunk kernel."""
    lengths = [0, 1, 2, 3, 63, 64, 65, 130, 5]
    S = 12
    slots = [3, 0, 7, 11, -1, 5, 9, 2, 13]
    c = W.random_case(201 + dk + dv, lengths, H=3, d_k=dk, d_v=dv, io_dtype=io, num_slots=S,
                      slots=slots, scale=0.8)
    weight, window = W.draw_conv(202, S, 3, dk, dv, io)
    dt = torch_dtype(io)
    o_init = np.full((c.T, c.H, c.d_v), 2.0, dtype=np.float32)
    announce("prefill conv %s act=%s fuse=%d" % (c.name, act, fuse))
    win_d = dev(window, dt)
    o_g, pool_g = run_prefill_conv(c, weight, win_d, dt, act, o_init=o_init, fuse_chunks=fuse)
    win_g = win_d.float().cpu().numpy()
    o_r, pool_r, _, win_r = oracle.chunk_prefill_conv(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens,
                                                      weight, window, c.state_pool, c.slots,
                                                      scale=c.scale, o_init=o_init,
                                                      activation=act)
    live = (c.slots >= 0) & (c.slots < S)
    eo, es = per_sequence_errors(c, o_g, o_r, pool_g, pool_r, live=live)
    announce("  o err %.3e  state err %.3e" % (eo, es))
    assert eo <= TOL[io] and es <= TOL[io], (eo, es)
    np.testing.assert_array_equal(win_g, win_r.astype(np.float32))
    cu = c.cu_seqlens
    assert np.all(o_g[cu[4]:cu[5]] == 2.0)          # padded sequence untouched


@pytest.mark.parametrize("d,act,window_chunks", [(128, "silu", 0), (128, "none", 3), (64, "silu", 0)])
def test_folded_conv_matches_conv_pass_bit_for_bit(d, act, window_chunks):
    """bf16 with d_k = d_v: with nothing fused the conv is folded into the
    intra-chunk kernel's loads; fuse_chunks = 1 on sequences that all exceed
    one chunk fuses none of them but runs the conv as a pass of its own.  The
    fold rounds each convolved row to bf16 as the pass writes it, so o, the
    states and the windows agree bit for bit (window_chunks = 3: the records
    of several windows, the conv windows read by every one of them)."""
    lengths = [65, 130, 64 * 5 + 7, 200, 66, 129]
    S = 9
    slots = [3, 0, -1, 8, 5, 20]                    # a padded and an out-of-range slot
    c = W.random_case(231 + d, lengths, H=4, d_k=d, d_v=d, io_dtype="bf16", num_slots=S,
                      slots=slots, scale=0.7)
    weight, window = W.draw_conv(232 + d, S, 4, d, d, "bf16")
    dt = torch.bfloat16
    announce("prefill conv fold vs pass %s act=%s window_chunks=%d" % (c.name, act, window_chunks))
    assert lap.prefill_fuse_chunks(c.T, c.N, c.H, d, d, fuse_chunks=-1) == -1
    w1, w2 = dev(window, dt), dev(window, dt)
    o1, p1 = run_prefill_conv(c, weight, w1, dt, act, fuse_chunks=-1, window_chunks=window_chunks)
    o2, p2 = run_prefill_conv(c, weight, w2, dt, act, fuse_chunks=1, window_chunks=window_chunks)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(w1.float().cpu().numpy(), w2.float().cpu().numpy())


def _tap_major(window, H, dk, dv):
    """Dense [S][H][3][C] -> SGLang's [S][3][q(H dk) | k(H dk) | v(H dv)]."""
    S = window.shape[0]
    q = window[:, :, :, :dk].transpose(0, 2, 1, 3).reshape(S, 3, H * dk)
    k = window[:, :, :, dk:2 * dk].transpose(0, 2, 1, 3).reshape(S, 3, H * dk)
    v = window[:, :, :, 2 * dk:].transpose(0, 2, 1, 3).reshape(S, 3, H * dv)
    return np.concatenate([q, k, v], axis=2).copy()


@pytest.mark.parametrize("fuse", [0, -1])
def test_prefill_conv_tap_major_window_matches_dense(fuse):
    """fuse = 0 fuses the short sequences here and runs the conv as a pass;
    -1 folds it into the intra-chunk kernel, which then reads the windows
    through the same strides."""
    H, d, S = 4, 128, 6
    c = W.random_case(211, [70, 3, 200], H=H, d_k=d, d_v=d, io_dtype="bf16", num_slots=S,
                      slots=[4, 1, 0])
    weight, window = W.draw_conv(212, S, H, d, d, "bf16")
    dt = torch.bfloat16
    announce("prefill conv tap-major %s fuse=%d" % (c.name, fuse))
    win_dense = dev(window, dt)
    o1, p1 = run_prefill_conv(c, weight, win_dense, dt, "silu", fuse_chunks=fuse)
    C = 3 * d
    tm = dev(_tap_major(window, H, d, d), dt)
    strides = (3 * H * C, d, H * C, H * d)
    o2, p2 = run_prefill_conv(c, weight, tm, dt, "silu", strides=strides, fuse_chunks=fuse)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(tm.float().cpu().numpy(),
                                  _tap_major(win_dense.float().cpu().numpy(), H, d, d))


@pytest.mark.parametrize("dk,dv,io,act", [(128, 128, "bf16", "silu"), (64, 128, "f32", "none")])
def test_decode_conv_parity_and_prefill_continuity(dk, dv, io, act):
    """Prefill 37 rows with the conv, then 4 decode steps with the conv fused:
    every output and the final state and window against the oracle run over
    all 41 rows at once."""
    H, S = 3, 5
    lengths = [41, 41, 41]
    slots = np.array([2, 4, 0], dtype=np.int32)
    c = W.random_case(221 + dk, lengths, H=H, d_k=dk, d_v=dv, io_dtype=io, num_slots=S,
                      slots=slots)
    weight, window = W.draw_conv(222, S, H, dk, dv, io)
    dt = torch_dtype(io)
    o_r, pool_r, _, win_r = oracle.chunk_prefill_conv(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens,
                                                      weight, window, c.state_pool, c.slots,
                                                      activation=act)
    P = 37
    rows = np.concatenate([np.arange(41 * n, 41 * n + P) for n in range(3)])
    sub = W.Case("prefix", c.q[rows], c.k[rows], c.v[rows], c.g[rows], c.beta[rows],
                 np.array([0, P, 2 * P, 3 * P], dtype=np.int32), io, state_pool=c.state_pool,
                 slots=slots)
    win_d = dev(window, dt)
    announce("decode conv continuity %s act=%s" % (c.name, act))
    o_p, pool_g = run_prefill_conv(sub, weight, win_d, dt, act)
    pool_d = dev(pool_g)
    outs = []
    for t in range(P, 41):
        r = np.array([41 * n + t for n in range(3)])
        o = torch.zeros((3, H, dv), dtype=dt, device="cuda")
        lap.decode_step(dev(c.q[r], dt), dev(c.k[r], dt), dev(c.v[r], dt), dev(c.g[r]),
                        dev(c.beta[r]), pool_d, dev(slots), o=o, conv_weight=dev(weight),
                        conv_window=win_d, conv_activation=act)
        torch.cuda.synchronize()
        outs.append(o.float().cpu().numpy())
    for n in range(3):
        a = 41 * n
        assert per_head_error(o_p[P * n:P * n + P], o_r[a:a + P]) <= TOL[io]
        for j, t in enumerate(range(P, 41)):
            assert block_error(outs[j][n], o_r[a + t], 1) <= TOL[io]
        s = slots[n]
        assert block_error(pool_d.cpu().numpy()[s], pool_r[s], 2) <= TOL[io]
    np.testing.assert_array_equal(win_d.float().cpu().numpy(), win_r.astype(np.float32))


def test_decode_conv_full_size_with_padding():
    """64 sequences x 1 token, H=32, d=128, bf16, SiLU; one padded row."""
    N, H, d, S = 64, 32, 128, 64
    c = W.decode_case()
    slots = c.slots.copy()
    slots[9] = -1
    weight, window = W.draw_conv(231, S, H, d, d, "bf16")
    dt = torch.bfloat16
    win_d = dev(window, dt)
    pool = dev(c.state_pool)
    o = torch.full((N, H, d), 3.0, dtype=dt, device="cuda")
    announce("decode conv full N=64 H=32 d=128 bf16")
    lap.decode_step(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta), pool,
                    dev(slots), o=o, conv_weight=dev(weight), conv_window=win_d,
                    conv_activation="silu")
    torch.cuda.synchronize()
    o_r, pool_r, win_r = oracle.decode_step_conv(c.q, c.k, c.v, c.g, c.beta, c.state_pool, slots,
                                                 weight, window, activation="silu",
                                                 o_init=np.full((N, H, d), 3.0))
    o_g, pool_g = o.float().cpu().numpy(), pool.cpu().numpy()
    live = slots >= 0
    assert block_error(o_g[live], o_r[live], 1) <= TOL["bf16"]
    assert np.all(o_g[~live] == 3.0)
    assert block_error(pool_g, pool_r, 2) <= TOL["bf16"]
    np.testing.assert_array_equal(win_d.float().cpu().numpy(), win_r.astype(np.float32))


@pytest.mark.parametrize("fuse", [0, -1])
def test_conv_window_inside_hybrid_page_lines(fuse):
    """kern's hybrid-page line: per head a 64 KiB fp32 state followed by its
    3-row bf16 window (2,304 bytes), 12 heads on 884,736-byte pages.  Prefill
    and a decode step read and write both through one buffer (fuse = -1: the
    prefill's conv folded into the intra-chunk kernel)."""
    H, d, S = 12, 128, 4
    C = 3 * d
    hs = (d * d * 4 + 3 * C * 2) // 4          # 16,960 fp32 words per head
    ss = 884736 // 4
    c = W.random_case(241, [150, 2], H=H, d_k=d, d_v=d, io_dtype="bf16", num_slots=S,
                      slots=[3, 1])
    weight, window = W.draw_conv(242, S, H, d, d, "bf16")
    flat = np.zeros(S * ss, dtype=np.float32)     # whole pages: the last window lies past the
                                                  # last state block
    fb = flat.view(np.uint16)
    wb = (torch.from_numpy(window).to(torch.bfloat16).view(torch.int16).numpy()
          .view(np.uint16))
    for s in range(S):
        for h in range(H):
            a = s * ss + h * hs
            flat[a:a + d * d] = c.state_pool[s, h].reshape(-1)
            b = 2 * (a + d * d)
            fb[b:b + 3 * C] = wb[s, h].reshape(-1)
    buf = dev(flat)
    win_view = buf.view(torch.bfloat16)[2 * d * d:]
    strides = (2 * ss, 2 * hs, C, d)
    dt = torch.bfloat16
    o = torch.zeros((c.T, H, d), dtype=dt, device="cuda")
    announce("prefill+decode conv in hybrid page lines fuse=%d" % fuse)
    lap.chunk_prefill(dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta),
                      dev(c.cu_seqlens), state_in=buf, state_out=buf, o=o, slots=dev(c.slots),
                      num_slots=S, state_slot_stride=ss, state_head_stride=hs,
                      conv_weight=dev(weight), conv_window=win_view, conv_activation="silu",
                      conv_strides=strides, fuse_chunks=fuse)
    dc = W.random_case(243, [1, 1], H=H, d_k=d, d_v=d, io_dtype="bf16", num_slots=S,
                       slots=[3, 1])
    od = torch.zeros((2, H, d), dtype=dt, device="cuda")
    lap.decode_step(dev(dc.q, dt), dev(dc.k, dt), dev(dc.v, dt), dev(dc.g), dev(dc.beta), buf,
                    dev(dc.slots), o=od, num_slots=S, state_slot_stride=ss, state_head_stride=hs,
                    conv_weight=dev(weight), conv_window=win_view, conv_activation="silu",
                    conv_strides=strides)
    torch.cuda.synchronize()
    o_r, pool_r, _, win_r = oracle.chunk_prefill_conv(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens,
                                                      weight, window, c.state_pool, c.slots,
                                                      activation="silu")
    od_r, pool_r2, win_r2 = oracle.decode_step_conv(dc.q, dc.k, dc.v, dc.g, dc.beta, pool_r,
                                                    dc.slots, weight, win_r, activation="silu")
    out = buf.cpu().numpy()
    ob = out.view(np.uint16)
    assert per_head_error(o.float().cpu().numpy(), o_r) <= TOL["bf16"]
    assert block_error(od.float().cpu().numpy(), od_r, 1) <= TOL["bf16"]
    wr = (torch.from_numpy(win_r2.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
          .numpy().view(np.uint16))
    for s in range(S):
        for h in range(H):
            a = s * ss + h * hs
            assert rel_err(out[a:a + d * d].reshape(d, d), pool_r2[s, h]) <= TOL["bf16"]
            b = 2 * (a + d * d)
            np.testing.assert_array_equal(ob[b:b + 3 * C], wr[s, h].reshape(-1))


@pytest.mark.parametrize("workload", ["single", "packed"])
def test_prefill_conv_full_size(workload):
    """The conv front end at the full prefill shapes that bench.py times with
    the conv (8192 rows, H = 32, d = 128, bf16, SiLU): one sequence from a
    one-slot window pool, and the 16 packed sequences with their 64-slot state
    and window pools.  Windows bit for bit, o and states per (sequence, head)
    against the oracle."""
    c = W.single_seq_prefill() if workload == "single" else W.packed_varlen_prefill()
    S = 1 if c.state_pool is None else c.state_pool.shape[0]
    weight, window = W.draw_conv(11, S, c.H, c.d_k, c.d_v, c.io_dtype)
    dt = torch.bfloat16
    pool = (np.zeros((1, c.H, c.d_v, c.d_k), dtype=np.float32) if c.state_pool is None
            else c.state_pool)
    slots = np.zeros(1, dtype=np.int32) if c.slots is None else c.slots
    q, k, v = dev(c.q, dt), dev(c.k, dt), dev(c.v, dt)
    o = torch.zeros((c.T, c.H, c.d_v), dtype=dt, device="cuda")
    p = dev(pool)
    win_d = dev(window, dt)
    announce("prefill conv full size %s" % c.name)
    lap.chunk_prefill(q, k, v, dev(c.g), dev(c.beta), dev(c.cu_seqlens), state_in=p,
                      state_out=p, o=o, slots=dev(slots), num_slots=S, conv_weight=dev(weight),
                      conv_window=win_d, conv_activation="silu")
    torch.cuda.synchronize()
    o_g, pool_g, win_g = o.float().cpu().numpy(), p.cpu().numpy(), win_d.float().cpu().numpy()
    o_r, pool_r, _, win_r = oracle.chunk_prefill_conv(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens,
                                                      weight, window, pool, slots,
                                                      activation="silu")
    ref_case = W.Case(c.name, c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens, c.io_dtype,
                      state_pool=pool, slots=slots)
    eo, es = per_sequence_errors(ref_case, o_g, o_r, pool_g, pool_r)
    announce("  max relative error per (sequence, head): o %.3e  state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)
    np.testing.assert_array_equal(win_g, win_r.astype(np.float32))
