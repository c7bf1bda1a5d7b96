"""Calls enqueue on the caller's stream and can be captured into a HIP graph
(kda.h, "Ownership and execution"; the "kern" page, section "Hosts": launches
go on the host's stream, inside its graphs).

Graph replays are checked one by one against eager calls on copies of the
same buffers, with eager work and synchronisations between the replays; the
kernels are deterministic, so the comparison is bit for bit.
"""
import numpy as np
import pytest
import torch

from linear_attention_prefill_amd import workloads as W
from oracle import oracle
from kda_testlib import TOL, announce, dev, per_sequence_errors
import linear_attention_prefill_amd as lap

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _prefill_args(c, dt):
    return dict(q=dev(c.q, dt), k=dev(c.k, dt), v=dev(c.v, dt), g=dev(c.g), beta=dev(c.beta),
                cu_seqlens=dev(c.cu_seqlens), slots=dev(c.slots))


def test_conv_prefill_on_a_side_stream():
    c = W.random_case(301, [100, 3, 64], H=2, d_k=128, d_v=128, io_dtype="bf16", num_slots=5)
    weight, window = W.draw_conv(302, 5, 2, 128, 128, "bf16")
    dt = torch.bfloat16
    side = torch.cuda.Stream()
    announce("prefill with conv on a side stream")
    with torch.cuda.stream(side):
        a = _prefill_args(c, dt)
        pool = dev(c.state_pool)
        win = dev(window, dt)
        o = torch.zeros((c.T, c.H, c.d_v), dtype=dt, device="cuda")
        lap.chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                          state_in=pool, state_out=pool, o=o, slots=a["slots"],
                          conv_weight=dev(weight), conv_window=win, conv_activation="silu")
    side.synchronize()
    o_r, pool_r, _, win_r = oracle.chunk_prefill_conv(c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens,
                                                      weight, window, c.state_pool, c.slots,
                                                      activation="silu")
    eo, es = per_sequence_errors(c, o.float().cpu().numpy(), o_r, pool.cpu().numpy(), pool_r)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)
    np.testing.assert_array_equal(win.float().cpu().numpy(), win_r.astype(np.float32))


@pytest.mark.parametrize("fuse", [-1, 64])
def test_prefill_graph_replays_match_eager(fuse):
    """fuse = 64: every sequence in the fused prefill (no intra-chunk kernel
    or scan launched); -1: none."""
    c = W.random_case(311, [200, 1, 77], H=3, d_k=128, d_v=64, io_dtype="bf16", num_slots=4)
    dt = torch.bfloat16
    a = _prefill_args(c, dt)
    pin = dev(c.state_pool)
    pout = torch.zeros_like(pin)
    o = torch.zeros((c.T, c.H, c.d_v), dtype=dt, device="cuda")
    ws = torch.empty(lap.prefill_workspace_size(c.T, c.N, c.H, c.d_k, c.d_v, dt),
                     dtype=torch.uint8, device="cuda")

    def call():
        lap.chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                          state_in=pin, state_out=pout, o=o, slots=a["slots"], workspace=ws,
                          fuse_chunks=fuse)

    announce("prefill eager reference")
    call()
    torch.cuda.synchronize()
    o_ref, p_ref = o.clone(), pout.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    announce("prefill graph capture")
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        o.zero_()
        pout.zero_()
        torch.cuda.synchronize()
        announce("prefill graph replay %d" % rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), rep
        assert torch.equal(pout, p_ref), rep
        _ = (a["q"].float() * 2).sum().item()      # eager work between replays


def test_decode_and_conv_decode_graph_replays_match_eager():
    """In-place pools and windows: each replay advances them one token, as
    the eager calls on copies do."""
    c = W.random_case(321, [1] * 6, H=4, d_k=128, d_v=128, io_dtype="bf16", num_slots=8)
    weight, window = W.draw_conv(322, 8, 4, 128, 128, "bf16")
    dt = torch.bfloat16
    q, k, v, g, beta = dev(c.q, dt), dev(c.k, dt), dev(c.v, dt), dev(c.g), dev(c.beta)
    slots = dev(c.slots)
    w = dev(weight)

    def make():
        return dev(c.state_pool), dev(window, dt), torch.zeros((6, 4, 128), dtype=dt, device="cuda")

    def call(pool, win, o):
        lap.decode_step(q, k, v, g, beta, pool, slots, o=o)
        lap.decode_step(q, k, v, g, beta, pool, slots, o=o, conv_weight=w, conv_window=win,
                        conv_activation="silu")

    pool_e, win_e, o_e = make()
    pool_g, win_g, o_g = make()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    announce("decode graph capture")
    with torch.cuda.graph(graph, stream=side):
        call(pool_g, win_g, o_g)
    torch.cuda.synchronize()
    # capture does not run the kernels: both copies still hold the initial pools
    assert torch.equal(pool_g, pool_e)
    for rep in range(4):
        announce("decode graph replay %d" % rep)
        call(pool_e, win_e, o_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(pool_g, pool_e), rep
        assert torch.equal(win_g, win_e), rep
        _ = (pool_e * 0.5).sum().item()


def test_explicit_stream_argument_owns_its_allocations():
    """stream= names a stream other than the current one, with the default
    stream current throughout.  The workspace and o that the binding
    allocates belong to that stream's memory pool, so memory the default
    stream allocates and fills at once, while the call's kernels still run,
    cannot be the call's workspace: results match an eager call bit for
    bit."""
    c = W.random_case(321, [8192], H=8, d_k=128, d_v=128, io_dtype="bf16", num_slots=2)
    dt = torch.bfloat16
    a = _prefill_args(c, dt)
    announce("prefill reference on the current stream")
    p_ref = dev(c.state_pool)
    o_ref = lap.chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                              state_in=p_ref, state_out=p_ref, slots=a["slots"])
    torch.cuda.synchronize()
    ws_bytes = lap.prefill_workspace_size(c.T, c.N, c.H, c.d_k, c.d_v, dt)
    side = torch.cuda.Stream()
    pool = dev(c.state_pool)
    torch.cuda.synchronize()
    announce("prefill with stream=side, default stream allocating meanwhile")
    o = lap.chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                          state_in=pool, state_out=pool, slots=a["slots"], stream=side)
    junk = [torch.full((ws_bytes // 4 + 1024,), 1e30, dtype=torch.float32, device="cuda")
            for _ in range(2)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, o_ref)
    assert torch.equal(pool, p_ref)
