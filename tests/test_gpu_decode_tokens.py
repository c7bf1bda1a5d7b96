"""Multi-token decode and speculative verify / commit on the GPU
(``kda_decode_tokens``; the prhub report on SGLang PR #32890, section
"关键文件": multi-token verify beside the single-token step, and ReplaySSM's
exact fold of the accepted tokens at commit).

Two bars: against repeated single steps of the HIP path the outputs and the
committed states must be identical bit for bit (the exact-fold contract);
against the oracle they must meet the usual tolerance.
"""
import numpy as np
import pytest
import torch

from linear_attention_prefill_amd import workloads as W
from oracle import oracle
from kda_testlib import TOL, announce, block_error, dev, rel_err, torch_dtype
import linear_attention_prefill_amd as lap

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def tokens_case(seed, N, T, H, dk, dv, io, num_slots, slots, scale=1.0):
    """N sequences of T tokens each; arrays reshaped to [N, T, ...]."""
    c = W.random_case(seed, [T] * N, H=H, d_k=dk, d_v=dv, io_dtype=io, num_slots=num_slots,
                      slots=slots, scale=scale)
    r = lambda x: x.reshape((N, T) + x.shape[1:])
    return c, [r(x) for x in (c.q, c.k, c.v, c.g, c.beta)]


def steps_reference(args, pool, slots, scale, dt):
    """T single decode steps on the GPU; returns (o [N,T,H,dv] as io values,
    pools after each step: list of T+1 numpy pools)."""
    q, k, v, g, beta = args
    N, T = k.shape[:2]
    p = dev(pool)
    sl = dev(slots)
    pools = [pool.copy()]
    outs = []
    for t in range(T):
        o = torch.full((N,) + v.shape[2:], 5.0, dtype=dt, device="cuda")
        lap.decode_step(dev(q[:, t], dt), dev(k[:, t], dt), dev(v[:, t], dt), dev(g[:, t]),
                        dev(beta[:, t]), p, sl, o=o, scale=scale)
        torch.cuda.synchronize()
        outs.append(o.float().cpu().numpy())
        pools.append(p.cpu().numpy())
    return np.stack(outs, axis=1), pools


@pytest.mark.parametrize("dk,dv,io,T", [(128, 128, "bf16", 5), (64, 128, "f32", 3),
                                        (128, 64, "bf16", 16), (64, 64, "f32", 1)])
def test_tokens_bitwise_against_single_steps(dk, dv, io, T):
    N, S = 7, 10
    slots = [3, -1, 0, 9, 12, 5, 7]
    c, args = tokens_case(101 + T + dk, N, T, 3, dk, dv, io, S, slots, scale=0.9)
    dt = torch_dtype(io)
    rng = np.random.default_rng(T)
    acc = rng.integers(0, T + 1, size=N).astype(np.int32)
    acc[0], acc[2] = T, 0
    announce("decode_tokens bitwise %s T=%d acc=%s" % (c.name, T, acc.tolist()))
    o_ref, pools = steps_reference(args, c.state_pool, c.slots, c.scale, dt)
    q, k, v, g, beta = [dev(x, dt) if i < 3 else dev(x) for i, x in enumerate(args)]
    # fused verify + commit
    pool = dev(c.state_pool)
    o = torch.full((N, T, 3, dv), 5.0, dtype=dt, device="cuda")
    lap.decode_tokens(q, k, v, g, beta, pool, dev(c.slots), o=o, num_accepted=dev(acc),
                      scale=c.scale)
    torch.cuda.synchronize()
    o_f, pool_f = o.float().cpu().numpy(), pool.cpu().numpy()
    for n in range(N):
        s = int(c.slots[n])
        if 0 <= s < S:
            np.testing.assert_array_equal(o_f[n], o_ref[n])
            np.testing.assert_array_equal(pool_f[s], pools[int(acc[n])][s])
        else:
            assert np.all(o_f[n] == 5.0)
    named = {int(s) for s in c.slots}
    for s in range(S):
        if s not in named:
            np.testing.assert_array_equal(pool_f[s], c.state_pool[s])
    # verify (no commit), then commit the accepted tokens with no outputs
    pool2 = dev(c.state_pool)
    o2 = torch.full((N, T, 3, dv), 5.0, dtype=dt, device="cuda")
    lap.decode_tokens(q, k, v, g, beta, pool2, dev(c.slots), o=o2, commit=False, scale=c.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool2.cpu().numpy(), c.state_pool)
    np.testing.assert_array_equal(o2.float().cpu().numpy(), o_f)
    lap.decode_tokens(None, k, v, g, beta, pool2, dev(c.slots), num_accepted=dev(acc),
                      outputs=False, scale=c.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool2.cpu().numpy(), pool_f)
    # oracle parity of the fused call
    o_r, pool_r = oracle.decode_tokens(*args, c.state_pool, c.slots, num_accepted=acc,
                                       scale=c.scale, o_init=np.full((N, T, 3, dv), 5.0))
    for n in range(N):
        s = int(c.slots[n])
        if 0 <= s < S:
            assert block_error(o_f[n], o_r[n], 1) <= TOL[io]
            assert block_error(pool_f[s], pool_r[s], 2) <= TOL[io]


def test_tokens_full_size_with_acceptance():
    """64 sequences x 4 draft tokens, H=32, d=128, bf16, 64-slot pool."""
    N, T, H, d, S = 64, 4, 32, 128, 64
    slots = list(np.random.default_rng(5).permutation(S).astype(int))
    slots[7] = -1
    c, args = tokens_case(131, N, T, H, d, d, "bf16", S, slots)
    acc = np.random.default_rng(6).integers(0, T + 1, size=N).astype(np.int32)
    dt = torch.bfloat16
    q, k, v, g, beta = [dev(x, dt) if i < 3 else dev(x) for i, x in enumerate(args)]
    pool = dev(c.state_pool)
    announce("decode_tokens full N=64 T=4 H=32 d=128 bf16")
    o = lap.decode_tokens(q, k, v, g, beta, pool, dev(c.slots), num_accepted=dev(acc))
    torch.cuda.synchronize()
    o_r, pool_r = oracle.decode_tokens(*args, c.state_pool, c.slots, num_accepted=acc)
    o_g, pool_g = o.float().cpu().numpy(), pool.cpu().numpy()
    worst_o = worst_s = 0.0
    for n in range(N):
        s = int(c.slots[n])
        if s < 0:
            continue
        worst_o = max(worst_o, block_error(o_g[n], o_r[n], 1))
        worst_s = max(worst_s, block_error(pool_g[s], pool_r[s], 2))
    announce("  o err %.3e  state err %.3e" % (worst_o, worst_s))
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]


def test_tokens_with_line_addressed_pool():
    N, T, H, dk, dv, S = 5, 3, 2, 128, 128, 6
    c, args = tokens_case(141, N, T, H, dk, dv, "bf16", S, [4, 0, -1, 5, 2])
    hs = dk * dv + 576
    ss = H * hs + 1000
    fill = np.float32(4.5)
    flat = np.full(lap.line_extent(S, H, dk, dv, ss, hs), fill, dtype=np.float32)
    for s in range(S):
        for h in range(H):
            flat[s * ss + h * hs:s * ss + h * hs + dk * dv] = c.state_pool[s, h].reshape(-1)
    acc = np.array([3, 1, 2, 0, 2], dtype=np.int32)
    dt = torch.bfloat16
    q, k, v, g, beta = [dev(x, dt) if i < 3 else dev(x) for i, x in enumerate(args)]
    p = dev(flat)
    announce("decode_tokens lines %s" % c.name)
    o = lap.decode_tokens(q, k, v, g, beta, p, dev(c.slots), num_accepted=dev(acc), num_slots=S,
                          state_slot_stride=ss, state_head_stride=hs)
    torch.cuda.synchronize()
    out = p.cpu().numpy()
    o_r, pool_r = oracle.decode_tokens(*args, c.state_pool, c.slots, num_accepted=acc)
    o_g = o.float().cpu().numpy()
    mask = np.ones(out.shape, dtype=bool)
    for s in range(S):
        for h in range(H):
            a = s * ss + h * hs
            blk = out[a:a + dk * dv].reshape(dv, dk)
            assert rel_err(blk, pool_r[s, h]) <= TOL["bf16"]
            mask[a:a + dk * dv] = False
    np.testing.assert_array_equal(out[mask], np.full(mask.sum(), fill, dtype=np.float32))
    for n in range(N):
        if c.slots[n] >= 0:
            assert block_error(o_g[n], o_r[n], 1) <= TOL["bf16"]
