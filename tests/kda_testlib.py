"""Helpers shared by the GPU tests: move a seeded case to the device, run the
HIP path through the C ABI, run the oracle, and measure errors."""
import sys

import numpy as np
import torch

import linear_attention_prefill_amd as lap
from oracle import oracle

TOL = {"bf16": 2e-2, "f32": 1e-4}


# pytest's capture manager, set by conftest.py when running under pytest.
CAPTURE = None


def announce(msg: str):
    """Name the case before a GPU step.  pytest captures at the file
    descriptor level, so the line is written with capture suspended: it
    reaches the terminal (or the log a run is redirected to) at once, and
    survives a process that dies in the GPU step that follows."""
    line = "[gpu-case] %s\n" % msg
    if CAPTURE is not None:
        with CAPTURE.global_and_fixture_disabled():
            sys.stderr.write(line)
            sys.stderr.flush()
    else:
        sys.__stderr__.write(line)
        sys.__stderr__.flush()


def torch_dtype(io):
    return torch.bfloat16 if io == "bf16" else torch.float32


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t.to(dtype) if dtype is not None else t


def rel_err(x, ref):
    """Normwise error max|x - ref| / max|ref| (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def gpu_prefill(case, pool=None, o_init=None, in_place=True, state_in_null=False,
                state_out_null=False, num_slots=None, stream=None, fuse_chunks=0):
    """Run kda_chunk_prefill on a workloads.Case.  Returns (o f32 numpy,
    state_out numpy or None)."""
    dt = torch_dtype(case.io_dtype)
    q, k, v = dev(case.q, dt), dev(case.k, dt), dev(case.v, dt)
    g, beta = dev(case.g), dev(case.beta)
    cu = dev(case.cu_seqlens)
    slots = dev(case.slots) if case.slots is not None else None
    pool = case.state_pool if pool is None else pool
    pin = pout = None
    if pool is not None:
        pin = dev(pool)
        pout = pin if in_place else dev(pool)
    if state_in_null:
        pin = None
    if state_out_null:
        pout = None
    if o_init is None:
        o = torch.zeros((case.T, case.H, case.d_v), dtype=dt, device="cuda")
    else:
        o = dev(o_init, dt)
    lap.chunk_prefill(q, k, v, g, beta, cu, state_in=pin, state_out=pout, o=o, slots=slots,
                      num_slots=num_slots, scale=case.scale, stream=stream, fuse_chunks=fuse_chunks)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(),
            None if pout is None else pout.cpu().numpy())


def oracle_prefill(case, pool=None, o_init=None, num_slots=None):
    pool = case.state_pool if pool is None else pool
    return oracle.chunk_prefill(case.q, case.k, case.v, case.g, case.beta, case.cu_seqlens,
                                state_pool=pool, slots=case.slots, scale=case.scale,
                                o_init=o_init, num_slots=num_slots)


def per_sequence_errors(case, o_gpu, o_ref, pool_gpu=None, pool_ref=None, live=None):
    """Max over (sequence, head) pairs of the normwise error of o, and of the
    final state: each head is normalised by its own largest reference value,
    so a head with small outputs is held to the same relative bar as the
    largest one."""
    cu = case.cu_seqlens
    eo, es = 0.0, 0.0
    for n in range(case.N):
        if live is not None and not live[n]:
            continue
        a, b = int(cu[n]), int(cu[n + 1])
        s = int(case.slots[n]) if case.slots is not None else n
        for h in range(case.H):
            if b > a:
                eo = max(eo, rel_err(o_gpu[a:b, h], o_ref[a:b, h]))
            if pool_gpu is not None:
                es = max(es, rel_err(pool_gpu[s, h], pool_ref[s, h]))
    return eo, es


def per_head_error(x, ref):
    """Max over heads of the normwise error of outputs [..., H, d]: each head's
    block (all leading rows, all d columns) is normalised by its own largest
    reference value."""
    x = np.asarray(x)
    ref = np.asarray(ref)
    return max(rel_err(x[..., h, :], ref[..., h, :]) for h in range(x.shape[-2]))


def block_error(x, ref, block_dims):
    """Max of the normwise error over blocks made of the last `block_dims`
    axes: block_dims = 2 gives one error per (slot, head) state [d_v, d_k],
    block_dims = 1 one per (token, head) output row."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    n = int(np.prod(x.shape[-block_dims:]))
    xb, rb = x.reshape(-1, n), ref.reshape(-1, n)
    return max(rel_err(xb[i], rb[i]) for i in range(xb.shape[0]))
