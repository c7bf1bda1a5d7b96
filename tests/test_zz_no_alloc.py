"""The allocation-free prefill (``kda_chunk_prefill_static``) against the
workspace entry point (``kda_chunk_prefill``), through the C ABI.

Both run the same kernels on the same inputs, so their outputs and states
must agree bit for bit.  Two calls in a row use the static scratch, the
second smaller than the first, so stale records of the first call lie in the
part of the scratch the second does not overwrite; a call larger than the
scratch is rejected before anything runs.
"""
import numpy as np
import pytest
import torch

from linear_attention_prefill_amd import workloads as W
from kda_testlib import TOL, announce, dev, oracle_prefill, per_sequence_errors
import linear_attention_prefill_amd as lap

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _run(case, no_alloc):
    dt = torch.bfloat16 if case.io_dtype == "bf16" else torch.float32
    q, k, v = dev(case.q, dt), dev(case.k, dt), dev(case.v, dt)
    g, beta, cu, slots = dev(case.g), dev(case.beta), dev(case.cu_seqlens), dev(case.slots)
    pool = dev(case.state_pool)
    o = torch.full((case.T, case.H, case.d_v), 3.0, dtype=dt, device="cuda")
    if no_alloc:
        lap.chunk_prefill_no_alloc(q, k, v, g, beta, cu, o, state_in=pool, state_out=pool,
                                   slots=slots, scale=case.scale)
    else:
        lap.chunk_prefill(q, k, v, g, beta, cu, state_in=pool, state_out=pool, o=o, slots=slots,
                          scale=case.scale)
    torch.cuda.synchronize()
    return o, pool


def test_no_alloc_matches_workspace_entry_on_two_calls():
    first = W.packed_varlen_prefill()                       # the full packed chunk
    second = W.random_case(801, [300, 1, 0, 77], H=4, d_k=128, d_v=64, io_dtype="bf16",
                           num_slots=6, scale=0.5)
    assert (lap.prefill_workspace_size(first.T, first.N, first.H, first.d_k, first.d_v)
            <= lap.kda.STATIC_SCRATCH_BYTES)
    for case in (first, second):
        announce("prefill, workspace entry: %s" % case.name)
        o_ref, p_ref = _run(case, False)
        announce("prefill, allocation-free entry: %s" % case.name)
        o_na, p_na = _run(case, True)
        assert torch.equal(o_na, o_ref)
        assert torch.equal(p_na, p_ref)
    o_r, pool_r, _ = oracle_prefill(second, o_init=np.full((second.T, second.H, second.d_v), 3.0))
    eo, es = per_sequence_errors(second, o_na.float().cpu().numpy(), o_r, p_na.cpu().numpy(),
                                 pool_r)
    announce("  second call against the oracle: o %.3e  state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_no_alloc_rejects_calls_beyond_the_scratch():
    T, N, H, d = 16384, 16, 32, 128
    assert lap.prefill_workspace_size(T, N, H, d, d) > lap.kda.STATIC_SCRATCH_BYTES
    dt = torch.bfloat16
    q = torch.zeros((T, H, d), dtype=dt, device="cuda")
    g = torch.zeros((T, H, d), dtype=torch.float32, device="cuda")
    beta = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    o = torch.full((T, H, d), 3.0, dtype=dt, device="cuda")
    cu = torch.arange(0, T + 1, T // N, dtype=torch.int32, device="cuda")
    announce("allocation-free prefill, oversize call")
    with pytest.raises(lap.KdaError) as err:
        lap.chunk_prefill_no_alloc(q, q, q, g, beta, cu, o)
    assert err.value.status == 8
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)                                # nothing ran
