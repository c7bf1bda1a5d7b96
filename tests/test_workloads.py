"""Host-side checks of the seeded input generators (no method arithmetic)."""
import numpy as np
import torch

from linear_attention_prefill_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    # include exact ties
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32)
    x = np.concatenate([x, ties])
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_dirichlet_lengths_contract():
    for seed in range(20):
        L = W.dirichlet_lengths(np.random.default_rng(seed), 8192, 16)
        assert L.sum() == 8192 and len(L) == 16
        assert L.min() == 1
        assert np.sum(L % 64 != 0) >= 9


def test_packed_case_shapes_and_distributions():
    c = W.packed_varlen_prefill(T=1024, H=4, d=64, n=16, num_slots=64)
    assert c.cu_seqlens.dtype == np.int32 and c.cu_seqlens[-1] == 1024 and c.N == 16
    assert len(set(c.slots.tolist())) == 16 and c.slots.min() >= 0 and c.slots.max() < 64
    assert np.all(c.g <= 0) and np.all((c.beta > 0) & (c.beta < 1))
    # q, k unit norm up to bf16 rounding
    nq = np.linalg.norm(c.q.astype(np.float64), axis=-1)
    assert np.all(np.abs(nq - 1) < 2 ** -7)
    assert np.array_equal(W.round_to_bf16(c.v), c.v)
    assert abs(float(c.state_pool.std()) - 0.02) < 1e-3


def test_seeded_cases_are_deterministic():
    a = W.random_case(3, [5, 7], H=2, d_k=8, d_v=8)
    b = W.random_case(3, [5, 7], H=2, d_k=8, d_v=8)
    for x, y in ((a.q, b.q), (a.g, b.g), (a.state_pool, b.state_pool), (a.slots, b.slots)):
        np.testing.assert_array_equal(x, y)
