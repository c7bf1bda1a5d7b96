"""The parity gates against the noise floor of the oracle itself (the "kern"
page, section "The harness": a candidate is judged against a floor measured by
replaying the reference against itself).

The same token loop in fp32 against fp64 sits about two orders below the fp32
gate (1e-4), and rounding the fp64 output to bf16 alone costs about a tenth of
the bf16 gate (2e-2).  So both gates leave room above what the arithmetic and
the output dtype can reach, without being so loose that a dropped term would
pass (the pins in test_oracle_pins.py fail far above them).
"""
import numpy as np

from linear_attention_prefill_amd import workloads as W
from oracle import noise_floor, oracle


def test_fp32_loop_is_far_below_the_fp32_gate():
    c = W.tiny_prefill()
    r = noise_floor.one_call(c, threads=4)["fp32_vs_fp64"]
    # fp32 arithmetic really ran (a float build that silently used doubles
    # would give 0) and stays two orders below the gate
    assert 1e-9 < r["o"] < 1e-6 and 1e-9 < r["state"] < 1e-6, r


def test_bf16_floor_against_the_bf16_gate():
    c = W.single_seq_prefill(seed=9, T=1024, H=4)
    r = noise_floor.one_call(c, threads=4)
    assert r["fp32_vs_fp64"]["o"] < 1e-5 and r["fp32_vs_fp64"]["state"] < 1e-5, r
    # bf16 has 8 significant bits: output rounding alone costs between 2^-10
    # and 2^-8 of the largest value
    assert 2.0 ** -10 < r["bf16_output_rounding"]["o"] < 2.0 ** -8, r


def test_float_build_matches_double_build_on_exact_cases():
    """With g = 0 and beta = 0 the state never changes and o_t = S0^T q_t: a
    dot product of 64 terms, equal in both builds to within fp32 rounding."""
    rng = np.random.default_rng(3)
    T, H, d = 5, 1, 64
    q = rng.standard_normal((T, H, d)).astype(np.float32)
    z = np.zeros((T, H, d), dtype=np.float32)
    s0 = rng.standard_normal((1, H, d, d)).astype(np.float32)
    cu = np.array([0, T], dtype=np.int32)
    o64, s64 = oracle.recurrence(q, z, z, z, np.zeros((T, H), np.float32), cu, s0=s0)
    o32, s32 = oracle.recurrence(q, z, z, z, np.zeros((T, H), np.float32), cu, s0=s0,
                                 precision="f32")
    np.testing.assert_array_equal(s32, s0.astype(np.float64))
    np.testing.assert_allclose(o32, o64, rtol=0, atol=1e-5 * np.max(np.abs(o64)))
