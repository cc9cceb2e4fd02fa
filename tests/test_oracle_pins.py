"""The CPU oracle against closed forms, invariants, library routines and brute force."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads
from oracle_pins import ALL_PINS, brute_compare


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(
    B=st.integers(1, 2), Hkv=st.integers(1, 2), G=st.sampled_from([1, 2]),
    Nq=st.integers(1, 9), Nk=st.integers(1, 9), D=st.sampled_from([2, 4, 6]),
    seed=st.integers(0, 10_000), rope=st.booleans(), causal=st.booleans(),
    window=st.sampled_from([0, 1, 3]), alibi=st.booleans(), bias=st.booleans(),
    block=st.booleans(), q_pos0=st.integers(0, 5), k_pos0=st.integers(0, 5),
)
def test_oracle_matches_brute_force(B, Hkv, G, Nq, Nk, D, seed, rope, causal, window, alibi,
                                    bias, block, q_pos0, k_pos0):
    brute_compare(oracle, B, Hkv * G, Hkv, Nq, Nk, D, seed, rope, causal, window, alibi, bias,
                  block, q_pos0, k_pos0)


def test_brute_force_pins_itself_on_closed_forms():
    """The brute force also meets the D=2 rotation and the Q=0 prefix mean."""
    rng = np.random.default_rng(3)
    N = 6
    v = rng.standard_normal((1, 1, N, 2))
    out, lse = oracle.attention_brute(np.zeros((1, 1, N, 2)).tolist(),
                                      rng.standard_normal((1, 1, N, 2)).tolist(), v.tolist(),
                                      rope_theta=10.0, causal=True)
    np.testing.assert_allclose(np.array(out)[0, 0], np.cumsum(v[0, 0], 0) / np.arange(1, N + 1)[:, None],
                               atol=1e-14)
    # one key at position p, one query at position 0: score = <q, R(p) k> / sqrt(2)
    p = 3.0
    q = [[[[1.0, 0.0]]]]
    k = [[[[1.0, 0.0]]]]
    vv = [[[[2.0, 5.0]]]]
    _, l = oracle.attention_brute(q, k, vv, rope_theta=10.0, k_pos0=int(p))
    np.testing.assert_allclose(l[0][0][0], np.cos(p) / np.sqrt(2.0), atol=1e-14)


# ----------------------------------------------------------------------------
# The seeded input generators
# ----------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], np.float32)])
    bits = workloads.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f64(bits),
                                  torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_bigbird_csr_structure():
    rp, ci = workloads.bigbird_csr(64, 64, seed=4)
    assert rp[-1] == ci.size == 505
    counts = np.diff(rp)
    assert counts[0] == 5 and counts[1] == 6 and counts[2] == 7 and counts[63] == 7
    assert np.all(counts[3:63] == 8)
    for r in range(64):
        cols = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(cols) > 0) and cols.min() >= 0 and cols.max() < 64
        for need in {0, 1} | {c for c in (r - 1, r, r + 1) if 0 <= c < 64}:
            assert need in cols
    rp2, ci2 = workloads.bigbird_csr(64, 64, seed=4)
    np.testing.assert_array_equal(ci, ci2)


def test_alibi_slopes_values():
    s = workloads.alibi_slopes(16)
    np.testing.assert_allclose(s, [2.0 ** (-h / 2) for h in range(1, 17)], rtol=1e-7)
    assert s.dtype == np.float32


def test_make_inputs_shapes_and_exact_widening():
    w = workloads.WORKLOADS["llama3_8b_rope_causal_n4096"].with_(Nq=64, Nk=64)
    inp = workloads.make_inputs(w)
    assert inp.q_dev.shape == (1, 32, 64, 128) and inp.q_dev.dtype == np.uint16
    assert inp.k.shape == (1, 8, 64, 128)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f64(inp.v_dev), inp.v)
    w1 = workloads.WORKLOADS["rope_causal_fp32_n256"]
    i1 = workloads.make_inputs(w1)
    assert i1.q_dev.dtype == np.float32
    np.testing.assert_array_equal(i1.q_dev.astype(np.float64), i1.q)
