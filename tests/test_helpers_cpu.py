"""CPU checks of the test helpers the GPU parity tests rely on."""
import numpy as np

import oracle
import workloads
from gpu_helpers import check_lse, oracle_all_heads


def test_oracle_all_heads_equals_one_oracle_call():
    w = workloads.WORKLOADS["alibi_causal_window1024_n8192"].with_(B=2, Hq=4, Hkv=2, Nq=130, Nk=150,
                                                                  window=40, rope_theta=1e4)
    inp = workloads.make_inputs(w)
    rp, ci = workloads.random_csr(3, 3, 0.6, seed=2, n_heads=w.Hq)
    kw = dict(rope_theta=w.rope_theta, causal=True, window=w.window,
              alibi_slopes=workloads.alibi_slopes(w.Hq).astype(np.float64),
              block_mask=(rp, ci, 64, 64))
    a, la = oracle.attention(inp.q, inp.k, inp.v, **kw)
    b, lb = oracle_all_heads(inp.q, inp.k, inp.v, w.B, w.Hq, workers=3, **kw)
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    check_lse(lb, la, 1e-12, "helper")


def test_check_lse_accepts_matching_empty_rows_without_warnings():
    import warnings
    got = np.array([1.0, -np.inf, 2.0])
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        check_lse(got, got.copy(), 0.0, "empty rows")
