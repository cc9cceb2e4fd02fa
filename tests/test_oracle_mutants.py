"""Plant one plausible mistake in a copy of the oracle; some pin must fail.

The mistakes are planted in a private in-memory copy of ``oracle/attention.py``
on the CPU; the real oracle is untouched.  Each mutation is a mistake a reader
of the pages could plausibly make (wrong rotation sign or pairing, wrong
frequency exponent, wrong scale, an off-by-one mask, the ALiBi sign, the GQA
head mapping, the log base of the saved statistic, a dropped bias term, ...).
"""
import os
import types

import numpy as np
import pytest

from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")

MUTATIONS = {
    "rope_sign": ("lo * c - hi * s", "lo * c + hi * s"),
    "rope_second_half_sign": ("hi * c + lo * s", "hi * c - lo * s"),
    "rope_interleaved_pairs": ("lo, hi = x[..., :half], x[..., half:]",
                               "lo, hi = x[..., 0::2], x[..., 1::2]"),
    "rope_freq_exponent": ("-2.0 * r / D", "-1.0 * r / D"),
    "rope_q_uses_k_positions": ("rope_rotate(qq, q_pos0 + ri", "rope_rotate(qq, k_pos0 + ri"),
    "scale_one_over_d": ("scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
    "alibi_sign": ("(k_pos0 + k_idx)[None, :] - (q_pos0 + ri)[:, None]",
                   "(q_pos0 + ri)[:, None] - (k_pos0 + k_idx)[None, :]"),
    "alibi_wrong_head": ("alibi_slopes, dtype=np.float64)[h]",
                         "alibi_slopes, dtype=np.float64)[h // group]"),
    "causal_strict": ("ok &= pk <= pq", "ok &= pk < pq"),
    "window_off_by_one": ("(dist >= 0) & (dist < window)", "(dist >= 0) & (dist <= window)"),
    "window_noncausal_one_sided": ("ok &= np.abs(dist) < window", "ok &= (dist >= 0) & (dist < window)"),
    "gqa_modulo_mapping": ("kvh = h // group", "kvh = h % Hkv"),
    "lse_log2": ("ls = m + np.log(l)", "ls = m + np.log2(l)"),
    "lse_missing_max": ("ls = m + np.log(l)", "ls = np.log(l)"),
    "bias_dropped": ("s = s + bias[b, h][ri]", "s = s"),
    "bias_transposed": ("s = s + bias[b, h][ri]", "s = s + bias[b, h].T[ri]"),
    "block_row_overrun": ("cols = col_idx[row_ptr[b]:row_ptr[b + 1]]",
                          "cols = col_idx[row_ptr[b]:row_ptr[b + 1] + 1]"),
    "block_per_head_ignored": ("row_ptr = row_ptr[head]", "row_ptr = row_ptr[0]"),
    "empty_row_not_zeroed": ("o[~any_ok] = 0.0", "pass"),
    "softmax_unnormalised": ("o = (e @ vv) / l[:, None]", "o = (e @ vv)"),
    "values_from_wrong_head": ("vv = v[b, kvh]", "vv = v[b, (kvh + 1) % Hkv]"),
}


def _mutant(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            # a planted mistake may produce inf - inf; that is part of being caught
            with np.errstate(invalid="ignore"):
                pin(mod)
        except Exception:  # an assertion or a shape error both mean "caught"
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
