"""The FP8 E4M3 input formatting (OCP E4M3: bias 7, largest 448, no
infinities, 0x7f / 0xff NaN) that the fp8 KV-cache decode's inputs go
through: decoded values pinned to the format's definition, and the encoder's
rounding (nearest, ties to the even code, saturation at 448)."""
import numpy as np
import pytest

import workloads


def test_decoded_values_follow_the_format():
    v = workloads.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x38] == 1.0 and v[0xB8] == -1.0 and v[0x40] == 2.0 and v[0x30] == 0.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6                          # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9  # subnormals m * 2^-9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = v[:0x7F]
    assert np.all(np.diff(finite) > 0)                  # codes 0..126 ascend
    # every step inside a binade is 2^(e-10): 8 values per binade
    for e in range(1, 15):
        seg = finite[8 * e: 8 * e + 8]
        assert np.allclose(np.diff(seg), 2.0 ** (e - 10))


def test_encoder_round_trip_and_rounding():
    c = np.arange(256, dtype=np.uint8)
    v = workloads.e4m3_to_f64(c)
    ok = ~np.isnan(v) & (c != 0x80)                      # -0 encodes as +0
    assert np.array_equal(workloads.round_to_e4m3(v[ok]), c[ok])
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 500.0, -500.0, 447.0, 1e-30])
    want = np.array([0x38, 0x3A, 0x00, 0x02, 0x7E, 0xFE, 0x7E, 0x00], dtype=np.uint8)
    assert np.array_equal(workloads.round_to_e4m3(x), want)
    rng = np.random.default_rng(0)
    y = rng.standard_normal(10000) * 50
    got = workloads.e4m3_to_f64(workloads.round_to_e4m3(y))
    grid = workloads.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    grid = np.concatenate([-grid[::-1], grid])
    nearest = grid[np.abs(np.minimum(np.abs(y), 448)[:, None] * np.sign(y)[:, None] - grid[None, :]).argmin(axis=1)]
    assert np.all(np.abs(got - np.clip(y, -448, 448)) <= np.abs(nearest - np.clip(y, -448, 448)) + 1e-12)


def test_encoder_rejects_non_finite():
    with pytest.raises(ValueError):
        workloads.round_to_e4m3(np.array([np.inf]))
