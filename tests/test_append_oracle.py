"""Pins of the latent-append oracle (CPU).

Each check rests on something other than the oracle itself: closed forms of
the rotation, invariants every rotation obeys, a one-hot input whose product
is a column of the weight, brute-force rounding on small sets and torch's
float -> bfloat16 / float8_e4m3fn conversions (library routines).
"""
import math

import numpy as np
import pytest
import torch

from oracle import latent_append as A

BASE = 10000.0


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((3, 64))
    np.testing.assert_array_equal(A.rope_rotate(v, np.zeros(3, np.int64), BASE), v)


def test_rope_first_pair_closed_form():
    # pair 0 turns by exactly the position (base^0 = 1)
    v = np.zeros((4, 64))
    v[:, 0] = 1.0
    pos = np.array([1, 2, 100, 4097])
    out = A.rope_rotate(v, pos, BASE)
    for n, p in enumerate(pos):
        assert out[n, 0] == pytest.approx(math.cos(p), abs=1e-15)
        assert out[n, 1] == pytest.approx(math.sin(p), abs=1e-15)
    assert np.all(out[:, 2:] == 0.0)


@pytest.mark.parametrize("k,angle", [(0, 1.0), (16, 0.01), (31, 10000.0 ** (-62 / 64))])
def test_rope_pair_frequency(k, angle):
    # at position 1, pair k turns by base^(-2k/64): 1, 1/100 (k = 16), ...
    v = np.zeros((1, 64))
    v[0, 2 * k + 1] = 1.0                 # (0, 1) -> (-sin, cos)
    out = A.rope_rotate(v, np.array([1]), BASE)
    assert out[0, 2 * k] == pytest.approx(-math.sin(angle), abs=1e-15)
    assert out[0, 2 * k + 1] == pytest.approx(math.cos(angle), abs=1e-15)


def test_rope_relative_position_invariant():
    # <R_i a, R_j b> depends only on i - j, and rotations keep every pair's norm
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal((2, 1, 64))
    for i, j in [(5, 2), (1000, 997), (3, 0)]:
        lhs = A.rope_rotate(a, np.array([i]), BASE)[0] @ A.rope_rotate(b, np.array([j]), BASE)[0]
        rhs = A.rope_rotate(a, np.array([i - j]), BASE)[0] @ b[0]
        assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-12)
    r = A.rope_rotate(a, np.array([12345]), BASE)[0]
    np.testing.assert_allclose(r[0::2] ** 2 + r[1::2] ** 2, a[0, 0::2] ** 2 + a[0, 1::2] ** 2, rtol=1e-12)


def test_append_rows_one_hot_picks_a_weight_column():
    rng = np.random.default_rng(2)
    d = 96
    w = rng.standard_normal((576, d))
    x = np.zeros((3, d))
    x[0, 5] = 1.0
    x[1, 17] = 2.0
    x[2, 95] = -1.0
    rows = A.append_rows(x, w, np.zeros(3, np.int64), BASE)
    np.testing.assert_array_equal(rows[0], w[:, 5])
    np.testing.assert_array_equal(rows[1], 2.0 * w[:, 17])
    np.testing.assert_array_equal(rows[2], -w[:, 95])
    # the latent part ignores the position; the rope part turns with it
    moved = A.append_rows(x, w, np.array([7, 7, 7]), BASE)
    np.testing.assert_array_equal(moved[:, :512], rows[:, :512])
    assert not np.allclose(moved[:, 512:], rows[:, 512:])


def test_append_rows_linear_in_x():
    rng = np.random.default_rng(3)
    d = 64
    w = rng.standard_normal((576, d))
    x1, x2 = rng.standard_normal((2, 2, d))
    pos = np.array([3, 9])
    lhs = A.append_rows(2.0 * x1 - x2, w, pos, BASE)
    rhs = 2.0 * A.append_rows(x1, w, pos, BASE) - A.append_rows(x2, w, pos, BASE)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_nearest_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(A.e4m3_nearest(vals), codes)


def test_e4m3_nearest_midpoints_go_to_even():
    # midpoints of adjacent codes: 1 + 1/16 lies between 1 (0x38) and 1.125
    # (0x39) -> 0x38; 1.125 + 1/16 between 0x39 and 0x3A -> 0x3A; the
    # smallest subnormal's half -> 0
    got = A.e4m3_nearest(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -1.0625]))
    np.testing.assert_array_equal(got, [0x38, 0x3A, 0x00, 0x02, 0xB8])


def test_e4m3_nearest_clamps_and_matches_torch():
    assert A.e4m3_nearest(np.array([449.0, 463.9, 1e6, -1e6])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    np.testing.assert_array_equal(A.e4m3_nearest(v.astype(np.float64)), _torch_e4m3(v))


def test_quantize_rows_scale_and_bound():
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((6, 576)) * np.array([1, 1e-3, 50, 1, 1, 1])[:, None]
    rows[3] = 0.0
    codes, scale = A.quantize_rows(rows)
    assert scale.dtype == np.float32 and scale[3] == 1.0
    np.testing.assert_array_equal(codes[3], 0)
    amax = np.max(np.abs(rows), axis=1)
    for n in (0, 1, 2, 4, 5):
        assert scale[n] == np.float32(amax[n] / 448.0)
        k = int(np.argmax(np.abs(rows[n])))
        assert codes[n, k] & 0x7F == 0x7E          # the largest magnitude maps to 448
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale[:, None]
    # every value is within half a quantum of its code (the quantum is 2^-3
    # of the binade, 2^-9 * scale below 2^-6 * scale)
    err = np.abs(dec - rows) / scale[:, None]
    q = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(rows) / scale[:, None], 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(err <= 0.5 * q * (1 + 1e-9))


def test_bf16_nearest_matches_torch_and_ties():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(20000) * np.exp2(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(A.bf16_nearest(v.astype(np.float64)), ref)
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80);
    # 1 + 3 * 2^-8 -> 1 + 2^-6 (0x3F82)
    assert A.bf16_nearest(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])).tolist() == [0x3F80, 0x3F82]
