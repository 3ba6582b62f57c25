"""Storage encodings: the oracle's decoders and the generator's encoders (CPU).

The oracle's E4M3 decoder is pinned against torch's float8_e4m3fn (a library
implementation of the OCP format) over all 256 codes and against values the
OCP definition fixes.  The generator's encoders are pinned against torch's
float -> bfloat16 / float8_e4m3fn conversions (round to nearest even).
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from head_latent_attention_mla_amd import workloads as W


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0), (0x77, 240.0),
])
def test_e4m3_decode_definition_values(code, value):
    got = O.e4m3_to_f64(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    enc = W.to_e4m3_codes(vals)
    # +0 and -0 keep their sign bit; every other code maps back to itself
    np.testing.assert_array_equal(enc, codes)


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ours = W.to_e4m3_codes(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_ties_and_saturation():
    # 1 + 1/16 is halfway between 1 (mantissa 0, even) and 1.125: goes to 1
    # 1 + 3/16 is halfway between 1.125 (odd) and 1.25 (even): goes to 1.25
    v = np.array([1 + 1 / 16, 1 + 3 / 16, 460.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10])
    got = O.e4m3_to_f64(W.to_e4m3_codes(v))
    np.testing.assert_array_equal(got, [1.0, 1.25, 448.0, 448.0, -448.0, 0.0, 2 * 2.0 ** -9])


def test_row_quantisation_scale_rule():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((50, 576))
    rows[3] = 0
    codes, scale = W.quantize_rows_e4m3(rows)
    amax = np.abs(rows).max(1)
    np.testing.assert_allclose(scale[np.arange(50) != 3], (amax / 448)[np.arange(50) != 3], rtol=1e-7)
    assert scale[3] == 1.0 and not codes[3].any()
    deq = O.e4m3_to_f64(codes) * scale[:, None].astype(np.float64)
    # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 for normal values
    big = np.abs(rows) > 2 ** -6 * scale[:, None] * 2
    assert np.all(np.abs(deq - rows)[big] <= 2 ** -4 * np.abs(rows)[big] + 1e-12)
    assert np.abs(O.e4m3_to_f64(codes)).max() == 448.0


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32)
    ours = W.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(O.bf16_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())
