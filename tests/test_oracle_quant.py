"""Pins of the oracle's append-time quantisers (int8 and FP8 E4M3 with one
fp32 scale per token per KV head) against facts that do not come from them:
the generator's numpy / torch encoders, the E4M3 definition, round-half-to-even
ties, and the quantisation error bound."""

import math

import numpy as np
import pytest

import oracle
from synth.make import quantize_fp8, quantize_int8


def special_rows(D=128):
    rng = np.random.default_rng(99)
    rows = [
        np.zeros(D),                                   # all zero: scale 1e-5 / Q
        np.full(D, -3.0),                              # constant
        np.linspace(-5.0, 5.0, D),                     # symmetric ramp
        rng.standard_normal(D) * 1e-7,                 # below the scale floor
        np.concatenate([[1e4], rng.standard_normal(D - 1)]),   # one outlier
        rng.standard_normal(D) * 100.0,
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("kind", ["i8", "fp8"])
def test_quantiser_matches_generator_encoders(kind):
    rng = np.random.default_rng(3)
    x = np.concatenate([special_rows(), rng.standard_normal((300, 128)).astype(np.float32) * 2.0])
    codes, scales = oracle.quantize_rows(x, kind)
    ref_codes, ref_scales = (quantize_int8 if kind == "i8" else quantize_fp8)(x)
    assert (scales == ref_scales).all()
    assert (codes.view(np.uint8) == np.asarray(ref_codes).view(np.uint8)).all()


def test_scale_closed_forms():
    codes, scales = oracle.quantize_rows(special_rows()[:2], "i8")
    assert scales[0] == np.float32(np.float32(1e-5) / np.float32(127.0))
    assert (codes[0] == 0).all()
    assert scales[1] == np.float32(np.float32(3.0) / np.float32(127.0))
    assert (codes[1] == -127).all()
    _, s8 = oracle.quantize_rows(special_rows()[1:2], "fp8")
    assert s8[0] == np.float32(np.float32(3.0) / np.float32(448.0))


def test_int8_ties_round_to_even():
    # amax 127 makes the scale exactly 1, so x / s = x
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :8] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    codes, scales = oracle.quantize_rows(x, "i8")
    assert scales[0] == 1.0
    assert list(codes[0, :8]) == [127, 2, 4, -2, -4, 0, 2, 0]


def test_fp8_encode_round_trips_every_finite_code():
    for c in range(256):
        v = oracle.fp8e4m3_to_f64(c)
        if math.isnan(v):
            continue
        assert oracle.fp8e4m3_encode(v) == c, hex(c)


def test_fp8_encode_ties_and_saturation():
    enc = oracle.fp8e4m3_encode
    assert enc(1.0625) == 0x38          # halfway 1.0 | 1.125 -> even mantissa 0
    assert enc(1.1875) == 0x3A          # halfway 1.125 | 1.25 -> even mantissa 2
    assert enc(1.5 * 2.0 ** -9) == 0x02  # halfway 0x01 | 0x02 (subnormals) -> even
    assert enc(7.5 * 2.0 ** -9) == 0x08  # halfway largest subnormal | smallest normal
    assert enc(-1.0625) == 0xB8
    assert enc(452.0) == 0x7E and enc(463.9) == 0x7E and enc(1e6) == 0x7E
    assert enc(-500.0) == 0xFE
    assert enc(2.0 ** -11) == 0x00      # below half the smallest subnormal


@pytest.mark.parametrize("kind", ["i8", "fp8"])
def test_quantisation_error_bound(kind):
    """|s * code - x| <= s / 2 for int8; for E4M3 at most half a unit in the
    last place of the code (2^-4 relative for normals, 2^-10 absolute in the
    subnormal range), times s."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((200, 64)).astype(np.float32) * 5.0
    codes, scales = oracle.quantize_rows(x, kind)
    s = scales.astype(np.float64)[:, None]
    if kind == "i8":
        back = codes.astype(np.float64) * s
        assert (np.abs(back - x) <= s * 0.5 * (1 + 1e-6)).all()
    else:
        dec = np.vectorize(oracle.fp8e4m3_to_f64)(codes.astype(np.int64))
        y = x.astype(np.float64) / s
        bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10)
        assert (np.abs(dec - y) <= bound * (1 + 1e-6)).all()
