"""Pins of the oracle's element codecs.

E4M3 follows the OCP OFP8 definition (bias 7, 3 mantissa bits, subnormals,
S.1111.111 = NaN, no infinity, max 448); fp8 KV with b = 1 is the option the
pages name ("LLM inference basics and vLLM internals", §2 and §7).  The
encoder is checked against hand values, exhaustive round trips, and torch's
float8_e4m3fn cast (a library routine) after clamping to +-448 — torch's CPU
cast turns magnitudes >= 480 into NaN, so the clamp makes it satfinite.
bf16 / fp16 decode are checked against numpy / torch conversions.
"""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3_hand_values():
    t = oracle.e4m3_table()
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0**-9                      # smallest subnormal
    assert t[0x07] == 7 * 2.0**-9                  # largest subnormal
    assert t[0x08] == 2.0**-6                      # smallest normal
    assert t[0x38] == 1.0
    assert t[0x39] == 1.125
    assert t[0x7E] == 448.0
    assert t[0xFE] == -448.0
    assert t[0x77] == 240.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2
    assert np.isfinite(t).sum() == 254


def test_e4m3_monotone_and_symmetric():
    t = oracle.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_e4m3_round_trip_all_codes():
    t = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    enc = oracle.e4m3_encode(t[codes].astype(np.float32))
    assert np.array_equal(enc, codes)


def test_e4m3_ties_saturation_nan():
    cases = [
        (1.0625, 0x38),      # tie between 1.0 (even) and 1.125 -> 1.0
        (1.1875, 0x3A),      # tie between 1.125 and 1.25 (even) -> 1.25
        (1.07, 0x39),
        (2.0**-10, 0x00),    # half the smallest subnormal: tie -> even 0
        (1.5 * 2.0**-10, 0x01),
        (2.0**-11, 0x00),
        (-2.0**-11, 0x80),   # sign kept on underflow
        (464.0, 0x7E),       # would round past 448: saturate
        (500.0, 0x7E),
        (1e30, 0x7E),
        (-1e30, 0xFE),
        (float("inf"), 0x7E),
        (float("-inf"), 0xFE),
        (440.0, 0x7E),       # tie between 416 and 448 (even 448 = ...110)
        (-0.0, 0x80),
    ]
    x = np.array([c[0] for c in cases], np.float32)
    got = oracle.e4m3_encode(x)
    for (v, want), g in zip(cases, got):
        assert g == want, (v, hex(g), hex(want))
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def _torch_e4m3(x32):
    t = torch.from_numpy(np.clip(x32, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0, 0.0123, 1.0 / 64])
def test_e4m3_encode_matches_torch_on_all_bf16(scale):
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x)]
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore"):                 # large inputs overflow to inf, dropped next
        xs = (x * inv).astype(np.float32)
    xs = xs[np.isfinite(xs)]
    assert np.array_equal(oracle.e4m3_encode(xs), _torch_e4m3(xs))


def test_e4m3_encode_matches_torch_random_fp32():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * rng.choice([1e-3, 1, 30, 300], 200000)).astype(
        np.float32)
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3(x))


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")   # the NaN codes
def test_bf16_and_fp16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    want16 = bits.view(np.float16).astype(np.float64)
    got16 = oracle.decode_values(bits, oracle.FP16)
    same = (got16 == want16) | (np.isnan(got16) & np.isnan(want16))
    assert same.all()
    wantb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    gotb = oracle.decode_values(bits, oracle.BF16)
    same = (gotb == wantb) | (np.isnan(gotb) & np.isnan(wantb))
    assert same.all()
