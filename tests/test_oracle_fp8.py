"""Pins for the oracle's FP8 E4M3fn codec and per-row quantiser.

Pinned against: the OCP E4M3 value table (tests/golden/e4m3fn_values.json),
PyTorch's float8_e4m3fn casts (an independent library routine), and the
error bounds of round-to-nearest on a 3-bit mantissa."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_values.json")


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32).copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_table():
    g = json.load(open(GOLDEN))
    for code, val in g["codes_to_values"]:
        got = fp8.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        assert got == float(val), (code, got, val)
        assert np.signbit(got) == val.startswith("-")
    for code in g["nan_codes"]:
        assert np.isnan(fp8.e4m3_decode(np.array([int(code, 16)], np.uint8))[0])


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert (np.signbit(ours[~nan]) == np.signbit(ref[~nan])).all()


def test_roundtrip_identity_on_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert (fp8.e4m3_encode(fp8.e4m3_decode(codes)) == codes).all()


def test_midpoints_round_to_even_code():
    grid = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2  # exactly representable in float64 and fp32
    got = fp8.e4m3_encode(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert (got == expect).all()
    assert (fp8.e4m3_encode(-mids) == (expect | 0x80)).all()
    assert (got == torch_encode(mids)).all()


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(400_000) * 100,
        rng.standard_normal(300_000) * 1e-2,
        rng.uniform(-448, 448, 200_000),
        rng.standard_normal(100_000) * 3e-3,  # subnormal region
    ]
    x = np.concatenate(parts).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert (fp8.e4m3_encode(x) == torch_encode(x)).all()


def test_saturation_and_signed_zero():
    x = np.array([448.0, 460.0, 470.0, 1e6, -470.0, -1e30, 1e-9, -1e-9, 0.0, -0.0], np.float32)
    got = fp8.e4m3_encode(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x00, 0x80]
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([np.nan]))


def test_quantize_rows_error_bound_and_scale():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((257, 128)).astype(np.float32)
    x[3] = 0.0
    codes, scale = fp8.quantize_rows(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[3] == 1.0 and (codes[3] == 0).all()
    amax = np.abs(x).max(axis=1)
    ok = amax > 0
    assert (scale[ok] == (amax[ok] / np.float32(448)).astype(np.float32)).all()
    deq = fp8.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    err = np.abs(deq - x.astype(np.float64))
    y = np.abs(x.astype(np.float64)) / scale[:, None]
    normal = y >= 2.0 ** -6
    # half an ulp of a 3-bit mantissa: 2^-4 relative (plus the fp32 division's rounding)
    assert (err[normal] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(x.astype(np.float64))[normal]).all()
    # subnormal region: half of the 2^-9 spacing, times the row scale
    sub_bound = (2.0 ** -10 + 2.0 ** -30) * np.broadcast_to(scale[:, None], x.shape)
    assert (err[~normal] <= sub_bound[~normal]).all()
    # the row maximum lands on (or next to) +-448
    top = np.abs(fp8.e4m3_decode(codes[ok][np.arange(ok.sum()), np.abs(x[ok]).argmax(axis=1)]))
    assert (top >= 416).all()


# --------------------------------------------------------------- E8M0 variant
# Pinned against the definition's closed-form properties and against PyTorch's
# float8_e4m3fn cast of x / 2^e (an exact division, so the library cast of the
# quotient is an independent check of the codes).


def test_e8m0_decode_closed_form():
    b = np.arange(255, dtype=np.uint8)
    v = fp8.e8m0_decode(b)
    assert (v == 2.0 ** (b.astype(np.int64) - 127)).all()
    with pytest.raises(ValueError):
        fp8.e8m0_decode(np.array([255], np.uint8))


def test_e8m0_scale_is_the_smallest_power_of_two():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-40, 40, size=(2000, 1)).astype(np.float32)
    codes, b, scale = fp8.quantize_rows_e8m0(x)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    assert (scale == np.ldexp(1.0, b.astype(np.int64) - 127)).all()
    assert (amax <= 448.0 * scale).all()          # nothing saturates
    assert (amax > 224.0 * scale).all()           # a smaller power of two would
    # codes: the library cast of the exact quotient
    q = (x.astype(np.float64) / scale[:, None]).astype(np.float32)
    assert (codes == torch_encode(q)).all()


def test_e8m0_boundaries_and_special_rows():
    base = np.zeros((6, 64), np.float32)
    base[0, 3] = 448.0                            # absmax = 448 * 2^0 -> e = 0, code 0x7E
    base[1, 5] = np.float32(448.0 * 2.0 ** 10)    # exactly on a power of two -> e = 10
    base[2, 7] = np.nextafter(np.float32(448.0 * 2.0 ** -5), np.float32(np.inf))  # just above -> e = -4
    base[3] = 0.0                                 # all zero -> e = 0, codes 0
    base[4, 0] = np.float32(1e-40)                # subnormal absmax -> exponent clamped at -127
    base[5, 1] = np.float32(3e38)                 # near the fp32 maximum
    codes, b, scale = fp8.quantize_rows_e8m0(base)
    e = b.astype(np.int64) - 127
    assert list(e[:4]) == [0, 10, -4, 0]
    assert codes[0, 3] == 0x7E and codes[1, 5] == 0x7E
    assert (codes[3] == 0).all()
    assert e[4] == -127 and 1e-40 / scale[4] <= 448.0
    assert 3e38 / scale[5] <= 448.0 and 3e38 / scale[5] > 224.0
    assert (codes == torch_encode((base.astype(np.float64) / scale[:, None]).astype(np.float32))).all()


def test_e8m0_dequantisation_error_bound():
    """Round-to-nearest on a 3-bit mantissa: |decode(code) * 2^e - x| <= 2^-4 |x|
    for quotients in the normal range, <= 2^-10 * 2^e below it."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((500, 256)) * 3.0).astype(np.float32)
    codes, b, scale = fp8.quantize_rows_e8m0(x)
    back = fp8.e4m3_decode(codes) * scale[:, None]
    err = np.abs(back - x.astype(np.float64))
    normal = np.abs(x) / scale[:, None] >= 2.0 ** -6
    assert (err[normal] <= 2.0 ** -4 * np.abs(x.astype(np.float64))[normal]).all()
    assert (err[~normal] <= (2.0 ** -10 * scale[:, None] * np.ones_like(err))[~normal]).all()
