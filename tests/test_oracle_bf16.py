"""Pins for the oracle's bfloat16 decoder: closed-form values of the format
(1 sign, 8 exponent, 7 mantissa bits, bias 127) and agreement on every one of
the 65536 codes with torch's own bfloat16 conversion."""

import numpy as np
import torch

from oracle.bf16 import bf16_decode


def test_closed_form_values():
    codes = np.array([0x0000, 0x8000, 0x3F80, 0xC000, 0x3F81, 0x0001, 0x0080, 0x7F7F, 0x7F80, 0xFF80],
                     dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, 2.0 ** -126,
            (2.0 - 2.0 ** -7) * 2.0 ** 127, np.inf, -np.inf]
    got = bf16_decode(codes)
    assert got.dtype == np.float64
    assert list(got) == want
    assert np.signbit(got[1])


def test_every_code_matches_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()
