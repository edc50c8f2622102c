"""OCP FP8 E4M3 ("e4m3fn") codec and per-row quantiser, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Where the pages stand: the lightning indexer runs in FP8 (page "arXiv'25 | DSA ...
DeepSeek-V3.2" on marsggbo.github.io, section 3; page "DeepSeekV3.2之DSA" on
yuyanqi.com, part 4.3: FP8 q times FP8 k into fp32 logits, with a per-key scale
applied after the head sum).  The pages fix neither the FP8 variant nor the
rounding rule nor the scale rule.  Readings taken here:

* variant: E4M3 with a maximum of 448 and no infinities (the OCP "fn" variant),
  the only E4M3 flavour whose maximum is 448;
* scale per row: fp32(absmax(row)) / 448 as an IEEE fp32 division; an all-zero
  row gets scale 1 (its codes are all zero);
* code = E4M3(fp32(x) / scale): the fp32 division first, then
  round-to-nearest-even onto the E4M3 grid, saturating at +-448; the sign of a
  result that rounds to zero is kept (0x80 for negative inputs).

Decode of code c = S.EEEE.MMM:
    E > 0 : (-1)^S * 2^(E-7) * (1 + M/8)
    E = 0 : (-1)^S * 2^-6   * (M/8)
    S.1111.111 is NaN (never produced by the encoder).
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode E4M3fn codes (uint8 array) to float64 with the closed form above."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = np.ldexp(1.0 + man / 8.0, (exp - 7).astype(np.int64))
    subnormal = np.ldexp(man / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    val = np.where(sign == 1, -mag, mag)
    return np.where((exp == 15) & (man == 7), np.nan, val)


def _positive_grid():
    """All finite non-negative E4M3fn values, indexed by their code 0..126."""
    return e4m3_decode(np.arange(127, dtype=np.uint8))


_GRID = _positive_grid()  # strictly increasing in the code


def e4m3_encode(x):
    """Round float values onto the E4M3fn grid: nearest value, ties to the even
    code (even mantissa), saturating at +-448.  Input is taken as float64 (an
    fp32 input is represented exactly).  NaN input is rejected."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no E4M3 encoding in this reading")
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_GRID, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _GRID[hi], hi, code)  # exact hits
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


E8M0_BIAS = 127


def e8m0_decode(b):
    """E8M0 byte (an 8-bit biased exponent, no sign or mantissa) to its float64
    value 2^(b - 127).  255 is NaN in the format and is rejected here."""
    b = np.asarray(b, dtype=np.int64)
    if (b == 255).any():
        raise ValueError("E8M0 255 is NaN")
    return np.ldexp(1.0, b - E8M0_BIAS)


def quantize_rows_e8m0(x):
    """Per-row FP8 quantisation with a power-of-two scale per row, the E8M0 key
    scale of page "DeepSeekV3.2之DSA", part 4.3 (the last step multiplies the head
    sum by k_s in e8m0).  The page does not give the rule that picks the
    exponent; the reading taken here is the smallest power of two that keeps
    every |x| / scale within 448, so no code saturates:

        e     = min { e integer : absmax(row) <= 448 * 2^e }, clamped to [-127, 127]
                (e = 0 for an all-zero row)
        scale = 2^e                      (exact in fp32 and float64)
        code  = E4M3(x / 2^e)            (an exact division, then round to nearest-even)
        byte  = e + 127

    Returns (codes uint8 [N, D], bytes uint8 [N], scales float64 [N])."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if x32.ndim != 2:
        raise ValueError("quantize_rows_e8m0 expects a 2-D array")
    amax = np.max(np.abs(x32.astype(np.float64)), axis=1) if x32.shape[1] else np.zeros(x32.shape[0])
    exps = np.zeros(x32.shape[0], np.int64)
    for i, a in enumerate(amax):
        if a == 0.0:
            continue
        # Start from a float estimate, then settle it with exact comparisons
        # (448 * 2^e is exact in float64 over the whole range).
        e = int(np.ceil(np.log2(a / E4M3_MAX)))
        while a > np.ldexp(E4M3_MAX, e):
            e += 1
        while a <= np.ldexp(E4M3_MAX, e - 1):
            e -= 1
        exps[i] = min(max(e, -E8M0_BIAS), E8M0_BIAS)
    scale = np.ldexp(1.0, exps)
    y = x32.astype(np.float64) / scale[:, None]
    return e4m3_encode(y), (exps + E8M0_BIAS).astype(np.uint8), scale


def quantize_rows(x):
    """Per-row FP8 quantisation of an fp32 matrix [N, D].

    Returns (codes uint8 [N, D], scales float32 [N]) with
    scale = fp32(absmax / 448) (1 for an all-zero row) and
    code = E4M3(fp32(x / scale))."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if x32.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D array")
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (x32 / scale[:, None]).astype(np.float32)
    return e4m3_encode(y), scale
