"""GPU parity of dsa_quantize_fp8 against the oracle's quantiser: codes and
scales must be bit-exact (integer / byte work)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_dsa_amd as dsa
from gpu_util import banner

pytestmark = pytest.mark.gpu


def run(x):
    xd = torch.from_numpy(x).cuda()
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    dsa.dsa_quantize_fp8(xd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("cols", [64, 128, 256, 512])
def test_random_rows_bit_exact(cols):
    banner(f"quantize random rows cols={cols}")
    rng = np.random.default_rng(cols)
    x = rng.standard_normal((3001, cols)).astype(np.float32)
    x[::7] *= 1e-3
    x[::11] *= 1e3
    codes, scales = run(x)
    rc, rs = oracle.quantize_rows(x)
    assert (scales.view(np.uint32) == rs.view(np.uint32)).all()
    mism = (codes != rc).sum()
    assert mism == 0, f"{mism} codes differ"


def test_special_rows_bit_exact():
    banner("quantize special rows")
    rng = np.random.default_rng(5)
    rows = [
        np.zeros(128, np.float32),                         # all zero -> scale 1
        -np.zeros(128, np.float32),                        # all -0
        np.full(128, 3.0, np.float32),                     # constant row
        np.linspace(-1, 1, 128).astype(np.float32),
        (rng.standard_normal(128) * 1e-30).astype(np.float32),  # tiny magnitudes
        np.concatenate([[1.0], rng.standard_normal(127) * 1e-4]).astype(np.float32),  # subnormal codes
        np.concatenate([[448.0], np.arange(127) * 3.5]).astype(np.float32),  # exact grid points
    ]
    # values whose quotient lands exactly on midpoints of the E4M3 grid (scale = 1 when absmax = 448)
    grid = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    mid_rows = np.concatenate([mids, -mids, np.zeros(256 - 2 * mids.size, np.float32)]).reshape(2, 128)
    mid_rows[:, 0] = 448.0
    x = np.vstack(rows + [mid_rows]).astype(np.float32)
    x[1] = -0.0
    codes, scales = run(x)
    rc, rs = oracle.quantize_rows(x)
    assert (scales.view(np.uint32) == rs.view(np.uint32)).all()
    assert (codes == rc).all(), np.argwhere(codes != rc)[:10]


def run_e8m0(x, with_scales=True):
    xd = torch.from_numpy(x).cuda()
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    e8m0 = torch.empty(x.shape[0], dtype=torch.uint8, device="cuda")
    scales = torch.empty(x.shape[0], dtype=torch.float32, device="cuda") if with_scales else None
    dsa.dsa_quantize_fp8_e8m0(xd, codes, e8m0, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), e8m0.cpu().numpy(), (scales.cpu().numpy() if with_scales else None)


@pytest.mark.parametrize("cols", [64, 128, 512])
def test_e8m0_random_rows_bit_exact(cols):
    banner(f"quantize e8m0 random rows cols={cols}")
    rng = np.random.default_rng(100 + cols)
    x = rng.standard_normal((3001, cols)).astype(np.float32)
    x *= (np.float32(2.0) ** rng.integers(-60, 60, size=(3001, 1))).astype(np.float32)
    codes, b, scales = run_e8m0(x)
    rc, rb, rs = oracle.quantize_rows_e8m0(x)
    assert (b == rb).all(), np.argwhere(b != rb)[:10]
    assert (scales.astype(np.float64) == rs).all()
    assert (codes == rc).all(), f"{(codes != rc).sum()} codes differ"


def test_e8m0_special_rows_bit_exact():
    banner("quantize e8m0 special rows")
    x = np.zeros((8, 64), np.float32)
    x[0, 3] = 448.0                                   # e = 0, code 0x7E
    x[1, 5] = np.float32(448.0 * 2.0 ** 10)           # exactly 448 * 2^10
    x[2, 7] = np.nextafter(np.float32(448.0 * 2.0 ** -5), np.float32(np.inf))  # just above a boundary
    x[3] = -0.0                                       # all -0: e = 0, codes 0x80
    x[4, 0] = np.float32(1e-40)                       # subnormal absmax: exponent clamped at -127
    x[5, 1] = np.float32(-3e38)                       # near the fp32 maximum
    x[6] = np.linspace(-7, 7, 64).astype(np.float32)  # m > 1.75 case (absmax 7 = 1.75 * 4)
    x[7] = np.linspace(-7.5, 7.5, 64).astype(np.float32)
    codes, b, scales = run_e8m0(x)
    rc, rb, rs = oracle.quantize_rows_e8m0(x)
    assert (b == rb).all() and (scales.astype(np.float64) == rs).all()
    assert (codes == rc).all(), np.argwhere(codes != rc)[:10]
    codes2, b2, _ = run_e8m0(x, with_scales=False)    # scales are optional
    assert (codes2 == codes).all() and (b2 == b).all()
