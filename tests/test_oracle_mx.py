"""Pins of the MX-FP8 quantization oracle (CPU).

- E4M3 rounding equals torch's float8_e4m3fn conversion (round to nearest
  even) on every in-range value tried, including all 254 finite code points
  and the midpoints between neighbours.
- Closed forms: code points are fixed points; ties go to the even mantissa;
  magnitudes past 448 clamp to 448.
- Block scales: the block maximum lands in [256, 448]; scaling a block by 2^k
  shifts its exponent by k and leaves its elements; powers of two and zero
  blocks round-trip exactly; the error of every element is at most half a
  unit in the last place of its E4M3 binade times the block scale.
"""
import numpy as np
import torch

from oracle import mx_fp8 as M


def _code_points():
    u = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    v = u.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.unique(v[np.isfinite(v)])


def test_code_points_are_fixed_and_match_torch_cast():
    cp = _code_points()
    assert len(cp) == 253 and cp.max() == 448.0     # +-0 collapse: 254 codes, 253 values
    np.testing.assert_array_equal(M.round_e4m3(cp), cp)
    mids = (cp[1:] + cp[:-1]) / 2
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(M.round_e4m3(mids), ref)


def test_random_values_match_torch_cast():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000))
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(M.round_e4m3(x), ref)


def test_ties_to_even_and_clamp():
    # 1 + 1/16 lies halfway between 1 and 1.125: even mantissa is 1.0
    assert M.round_e4m3(1.0625) == 1.0
    assert M.round_e4m3(1.1875) == 1.25
    assert M.round_e4m3(-1.0625) == -1.0
    assert M.round_e4m3(460.0) == 448.0 and M.round_e4m3(-1e9) == -448.0
    assert M.round_e4m3(2.0 ** -10) == 0.0          # half of the smallest subnormal: even -> 0
    assert M.round_e4m3(3 * 2.0 ** -10) == 2.0 ** -8


def test_block_scales():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 96)) * np.exp2(rng.integers(-20, 20, (7, 96)))
    P, X = M.mx_quantize(x)
    Pb = np.abs(P.reshape(7, 3, 32)).max(-1)
    assert np.all((Pb >= 256) & (Pb <= 448))
    P2, X2 = M.mx_quantize(x * 2.0 ** 5)
    np.testing.assert_array_equal(P2, P)
    np.testing.assert_array_equal(X2, X + 5)
    # error bound: half an E4M3 ulp of each element, times the block scale
    deq = M.mx_dequantize(P, X)
    s = np.repeat(2.0 ** X, 32, axis=-1)
    a = np.abs(x) / s
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1))), -6)
    assert np.all(np.abs(deq - x) <= 0.5 * 2.0 ** (e - 3) * s * (1 + 1e-12) + (a > 448) * (a - 448) * s)


def test_exact_blocks_round_trip():
    x = np.zeros((2, 64))
    x[0, :32] = 2.0 ** np.arange(-10, 22)[:32] / 2 ** 20
    x[0, 32:] = np.linspace(-1, 1, 32) * 0   # zero block
    P, X = M.mx_quantize(x)
    assert X[0, 1] == 0 and np.all(P[0, 32:] == 0)
    np.testing.assert_array_equal(M.mx_dequantize(P, X)[0, 32:], 0)
    # three mantissa bits and binades within the E4M3 range of each block
    rng = np.random.default_rng(2)
    x[1] = rng.choice([-1, 1], 64) * (1 + rng.integers(0, 8, 64) / 8) * 2.0 ** rng.integers(-5, 1, 64)
    P, X = M.mx_quantize(x[1:])
    np.testing.assert_array_equal(M.mx_dequantize(P, X), x[1:])


def test_fp8_projection_of_representable_operands_is_exact():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, (5, 64)).astype(np.float64)
    w = rng.integers(-8, 9, (6, 64)).astype(np.float64) / 4
    np.testing.assert_array_equal(M.output_projection_mxfp8(x, w), x @ w.T)
