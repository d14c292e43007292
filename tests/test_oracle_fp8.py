"""Pins for the oracle's FP8 (E4M3) W8A8 baseline (CPU only).

Each test checks the oracle against something it does not compute itself:
PyTorch's float8_e4m3fn conversion (an independent library routine),
exact rational arithmetic, brute-force sums on tiny inputs and closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import fp8 as Q8


def _bf16(a):
    return F.round_to_bf16(np.asarray(a, dtype=np.float64))


def test_codes_match_torch_float8_cast():
    # E4M3(float32(|x| / g)) with the sign bit of x is what torch's
    # float8_e4m3fn cast gives for float32(x / g) (below its NaN threshold,
    # which the scaled values never reach)
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_t(3, size=(64, 96)) * rng.lognormal(0, 2, size=96))
    x[0, :4] = [0.0, -0.0, 1e-30, -1e-30]
    codes, g, A = Q8.quantize(x)
    assert A == np.float32(np.max(np.abs(x)))
    v = torch.from_numpy(x.astype(np.float32)) / torch.tensor(g)
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_amax_maps_to_448_and_scale_is_exact_division():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((8, 32)) * 3.0)
    codes, g, A = Q8.quantize(x)
    q = Fraction(float(A)) / 448
    # g is the float32 nearest to A / 448
    assert abs(Fraction(float(g)) - q) <= abs(Fraction(float(np.nextafter(g, np.float32(1e9)))) - q)
    assert abs(Fraction(float(g)) - q) <= abs(Fraction(float(np.nextafter(g, np.float32(0)))) - q)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] & 0x7F == 0x7E                      # 448
    assert np.all((codes & 0x7F) <= 0x7E)               # never NaN


def test_round_to_nearest_even_on_constructed_ties():
    # With A = 448 and g = 1 the scaled value is x itself.  Between 1 and 2
    # E4M3 steps by 1/8: 1 + 1/16 ties to 1 (even code), 1 + 3/16 to 1.25
    # (code 0x3A, even); 0.75 * 2^-9 (between the subnormal steps 2^-9 and
    # 2 * 2^-9) ... rounds to the nearest multiple of 2^-9
    x = np.array([448.0, 1.0625, 1.1875, -1.0625, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9,
                  2.5 * 2.0 ** -9, 2.0 ** -6 + 2.0 ** -10, 240.0, 232.0])
    codes, g, _ = Q8.quantize(x)
    assert g == np.float32(1.0)
    dec = F.e4m3_decode(codes)
    assert list(dec) == [448.0, 1.0, 1.25, -1.0, 0.0, 2.0 * 2.0 ** -9, 2.0 * 2.0 ** -9,
                         2.0 ** -6, 240.0, 224.0]


def test_error_bound_and_zero_tensor():
    # relative error of a normal-range E4M3 value <= 2^-4; absolute error
    # below the normal range <= 2^-10 * g
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((32, 64)) * rng.lognormal(0, 1.5, size=64))
    codes, g, _ = Q8.quantize(x)
    xh = Q8.dequantize(codes, g)
    normal = np.abs(x) >= 2.0 ** -6 * float(g)
    assert np.all(np.abs(xh - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-6))
    assert np.all(np.abs(xh - x)[~normal] <= 2.0 ** -10 * float(g) * (1 + 1e-6))
    z = np.array([[0.0, -0.0], [0.0, 0.0]])
    cz, gz, Az = Q8.quantize(z)
    assert Az == 0 and gz == 0 and list(cz.ravel()) == [0, 0x80, 0, 0]


def test_stacked_scales_are_per_expert():
    rng = np.random.default_rng(4)
    w = _bf16(rng.standard_normal((3, 16, 32)) * np.array([0.01, 1.0, 100.0])[:, None, None])
    codes, g = Q8.quantize_stacked(w)
    for e in range(3):
        c1, g1, _ = Q8.quantize(w[e])
        assert g[e] == g1 and np.array_equal(codes[e], c1)
    assert g[0] < g[1] < g[2]


def test_grouped_gemm_brute_force_tiny():
    # sums written out term by term in exact rationals, then one rounding
    rng = np.random.default_rng(5)
    M_src, K, N, E = 5, 16, 3, 2
    x = _bf16(rng.standard_normal((M_src, K)))
    w = _bf16(rng.standard_normal((E, N, K)) * 0.1)
    ac, gx, _ = Q8.quantize(x)
    wc, gw = Q8.quantize_stacked(w)
    offs = np.array([0, 3, 6])
    a_rows = np.array([4, 0, 2, 1, 1, 3])
    y = Q8.grouped_gemm_fp8(ac, gx, a_rows, wc, gw, offs)
    av = F.e4m3_decode(ac)
    for p in range(6):
        e = 0 if p < 3 else 1
        wv = F.e4m3_decode(wc[e])
        for n in range(N):
            s = sum(Fraction(float(av[a_rows[p], k])) * Fraction(float(wv[n, k])) for k in range(K))
            s *= Fraction(float(gx)) * Fraction(float(gw[e]))
            assert y[p, n] == F.round_to_bf16(np.float64(s)), (p, n)


def test_grouped_gemm_exact_integer_case_and_empty_expert():
    # values that are E4M3-exact with power-of-two scales: A = 448 * 2^j makes
    # g = 2^j exactly, and the product is the integer matmul times the scales
    rng = np.random.default_rng(6)
    K, N = 64, 8
    a = rng.integers(-8, 9, size=(10, K)).astype(np.float64)
    a[0, 0] = 448.0
    w = rng.integers(-8, 9, size=(3, N, K)).astype(np.float64) * 0.25
    w[:, 0, 0] = 112.0                                   # 448 / 4
    ac, gx, _ = Q8.quantize(a)
    wc, gw = Q8.quantize_stacked(w)
    assert gx == 1.0 and np.all(gw == 0.25)
    offs = np.array([0, 4, 4, 10])                       # expert 1 empty
    y = Q8.grouped_gemm_fp8(ac, gx, None, wc, gw, offs)
    ref = np.concatenate([a[:4] @ w[0].T, a[4:] @ w[2].T])
    assert np.array_equal(y, F.round_to_bf16(ref))


@pytest.mark.parametrize("seed", [7, 8])
def test_grouped_gemm_gather_equals_dense_per_expert(seed):
    rng = np.random.default_rng(seed)
    M_src, K, N, E = 12, 32, 5, 3
    x = _bf16(rng.standard_normal((M_src, K)))
    w = _bf16(rng.standard_normal((E, N, K)))
    ac, gx, _ = Q8.quantize(x)
    wc, gw = Q8.quantize_stacked(w)
    a_rows = rng.integers(0, M_src, size=20)
    offs = np.array([0, 7, 15, 20])
    y = Q8.grouped_gemm_fp8(ac, gx, a_rows, wc, gw, offs)
    xh = Q8.dequantize(ac, gx)
    for e in range(E):
        p = np.arange(offs[e], offs[e + 1])
        ref = F.round_to_bf16(xh[a_rows[p]] @ Q8.dequantize(wc[e], gw[e]).T)
        assert np.array_equal(y[p], ref)
    sub = Q8.grouped_gemm_fp8(ac, gx, a_rows, wc, gw, offs, rows=np.array([3, 16]))
    assert np.array_equal(sub[[3, 16]], y[[3, 16]]) and np.isnan(sub[0]).all()


def test_slice_with_the_tensor_amax_equals_slice_of_the_whole():
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_t(3, size=(40, 64)))
    codes, g, A = Q8.quantize(x)
    c2, g2, _ = Q8.quantize(x[10:17], A=A)
    assert g2 == g and np.array_equal(c2, codes[10:17])
    with pytest.raises(ValueError):
        Q8.quantize(x, A=A / 2)
