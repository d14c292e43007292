"""Pins for the oracle's NVFP4 quantizer, residual, channel scores and
selection (CPU only)."""
from fractions import Fraction
import itertools

import numpy as np
import pytest

from oracle import formats as F
from oracle import nvfp4 as Q
from tests import exact


def _bf16_values(a):
    return F.round_to_bf16(np.asarray(a, dtype=np.float64))


def _rand_x(rng, M, K, heavy=True):
    x = rng.standard_t(3, size=(M, K)) if heavy else rng.standard_normal((M, K))
    x *= rng.lognormal(0, 1, size=K)[None, :]
    x = _bf16_values(x)
    x[x == 0] = 0.0            # no negative zeros: Fractions carry no zero sign
    return x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_matches_exact_rational_rederivation(seed):
    rng = np.random.default_rng(seed)
    x = _rand_x(rng, 3, 48)
    codes, scales, g, A = Q.quantize(x)
    Af = Fraction(float(np.abs(x).max()))
    assert Fraction(float(A)) == Af
    assert Fraction(float(g)) == exact.to_f32(Af / 2688)
    for i in range(3):
        for b in range(3):
            blk = [Fraction(float(v)) for v in x[i, 16 * b:16 * b + 16]]
            c, s = exact.quantize_block_exact(blk, Af)
            assert scales[i, b] == s
            assert list(codes[i, 16 * b:16 * b + 16]) == c


def test_hand_worked_block():
    # One block, worked by hand.  A = 6 (the block max), so
    #   u = 6*448/6 = 448 -> s = 448 (0x7E);  s*A = 2688;  rho = 2688/2688 = 1
    #   v = x, and the codes are the E2M1 roundings of x itself.
    x = np.array([[6, -0.3, 0.25, 0.75, 1.25, 1.75, 2.5, -3.5, 5, 4.9, 0, 1, 2, 3, 4, -6]],
                 dtype=np.float64)
    codes, scales, g, A = Q.quantize(x)
    assert A == 6 and scales[0, 0] == 0x7E
    assert g == np.float32(6 / 2688)
    want = [0x7, 0x9, 0x0, 0x2, 0x2, 0x4, 0x4, 0xE, 0x6, 0x6, 0x0, 0x2, 0x4, 0x5, 0x6, 0xF]
    assert list(codes[0]) == want
    # second worked block: A = 8 elsewhere in the tensor, block max 1
    #   u = 448/8 = 56 = 1.75 * 2**5 -> exponent field 12, mantissa 6 -> s = 0x66
    #   s*A = 448;  rho = 2688/448 = 6
    #   v = 6x: x = 1 -> 6 (code 7), x = 0.5 -> 3 (5), x = 0.3 -> 1.8 (4), x = 0.05 -> 0.3 (1)
    x2 = np.zeros((1, 32))
    x2[0, 0] = 8.0
    x2[0, 16:20] = [1.0, 0.5, -0.300048828125, 0.0500488281250]   # bf16-exact values
    codes, scales, g, A = Q.quantize(x2)
    assert scales[0, 1] == 0x66 and F.e4m3_decode(np.uint8(0x66)) == 56
    assert list(codes[0, 16:20]) == [0x7, 0x5, 0xC, 0x1]


def test_block_max_maps_to_six_when_scale_is_normal():
    rng = np.random.default_rng(5)
    x = _rand_x(rng, 64, 256)
    codes, scales, g, A = Q.quantize(x)
    xb = np.abs(x).reshape(64, 16, 16)
    cb = codes.reshape(64, 16, 16)
    normal = scales >= 0x08
    imax = xb.argmax(axis=-1)
    cmax = np.take_along_axis(cb, imax[..., None], axis=-1)[..., 0] & 7
    assert normal.sum() > 500
    assert np.all(cmax[normal] == 7)


def test_dequantization_error_bound():
    # |x - x^| <= s*g*(half grid gap at |v|) up to float32 rounding of rho/g
    rng = np.random.default_rng(6)
    x = _rand_x(rng, 64, 512)
    codes, scales, g, A = Q.quantize(x)
    xh = Q.dequantize(codes, scales, g)
    s = np.repeat(F.e4m3_decode(scales), 16, axis=1)
    v = np.abs(x) / (s * np.float64(g))
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    bound = s * np.float64(g) * half_gap * (1 + 2 ** -18) + 1e-300
    assert np.all(np.abs(x - xh) <= bound)


def test_scale_invariance_by_powers_of_two():
    rng = np.random.default_rng(7)
    x = _rand_x(rng, 16, 128)
    c0, s0, g0, _ = Q.quantize(x)
    for j in (-5, 3, 11):
        c1, s1, g1, _ = Q.quantize(x * 2.0 ** j)
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert g1 == np.float32(g0 * 2.0 ** j)


def test_sign_symmetry_and_row_permutation():
    rng = np.random.default_rng(8)
    x = _rand_x(rng, 16, 128)
    c0, s0, g0, _ = Q.quantize(x)
    c1, s1, g1, _ = Q.quantize(-x)
    nz = x != 0
    assert np.array_equal(c1[nz], c0[nz] ^ 8) and np.array_equal(s0, s1) and g0 == g1
    p = rng.permutation(16)
    c2, s2, g2, _ = Q.quantize(x[p])
    assert np.array_equal(c2, c0[p]) and np.array_equal(s2, s0[p]) and g2 == g0


def test_qdq_idempotence_on_normal_scale_blocks():
    rng = np.random.default_rng(9)
    x = _rand_x(rng, 32, 256, heavy=False)
    c0, s0, g0, _ = Q.quantize(x)
    xq = _bf16_values(Q.dequantize(c0, s0, g0))
    c1, s1, g1, _ = Q.quantize(xq)
    assert g1 == g0
    normal = np.repeat(s0 >= 0x08, 16, axis=1)
    assert np.array_equal(s1[s0 >= 0x08], s0[s0 >= 0x08])
    assert np.array_equal((c1 & 7)[normal], (c0 & 7)[normal])


def test_zero_tensor_and_zero_block():
    codes, scales, g, A = Q.quantize(np.zeros((2, 32)))
    assert A == 0 and g == 0 and not codes.any() and not scales.any()
    x = np.zeros((1, 32))
    x[0, 0] = 1.0
    codes, scales, g, A = Q.quantize(x)
    assert scales[0, 1] == 0 and not codes[0, 16:].any()


def test_residual_matches_exact_rederivation():
    rng = np.random.default_rng(10)
    x = _rand_x(rng, 4, 64)
    codes, scales, g, A = Q.quantize(x)
    r = Q.residual(x, codes, scales, g)
    for i in range(4):
        for j in range(64):
            q = Fraction(float(F.e2m1_decode(codes[i, j])))
            s = Fraction(float(F.e4m3_decode(scales[i, j // 16])))
            want = exact.to_bf16(exact.to_f32(Fraction(float(x[i, j])) - q * s * Fraction(float(g))))
            assert Fraction(float(r[i, j])) == want


def test_scores_exact_and_order_free():
    rng = np.random.default_rng(11)
    x = _rand_x(rng, 40, 64)
    codes, scales, g, A = Q.quantize(x)
    r = Q.residual(x, codes, scales, g)
    sc = Q.channel_scores(r, A)
    m, E = np.frexp(float(A))
    assert 0.5 <= m < 1
    for j in (0, 7, 33, 63):
        want = sum(int((abs(Fraction(float(r[i, j]))) * Fraction(2) ** (31 - E)).__floor__())
                   for i in range(40))
        assert int(sc[j]) == want
    p = rng.permutation(40)
    assert np.array_equal(Q.channel_scores(r[p], A), sc)


def test_select_ties_lower_index_and_dominance():
    score = np.array([5, 9, 9, 1, 9, 0, 5, 7], dtype=np.uint64)
    assert list(Q.select_channels(score, 2)) == [1, 2]
    assert list(Q.select_channels(score, 3)) == [1, 2, 4]
    assert list(Q.select_channels(score, 5)) == [0, 1, 2, 4, 7]
    assert list(Q.select_channels(score, 0)) == []
    assert list(Q.select_channels(score, 8)) == list(range(8))
    rng = np.random.default_rng(12)
    for _ in range(50):
        s = rng.integers(0, 6, 12).astype(np.uint64)
        k = int(rng.integers(0, 13))
        S = set(Q.select_channels(s, k).tolist())
        assert len(S) == k
        for a, b in itertools.product(S, set(range(12)) - S):
            assert s[a] > s[b] or (s[a] == s[b] and a < b)


def test_duplicated_channels_tie_to_lower_index():
    # block 2 is an exact copy of block 0, so channels j and j+32 have equal
    # residuals in every row and hence equal scores: the lower index must win
    rng = np.random.default_rng(13)
    x = _rand_x(rng, 32, 64)
    x[:, 32:48] = x[:, 0:16]
    qa = Q.quantize_activation(x, 64)
    assert np.array_equal(qa["score"][32:48], qa["score"][0:16])
    for k in range(0, 65):
        S = set(Q.select_channels(qa["score"], k).tolist())
        for j in range(16):
            assert not (j + 32 in S and j not in S)


def test_pack_roundtrip_and_nibble_order():
    c = np.array([[0x1, 0x2, 0xF, 0x8]], dtype=np.uint8)
    p = Q.pack_codes(c)
    assert list(p[0]) == [0x21, 0x8F]
    assert np.array_equal(Q.unpack_codes(p), c)


def test_weight_qdq_is_trainer_fake_quant():
    rng = np.random.default_rng(14)
    w = _bf16_values(rng.standard_normal((3, 8, 64)) * 0.02)
    codes, scales, g_w, w_qdq = Q.qdq_weights(w)
    for e in range(3):
        c, s, g, _ = Q.quantize(w[e])
        assert np.array_equal(codes[e], c) and g_w[e] == g
        # w_qdq is one float32 product rounded once to bf16
        qs = [Fraction(float(v)) for v in Q.dequantize_unscaled(c, s).ravel()]
        want = [exact.to_bf16(exact.to_f32(v * Fraction(float(g)))) for v in qs]
        assert [Fraction(float(v)) for v in w_qdq[e].ravel()] == want
    # the fake-quantized weight is a fixed point of QDQ (same codes and scales)
    c2, s2, g2, w2 = Q.qdq_weights(w_qdq)
    assert np.array_equal(g2, g_w)
    ok = np.repeat(scales >= 0x08, 16, axis=-1)
    assert np.array_equal((c2 & 7)[ok], (codes & 7)[ok])


def test_quantize_slices_with_given_amax_match_whole_tensor():
    rng = np.random.default_rng(15)
    x = _rand_x(rng, 24, 96)
    codes, scales, g, A = Q.quantize(x)
    c1, s1, g1, _ = Q.quantize(x[5:11], A=A)                       # a row slice
    assert np.array_equal(c1, codes[5:11]) and np.array_equal(s1, scales[5:11]) and g1 == g
    c2, s2, _, _ = Q.quantize(x[:, 32:64], A=A)                    # a column-block slice
    assert np.array_equal(c2, codes[:, 32:64]) and np.array_equal(s2, scales[:, 2:4])
    with pytest.raises(ValueError):
        Q.quantize(x, A=A / 2)
