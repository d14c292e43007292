"""Pins for the oracle's compensation variants (CPU only): the residual of
the selected channels quantized a second time to NVFP4 before it is added
back (gist.science technical summary §2.2 B, 'second-pass quantization'),
and the compensation strength as a function of k."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import nvfp4 as Q
from tests import exact


def _bf16(a):
    return F.round_to_bf16(np.asarray(a, dtype=np.float64))


def _problem(rng, M, N, K, heavy=True):
    x = rng.standard_t(3, size=(M, K)) if heavy else rng.standard_normal((M, K))
    x = _bf16(x * rng.lognormal(0, 1, size=K)[None, :])
    w = _bf16(rng.standard_normal((1, N, K)) * 0.02)
    return x, w


def _rownorm_err(y, ref):
    return np.max(np.linalg.norm(y - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300))


def test_residual_qdq_matches_exact_rederivation():
    # codes and scales come from the block recipe applied to R_S as a tensor
    # of its own (its own amax), and r^ is one float32 product q*s*g rounded
    # once to bf16
    rng = np.random.default_rng(40)
    x, _ = _problem(rng, 6, 8, 128)
    qa = Q.quantize_activation(x, 32)
    R = qa["R_S"]
    codes, scales, g, r_hat = Q.qdq_residual(R)
    Af = max(abs(Fraction(float(v))) for v in R.ravel())
    assert Fraction(float(g)) == exact.to_f32(Af / 2688)
    for i in range(6):
        for b in range(2):
            blk = [Fraction(float(v)) for v in R[i, 16 * b:16 * b + 16]]
            c, s = exact.quantize_block_exact(blk, Af)
            assert scales[i, b] == s
            assert [int(v) & 7 for v in codes[i, 16 * b:16 * b + 16]] == [v & 7 for v in c]
            sv = exact.e4m3_values()[s]
            for j in range(16):
                q = exact.E2M1_MAGS[c[j] & 7] * (-1 if blk[j] < 0 else 1)
                want = exact.to_bf16(exact.to_f32(q * sv * Fraction(float(g))))
                assert Fraction(float(r_hat[i, 16 * b + j])) == want


def test_residual_qdq_error_bound():
    # |r - r^| <= half an E2M1 gap at |r|/(s g), times s g (up to the float32
    # rounding of the recipe), plus the final bf16 rounding of r^
    rng = np.random.default_rng(41)
    x, _ = _problem(rng, 64, 8, 512)
    R = Q.quantize_activation(x, 128)["R_S"]
    codes, scales, g, r_hat = Q.qdq_residual(R)
    s = np.repeat(F.e4m3_decode(scales), 16, axis=1)
    sg = s * np.float64(g)
    v = np.abs(R) / np.where(sg > 0, sg, 1)
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    bound = sg * half_gap * (1 + 2 ** -18) + np.abs(r_hat) * 2 ** -8 + 1e-300
    assert np.all(np.abs(R - r_hat) <= bound)
    # and it is a real approximation, not a copy
    assert 0 < np.count_nonzero(R != r_hat) < R.size


def test_residual_qdq_is_a_fixed_point():
    # feeding r^ back through the same QDQ gives r^ again on blocks whose
    # scale is an E4M3 normal (the tensor amax is preserved exactly)
    rng = np.random.default_rng(42)
    x, _ = _problem(rng, 32, 8, 256, heavy=False)
    R = Q.quantize_activation(x, 64)["R_S"]
    c0, s0, g0, r0 = Q.qdq_residual(R)
    c1, s1, g1, r1 = Q.qdq_residual(r0)
    assert g1 == g0
    normal = np.repeat(s0 >= 0x08, 16, axis=1)
    assert normal.mean() > 0.9
    assert np.array_equal(r1[normal], r0[normal])


def test_residual_qdq_sign_symmetry_and_scale_invariance():
    rng = np.random.default_rng(43)
    x, _ = _problem(rng, 16, 8, 128)
    R = Q.quantize_activation(x, 32)["R_S"]
    _, _, g0, r0 = Q.qdq_residual(R)
    _, _, g1, r1 = Q.qdq_residual(-R)
    assert g1 == g0 and np.array_equal(r1, -r0)
    _, _, g2, r2 = Q.qdq_residual(R * 2.0 ** -7)
    assert g2 == np.float32(g0 * 2.0 ** -7) and np.array_equal(r2, r0 * 2.0 ** -7)


def test_gemm_with_quantized_residual_is_linear_and_between_the_extremes():
    # y = bf16(X^ W^ + R^_S W^_S): the correction enters linearly; its error
    # against the W4A16 product X W^ lies between the plain W4A4 GEMM's and
    # the bf16 residual's (every channel selected)
    rng = np.random.default_rng(44)
    x, w = _problem(rng, 48, 40, 256)
    qa = Q.quantize_activation(x, 256)
    wc, ws, gw, _ = Q.qdq_weights(w)
    _, _, _, r_hat = Q.qdq_residual(qa["R_S"])
    args = (qa["codes"], qa["scales"], qa["g"], None)
    y2 = G.grouped_gemm_rac(*args, r_hat, qa["S"], wc, ws, gw, [0, 48])
    y1 = G.grouped_gemm_rac(*args, qa["R_S"], qa["S"], wc, ws, gw, [0, 48])
    y0 = G.grouped_gemm_rac(*args, None, [], wc, ws, gw, [0, 48])
    w_hat = Q.dequantize(wc[0], ws[0], gw[0])
    x_hat = Q.dequantize(qa["codes"], qa["scales"], qa["g"])
    assert np.array_equal(y2, _bf16(x_hat @ w_hat.T + r_hat @ w_hat[:, qa["S"]].T))
    ref = _bf16(x @ w_hat.T)
    e0, e1, e2 = (np.linalg.norm(y - ref) / np.linalg.norm(ref) for y in (y0, y1, y2))
    assert e1 < e2 < e0
    assert e2 < e0 / 4           # the second pass keeps most of the gain


@pytest.mark.parametrize("k", [16, 48])
def test_quantized_residual_on_a_k_subset(k):
    # the second pass quantizes the gathered [M][k] tensor, blocks of 16
    # running along the selected channels in ascending channel order
    rng = np.random.default_rng(45 + k)
    x, _ = _problem(rng, 24, 8, 128)
    qa = Q.quantize_activation(x, k)
    codes, scales, g, r_hat = Q.qdq_residual(qa["R_S"])
    assert codes.shape == (24, k) and scales.shape == (24, k // 16)
    c_ref, s_ref, g_ref, _ = Q.quantize(qa["r"][:, qa["S"]])
    assert np.array_equal(codes, c_ref) and np.array_equal(scales, s_ref) and g == g_ref
    assert np.array_equal(r_hat, Q.fake_quant(c_ref, s_ref, g_ref))


# ---------------------------------------------------------- W4A16 forward

def test_w4a16_matches_exact_rational_sum():
    rng = np.random.default_rng(50)
    x, w = _problem(rng, 3, 4, 64)
    wc, ws, gw, _ = Q.qdq_weights(w)
    y = G.grouped_gemm_w4a16(x, None, wc, ws, gw, [0, 3])
    g0 = Fraction(float(gw[0]))
    for m in range(3):
        for n in range(4):
            acc = Fraction(0)
            for kk in range(64):
                wv = (Fraction(float(F.e2m1_decode(wc[0, n, kk])))
                      * Fraction(float(F.e4m3_decode(ws[0, n, kk // 16]))) * g0)
                acc += Fraction(float(x[m, kk])) * wv
            assert Fraction(float(y[m, n])) == exact.to_bf16(acc)


def test_w4a16_equals_w4a4_on_nvfp4_exact_activations():
    # activations that are their own NVFP4 dequantization (tensor amax
    # 2688 * 2^-10, so g = 2^-10 and every q*s*g is a bf16 value): the W4A16
    # product and the plain W4A4 GEMM are then the same sum
    rng = np.random.default_rng(51)
    x0, w = _problem(rng, 40, 24, 256, heavy=False)
    x0 = x0 / np.abs(x0).max() * (2688 * 2.0 ** -10)
    x0 = _bf16(x0)
    assert np.abs(x0).max() == 2688 * 2.0 ** -10
    c, s, g, A = Q.quantize(x0)
    assert g == np.float32(2.0 ** -10)
    x = Q.dequantize(c, s, g)
    assert np.array_equal(_bf16(x), x)
    c1, s1, g1, _ = Q.quantize(x)
    assert g1 == g and np.array_equal(s1, s)
    wc, ws, gw, _ = Q.qdq_weights(w)
    y16 = G.grouped_gemm_w4a16(x, None, wc, ws, gw, [0, 40])
    y4 = G.grouped_gemm_rac(c1, s1, g1, None, None, [], wc, ws, gw, [0, 40])
    assert np.array_equal(y16, y4)


def test_w4a16_grouped_gather_and_the_compensation_limit():
    rng = np.random.default_rng(52)
    x, _ = _problem(rng, 20, 16, 128)
    w = _bf16(rng.standard_normal((3, 16, 128)) * 0.02)
    wc, ws, gw, _ = Q.qdq_weights(w)
    offs = [0, 9, 9, 31]
    a_rows = rng.integers(0, 20, 31)
    y = G.grouped_gemm_w4a16(x, a_rows, wc, ws, gw, offs)
    for e, (lo, hi) in enumerate(zip(offs[:-1], offs[1:])):
        if lo == hi:
            continue
        w_hat = Q.dequantize(wc[e], ws[e], gw[e])
        assert np.array_equal(y[lo:hi], _bf16(x[a_rows[lo:hi]] @ w_hat.T))
    # compensating every channel approaches the W4A16 product (bf16 residual)
    qa = Q.quantize_activation(x, 128)
    yk = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, qa["R_S"], qa["S"],
                            wc, ws, gw, offs)
    y0 = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, None, [], wc, ws, gw, offs)
    assert _rownorm_err(yk, y) <= 2e-3 < _rownorm_err(y0, y)


# ------------------------------------------------- per-expert selection

def _routed(rng, M_src, counts):
    offs = np.zeros(len(counts) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(counts)
    a_rows = rng.integers(0, M_src, int(offs[-1]))
    return offs, a_rows


def test_per_expert_selection_with_one_expert_is_the_shared_selection():
    rng = np.random.default_rng(60)
    x, _ = _problem(rng, 48, 8, 256)
    qa = Q.quantize_activation(x, 40)
    S, R, score = Q.select_channels_per_expert(x, qa["codes"], qa["scales"], qa["g"], qa["A"],
                                               None, [0, 48], 40)
    assert np.array_equal(score[0], qa["score"])
    assert np.array_equal(S[0], qa["S"]) and np.array_equal(R, qa["R_S"])


def test_per_expert_scores_exact_and_dominant():
    rng = np.random.default_rng(61)
    x, _ = _problem(rng, 30, 8, 64)
    codes, scales, g, A = Q.quantize(x)
    offs, a_rows = _routed(rng, 30, [11, 0, 25, 7])
    S, R, score = Q.select_channels_per_expert(x, codes, scales, g, A, a_rows, offs, 9)
    r = Q.residual(x, codes, scales, g)
    m, E_A = np.frexp(float(A))
    for e in (0, 2, 3):
        t = a_rows[offs[e]:offs[e + 1]]
        for j in (0, 5, 40, 63):
            want = sum(int((abs(Fraction(float(r[i, j]))) * Fraction(2) ** (31 - E_A)).__floor__())
                       for i in t)
            assert int(score[e, j]) == want
        sel = set(S[e].tolist())
        for a in sel:
            for b in set(range(64)) - sel:
                assert score[e, a] > score[e, b] or (score[e, a] == score[e, b] and a < b)
        assert np.array_equal(R[offs[e]:offs[e + 1]], r[t][:, S[e]])
        # the order of an expert's rows does not matter
        perm = rng.permutation(t.size)
        a2 = a_rows.copy()
        a2[offs[e]:offs[e + 1]] = t[perm]
        S2, _, sc2 = Q.select_channels_per_expert(x, codes, scales, g, A, a2, offs, 9)
        assert np.array_equal(S2, S) and np.array_equal(sc2, score)
    # an expert with no rows scores zero everywhere and takes channels 0..k-1
    assert not score[1].any() and list(S[1]) == list(range(9))


def test_per_expert_gemm_with_a_common_set_is_the_shared_gemm():
    rng = np.random.default_rng(62)
    x, _ = _problem(rng, 40, 8, 128)
    w = _bf16(rng.standard_normal((3, 16, 128)) * 0.02)
    wc, ws, gw, _ = Q.qdq_weights(w)
    offs, a_rows = _routed(rng, 40, [13, 20, 9])
    qa = Q.quantize_activation(x, 24)
    y_shared = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, qa["R_S"], qa["S"],
                                  wc, ws, gw, offs)
    S_E = np.tile(qa["S"], (3, 1))
    y_pe = G.grouped_gemm_rac_per_expert(qa["codes"], qa["scales"], qa["g"], a_rows,
                                         qa["R_S"][a_rows], S_E, wc, ws, gw, offs)
    assert np.array_equal(y_pe, y_shared)
    # with each expert's own channels, the correction is linear in R_P
    S, R, _ = Q.select_channels_per_expert(x, qa["codes"], qa["scales"], qa["g"], qa["A"], a_rows,
                                           offs, 24)
    y = G.grouped_gemm_rac_per_expert(qa["codes"], qa["scales"], qa["g"], a_rows, R, S, wc, ws, gw,
                                      offs)
    x_hat = Q.dequantize(qa["codes"], qa["scales"], qa["g"])
    for e in range(3):
        p = np.arange(offs[e], offs[e + 1])
        w_hat = Q.dequantize(wc[e], ws[e], gw[e])
        assert np.array_equal(y[p], _bf16(x_hat[a_rows[p]] @ w_hat.T + R[p] @ w_hat[:, S[e]].T))
