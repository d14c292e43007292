"""Pins for the oracle's grouped GEMM with residual compensation, and for
routing, permutation, SwiGLU and combine (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import moe as MOE
from oracle import nvfp4 as Q
from tests import exact


def _bf16(a):
    return F.round_to_bf16(np.asarray(a, dtype=np.float64))


def _problem(rng, M, N, K, E=1, heavy=True):
    x = rng.standard_t(3, size=(M, K)) if heavy else rng.standard_normal((M, K))
    x = _bf16(x * rng.lognormal(0, 1, size=K)[None, :])
    w = _bf16(rng.standard_normal((E, N, K)) * 0.02)
    return x, w


def _rownorm_err(y, ref):
    return np.max(np.linalg.norm(y - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300))


@pytest.mark.parametrize("k", [0, 3, 64])
def test_gemm_matches_exact_rational_sum(k):
    rng = np.random.default_rng(20 + k)
    x, w = _problem(rng, 4, 3, 64)
    qa = Q.quantize_activation(x, k)
    wc, ws, gw, _ = Q.qdq_weights(w)
    y = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], None, qa["R_S"], qa["S"],
                           wc, ws, gw, [0, 4])
    gx, g0 = Fraction(float(qa["g"])), Fraction(float(gw[0]))
    for m in range(4):
        for n in range(3):
            acc = Fraction(0)
            for kk in range(64):
                xv = (Fraction(float(F.e2m1_decode(qa["codes"][m, kk])))
                      * Fraction(float(F.e4m3_decode(qa["scales"][m, kk // 16]))) * gx)
                wv = (Fraction(float(F.e2m1_decode(wc[0, n, kk])))
                      * Fraction(float(F.e4m3_decode(ws[0, n, kk // 16]))) * g0)
                acc += xv * wv
            for jj, j in enumerate(qa["S"]):
                wv = (Fraction(float(F.e2m1_decode(wc[0, n, j])))
                      * Fraction(float(F.e4m3_decode(ws[0, n, j // 16]))) * g0)
                acc += Fraction(float(qa["R_S"][m, jj])) * wv
            assert Fraction(float(y[m, n])) == exact.to_bf16(acc)


def test_all_channels_reproduce_the_w4a16_product():
    # with every channel selected, x^ + r = x up to the bf16 rounding of r, so
    # the result is the trainer's W4A16 forward X @ W^ (W^ = dequantized weight)
    rng = np.random.default_rng(30)
    x, w = _problem(rng, 48, 40, 256)
    qa = Q.quantize_activation(x, 256)
    wc, ws, gw, _ = Q.qdq_weights(w)
    y = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], None, qa["R_S"], qa["S"],
                           wc, ws, gw, [0, 48])
    ref = _bf16(x @ Q.dequantize(wc[0], ws[0], gw[0]).T)
    assert _rownorm_err(y, ref) <= 2e-3
    y0 = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], None, None, [], wc, ws, gw, [0, 48])
    assert _rownorm_err(y0, ref) > 10 * _rownorm_err(y, ref)     # the correction matters


def test_correction_is_linear_in_the_selected_residual():
    rng = np.random.default_rng(31)
    x, w = _problem(rng, 32, 24, 128)
    qa = Q.quantize_activation(x, 16)
    wc, ws, gw, _ = Q.qdq_weights(w)
    args = (qa["codes"], qa["scales"], qa["g"], None)
    yk = G.grouped_gemm_rac(*args, qa["R_S"], qa["S"], wc, ws, gw, [0, 32])
    y0 = G.grouped_gemm_rac(*args, None, [], wc, ws, gw, [0, 32])
    w_hat = Q.dequantize(wc[0], ws[0], gw[0])
    corr = qa["R_S"] @ w_hat[:, qa["S"]].T
    x_hat = Q.dequantize(qa["codes"], qa["scales"], qa["g"])
    assert np.array_equal(yk, _bf16(x_hat @ w_hat.T + corr))
    # and each selected channel's residual really is x - x^ on that channel
    d = (x - x_hat)[:, qa["S"]]
    assert np.all(np.abs(qa["R_S"] - d) <= np.abs(d) * 2 ** -8)
    assert not np.array_equal(yk, y0)


def test_grouped_equals_per_expert_dense_and_gather():
    rng = np.random.default_rng(32)
    x, w = _problem(rng, 20, 16, 64, E=3)
    qa = Q.quantize_activation(x, 8)
    wc, ws, gw, _ = Q.qdq_weights(w)
    offs = [0, 7, 7, 30]                     # expert 1 empty
    a_rows = rng.integers(0, 20, 30)
    y = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, qa["R_S"], qa["S"],
                           wc, ws, gw, offs)
    for e, (lo, hi) in enumerate(zip(offs[:-1], offs[1:])):
        if lo == hi:
            continue
        t = a_rows[lo:hi]
        yd = G.grouped_gemm_rac(qa["codes"][t], qa["scales"][t], qa["g"], None, qa["R_S"][t],
                                qa["S"], wc[e:e + 1], ws[e:e + 1], gw[e:e + 1], [0, hi - lo])
        assert np.array_equal(y[lo:hi], yd)


def test_zero_weights_give_zero():
    rng = np.random.default_rng(33)
    x, _ = _problem(rng, 8, 4, 32)
    qa = Q.quantize_activation(x, 4)
    wc, ws, gw, _ = Q.qdq_weights(np.zeros((1, 4, 32)))
    y = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], None, qa["R_S"], qa["S"],
                           wc, ws, gw, [0, 8])
    assert not np.any(y)


def test_compensation_error_shrinks_with_k_on_average():
    # diagnostic form of 'moves the rollout output towards the BF16 reference'
    rng = np.random.default_rng(34)
    x, w = _problem(rng, 64, 64, 256)
    wc, ws, gw, _ = Q.qdq_weights(w)
    ref = x @ Q.dequantize(wc[0], ws[0], gw[0]).T
    errs = []
    for k in (0, 16, 64, 256):
        qa = Q.quantize_activation(x, k)
        y = G.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], None, qa["R_S"], qa["S"],
                               wc, ws, gw, [0, 64])
        errs.append(np.linalg.norm(y - ref))
    assert errs[0] > errs[1] > errs[2] > errs[3]


# ------------------------------ routing -------------------------------------

def test_route_brute_force_and_ties():
    rng = np.random.default_rng(40)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    logits[0, :] = 0.5                                 # all tied -> experts 0..tk-1
    logits[1, [3, 9]] = 7.0                            # tie at the top -> 3 before 9
    bias = rng.standard_normal(16).astype(np.float32)
    for b in (None, bias):
        ids, w = MOE.route(logits, 4, b)
        for t in range(50):
            lp = [float(np.float32(logits[t, e] + (0 if b is None else b[e]))) for e in range(16)]
            want = sorted(range(16), key=lambda e: (-lp[e], e))[:4]
            assert list(ids[t]) == want
            z = [np.exp(lp[e] - lp[want[0]]) for e in want]
            assert np.allclose(w[t], np.array(z) / sum(z), rtol=1e-6)
    ids, _ = MOE.route(logits, 4)
    assert list(ids[0]) == [0, 1, 2, 3] and list(ids[1][:2]) == [3, 9]


def test_route_closed_forms():
    logits = np.array([[1.0, 3.0, -2.0]], dtype=np.float32)
    ids, w = MOE.route(logits, 1)
    assert list(ids[0]) == [1] and w[0, 0] == 1.0
    ids, w = MOE.route(logits, 2)
    assert list(ids[0]) == [1, 0]
    assert w[0, 0] == np.float32(1 / (1 + np.exp(-2.0)))   # logistic of the gap


def test_permute_bijection_and_order():
    rng = np.random.default_rng(41)
    T, E, tk = 200, 12, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = MOE.route(logits, tk)
    offs, perm, inv = MOE.permute(ids, E)
    assert offs[0] == 0 and offs[-1] == T * tk and np.all(np.diff(offs) >= 0)
    assert sorted(perm.tolist()) == sorted(np.repeat(np.arange(T), tk).tolist())
    assert sorted(inv.ravel().tolist()) == list(range(T * tk))
    for t in range(T):
        for j in range(tk):
            p = inv[t, j]
            assert perm[p] == t
            e = np.searchsorted(offs, p, side="right") - 1
            assert ids[t, j] == e
    for e in range(E):
        seg = perm[offs[e]:offs[e + 1]]
        assert np.all(np.diff(seg) > 0)                # tokens ascending within an expert


def test_swiglu_against_torch_silu():
    rng = np.random.default_rng(42)
    y = _bf16(rng.standard_normal((16, 64)) * 3)
    h = MOE.swiglu(y, 32)
    t = torch.from_numpy(y)
    want = _bf16((torch.nn.functional.silu(t[:, :32]) * t[:, 32:]).numpy())
    assert np.max(np.abs(h - want) / np.maximum(np.abs(want), 1e-30)) <= 2 ** -7
    assert np.mean(h == want) > 0.99
    assert not MOE.swiglu(np.zeros((1, 4)), 2).any()


def test_combine_copy_and_weights():
    rng = np.random.default_rng(43)
    y = _bf16(rng.standard_normal((10, 8)))
    inv = rng.permutation(10).reshape(10, 1)
    out = MOE.combine(y, inv, np.ones((10, 1), np.float32))
    assert np.array_equal(out, y[inv[:, 0]])
    inv2 = np.stack([np.arange(5), np.arange(5, 10)], axis=1)
    w = np.full((5, 2), 0.5, np.float32)
    out = MOE.combine(y, inv2, w)
    assert np.array_equal(out, _bf16((y[:5] + y[5:]) / 2))
