"""NVFP4 quantize / dequantize, residual, channel scores and channel selection.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain and slow on purpose.

What the QUADS pages fix, and where:
  * Activations are quantized online, every forward, onto the coarse E2M1
    grid (arXiv abstract; gist.science technical summary §2.1).
  * Weights reach the rollout through the same quantize-dequantize (QDQ)
    path the trainer fake-quantizes with (abstract; summary §2.1 and §2.2 A).
  * Residual Activation Compensation picks the channels with the largest
    quantization residual with a binary channel mask, and adds the residual
    back on top of the W4A4 product (summary §2.2 B, both languages).

What the pages leave open and is read here (each reading is listed in the
design notes): the scale recipe's float32 operation order, the sign of codes
that round to zero, the channel statistic (sum of |residual| over all rows,
accumulated exactly in fixed point), and ties (lower channel index wins).

All inputs are bfloat16 values carried as float64 (exactly).  A tensor's
absolute maximum must lie in [2**-100, 2**100] or be exactly 0.
"""
from __future__ import annotations

import numpy as np

from .formats import (e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode_nonneg,
                      round_to_bf16)

BLOCK = 16          # elements per scale block, along the contraction dimension
E2M1_MAX = 6.0      # largest E2M1 magnitude
E4M3_MAX = 448.0    # largest finite E4M3 value
SCALE_DEN = np.float32(E2M1_MAX * E4M3_MAX)   # 2688, exact in float32


def tensor_amax(x) -> np.float32:
    """A = max |x| over the whole tensor (exact: a max of bf16 values)."""
    x = np.asarray(x, dtype=np.float64)
    return np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)


def tensor_scale(A: np.float32) -> np.float32:
    """g = float32(A / 2688): the per-tensor scale that is stored and used to
    decode.  numpy's float32 division is correctly rounded."""
    return np.float32(np.float32(A) / SCALE_DEN)


def quantize(x, A=None):
    """Quantize a [M][K] tensor (K % 16 == 0) to NVFP4.

    A: the tensor's absolute maximum, when x is a slice (rows or 16-aligned
    column blocks) of a larger tensor; by default max |x|.

    Returns (codes uint8 [M][K] one code per element, scales uint8
    [M][K/16] E4M3 bytes, g float32, A float32).

    Per 16-element block b with a_b = max |x_i| (float32 steps, each rounded
    to nearest even):
        u_b  = (a_b * 448) / A              -> E4M3 scale s_b (round, ties even)
        if s_b == 0: every magnitude in the block is 0
        rho  = 2688 / (s_b * A)             (s_b * A is exact in float32)
        v_i  = x_i * rho                    -> E2M1 code (round, ties even)
    The sign bit of every code is the sign bit of x_i.
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    A = tensor_amax(x) if A is None else np.float32(A)
    if x.size and tensor_amax(x) > A:
        raise ValueError("A is below max |x|")
    g = tensor_scale(A)
    xf = x.astype(np.float32)                      # exact (bf16 values)
    xb = xf.reshape(M, K // BLOCK, BLOCK)
    a_b = np.max(np.abs(xb), axis=-1)              # float32, exact
    codes = np.zeros((M, K // BLOCK, BLOCK), dtype=np.uint8)
    scales = np.zeros((M, K // BLOCK), dtype=np.uint8)
    if A > 0:
        u = np.float32(a_b * np.float32(E4M3_MAX)) / A            # float32 ops
        scales = e4m3_encode_nonneg(u)
        s = e4m3_decode(scales).astype(np.float32)                 # exact
        sA = (s * A).astype(np.float32)                            # exact product
        with np.errstate(divide="ignore"):
            rho = np.where(s > 0, SCALE_DEN / np.where(s > 0, sA, np.float32(1)),
                           np.float32(0)).astype(np.float32)
        v = (xb * rho[..., None]).astype(np.float32)
        codes = e2m1_encode(v)
        codes = np.where((s > 0)[..., None], codes, 0)
    sign = (np.signbit(xb).astype(np.uint8) << 3)
    codes = (codes & 7) | sign
    return codes.reshape(M, K).astype(np.uint8), scales.astype(np.uint8), g, A


def dequantize_unscaled(codes, scales) -> np.ndarray:
    """x~ = q * s_b (no tensor scale), float64 and exact: q has two
    significant bits and s_b four."""
    codes = np.asarray(codes)
    M, K = codes.shape
    q = e2m1_decode(codes).reshape(M, K // BLOCK, BLOCK)
    s = e4m3_decode(scales)[..., None]
    return (q * s).reshape(M, K)


def dequantize(codes, scales, g) -> np.ndarray:
    """x^ = q * s_b * g, float64 (exact: at most 6 + 24 significant bits)."""
    return dequantize_unscaled(codes, scales) * np.float64(g)


def residual(x, codes, scales, g) -> np.ndarray:
    """r = bf16(float32(x - x^)).  x - x^ is exact in float64 here because x
    and x^ lie within a few binades of each other (or x^ = 0); the float32 and
    bf16 roundings are both to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    d = x - dequantize(codes, scales, g)
    return round_to_bf16(d.astype(np.float32).astype(np.float64))


def frexp_exponent(A: np.float32) -> int:
    """E with A = m * 2**E, m in [0.5, 1)."""
    return int(np.frexp(np.float64(A))[1])


def channel_scores(r, A) -> np.ndarray:
    """score_j = sum over rows of floor(|r_ij| * 2**(31 - E_A)), an exact
    integer sum (uint64).  This is the 'residual magnitude' ranking statistic:
    the mean |r| over all rows, up to a positive factor, truncated below
    2**-31 * 2**E_A per element so that any summation order gives the same
    bits.  |r| <= 2**E_A, so each term fits in 32 bits."""
    r = np.asarray(r, dtype=np.float64)
    if A == 0:
        return np.zeros(r.shape[1], dtype=np.uint64)
    E = frexp_exponent(A)
    t = np.floor(np.ldexp(np.abs(r), 31 - E))
    assert np.all(t <= 2.0 ** 31)
    return t.astype(np.uint64).sum(axis=0, dtype=np.uint64)


def select_channels(score, k: int) -> np.ndarray:
    """The k channels with the largest score (ties: lower index first),
    returned in ascending index order as int32."""
    score = [int(s) for s in np.asarray(score, dtype=np.uint64)]
    K = len(score)
    if not 0 <= k <= K:
        raise ValueError("k out of range")
    order = sorted(range(K), key=lambda j: (-score[j], j))
    return np.array(sorted(order[:k]), dtype=np.int32)


def quantize_activation(x, k: int):
    """One activation tensor through quantize -> residual -> scores -> select.

    Returns a dict with codes, scales, g, A, r (full residual), score, S and
    R_S = r[:, S] (bf16 values as float64)."""
    codes, scales, g, A = quantize(x)
    r = residual(x, codes, scales, g)
    score = channel_scores(r, A)
    S = select_channels(score, k)
    return dict(codes=codes, scales=scales, g=g, A=A, r=r, score=score, S=S, R_S=r[:, S])


def fake_quant(codes, scales, g) -> np.ndarray:
    """The QDQ output handed to bf16 arithmetic: bf16(float32(q * s_b) * g).
    q * s_b is exact in float32, so this is one float32 product with the
    tensor scale, then one rounding to bf16."""
    qs = dequantize_unscaled(codes, scales).astype(np.float32)           # exact
    return round_to_bf16((qs * np.float32(g)).astype(np.float32).astype(np.float64))


def qdq_weights(w):
    """Weight QDQ for each expert of w [E][N][K] (bf16 values as float64).

    One tensor scale per expert matrix.  Returns codes [E][N][K], scales
    [E][N][K/16], g_w float32 [E], and the trainer-side fake-quantized
    weight w_qdq = bf16(float32(q * s_b * g)) [E][N][K] (q * s_b is exact in
    float32, so this is one float32 product then one bf16 rounding)."""
    w = np.asarray(w, dtype=np.float64)
    E, N, K = w.shape
    codes = np.zeros((E, N, K), dtype=np.uint8)
    scales = np.zeros((E, N, K // BLOCK), dtype=np.uint8)
    g_w = np.zeros(E, dtype=np.float32)
    w_qdq = np.zeros((E, N, K), dtype=np.float64)
    for e in range(E):
        c, s, g, _ = quantize(w[e])
        codes[e], scales[e], g_w[e] = c, s, g
        w_qdq[e] = fake_quant(c, s, g)
    return codes, scales, g_w, w_qdq


def qdq_residual(R_S):
    """Second-pass quantization of the compensated residual (the variant in
    which the selected residual is itself quantized to NVFP4 before it is
    added back; gist.science technical summary §2.2 B, 'second-pass
    quantization').

    R_S [M][k] (k % 16 == 0, bf16 values as float64) goes through the same
    QDQ path as the weights: one tensor scale over the whole [M][k] tensor,
    16-element blocks along the selected-channel axis (channel order of S),
    and the bf16 fake-quantized value r^ = bf16(float32(q * s_b) * g_r) is
    what the GEMM's correction multiplies with the weights.

    Returns (codes [M][k], scales [M][k/16], g_r float32, r_qdq [M][k])."""
    codes, scales, g, _ = quantize(R_S)
    return codes, scales, g, fake_quant(codes, scales, g)


def pack_codes(codes) -> np.ndarray:
    """[..][K] codes -> [..][K/2] bytes: element 2j in bits 3:0, element 2j+1
    in bits 7:4."""
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def select_channels_per_expert(x, codes, scales, g, A, a_rows, expert_offsets, k: int):
    """Per-expert channel selection (a variant of the binary channel mask of
    gist.science technical summary §2.2 B in which each expert ranks the
    channels by the residual of its own rows).

    x, codes, scales, g, A: the quantized activation [M_src][K] as from
    quantize(); a_rows int [M_total] or None (identity): the activation row
    of each permuted row; expert_offsets int [E+1].  For expert e with
    permuted rows p in [off[e], off[e+1]) taking rows t = a_rows[p]:
        score_e[j] = sum over its rows of floor(|r[t, j]| * 2**(31 - E_A))
    (the channel_scores statistic restricted to those rows, E_A from the
    tensor amax A), S_e = the k channels of largest score_e (ties: lower
    index) ascending, and R[p] = r[t, S_e].

    Returns (S int32 [E][k], R float64 [M_total][k], score uint64 [E][K])."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    E = len(offs) - 1
    M_total = int(offs[-1])
    K = np.asarray(codes).shape[1]
    r = residual(x, codes, scales, g)
    rows = np.arange(M_total) if a_rows is None else np.asarray(a_rows, dtype=np.int64)
    S = np.zeros((E, k), dtype=np.int32)
    R = np.zeros((M_total, k))
    score = np.zeros((E, K), dtype=np.uint64)
    for e in range(E):
        t = rows[offs[e]:offs[e + 1]]
        score[e] = channel_scores(r[t], A) if t.size else np.zeros(K, dtype=np.uint64)
        S[e] = select_channels(score[e], k)
        R[offs[e]:offs[e + 1]] = r[t][:, S[e]]
    return S, R, score
