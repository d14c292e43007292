"""Expert-grouped W4A4 GEMM with Residual Activation Compensation.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The method (gist.science technical summary §2.2 B, both languages; arXiv
abstract): keep the native W4A4 product for all of K, and for the channels
picked by the binary residual mask add the residual activation's product with
the same quantized weights.  The correction is added to the product, which by
linearity equals quantizing nothing on those channels (the 'add it back'
reading).  With the mask empty the result is the plain W4A4 GEMM; with every
channel selected it is the product of the bf16-rounded activation with the
dequantized weight, the trainer's asymmetric W4A16 forward (summary §2.2 A).

For output row p of expert e, taking activation row t = a_rows[p]:

    y64[p, n] = sum_k x^[t, k] * w^_e[n, k]  +  sum_{j in S} r[t, j] * w^_e[n, j]
    y[p, n]   = bf16(y64[p, n])       (one rounding from float64)
"""
from __future__ import annotations

import numpy as np

from .formats import round_to_bf16
from .nvfp4 import dequantize


def grouped_gemm_rac(a_codes, a_scales, g_x, a_rows, R_S, S, w_codes, w_scales, g_w,
                     expert_offsets, rows=None):
    """a_codes [M_src][K] (one code per element), a_scales [M_src][K/16], g_x;
    a_rows int [M_total] or None (identity); R_S [M_src][k] bf16 values as
    float64 (may be None when k == 0); S int [k]; w_codes [E][N][K];
    w_scales [E][N][K/16]; g_w float32 [E]; expert_offsets int [E+1].

    rows: optional sorted array of output row indices to evaluate (the rest
    are returned as NaN), so full-size checks can sample.

    Returns float64 [M_total][N] holding bf16 values."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    E = len(offs) - 1
    M_total = int(offs[-1])
    N = w_codes.shape[1]
    S = np.asarray(S, dtype=np.int64)
    x_hat = dequantize(a_codes, a_scales, g_x)
    out = np.full((M_total, N), np.nan)
    want = np.ones(M_total, dtype=bool) if rows is None else np.isin(np.arange(M_total), rows)
    for e in range(E):
        p = np.arange(offs[e], offs[e + 1])
        p = p[want[p]]
        if p.size == 0:
            continue
        t = p if a_rows is None else np.asarray(a_rows, dtype=np.int64)[p]
        w_hat = dequantize(w_codes[e], w_scales[e], g_w[e])          # [N][K]
        y = x_hat[t] @ w_hat.T
        if S.size:
            y = y + np.asarray(R_S, dtype=np.float64)[t] @ w_hat[:, S].T
        out[p] = round_to_bf16(y)
    return out


def grouped_gemm_w4a16(x, a_rows, w_codes, w_scales, g_w, expert_offsets, rows=None):
    """The trainer-side forward of asymmetric W4A16 QAT (gist.science
    technical summary §2.2 A): bf16 activations times the dequantized NVFP4
    weights of each row's expert, the same weights the rollout's W4A4 GEMM
    uses (one QDQ path for both sides; arXiv abstract).

    x [M_src][K] bf16 values as float64; a_rows int [M_total] or None
    (identity); w_codes [E][N][K]; w_scales [E][N][K/16]; g_w float32 [E];
    expert_offsets int [E+1].  For output row p of expert e taking row
    t = a_rows[p]:
        y[p, n] = bf16( sum_k x[t, k] * w^_e[n, k] )   (float64, one rounding)
    rows: optional output rows to evaluate (others NaN).
    Returns float64 [M_total][N] holding bf16 values."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    E = len(offs) - 1
    M_total = int(offs[-1])
    N = w_codes.shape[1]
    x = np.asarray(x, dtype=np.float64)
    out = np.full((M_total, N), np.nan)
    want = np.ones(M_total, dtype=bool) if rows is None else np.isin(np.arange(M_total), rows)
    for e in range(E):
        p = np.arange(offs[e], offs[e + 1])
        p = p[want[p]]
        if p.size == 0:
            continue
        t = p if a_rows is None else np.asarray(a_rows, dtype=np.int64)[p]
        w_hat = dequantize(w_codes[e], w_scales[e], g_w[e])          # [N][K]
        out[p] = round_to_bf16(x[t] @ w_hat.T)
    return out


def grouped_gemm_rac_per_expert(a_codes, a_scales, g_x, a_rows, R_P, S_E, w_codes, w_scales, g_w,
                                expert_offsets, rows=None):
    """grouped_gemm_rac with a channel set per expert: S_E int [E][k], and
    the residual indexed by permuted row, R_P [M_total][k] (R_P[p] holds the
    residual of row a_rows[p] on the channels S_E[e] of p's expert e):
        y64[p, n] = sum_k x^[t, k] w^_e[n, k] + sum_j R_P[p, j] w^_e[n, S_E[e, j]]
    and y = bf16(y64)."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    E = len(offs) - 1
    M_total = int(offs[-1])
    N = w_codes.shape[1]
    x_hat = dequantize(a_codes, a_scales, g_x)
    out = np.full((M_total, N), np.nan)
    want = np.ones(M_total, dtype=bool) if rows is None else np.isin(np.arange(M_total), rows)
    S_E = np.asarray(S_E, dtype=np.int64)
    for e in range(E):
        p = np.arange(offs[e], offs[e + 1])
        p = p[want[p]]
        if p.size == 0:
            continue
        t = p if a_rows is None else np.asarray(a_rows, dtype=np.int64)[p]
        w_hat = dequantize(w_codes[e], w_scales[e], g_w[e])
        y = x_hat[t] @ w_hat.T
        if S_E.shape[1]:
            y = y + np.asarray(R_P, dtype=np.float64)[p] @ w_hat[:, S_E[e]].T
        out[p] = round_to_bf16(y)
    return out
