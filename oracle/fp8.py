"""FP8 (E4M3) W8A8 expert-grouped GEMM: the low-precision rollout baseline
that QUADS compares NVFP4 against.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name FP8 rollout as the stable baseline that NVFP4 is measured
against (arXiv abstract; gist.science technical summary §1, and §4 on
throughput, where QUADS is ~16% faster than FP8) but give no FP8 recipe.
The reading taken here is the plainest one: OCP FP8 E4M3 for both operands,
one float32 scale per tensor (per activation tensor, and per expert for the
weights), chosen so that the tensor's absolute maximum maps to 448:

    A = max |x|                        (exact: a max of bf16 values)
    g = float32(A / 448)               (correctly rounded float32 division)
    v = float32(|x| / g)               (correctly rounded float32 division)
    code = sign(x) << 7 | E4M3(v)      (round to nearest, ties to the even
                                        code, saturating at 448)

with every magnitude code 0 when A = 0 (then g = 0).  The sign bit of a code
is the sign bit of x, so -0.0 keeps it.  The product, for output row p of
expert e taking activation row t = a_rows[p]:

    y[p, n] = bf16( g_x * g_w[e] * sum_k E4M3(a[t, k]) * E4M3(w_e[n, k]) )

computed in float64 and rounded once.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, e4m3_decode, e4m3_encode_nonneg, round_to_bf16


def tensor_scale(A) -> np.float32:
    """g = float32(A / 448) (numpy's float32 division is correctly rounded)."""
    return np.float32(np.float32(A) / np.float32(E4M3_MAX))


def quantize(x, A=None):
    """x: bf16 values as float64, any shape, one tensor.  A: the tensor's
    absolute maximum when x is a slice (rows) of a larger tensor; by
    default max |x|.  Returns (codes uint8 of x's shape, g float32,
    A float32)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if A is None:
        A = amax
    A = np.float32(A)
    if amax > A:
        raise ValueError("A is below max |x|")
    g = tensor_scale(A)
    xf = x.astype(np.float32)                       # exact (bf16 values)
    if A > 0:
        v = (np.abs(xf) / g).astype(np.float32)     # float32 division
        mag = e4m3_encode_nonneg(v)
    else:
        mag = np.zeros(x.shape, dtype=np.uint8)
    sign = np.signbit(xf).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8), g, A


def quantize_stacked(x):
    """x [E][...]: each x[e] its own tensor (the weights of one expert).
    Returns (codes uint8 [E][...], g float32 [E])."""
    x = np.asarray(x, dtype=np.float64)
    codes = np.empty(x.shape, dtype=np.uint8)
    g = np.empty(x.shape[0], dtype=np.float32)
    for e in range(x.shape[0]):
        codes[e], g[e], _ = quantize(x[e])
    return codes, g


def dequantize(codes, g) -> np.ndarray:
    """x^ = E4M3(code) * g, float64 (exact: 4 + 24 significant bits)."""
    return e4m3_decode(codes) * np.float64(g)


def grouped_gemm_fp8(a_codes, g_x, a_rows, w_codes, g_w, expert_offsets, rows=None):
    """a_codes [M_src][K] E4M3 bytes, g_x float32; a_rows int [M_total] or None
    (identity); w_codes [E][N][K] E4M3 bytes; g_w float32 [E];
    expert_offsets int [E+1].  rows: optional output rows to evaluate (the
    others are NaN).  Returns float64 [M_total][N] holding bf16 values."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    E = len(offs) - 1
    M_total = int(offs[-1])
    N = w_codes.shape[1]
    a = e4m3_decode(a_codes)                                  # unscaled values
    out = np.full((M_total, N), np.nan)
    want = np.ones(M_total, dtype=bool) if rows is None else np.isin(np.arange(M_total), rows)
    for e in range(E):
        p = np.arange(offs[e], offs[e + 1])
        p = p[want[p]]
        if p.size == 0:
            continue
        t = p if a_rows is None else np.asarray(a_rows, dtype=np.int64)[p]
        w = e4m3_decode(w_codes[e])                           # [N][K]
        acc = a[t] @ w.T                                      # exact in float64 for K < 2^22
        out[p] = round_to_bf16(acc * np.float64(g_x) * np.float64(g_w[e]))
    return out
