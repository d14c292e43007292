"""Number formats of the NVFP4 path, written out from their definitions.

TEST INFRASTRUCTURE ONLY. This package is the slow CPU oracle that the HIP
library is checked against; only tests, the smoke check and the benchmark's
CPU-baseline leg may import it. The library never calls into it.

Source of the formats. The QUADS pages (gist.science technical summary §1,
both language versions) only say that FP4 uses the coarse E2M1 grid with
eight magnitudes per sign, and the arXiv abstract says NVFP4 adds
fine-grained scaling. The block layout used here is the public NVFP4
definition: E2M1 elements in blocks of 16, one FP8 E4M3 scale per block and
one FP32 scale per tensor.

Every function works on numpy arrays, computes in float64 unless a float32
step is named, and favours the plain definition over speed.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  Code bits are
# s e1 e0 m.  Exponent field 0 is subnormal: magnitude m * 0.5.  Otherwise
# magnitude 2**(e-1) * (1 + m/2).  This yields the eight magnitudes below.
# --------------------------------------------------------------------------


def _e2m1_magnitude_from_bits(c: int) -> float:
    e, m = (c >> 1) & 3, c & 1
    if e == 0:
        return 0.5 * m
    return 2.0 ** (e - 1) * (1.0 + 0.5 * m)


E2M1_MAG = np.array([_e2m1_magnitude_from_bits(c) for c in range(8)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """4-bit codes (uint8, low nibble used) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """float32 values -> E2M1 codes, round to nearest, ties to the even code,
    saturating at 6; the sign bit is the sign bit of v (so -0.1 -> 0x8).

    Written as a nearest-point search over the 8 grid magnitudes (exact in
    float64 because v is float32 and the grid points are dyadic)."""
    v = np.asarray(v, dtype=np.float32)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    idx = np.arange(8)
    step = 1 << 20
    for lo in range(0, flat.size, step):
        vc = flat[lo:lo + step]
        a = np.abs(vc.astype(np.float64))
        d = np.abs(a[:, None] - E2M1_MAG)                # distance to every grid point
        is_best = d == d.min(axis=1, keepdims=True)
        # among the nearest points prefer an even code index (ties to even)
        even_best = is_best & (idx % 2 == 0)
        mag_code = np.where(even_best.any(axis=1), np.argmax(even_best, axis=1),
                            np.argmax(is_best, axis=1))
        mag_code = np.where(a > 6.0, 7, mag_code)        # saturate
        sign = np.signbit(vc).astype(np.uint8) << 3
        out[lo:lo + step] = sign | mag_code.astype(np.uint8)
    return out.reshape(v.shape)


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP "E4M3FN"): bias 7, no infinities, S.1111.111 is NaN.
# Normal: (1 + f/8) * 2**(e-7), e = 1..15.  Subnormal: (f/8) * 2**-6.
# Scales are non-negative, so only codes 0x00..0x7E are produced.
# --------------------------------------------------------------------------


def _e4m3_value_from_bits(c: int) -> float:
    e, f = (c >> 3) & 0xF, c & 7
    if e == 0:
        return (f / 8.0) * 2.0 ** -6
    return (1.0 + f / 8.0) * 2.0 ** (e - 7)


E4M3_POS = np.array([_e4m3_value_from_bits(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = E4M3_POS[-1]          # 448


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 bytes -> float64.  Sign bit honoured; NaN codes map to NaN."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, E4M3_POS[np.minimum(c & 0x7F, 0x7E)])
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode_nonneg(u) -> np.ndarray:
    """Non-negative float32 -> E4M3 byte: round to nearest, ties to the even
    code, saturate to 448.  Written as a nearest-point search over the 127
    finite non-negative E4M3 values."""
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    if np.any(u < 0) or np.any(np.isnan(u)):
        raise ValueError("e4m3_encode_nonneg: negative or NaN input")
    hi = np.searchsorted(E4M3_POS, u, side="left")       # first grid value >= u
    hi = np.minimum(hi, len(E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = u - E4M3_POS[lo]
    d_hi = E4M3_POS[hi] - u
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(u >= E4M3_MAX, 0x7E, code)           # saturate
    code = np.where(u == E4M3_POS[hi], hi, code)         # exact hit
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# bfloat16: the upper 16 bits of an IEEE float32.  8 significant bits.
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """float64 (or float32) -> nearest bfloat16 value, ties to even, in one
    rounding straight from the input precision (no float32 detour).

    x = m * 2**e with m in [0.5, 1); a bf16 has 8 significant bits, so its
    spacing near x is 2**(e-8) (2**-133 below the normal range).  Dividing by
    a power of two is exact and np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)                              # bf16 normal floor 2**-126
    ulp = np.ldexp(1.0, e - 8)
    y = np.rint(x / ulp) * ulp
    with np.errstate(over="ignore"):
        y = np.where(np.abs(y) > 3.3895313892515355e38, np.copysign(np.inf, x), y)
    return np.where(x == 0, x, y)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round (as round_to_bf16) and return the 16-bit pattern."""
    y = round_to_bf16(x).astype(np.float32)              # exact: y is a bf16 value
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def f32(x) -> np.ndarray:
    """Round float64 to float32, to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
