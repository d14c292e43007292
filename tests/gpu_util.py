"""Host <-> device helpers for the GPU parity tests (no method arithmetic)."""
import numpy as np
import torch

from oracle import formats as OF


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_vals(t: torch.Tensor) -> np.ndarray:
    return OF.bf16_bits_to_f64(host_bits(t))


def tile_wscales(s: np.ndarray) -> np.ndarray:
    """Row-major weight block scales [E][N][K/16] -> the library's tiles
    [E][N/16][K/64][16][4] (a layout change only)."""
    E, N, KB = s.shape
    return np.ascontiguousarray(s.reshape(E, N // 16, 16, KB // 4, 4).transpose(0, 1, 3, 2, 4))


def untile_wscales(t: np.ndarray) -> np.ndarray:
    """The library's weight-scale tiles [E][N/16][K/64][16][4] -> [E][N][K/16]."""
    E, NB, KG, _, _ = t.shape
    return np.ascontiguousarray(t.transpose(0, 1, 3, 2, 4)).reshape(E, NB * 16, KG * 4)


def tile_wcodes(c: np.ndarray) -> np.ndarray:
    """Packed row-major weight codes [E][N][K/2] -> the library's tiles: per
    16 rows x 64 columns, the 32-column halves, each [16 rows][16 bytes]
    ([E][N/16][K/64][2][16][16], returned as [E][N/16][K/64][16][32]; a
    layout change only)."""
    E, N, KH = c.shape
    t = c.reshape(E, N // 16, 16, KH // 32, 2, 16).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(t).reshape(E, N // 16, KH // 32, 16, 32)


def untile_wcodes(t: np.ndarray) -> np.ndarray:
    """The library's weight-code tiles -> [E][N][K/2]."""
    E, NB, KG, _, _ = t.shape
    u = t.reshape(E, NB, KG, 2, 16, 16).transpose(0, 1, 4, 2, 3, 5)
    return np.ascontiguousarray(u).reshape(E, NB * 16, KG * 32)


def channel_major_codes(c: np.ndarray) -> np.ndarray:
    """Packed row-major weight codes [E][N][K/2] -> [E][K][N/2]: byte n/2 of
    column k holds rows n (bits 3:0) and n+1 (bits 7:4) (a layout change
    only)."""
    lo, hi = c & 0xF, c >> 4
    E, N, KH = c.shape
    cols = np.empty((E, N, 2 * KH), dtype=np.uint8)
    cols[:, :, 0::2], cols[:, :, 1::2] = lo, hi
    t = np.ascontiguousarray(cols.transpose(0, 2, 1))           # [E][K][N] nibbles
    return (t[:, :, 0::2] | (t[:, :, 1::2] << 4)).astype(np.uint8)


def gemm_wcodes(c: np.ndarray) -> np.ndarray:
    """Packed row-major weight codes [E][N][K/2] -> the GEMMs' packed copy
    [E][2][N/16][K/64][16][32]: the tiles, then the channel-major codes."""
    E, N, KH = c.shape
    cm = channel_major_codes(c).reshape(E, N // 16, KH // 32, 16, 32)
    return np.ascontiguousarray(np.stack([tile_wcodes(c), cm], axis=1))


def gemm_wscales(s: np.ndarray) -> np.ndarray:
    """Row-major weight block scales [E][N][K/16] -> the GEMMs' packed copy
    [E][2][N/16][K/64][16][4]: the tiles, then the channel-major scales
    [K/16][N]."""
    E, N, KB = s.shape
    cm = np.ascontiguousarray(s.transpose(0, 2, 1)).reshape(E, N // 16, KB // 4, 16, 4)
    return np.ascontiguousarray(np.stack([tile_wscales(s), cm], axis=1))


def bits_of(vals: np.ndarray) -> np.ndarray:
    return OF.f64_to_bf16_bits(vals)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def heavy_bf16(rng, shape, df=3.0, ch_sigma=1.0):
    x = rng.standard_t(df, size=shape) * rng.lognormal(0, ch_sigma, size=shape[-1])
    return OF.round_to_bf16(x)


def rownorm_err(y, ref):
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    ok = den > 0
    worst = np.max(num[ok] / den[ok]) if ok.any() else 0.0
    return max(worst, np.max(num[~ok]) if (~ok).any() else 0.0)


def maxabs_err(y, ref):
    m = np.max(np.abs(ref))
    return np.max(np.abs(y - ref)) / m if m > 0 else np.max(np.abs(y))


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (8 significant bits)."""
    m, e = np.frexp(np.abs(v))
    return np.where(m == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e, -125) - 8))


def assert_gemm_close(y, ref, tol=2e-3, min_exact=0.98):
    """The output tolerance, against the oracle's float64 result rounded once
    to bf16.  The GPU accumulates in float32 and rounds once to bf16, so an
    element may land one bf16 step (up to 2^-7 relative) from the oracle's
    when the two sums straddle a rounding boundary; near-zero outputs may
    differ by float32 accumulation error, small on the row's scale.  So:
      * row-normwise relative error <= tol;
      * every element within one bf16 step of the oracle's value, or within
        tol times the row's RMS;
      * at least min_exact of the elements bit-identical."""
    assert y.shape == ref.shape
    assert np.all(np.isfinite(y))
    e1, e2 = rownorm_err(y, ref), maxabs_err(y, ref)
    exact = np.mean(y == ref)
    assert e1 <= tol, f"row-normwise error {e1:.3e}"
    d = np.abs(y - ref)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)) if ref.ndim > 1 else np.sqrt(np.mean(ref * ref))
    allowed = np.maximum(bf16_ulp(ref), tol * rms)
    bad = d > allowed
    if bad.any():
        i = np.unravel_index(np.argmax(d / allowed), d.shape)
        raise AssertionError(f"{int(bad.sum())} elements beyond one bf16 step; worst at {i}: "
                             f"got {y[i]!r} want {ref[i]!r} (step {bf16_ulp(ref[i])!r})")
    assert exact >= min_exact, f"only {exact:.4f} of elements bit-identical"
    return e1, e2, exact
