"""GPU parity of the FP8 (E4M3) W8A8 baseline (fp8_quantize,
grouped_fp8_gemm; the format the pages compare NVFP4 against, arXiv
abstract and gist.science technical summary §1) against the oracle: codes
and scales bit-exact, products within the GEMM tolerance, on small cases
spanning several tiles, empty and single-row experts, N tails and an odd
number of K steps, and on the first GEMM of the decode and large-prefill
workloads at full size (sampled rows and columns)."""
import sys

import numpy as np
import pytest
import torch

import fp4_quantized_gemm_amd as F
import synth
from oracle import formats as OF
from oracle import fp8 as O8
from tests.gpu_util import assert_gemm_close, heavy_bf16, host_vals, to_dev_bf16
from tests.test_gpu_full import sample_rows

pytestmark = pytest.mark.gpu

# The row-norm and per-element bounds are the NVFP4 GEMM's.  The share of
# bit-identical elements is lower: the 64-product FP8 MFMA sums inside the
# matrix core with its own rounding, so more float32 sums land across a bf16
# rounding boundary from the exact one (96.8-97.5% identical on these cases,
# against >= 98% for the f16 path).
FP8_MIN_EXACT = 0.95


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("M,K", [(1, 8), (37, 136), (256, 4096), (1000, 24)])
def test_fp8_quantize_activation(dev, M, K):
    say(f"fp8 quantize M={M} K={K}")
    rng = np.random.default_rng(M + K)
    x = heavy_bf16(rng, (M, K), ch_sigma=2.0)
    x[0, 0] = -0.0
    if M > 1:
        x[1, :] = 0.0
    codes, g = F.fp8_quantize(to_dev_bf16(OF.f64_to_bf16_bits(x)))
    torch.cuda.synchronize()
    rc, rg, _ = O8.quantize(x)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert g.cpu().numpy()[0] == rg


def test_fp8_quantize_stacked_and_zero(dev):
    say("fp8 quantize stacked")
    rng = np.random.default_rng(11)
    w = OF.round_to_bf16(rng.standard_normal((5, 48, 256)) *
                         np.array([1e-3, 0.02, 1.0, 0.0, 300.0])[:, None, None])
    codes, g = F.fp8_quantize(to_dev_bf16(OF.f64_to_bf16_bits(w)), stacked=True)
    torch.cuda.synchronize()
    rc, rg = O8.quantize_stacked(w)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(g.cpu().numpy(), rg)
    assert rg[3] == 0


@pytest.mark.parametrize("M_src,counts,N,K,gather", [
    (64, [64], 256, 512, False),
    (300, [100, 200], 256, 1024, True),               # 1 tile each, half-empty row halves
    (500, [17, 0, 0, 400, 83], 272, 384, True),       # empty experts, N tail, odd K steps
    (700, [300, 1, 511, 0, 255], 528, 768, True),     # several 256-row tiles
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 512, 1024, True),
    (300, [300], 256, 4096, False),
])
def test_fp8_gemm(dev, M_src, counts, N, K, gather):
    say(f"fp8 gemm counts={counts} N={N} K={K} gather={gather}")
    rng = np.random.default_rng(sum(counts) + N + K)
    E = len(counts)
    x = heavy_bf16(rng, (M_src, K))
    w = OF.round_to_bf16(rng.standard_normal((E, N, K)) * 0.02)
    ac, gx, _ = O8.quantize(x)
    wc, gw = O8.quantize_stacked(w)
    offs = np.zeros(E + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    M_total = int(offs[-1])
    a_rows = rng.integers(0, M_src, M_total).astype(np.int32) if gather else None
    ref = O8.grouped_gemm_fp8(ac, gx, a_rows, wc, gw, offs)
    y = F.grouped_fp8_gemm(cu(ac), cu(np.array([gx])), cu(a_rows) if gather else None, cu(wc),
                           cu(gw), cu(offs), M_total=M_total)
    torch.cuda.synchronize()
    e1, e2, ex = assert_gemm_close(host_vals(y), ref, min_exact=FP8_MIN_EXACT)
    say(f"   rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.5f}")


def test_fp8_gemm_empty(dev):
    say("fp8 gemm empty")
    a = torch.zeros((4, 256), dtype=torch.uint8, device="cuda")
    w = torch.zeros((2, 32, 256), dtype=torch.uint8, device="cuda")
    g = torch.ones(2, dtype=torch.float32, device="cuda")
    offs = torch.zeros(3, dtype=torch.int32, device="cuda")
    y = F.grouped_fp8_gemm(a, g[:1], None, w, g, offs, M_total=0)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


@pytest.mark.parametrize("idx", [4, 5])
def test_full_size_first_gemm_fp8(dev, idx):
    cfg = synth.get(idx)
    say(f"workload {cfg.name}: generating")
    wl = synth.make(cfg)
    rng = np.random.default_rng(3)
    logits = torch.from_numpy(wl.logits).cuda()
    bias = torch.from_numpy(wl.bias).cuda() if wl.bias is not None else None
    say(f"workload {cfg.name}: running the library")
    ac, gx = F.fp8_quantize(to_dev_bf16(wl.x))
    wc, gw = F.fp8_quantize(to_dev_bf16(wl.w_first), stacked=True)
    ids, tw, offs, perm, inv = F.moe_permute(logits, cfg.topk, bias)
    y = F.grouped_fp8_gemm(ac, gx, perm, wc, gw, offs, M_total=perm.numel())
    torch.cuda.synchronize()
    x = OF.bf16_bits_to_f64(wl.x)
    A = np.float32(np.max(np.abs(x)))
    assert gx.cpu().numpy()[0] == O8.tensor_scale(A)
    offs_np, perm_np = offs.cpu().numpy(), perm.cpu().numpy()
    rows_p = sample_rows(offs_np, rng)
    say(f"  rows: {len(rows_p)}")
    N = wl.w_first.shape[1]
    cols = np.sort(rng.choice(N, min(N, 256), replace=False))
    y_h = host_vals(y)
    got, ref = [], []
    for e in np.unique(np.searchsorted(offs_np, rows_p, side="right") - 1):
        ps = rows_p[(rows_p >= offs_np[e]) & (rows_p < offs_np[e + 1])]
        w_e = OF.bf16_bits_to_f64(wl.w_first[e])
        we_c, we_g, _ = O8.quantize(w_e[cols], A=np.float32(np.max(np.abs(w_e))))
        assert gw.cpu().numpy()[e] == we_g
        a_c, a_g, _ = O8.quantize(x[perm_np[ps]], A=A)
        ref.append(O8.grouped_gemm_fp8(a_c, a_g, None, we_c[None], np.array([we_g]),
                                       [0, len(ps)]))
        got.append(y_h[ps][:, cols])
    e1, e2, ex = assert_gemm_close(np.concatenate(got), np.concatenate(ref),
                                   min_exact=FP8_MIN_EXACT)
    say(f"    rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.4f}")
