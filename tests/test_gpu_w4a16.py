"""GPU parity of the trainer-side W4A16 product (grouped_w4a16_gemm: bf16
activations times the dequantized NVFP4 weights; gist.science technical
summary §2.2 A) against the oracle, on small cases spanning several tiles,
empty and single-row experts and N tails, and on the first GEMM of the
decode and large-prefill workloads at full size (sampled rows)."""
import sys

import numpy as np
import pytest
import torch

import fp4_quantized_gemm_amd as F
import synth
from fp4_quantized_gemm_amd import pipeline
from oracle import formats as OF
from oracle import gemm as OG
from oracle import nvfp4 as OQ
from tests.gpu_util import (assert_gemm_close, gemm_wcodes, gemm_wscales, heavy_bf16, host_vals,
                            to_dev_bf16)
from tests.test_gpu_full import sample_rows, weight_host

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(params=["auto", "big", "decode"])
def w16_kernel(request, monkeypatch):
    # "auto": the library's own choice; "big" / "decode" force the large-tile
    # or the weight-streaming kernel
    if request.param == "auto":
        monkeypatch.delenv("NVFP4RAC_GEMM", raising=False)
    else:
        monkeypatch.setenv("NVFP4RAC_GEMM", request.param)
    return request.param


@pytest.mark.parametrize("M_src,counts,N,K,gather", [
    (64, [64], 512, 512, False),
    (200, [0, 130, 1, 257], 144, 256, True),          # empty / single-row experts, N tail
    (700, [300, 1, 511, 0, 255], 528, 768, True),      # several 256-row tiles, N tail
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 512, 1024, True),   # decode-sized: 0-40 rows each
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 272, 384, True),    # last chunk of 128 columns, N tail
    (48, [20, 9, 0, 19], 256, 640, True),               # two full chunks, then a half one
    (300, [300], 256, 4096, False),
])
def test_w4a16_gemm(dev, w16_kernel, M_src, counts, N, K, gather):
    say(f"w4a16[{w16_kernel}] counts={counts} N={N} K={K} gather={gather}")
    rng = np.random.default_rng(sum(counts) + N + K)
    E = len(counts)
    x = heavy_bf16(rng, (M_src, K))
    x[0, :7] = 0.0
    w = OF.round_to_bf16(rng.standard_normal((E, N, K)) * 0.02)
    wc, ws, gw, _ = OQ.qdq_weights(w)
    offs = np.zeros(E + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    M_total = int(offs[-1])
    a_rows = rng.integers(0, M_src, M_total).astype(np.int32) if gather else None
    ref = OG.grouped_gemm_w4a16(x, a_rows, wc, ws, gw, offs)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = F.grouped_w4a16_gemm(to_dev_bf16(OF.f64_to_bf16_bits(x)), cu(a_rows) if gather else None,
                             cu(gemm_wcodes(OQ.pack_codes(wc))), cu(gemm_wscales(ws)), cu(gw), cu(offs),
                             M_total=M_total)
    torch.cuda.synchronize()
    e1, e2, ex = assert_gemm_close(host_vals(y), ref)
    say(f"   rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.5f}")


def test_w4a16_empty(dev):
    say("w4a16 empty")
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, 32, 256), dtype=torch.bfloat16, device="cuda")
    wq = F.nvfp4_qdq_weights(w, want_qdq=False)
    offs = torch.zeros(3, dtype=torch.int32, device="cuda")
    y = F.grouped_w4a16_gemm(x, None, wq.packed_codes, wq.packed_scales, wq.g, offs, M_total=0)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


@pytest.mark.parametrize("idx", [4, 5])
def test_full_size_first_gemm_w4a16(dev, idx):
    cfg = synth.get(idx)
    say(f"workload {cfg.name}: generating")
    wl = synth.make(cfg)
    rng = np.random.default_rng(2)
    x_dev = to_dev_bf16(wl.x)
    w1 = pipeline.prepare_weights(to_dev_bf16(wl.w_first))
    logits = torch.from_numpy(wl.logits).cuda()
    bias = torch.from_numpy(wl.bias).cuda() if wl.bias is not None else None
    say(f"workload {cfg.name}: running the library")
    ids, tw, offs, perm, inv = F.moe_permute(logits, cfg.topk, bias)
    y = F.grouped_w4a16_gemm(x_dev, perm, w1.packed_codes, w1.packed_scales, w1.g, offs,
                             M_total=perm.numel())
    torch.cuda.synchronize()
    x = OF.bf16_bits_to_f64(wl.x)
    offs_np, perm_np = offs.cpu().numpy(), perm.cpu().numpy()
    rows_p = sample_rows(offs_np, rng)
    say(f"  rows: {len(rows_p)}")
    wq_host = weight_host(wl.w_first, rng)
    y_h = host_vals(y)
    got, ref = [], []
    for e in np.unique(np.searchsorted(offs_np, rows_p, side="right") - 1):
        ps = rows_p[(rows_p >= offs_np[e]) & (rows_p < offs_np[e + 1])]
        wc, ws, gw = wq_host(e)
        ref.append(OG.grouped_gemm_w4a16(x[perm_np[ps]], None, wc[None], ws[None], gw[None],
                                         [0, len(ps)]))
        got.append(y_h[ps][:, wq_host.cols])
    e1, e2, ex = assert_gemm_close(np.concatenate(got), np.concatenate(ref))
    say(f"    rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.4f}")
