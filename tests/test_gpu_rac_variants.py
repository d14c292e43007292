"""GPU parity of the compensation variant with an NVFP4-quantized residual
(gist.science technical summary §2.2 B, 'second-pass quantization'):
nvfp4_qdq_residual bit-exact against the oracle, and the grouped GEMM fed
its fake-quantized residual within the GEMM tolerance, on small cases for
every GEMM kernel and on the first GEMM of the decode and large-prefill
workloads at full size (sampled rows)."""
import sys

import numpy as np
import pytest
import torch

import fp4_quantized_gemm_amd as F
import synth
from fp4_quantized_gemm_amd import pipeline
from oracle import formats as OF
from oracle import gemm as OG
from oracle import moe as OM
from oracle import nvfp4 as OQ
from tests.gpu_util import (assert_gemm_close, f32_bits, heavy_bf16, host_bits, host_vals,
                            gemm_wcodes, gemm_wscales, to_dev_bf16)
from tests.test_gpu_full import sample_rows, weight_host

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_qdq_residual(R_vals, got):
    codes, scales, g, r_hat = got
    rc, rs, rg, rq = OQ.qdq_residual(R_vals)
    assert np.array_equal(OQ.unpack_codes(codes.cpu().numpy()), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert f32_bits(g.cpu().numpy()[0]) == f32_bits(rg)
    assert np.array_equal(host_bits(r_hat), OF.f64_to_bf16_bits(rq))
    return rq


@pytest.mark.parametrize("M,K,k", [(1, 64, 16), (37, 512, 48), (300, 768, 128), (2048, 4096, 64),
                                   (5, 1024, 256)])
def test_qdq_residual_bitexact(dev, M, K, k):
    say(f"qdq residual M={M} K={K} k={k}")
    rng = np.random.default_rng(M + K + k)
    x = heavy_bf16(rng, (M, K))
    R = OQ.quantize_activation(x, k)["R_S"]
    Rd = to_dev_bf16(OF.f64_to_bf16_bits(R))
    got = F.nvfp4_qdq_residual(Rd)
    torch.cuda.synchronize()
    check_qdq_residual(R, got)


def test_qdq_residual_zero_and_empty(dev):
    say("qdq residual zeros / empty")
    Rd = torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")
    codes, scales, g, r_hat = F.nvfp4_qdq_residual(Rd)
    torch.cuda.synchronize()
    assert g.item() == 0.0 and not codes.cpu().numpy().any() and not scales.cpu().numpy().any()
    assert not host_bits(r_hat).any()
    codes, scales, g, r_hat = F.nvfp4_qdq_residual(torch.empty((0, 64), dtype=torch.bfloat16,
                                                               device="cuda"))
    torch.cuda.synchronize()
    assert g.item() == 0.0


@pytest.fixture(params=["generic", "big", "decode"])
def gemm_kernel(request, monkeypatch):
    monkeypatch.setenv("NVFP4RAC_GEMM", request.param)
    return request.param


@pytest.mark.parametrize("M_src,counts,N,K,k", [
    (64, [64], 512, 512, 16),
    (500, [17, 0, 0, 400, 83], 272, 1024, 128),
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 512, 1024, 64),
])
def test_gemm_with_quantized_residual(dev, gemm_kernel, M_src, counts, N, K, k):
    say(f"gemm[{gemm_kernel}] nvfp4 residual counts={counts} N={N} K={K} k={k}")
    rng = np.random.default_rng(sum(counts) + N + K + k)
    E = len(counts)
    x = heavy_bf16(rng, (M_src, K))
    w = OF.round_to_bf16(rng.standard_normal((E, N, K)) * 0.02)
    offs = np.zeros(E + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    M_total = int(offs[-1])
    a_rows = rng.integers(0, M_src, M_total).astype(np.int32)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # the library chain
    q = F.nvfp4_quantize_act(to_dev_bf16(OF.f64_to_bf16_bits(x)))
    S, R = F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"], q["score"], k)
    rq = F.nvfp4_qdq_residual(R)
    wqd = F.nvfp4_qdq_weights(to_dev_bf16(OF.f64_to_bf16_bits(w)), want_qdq=False)
    wc_d, ws_d, gw_d = wqd.packed_codes, wqd.packed_scales, wqd.g
    y = F.grouped_w4a4_gemm_rac(q["codes"], q["scales"], q["g"], cu(a_rows), rq[3], S, wc_d, ws_d,
                                gw_d, cu(offs), M_total=M_total)
    torch.cuda.synchronize()
    # the oracle chain
    qa = OQ.quantize_activation(x, k)
    assert np.array_equal(S.cpu().numpy(), qa["S"])
    assert np.array_equal(host_bits(R), OF.f64_to_bf16_bits(qa["R_S"]))
    r_hat = check_qdq_residual(qa["R_S"], rq)
    wc, ws, gw, _ = OQ.qdq_weights(w)
    ref = OG.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, r_hat, qa["S"], wc, ws,
                              gw, offs)
    e1, e2, ex = assert_gemm_close(host_vals(y), ref)
    say(f"   rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.5f}")


@pytest.mark.parametrize("idx", [4, 5])
def test_full_size_first_gemm_with_quantized_residual(dev, idx):
    # the decode and large-prefill workloads' first GEMM, in the launch
    # configuration the benchmark uses, with the residual quantized again
    cfg = synth.get(idx)
    say(f"workload {cfg.name}: generating")
    wl = synth.make(cfg)
    rng = np.random.default_rng(1)
    x_dev = to_dev_bf16(wl.x)
    w1 = pipeline.prepare_weights(to_dev_bf16(wl.w_first))
    logits = torch.from_numpy(wl.logits).cuda()
    bias = torch.from_numpy(wl.bias).cuda() if wl.bias is not None else None
    say(f"workload {cfg.name}: running the library")
    ids, tw, offs, perm, inv = F.moe_permute(logits, cfg.topk, bias)
    q = F.nvfp4_quantize_act(x_dev)
    S, R = F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"], q["score"],
                                      cfg.k_first)
    rq = F.nvfp4_qdq_residual(R)
    y = F.grouped_w4a4_gemm_rac(q["codes"], q["scales"], q["g"], perm, rq[3], S, w1.packed_codes,
                                w1.packed_scales, w1.g, offs, M_total=perm.numel())
    torch.cuda.synchronize()
    # the quantized residual, in full, teacher-forced on the GPU's R_S (which
    # the full-size pipeline test checks against the oracle)
    say("  residual QDQ (full)")
    R_vals = host_vals(R)
    r_hat = check_qdq_residual(R_vals, rq)
    # sampled GEMM rows
    x = OF.bf16_bits_to_f64(wl.x)
    A = OQ.tensor_amax(x)
    g = OQ.tensor_scale(A)
    S_np = S.cpu().numpy()
    offs_np, perm_np = offs.cpu().numpy(), perm.cpu().numpy()
    rows_p = sample_rows(offs_np, rng)
    say(f"  GEMM rows: {len(rows_p)}")
    wq_host = weight_host(wl.w_first, rng)
    y_h = host_vals(y)
    got, ref = [], []
    for e in np.unique(np.searchsorted(offs_np, rows_p, side="right") - 1):
        ps = rows_p[(rows_p >= offs_np[e]) & (rows_p < offs_np[e + 1])]
        t = perm_np[ps]
        c, s, _, _ = OQ.quantize(x[t], A=A)
        r = OQ.residual(x[t], c, s, g)[:, S_np]
        assert np.array_equal(OF.f64_to_bf16_bits(r), host_bits(R)[t])
        wc, ws, gw = wq_host(e)
        ref.append(OG.grouped_gemm_rac(c, s, g, None, r_hat[t], S_np, wc[None], ws[None],
                                       gw[None], [0, len(ps)]))
        got.append(y_h[ps][:, wq_host.cols])
    e1, e2, ex = assert_gemm_close(np.concatenate(got), np.concatenate(ref))
    say(f"    rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.4f}")


# ------------------------------------------------- per-expert selection

def _routing(rng, M_src, counts, gather):
    offs = np.zeros(len(counts) + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    M_total = int(offs[-1])
    a_rows = rng.integers(0, M_src, M_total).astype(np.int32) if gather else None
    return offs, a_rows, M_total


@pytest.mark.parametrize("M_src,counts,K,k,gather", [
    (64, [64], 512, 16, False),
    (200, [0, 130, 1, 257, 0], 256, 37, True),
    (100, [3, 0, 17, 33, 1, 0, 16, 40], 1024, 64, True),
    (40, [20, 20], 96, 96, True),                        # every channel
    (300, [120, 200, 80], 4096, 128, True),
    (60, [25, 0, 35], 8192, 64, True),                   # two 4096-channel score slices
])
def test_select_per_expert_bitexact(dev, M_src, counts, K, k, gather):
    say(f"select per expert counts={counts} K={K} k={k}")
    rng = np.random.default_rng(M_src + K + k)
    x = heavy_bf16(rng, (M_src, K))
    offs, a_rows, M_total = _routing(rng, M_src, counts, gather)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = F.nvfp4_quantize_act(to_dev_bf16(OF.f64_to_bf16_bits(x)), want_score=False)
    S, R = F.select_residual_channels_per_expert(q["x_used"], q["codes"], q["scales"], q["g"], None,
                                                 k, cu(a_rows) if gather else None, cu(offs),
                                                 M_total=M_total)
    torch.cuda.synchronize()
    codes, scales, g, A = OQ.quantize(x)
    S_ref, R_ref, _ = OQ.select_channels_per_expert(x, codes, scales, g, A, a_rows, offs, k)
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(host_bits(R), OF.f64_to_bf16_bits(R_ref))


@pytest.mark.parametrize("M_src,counts,N,K,k", [
    (64, [64], 512, 512, 16),
    (500, [17, 0, 0, 400, 83], 272, 1024, 128),
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 512, 1024, 64),
    (300, [100, 200], 256, 1024, 256),                  # large k: streamed columns per expert
])
def test_gemm_per_expert(dev, gemm_kernel, M_src, counts, N, K, k):
    say(f"gemm[{gemm_kernel}] per expert counts={counts} N={N} K={K} k={k}")
    rng = np.random.default_rng(sum(counts) + N + K + k + 1)
    E = len(counts)
    x = heavy_bf16(rng, (M_src, K))
    w = OF.round_to_bf16(rng.standard_normal((E, N, K)) * 0.02)
    offs, a_rows, M_total = _routing(rng, M_src, counts, True)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = F.nvfp4_quantize_act(to_dev_bf16(OF.f64_to_bf16_bits(x)), want_score=False)
    S, R = F.select_residual_channels_per_expert(q["x_used"], q["codes"], q["scales"], q["g"], None,
                                                 k, cu(a_rows), cu(offs), M_total=M_total)
    wc, ws, gw, _ = OQ.qdq_weights(w)
    y = F.grouped_w4a4_gemm_rac_per_expert(q["codes"], q["scales"], q["g"], cu(a_rows), R, S,
                                           cu(gemm_wcodes(OQ.pack_codes(wc))), cu(gemm_wscales(ws)), cu(gw),
                                           cu(offs), M_total=M_total)
    torch.cuda.synchronize()
    codes, scales, g, A = OQ.quantize(x)
    S_ref, R_ref, _ = OQ.select_channels_per_expert(x, codes, scales, g, A, a_rows, offs, k)
    assert np.array_equal(S.cpu().numpy(), S_ref)
    ref = OG.grouped_gemm_rac_per_expert(codes, scales, g, a_rows, R_ref, S_ref, wc, ws, gw, offs)
    e1, e2, ex = assert_gemm_close(host_vals(y), ref)
    say(f"   rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.5f}")


def test_full_size_first_gemm_per_expert(dev):
    # the large-prefill workload's first GEMM with per-expert channel sets:
    # S of sampled experts from the oracle's scores over their rows, R and
    # the GEMM on sampled rows
    cfg = synth.get(5)
    say(f"workload {cfg.name}: generating")
    wl = synth.make(cfg)
    rng = np.random.default_rng(3)
    x_dev = to_dev_bf16(wl.x)
    w1 = pipeline.prepare_weights(to_dev_bf16(wl.w_first))
    logits = torch.from_numpy(wl.logits).cuda()
    say(f"workload {cfg.name}: running the library")
    ids, tw, offs, perm, inv = F.moe_permute(logits, cfg.topk, None)
    y, st = pipeline.quantized_linear_rac(x_dev, w1, cfg.k_first, a_rows=perm, offsets=offs,
                                          M_total=perm.numel(), select="per_expert")
    torch.cuda.synchronize()
    x = OF.bf16_bits_to_f64(wl.x)
    A = OQ.tensor_amax(x)
    g = OQ.tensor_scale(A)
    offs_np, perm_np = offs.cpu().numpy(), perm.cpu().numpy()
    S_gpu, R_gpu = st["S"].cpu().numpy(), host_bits(st["R"])
    rows_p = sample_rows(offs_np, rng, n_experts=3)
    wq_host = weight_host(wl.w_first, rng)
    y_h = host_vals(y)
    got, ref = [], []
    for e in np.unique(np.searchsorted(offs_np, rows_p, side="right") - 1):
        say(f"  expert {e}: {offs_np[e + 1] - offs_np[e]} rows")
        t_all = perm_np[offs_np[e]:offs_np[e + 1]]
        c, s, _, _ = OQ.quantize(x[t_all], A=A)
        r = OQ.residual(x[t_all], c, s, g)
        S_e = OQ.select_channels(OQ.channel_scores(r, A), cfg.k_first)
        assert np.array_equal(S_gpu[e], S_e), f"expert {e} S"
        ps = rows_p[(rows_p >= offs_np[e]) & (rows_p < offs_np[e + 1])]
        loc = ps - offs_np[e]
        assert np.array_equal(R_gpu[ps], OF.f64_to_bf16_bits(r[loc][:, S_e]))
        wc, ws, gw = wq_host(e)
        ref.append(OG.grouped_gemm_rac(c[loc], s[loc], g, None, r[loc][:, S_e], S_e, wc[None],
                                       ws[None], gw[None], [0, len(ps)]))
        got.append(y_h[ps][:, wq_host.cols])
    e1, e2, ex = assert_gemm_close(np.concatenate(got), np.concatenate(ref))
    say(f"    rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.4f}")


# ------------------------------------------------- fused SwiGLU output

@pytest.mark.parametrize("M_src,counts,I,K,k", [
    (64, [64], 256, 512, 16),
    (500, [17, 0, 0, 400, 83], 160, 1024, 128),          # I not a multiple of 128: a partial tile
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 256, 1024, 64),
    (300, [100, 200], 128, 512, 256),                     # large k
])
def test_gemm_swiglu_fused(dev, gemm_kernel, monkeypatch, M_src, counts, I, K, k):
    # h from the fused call is bit-identical to the plain GEMM followed by the
    # quantizer's SwiGLU, and within one bf16 step of the oracle's SwiGLU of
    # the oracle's GEMM output.  The fused call never splits K, so the plain
    # GEMM is held to one slice here (a K split sums in another order)
    monkeypatch.setenv("NVFP4RAC_SPLIT", "1")
    say(f"gemm[{gemm_kernel}] swiglu counts={counts} I={I} K={K} k={k}")
    rng = np.random.default_rng(sum(counts) + I + K + k + 7)
    E = len(counts)
    x = heavy_bf16(rng, (M_src, K))
    w = OF.round_to_bf16(rng.standard_normal((E, 2 * I, K)) * 0.02)
    offs, a_rows, M_total = _routing(rng, M_src, counts, True)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = F.nvfp4_quantize_act(to_dev_bf16(OF.f64_to_bf16_bits(x)))
    S, R = F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"], q["score"], k)
    wc, ws, gw, _ = OQ.qdq_weights(w)
    args = (q["codes"], q["scales"], q["g"], cu(a_rows), R, S, cu(gemm_wcodes(OQ.pack_codes(wc))),
            cu(gemm_wscales(ws)), cu(gw), cu(offs))
    h, amax = F.grouped_w4a4_gemm_rac_swiglu(*args, M_total=M_total, with_amax=True)
    y = F.grouped_w4a4_gemm_rac(*args, M_total=M_total)
    hq = F.nvfp4_quantize_act(y, glu=True)
    ha = F.nvfp4_quantize_act_amax(h, amax)
    torch.cuda.synchronize()
    assert h.shape == (M_total, I)
    assert np.array_equal(host_bits(h), host_bits(hq["x_used"]))
    assert int(amax.item()) == int(np.max(host_bits(h) & 0x7FFF))
    for key in ("codes", "scales", "score"):
        assert torch.equal(ha[key], hq[key]), key
    assert np.array_equal(f32_bits(ha["g"].cpu().numpy()), f32_bits(hq["g"].cpu().numpy()))
    qa = OQ.quantize_activation(x, k)
    y_ref = OG.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, qa["R_S"], qa["S"],
                                wc, ws, gw, offs)
    assert_gemm_close(host_vals(y), y_ref)
    h_ref = OM.swiglu(host_vals(y), I)                    # teacher-forced on the GPU's y
    hv = host_vals(h)
    rel = np.abs(hv - h_ref) / np.maximum(np.abs(h_ref), 1e-30)
    assert np.all(rel <= 2.0 ** -7) and np.mean(hv == h_ref) > 0.99


def test_full_size_fused_swiglu_block(dev):
    # the large-prefill block with the SwiGLU fused into the gate+up GEMM:
    # h and the block output bit-identical to the unfused chain
    cfg = synth.get(5)
    say(f"workload {cfg.name}: generating")
    wl = synth.make(cfg)
    x_dev = to_dev_bf16(wl.x)
    w1 = pipeline.prepare_weights(to_dev_bf16(wl.w_first))
    w2 = pipeline.prepare_weights(to_dev_bf16(wl.w_down))
    logits = torch.from_numpy(wl.logits).cuda()
    say("  unfused")
    o0, s0 = pipeline.moe_forward(x_dev, logits, cfg.topk, w1, w2, cfg.k_first, cfg.k_down,
                                  keep=True)
    h0 = host_bits(s0["st2"]["q"]["x_used"])
    o0 = host_bits(o0)
    del s0
    say("  fused")
    o1, s1 = pipeline.moe_forward(x_dev, logits, cfg.topk, w1, w2, cfg.k_first, cfg.k_down,
                                  keep=True, fuse_swiglu=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(s1["y1"]), h0)
    assert np.array_equal(host_bits(o1), o0)
