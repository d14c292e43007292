"""Parity at the five workloads' full sizes, through the same calls and launch
configuration the benchmark times (fp4_quantized_gemm_amd.pipeline).

The two smaller workloads are checked in full against the oracle chain.  For
the large ones the oracle checks what it can compute in seconds:
  * routing and permutation: in full (bit-exact);
  * weight QDQ: g of every tensor and the codes/scales of sampled rows on a
    few sampled experts (each slice quantized with its expert's amax);
  * activation quantization: sampled rows (with the tensor amax given, so a
    slice quantizes exactly as inside the whole tensor) and the channel scores
    of sampled 16-column blocks, summed over all rows;
  * selection: S is the top-k of the (verified) scores, R_S on sampled rows;
  * GEMMs and combine: sampled output rows (and, for large N, sampled output
    columns), evaluated one by one.
Stages downstream of a GEMM are teacher-forced on the GPU's own output (the
SwiGLU of y1, the combine of y2), since a one-ulp difference upstream can
legitimately move a downstream code.
"""
import sys
import time

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
from tests.gpu_util import (assert_gemm_close, f32_bits, host_bits, host_vals, to_dev_bf16,
                             untile_wcodes, untile_wscales)

pytestmark = pytest.mark.gpu


_T0 = time.time()


def say(msg):
    print(f"[{time.time() - _T0:7.1f}s] {msg}", flush=True)
    sys.stdout.flush()


def _topk_ref(score, k):
    return OQ.select_channels(score, k)


def check_weights(w_bits, wq, experts, rng, n_rows=256):
    g_gpu = wq.g.cpu().numpy()
    for e in range(w_bits.shape[0]):
        # finite bf16 magnitudes order like their 15 low bits
        A = float(OF.bf16_bits_to_f64(np.max(w_bits[e] & 0x7FFF)))
        assert f32_bits(g_gpu[e]) == f32_bits(OQ.tensor_scale(A)), f"expert {e} g"
    for e in experts:
        w = OF.bf16_bits_to_f64(w_bits[e])
        N = w.shape[0]
        r = np.arange(N) if N <= n_rows else np.sort(rng.choice(N, n_rows, replace=False))
        c, s, _, _ = OQ.quantize(w[r], A=OQ.tensor_amax(w))
        c_gpu = wq.codes[e].cpu().numpy()
        assert np.array_equal(OQ.unpack_codes(c_gpu[r]), c), f"expert {e} codes"
        s_gpu = wq.scales[e].cpu().numpy()
        assert np.array_equal(s_gpu[r], s), f"expert {e} scales"
        # the packed copy holds the same bytes
        assert np.array_equal(untile_wcodes(wq.packed_codes[e:e + 1, 0].cpu().numpy())[0][r],
                              c_gpu[r]), f"expert {e} packed codes"
        assert np.array_equal(untile_wscales(wq.packed_scales[e:e + 1, 0].cpu().numpy())[0][r],
                              s_gpu[r]), f"expert {e} packed scales"


def check_activation(x, st, k, rows, blocks):
    """x: host float64 values of the quantized tensor; st: the stage dict."""
    q = st["q"]
    A = OQ.tensor_amax(x)
    g = OQ.tensor_scale(A)
    assert f32_bits(q["g"].cpu().numpy()[0]) == f32_bits(g)
    codes_gpu = q["codes"].cpu().numpy()
    scales_gpu = q["scales"].cpu().numpy()
    c, s, _, _ = OQ.quantize(x[rows], A=A)
    assert np.array_equal(OQ.unpack_codes(codes_gpu[rows]), c)
    assert np.array_equal(scales_gpu[rows], s)
    score_gpu = q["score"].cpu().numpy()
    for b in blocks:
        cols = slice(16 * b, 16 * b + 16)
        cb, sb, _, _ = OQ.quantize(x[:, cols], A=A)
        r = OQ.residual(x[:, cols], cb, sb, g)
        assert np.array_equal(score_gpu[cols], OQ.channel_scores(r, A)), f"scores of block {b}"
    S_gpu = st["S"].cpu().numpy()
    assert np.array_equal(S_gpu, _topk_ref(score_gpu, k))
    # R_S on the sampled rows
    r_rows = OQ.residual(x[rows], c, s, g)
    assert np.array_equal(host_bits(st["R"])[rows], OF.f64_to_bf16_bits(r_rows[:, S_gpu]))
    return A, g, S_gpu


def check_gemm_rows(y_gpu, x, A, g, S, wq_host, offsets, perm, rows_p, R_S_gpu):
    """Oracle rows of the grouped GEMM for permuted rows rows_p, one expert at
    a time, from the oracle's own quantization of the activation rows; only
    the output columns wq_host covers."""
    offs = np.asarray(offsets)
    got, ref = [], []
    for e in np.unique(np.searchsorted(offs, rows_p, side="right") - 1):
        ps = rows_p[(rows_p >= offs[e]) & (rows_p < offs[e + 1])]
        t = perm[ps] if perm is not None else ps
        c, s, _, _ = OQ.quantize(x[t], A=A)
        r = OQ.residual(x[t], c, s, g)[:, S]
        assert np.array_equal(OF.f64_to_bf16_bits(r), host_bits(R_S_gpu)[t])
        wc, ws, gw = wq_host(e)
        yr = OG.grouped_gemm_rac(c, s, g, None, r, S, wc[None], ws[None], gw[None], [0, len(ps)])
        got.append(y_gpu[ps][:, wq_host.cols])
        ref.append(yr)
    return np.concatenate(got), np.concatenate(ref)


N_SAMPLE_ROWS = 64


def run_workload(idx, seed=0):
    cfg = synth.get(idx)
    say(f"workload {cfg.name}: generating")
    wl = synth.make(cfg)
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    x_dev = to_dev_bf16(wl.x)
    w1 = pipeline.prepare_weights(to_dev_bf16(wl.w_first))
    w2 = pipeline.prepare_weights(to_dev_bf16(wl.w_down)) if wl.w_down is not None else None
    say(f"workload {cfg.name}: running the library")
    if cfg.kind == "dense":
        y, st1 = pipeline.quantized_linear_rac(x_dev, w1, cfg.k_first)
        torch.cuda.synchronize()
        return cfg, wl, dict(y1=y, st1=st1), w1, w2, rng
    logits = torch.from_numpy(wl.logits).to(dev)
    bias = torch.from_numpy(wl.bias).to(dev) if wl.bias is not None else None
    out, st = pipeline.moe_forward(x_dev, logits, cfg.topk, w1, w2, cfg.k_first, cfg.k_down,
                                   bias=bias, keep=True)
    torch.cuda.synchronize()
    st["out"] = out
    return cfg, wl, st, w1, w2, rng


def weight_host(wl_bits, rng, n_cols=256, full_below=2 ** 23):
    """Oracle QDQ of output columns `cols` of one expert's weights (rows of
    the [N][K] matrix, quantized with the whole matrix's amax), computed on
    demand, last one kept."""
    N, K = wl_bits.shape[1:]
    cols = np.arange(N) if N * K <= full_below else np.sort(rng.choice(N, n_cols, replace=False))
    cache = {}

    def get(e):
        if e not in cache:
            cache.clear()
            w = OF.bf16_bits_to_f64(wl_bits[e])
            A = OQ.tensor_amax(w)
            c, s, g, _ = OQ.quantize(w[cols], A=A)
            cache[e] = (c, s, np.float32(g))
        return cache[e]
    get.cols = cols
    return get


def sample_rows(offs, rng, n_experts=4, per=16):
    """Up to `per` permuted rows from each of `n_experts` non-empty experts."""
    offs = np.asarray(offs)
    nonempty = np.nonzero(np.diff(offs) > 0)[0]
    picked = rng.choice(nonempty, min(n_experts, len(nonempty)), replace=False)
    rows = []
    for e in picked:
        span = np.arange(offs[e], offs[e + 1])
        rows.append(rng.choice(span, min(per, len(span)), replace=False))
    return np.sort(np.concatenate(rows))


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_full_size_workload(dev, idx):
    cfg, wl, st, w1, w2, rng = run_workload(idx)
    x = OF.bf16_bits_to_f64(wl.x)
    T = cfg.T
    # ---- weights
    experts = sorted(set([0, cfg.E - 1] + list(rng.integers(0, cfg.E, 1))))
    say(f"  weight QDQ on experts {experts}")
    check_weights(wl.w_first, w1, experts, rng)
    if w2 is not None:
        check_weights(wl.w_down, w2, experts, rng)
    # ---- routing
    if cfg.kind != "dense":
        say("  routing / permutation")
        ids, tw = OM.route(wl.logits, cfg.topk, wl.bias)
        offs, perm, inv = OM.permute(ids, cfg.E)
        assert np.array_equal(st["topk_ids"].cpu().numpy(), ids)
        assert np.allclose(st["topk_w"].cpu().numpy(), tw, rtol=1e-6, atol=0)
        assert np.array_equal(st["offsets"].cpu().numpy(), offs)
        assert np.array_equal(st["perm_token"].cpu().numpy(), perm)
        assert np.array_equal(st["inv_perm"].cpu().numpy(), inv)
    else:
        offs, perm = np.array([0, T]), None
    # ---- first activation
    small = T * cfg.H <= 2 ** 24
    rows = np.arange(T) if small else np.sort(rng.choice(T, N_SAMPLE_ROWS, replace=False))
    nb = cfg.H // 16
    blocks = range(nb) if small else sorted(set(rng.choice(nb, 4, replace=False).tolist()))
    say(f"  first activation ({'full' if small else 'sampled'})")
    A1, g1, S1 = check_activation(x, st["st1"], cfg.k_first, rows, blocks)
    # ---- first GEMM
    M1 = cfg.rows
    rows_p = np.arange(M1) if (M1 <= 4096 and cfg.E <= 8) else sample_rows(offs, rng)
    say(f"  first GEMM rows: {len(rows_p)}")
    y1 = host_vals(st["y1"])
    got, ref = check_gemm_rows(y1, x, A1, g1, S1, weight_host(wl.w_first, rng), offs, perm, rows_p,
                               st["st1"]["R"])
    e1, e2, ex = assert_gemm_close(got, ref)
    say(f"    rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.4f}")
    if w2 is None:
        return
    # ---- SwiGLU + second activation (teacher-forced on the GPU's y1)
    h = host_vals(st["st2"]["q"]["x_used"])
    hr = rows_p
    h_ref = OM.swiglu(y1[hr], cfg.inter)
    rel = np.abs(h[hr] - h_ref) / np.maximum(np.abs(h_ref), 1e-30)
    assert np.all(rel <= 2.0 ** -7) and np.mean(h[hr] == h_ref) > 0.99
    small2 = M1 * cfg.inter <= 2 ** 24
    rows2 = np.arange(M1) if small2 else rows_p
    nb2 = cfg.inter // 16
    blocks2 = range(nb2) if small2 else sorted(set(rng.choice(nb2, 4, replace=False).tolist()))
    say(f"  second activation ({'full' if small2 else 'sampled'})")
    A2, g2, S2 = check_activation(h, st["st2"], cfg.k_down, rows2, blocks2)
    # ---- down GEMM
    say("  down GEMM rows")
    y2 = host_vals(st["y2"])
    got, ref = check_gemm_rows(y2, h, A2, g2, S2, weight_host(wl.w_down, rng), offs, None, rows_p,
                               st["st2"]["R"])
    e1, e2, ex = assert_gemm_close(got, ref)
    say(f"    rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.4f}")
    # ---- combine (teacher-forced on the GPU's y2)
    toks = np.arange(T) if T <= 4096 else np.sort(rng.choice(T, N_SAMPLE_ROWS, replace=False))
    inv = st["inv_perm"].cpu().numpy()
    twg = st["topk_w"].cpu().numpy()
    out_ref = OM.combine(y2, inv[toks], twg[toks])
    assert_gemm_close(host_vals(st["out"])[toks], out_ref, min_exact=0.99)
    say("  combine ok")
