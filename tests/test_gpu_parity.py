"""GPU parity: every library call against the CPU oracle, stage by stage, on
seeded inputs that span several tiles, ragged tails and degenerate cases.

Bit-exact: codes, scales, tensor scales, channel scores, S, R_S, routing ids,
offsets and permutations, w_qdq.  Tolerance: softmax weights (1e-6 rel),
SwiGLU h (1 bf16 ulp), GEMM and combine outputs (row-normwise and max-abs
relative error <= 2e-3 against the oracle's bf16-rounded float64 result)."""
import sys

import numpy as np
import pytest
import torch

import fp4_quantized_gemm_amd as F
from oracle import formats as OF
from oracle import gemm as OG
from oracle import moe as OM
from oracle import nvfp4 as OQ
from tests.gpu_util import (assert_gemm_close, f32_bits, heavy_bf16, host_bits, host_vals,
                            channel_major_codes, gemm_wcodes, gemm_wscales, to_dev_bf16, untile_wcodes,
                            untile_wscales)

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_quant(x_vals, glu=False):
    xd = to_dev_bf16(OF.f64_to_bf16_bits(x_vals))
    q = F.nvfp4_quantize_act(xd, glu=glu)
    torch.cuda.synchronize()
    return q


def check_quant_against_oracle(q, x_vals):
    codes, scales, g, A = OQ.quantize(x_vals)
    got_codes = OQ.unpack_codes(q["codes"].cpu().numpy())
    assert np.array_equal(got_codes, codes), f"codes differ at {np.argwhere(got_codes != codes)[:5]}"
    assert np.array_equal(q["scales"].cpu().numpy(), scales)
    assert f32_bits(q["g"].cpu().numpy()[0]) == f32_bits(g)
    r = OQ.residual(x_vals, codes, scales, g)
    score = OQ.channel_scores(r, A)
    assert np.array_equal(q["score"].cpu().numpy(), score)
    return codes, scales, g, A, r, score


# ---------------------------------------------------------- E2M1 conversion

def test_e2m1_device_encoder_sweep(dev):
    # the hardware conversion every quantizer uses, over a fixed strided sweep
    # of all finite float32 bit patterns (every binade, normals, subnormals,
    # both signs) and the +-64-ulp neighbourhood of every grid point, every
    # midpoint between grid points and the saturation region, against the
    # oracle's nearest-point rule (ties to the even code, saturating, sign kept)
    say("e2m1 encoder sweep")
    pats = np.arange(0, 2 ** 32, 1021, dtype=np.uint64).astype(np.uint32)
    marks = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 8, 1e30],
                     dtype=np.float32).view(np.uint32)
    near = (marks[:, None].astype(np.int64) + np.arange(-64, 65)[None, :]).reshape(-1)
    near = near[near >= 0].astype(np.uint32)
    pats = np.concatenate([pats, near, near | np.uint32(0x80000000)])
    pats = pats[((pats >> 23) & 0xFF) != 0xFF]                    # finite values only
    v = pats.view(np.float32)
    got = F.nvfp4_e2m1_encode_f32(torch.from_numpy(v).cuda()).cpu().numpy()
    want = OF.e2m1_encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first {v[bad[:5]]} -> {got[bad[:5]]} want {want[bad[:5]]}"
    say(f"   {v.size} values bit-exact")


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (37, 512), (130, 768), (64, 4096), (3, 8192)])
def test_quantize_act_bitexact(dev, M, K):
    say(f"quantize M={M} K={K}")
    rng = np.random.default_rng(M * 1000 + K)
    x = heavy_bf16(rng, (M, K))
    check_quant_against_oracle(gpu_quant(x), x)


def test_quantize_act_edge_values(dev):
    say("quantize edge values")
    # hand-worked ties (A = 6 so rho = 1 in the first block), negative zeros,
    # an all-zero block, tiny blocks with subnormal E4M3 scales, saturation
    row = [6, -0.3, 0.25, 0.75, 1.25, 1.75, 2.5, -3.5, 5, 4.9, 0, 1, 2, 3, 4, -6]
    x = np.zeros((4, 64))
    x[0, :16] = row
    x[1, :16] = -0.0
    x[1, 16:32] = [2.0 ** -12 * (i + 1) for i in range(16)]
    x[2, 32:48] = 1e-3
    x[3, 48:64] = np.linspace(-6, 6, 16)
    x = OF.round_to_bf16(x)
    x[1, :16] = -0.0
    check_quant_against_oracle(gpu_quant(x), x)


def test_quantize_act_zero_and_empty(dev):
    say("quantize zeros / empty")
    x = np.zeros((3, 64))
    q = gpu_quant(x)
    assert not q["codes"].cpu().numpy().any() and not q["scales"].cpu().numpy().any()
    assert q["g"].item() == 0.0 and not q["score"].cpu().numpy().any()
    xd = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = F.nvfp4_quantize_act(xd)
    torch.cuda.synchronize()
    assert q["g"].item() == 0.0 and not q["score"].cpu().numpy().any()


@pytest.mark.parametrize("M,I", [(7, 32), (100, 768), (33, 1536)])
def test_quantize_glu(dev, M, I):
    say(f"quantize glu M={M} I={I}")
    rng = np.random.default_rng(M + I)
    y = OF.round_to_bf16(rng.standard_normal((M, 2 * I)) * 2)
    q = gpu_quant(y, glu=True)
    h_gpu = host_vals(q["x_used"])
    h_ref = OM.swiglu(y, I)
    rel = np.abs(h_gpu - h_ref) / np.maximum(np.abs(h_ref), 1e-30)
    assert np.all(rel <= 2.0 ** -7)                      # at most one bf16 step
    assert np.mean(h_gpu == h_ref) > 0.99
    check_quant_against_oracle(q, h_gpu)                 # teacher-forced on the GPU's h


@pytest.mark.parametrize("E,N,K", [(1, 16, 64), (3, 48, 192), (2, 144, 512), (40, 32, 128),
                                   (6, 256, 1536)])
def test_qdq_weights_bitexact(dev, E, N, K):
    say(f"qdq E={E} N={N} K={K}")
    rng = np.random.default_rng(E * N + K)
    w = OF.round_to_bf16(rng.standard_normal((E, N, K)) * 0.02)
    w[0, 0, :16] = 0.0
    if E > 3:
        w[2] = 0.0                                   # an all-zero expert: g = 0, codes 0
    wd = to_dev_bf16(OF.f64_to_bf16_bits(w))
    codes, scales, g_w, w_qdq, pc, ps = F.nvfp4_qdq_weights(wd, want_qdq=True)
    torch.cuda.synchronize()
    rc, rs, rg, rq = OQ.qdq_weights(w)
    # row-major codes and scales, compared with the oracle directly
    assert codes.shape == (E, N, K // 2) and scales.shape == (E, N, K // 16)
    assert np.array_equal(codes.cpu().numpy(), OQ.pack_codes(rc))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(f32_bits(g_w.cpu().numpy()), f32_bits(rg))
    assert np.array_equal(host_bits(w_qdq), OF.f64_to_bf16_bits(rq))
    # the GEMMs' packed copy: the same bytes, permuted into tiles, then the
    # channel-major copy
    assert pc.shape == (E, 2, N // 16, K // 64, 16, 32)
    assert np.array_equal(untile_wcodes(pc[:, 0].cpu().numpy()), OQ.pack_codes(rc))
    assert ps.shape == (E, 2, N // 16, K // 64, 16, 4)
    assert np.array_equal(untile_wscales(ps[:, 0].cpu().numpy()), rs)
    assert np.array_equal(pc[:, 1].cpu().numpy().reshape(E, K, N // 2),
                          channel_major_codes(OQ.pack_codes(rc)))
    assert np.array_equal(ps[:, 1].cpu().numpy().reshape(E, K // 16, N), rs.transpose(0, 2, 1))
    # nvfp4_pack_weights of the row-major outputs gives the same packed copy
    pc2, ps2 = F.nvfp4_pack_weights(codes, scales)
    assert torch.equal(pc2, pc) and torch.equal(ps2, ps)
    # without the packed copy, the row-major outputs are unchanged
    q2 = F.nvfp4_qdq_weights(wd, want_qdq=False, want_packed=False)
    assert q2.packed_codes is None and torch.equal(q2.codes, codes) and torch.equal(q2.scales, scales)


# ------------------------------------------------------------------ selection

@pytest.mark.parametrize("M,K,k", [(9, 64, 1), (50, 512, 16), (20, 768, 64), (4, 96, 96), (300, 4096, 128),
                                   (6, 8192, 100), (3, 16384, 300),
                                   (256, 4096, 64),    # the decode block's first selection
                                   (257, 1024, 64)])
def test_select_residual_bitexact(dev, M, K, k):
    say(f"select M={M} K={K} k={k}")
    rng = np.random.default_rng(M + K + k)
    x = heavy_bf16(rng, (M, K))
    q = gpu_quant(x)
    S, R = F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"], q["score"], k)
    torch.cuda.synchronize()
    ref = OQ.quantize_activation(x, k)
    assert np.array_equal(S.cpu().numpy(), ref["S"])
    assert np.array_equal(host_bits(R), OF.f64_to_bf16_bits(ref["R_S"]))


def test_select_ties_prefer_lower_index(dev):
    say("select ties")
    rng = np.random.default_rng(77)
    x = heavy_bf16(rng, (40, 128))
    x[:, 64:80] = x[:, 0:16]             # equal residuals -> equal scores
    q = gpu_quant(x)
    for k in (1, 5, 17, 40):
        S, _ = F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"], q["score"], k)
        ref = OQ.quantize_activation(x, k)
        assert np.array_equal(S.cpu().numpy(), ref["S"])


# ------------------------------------------------------------- route / permute

@pytest.mark.parametrize("T,E,tk,bias", [(1, 8, 2, False), (63, 8, 1, False), (64, 16, 4, True),
                                         (65, 128, 8, True), (300, 128, 8, False),
                                         (512, 256, 8, True),    # largest one-workgroup case
                                         (513, 128, 8, False),   # smallest multi-kernel case
                                         (1000, 1024, 32, True)])
def test_moe_permute_bitexact(dev, T, E, tk, bias):
    say(f"permute T={T} E={E} tk={tk} bias={bias}")
    rng = np.random.default_rng(T + E + tk)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = 0.25                       # a fully tied token
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    ld = torch.from_numpy(logits).cuda()
    bd = torch.from_numpy(b).cuda() if bias else None
    ids, w, offs, perm, inv = F.moe_permute(ld, tk, bd)
    torch.cuda.synchronize()
    rid, rw = OM.route(logits, tk, b)
    roffs, rperm, rinv = OM.permute(rid, E)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
    assert np.array_equal(offs.cpu().numpy(), roffs)
    assert np.array_equal(perm.cpu().numpy(), rperm)
    assert np.array_equal(inv.cpu().numpy(), rinv)


# ---------------------------------------------------------------------- GEMM

def _gemm_case(rng, M_src, counts, N, K, k, gather):
    E = len(counts)
    x = heavy_bf16(rng, (M_src, K))
    qa = OQ.quantize_activation(x, k)
    w = OF.round_to_bf16(rng.standard_normal((E, N, K)) * 0.02)
    wc, ws, gw, _ = OQ.qdq_weights(w)
    offs = np.zeros(E + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    M_total = int(offs[-1])
    a_rows = rng.integers(0, M_src, M_total).astype(np.int32) if gather else None
    ref = OG.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], a_rows, qa["R_S"], qa["S"],
                              wc, ws, gw, offs)
    cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = F.grouped_w4a4_gemm_rac(
        cu(OQ.pack_codes(qa["codes"])), cu(qa["scales"]), cu(np.array([qa["g"]], np.float32)),
        cu(a_rows) if gather else None,
        to_dev_bf16(OF.f64_to_bf16_bits(qa["R_S"])) if k else None,
        cu(qa["S"]) if k else None,
        cu(gemm_wcodes(OQ.pack_codes(wc))), cu(gemm_wscales(ws)), cu(gw), cu(offs), M_total=M_total)
    torch.cuda.synchronize()
    return host_vals(y), ref


@pytest.mark.parametrize("split", [1, 2, 4])
@pytest.mark.parametrize("M_src,counts,N,K,k,gather", [
    (300, [100, 200], 256, 1024, 128, True),           # correction staged like A (k % 64 == 0)
    (500, [17, 0, 0, 400, 83], 272, 1024, 32, True),  # correction from R rows directly
    (96, [50, 46], 128, 2048, 0, False),
])
def test_gemm_k_split(dev, monkeypatch, split, M_src, counts, N, K, k, gather):
    # the large-tile kernel with K split over 1, 2 or 4 workgroups (float32
    # partials reduced in a fixed order): every split is within the GEMM
    # tolerance of the oracle, and a repeated call is bit-identical
    monkeypatch.setenv("NVFP4RAC_GEMM", "big")
    monkeypatch.setenv("NVFP4RAC_SPLIT", str(split))
    say(f"gemm k-split {split} counts={counts} N={N} K={K} k={k}")
    rng = np.random.default_rng(sum(counts) + N + K + k)
    y, ref = _gemm_case(rng, M_src, counts, N, K, k, gather)
    e1, e2, ex = assert_gemm_close(y, ref)
    rng = np.random.default_rng(sum(counts) + N + K + k)
    y2, _ = _gemm_case(rng, M_src, counts, N, K, k, gather)
    assert np.array_equal(y, y2)
    say(f"   rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.5f}")


@pytest.fixture(params=["generic", "big", "decode"])
def gemm_kernel(request, monkeypatch):
    monkeypatch.setenv("NVFP4RAC_GEMM", request.param)
    return request.param


@pytest.mark.parametrize("M_src,counts,N,K,k,gather", [
    (64, [64], 512, 512, 16, False),                  # the dense 64x512x512 case
    (200, [0, 130, 1, 257], 144, 256, 37, True),      # empty / single-row experts, N and k tails
    (300, [300], 256, 384, 0, False),                 # no compensation
    (96, [50, 46], 128, 256, 256, False),             # every channel compensated
    (500, [17, 0, 0, 400, 83], 272, 1024, 128, True),
    (700, [300, 1, 511, 0, 255], 528, 768, 64, True),  # several 256-row tiles, N tail
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 512, 1024, 64, True),  # decode-sized: 0-40 rows each
    (64, [3, 0, 17, 33, 1, 0, 16, 40], 512, 384, 64, True),   # decode: last chunk of 128 columns
    (48, [20, 9, 0, 19], 256, 640, 64, True),                  # ... with two full chunks before it
    (300, [100, 200], 256, 1024, 256, True),           # large k: two 128-channel chunks
    (500, [17, 0, 0, 400, 83], 272, 1024, 384, True),  # three chunks, N tail
    (96, [50, 46], 128, 512, 512, False),              # large k = K: every channel
])
def test_grouped_gemm_rac(dev, gemm_kernel, M_src, counts, N, K, k, gather):
    say(f"gemm[{gemm_kernel}] counts={counts} N={N} K={K} k={k} gather={gather}")
    rng = np.random.default_rng(sum(counts) + N + K + k)
    y, ref = _gemm_case(rng, M_src, counts, N, K, k, gather)
    e1, e2, ex = assert_gemm_close(y, ref)
    say(f"   rownorm {e1:.2e} maxabs {e2:.2e} exact {ex:.5f}")


def test_grouped_gemm_deterministic(dev, gemm_kernel):
    say("gemm determinism")
    rng = np.random.default_rng(5)
    y1, _ = _gemm_case(rng, 300, [100, 200], 256, 512, 64, True)
    rng = np.random.default_rng(5)
    y2, _ = _gemm_case(rng, 300, [100, 200], 256, 512, 64, True)
    assert np.array_equal(y1, y2)


# ------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,tk,N", [(1, 1, 8), (37, 2, 64), (256, 8, 1024)])
def test_combine(dev, T, tk, N):
    say(f"combine T={T} tk={tk} N={N}")
    rng = np.random.default_rng(T * tk + N)
    y = OF.round_to_bf16(rng.standard_normal((T * tk, N)))
    inv = rng.permutation(T * tk).reshape(T, tk).astype(np.int32)
    w = rng.dirichlet(np.ones(tk), size=T).astype(np.float32)
    out = F.moe_unpermute_combine(to_dev_bf16(OF.f64_to_bf16_bits(y)), torch.from_numpy(inv).cuda(),
                                  torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ref = OM.combine(y, inv, w)
    got = host_vals(out)
    assert_gemm_close(got, ref, min_exact=0.99)
    if tk == 1:
        assert np.array_equal(got, y[inv[:, 0]])
