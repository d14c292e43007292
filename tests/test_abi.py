"""C-ABI library checks that need no GPU: it loads, exports every function
the header declares, and rejects bad arguments with the documented status
before enqueueing anything."""
import ctypes
import os
import re

import pytest

import fp4_quantized_gemm_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4rac.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WS = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_six_calls():
    names = declared_functions()
    for n in ["nvfp4_qdq_weights", "nvfp4_quantize_act", "select_residual_channels",
              "moe_permute", "grouped_w4a4_gemm_rac", "moe_unpermute_combine"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = F.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert sorted(F.EXPORTED_SYMBOLS) == names


def test_measurement_header_symbols_exported():
    L = F.lib()
    text = open(os.path.join(ROOT, "include", "nvfp4rac_bench.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))
    assert names == sorted(F.BENCH_SYMBOLS)
    for n in names:
        assert hasattr(L, n), n
    assert L.nvfp4_ceiling_mfma_flops(0) == 2 * 32 * 32 * 16
    assert L.nvfp4_ceiling_mfma_flops(3) == 2 * 32 * 32 * 64
    assert L.nvfp4_ceiling_mfma(7, 1, 1, FAKE, None) == ERR_SHAPE
    assert L.nvfp4_ceiling_mfma_operands(2, FAKE, 1, 1, FAKE, None) == ERR_SHAPE
    assert L.nvfp4_ceiling_mfma_operands(0, None, 1, 1, FAKE, None) == ERR_NULL
    assert L.nvfp4_ceiling_mfma(0, 1, 1, None, None) == ERR_NULL
    assert L.nvfp4_ceiling_read(FAKE, 24, FAKE, None) == ERR_SHAPE


def test_version_and_status_strings():
    L = F.lib()
    assert L.nvfp4_version() >= 100
    assert L.nvfp4_status_str(0) == b"NVFP4_OK"
    assert L.nvfp4_status_str(2) == b"NVFP4_ERR_SHAPE"
    assert L.nvfp4_status_str(99) == b"NVFP4_ERR_UNKNOWN"


# Fake, 256-aligned, never-dereferenced addresses: every call below must fail
# validation before it touches memory or launches anything.
FAKE = ctypes.c_void_p(0x10000)
FAKE_MIS = ctypes.c_void_p(0x10001)


def test_quantize_act_validation():
    L = F.lib()
    st = L.nvfp4_quantize_act(FAKE, 4, 48, 48, 0, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None)
    assert st == ERR_SHAPE and b"K" in L.nvfp4_last_error()
    st = L.nvfp4_quantize_act(FAKE, 4, 64, 64, 0, FAKE, FAKE, None, None, None, FAKE, 1 << 20, None)
    assert st == ERR_NULL
    st = L.nvfp4_quantize_act(FAKE, 4, 64, 64, 1, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None)
    assert st == ERR_SHAPE                       # glu needs ldx >= 2K
    st = L.nvfp4_quantize_act(FAKE, 4, 64, 128, 1, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None)
    assert st == ERR_NULL                        # glu needs x_used
    st = L.nvfp4_quantize_act(FAKE_MIS, 4, 64, 64, 0, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None)
    assert st == ERR_ALIGN
    st = L.nvfp4_quantize_act(FAKE, 4, 64, 64, 0, FAKE, FAKE, FAKE, None, None, FAKE, 8, None)
    assert st == ERR_WS


def test_quantize_act_noalloc_validation():
    L = F.lib()
    f = L.nvfp4_quantize_act_noalloc
    assert f(FAKE, 4, 48, 48, 0, FAKE, FAKE, FAKE, None, None, None) == ERR_SHAPE
    assert f(FAKE, 4, 65536 + 32, 65536 + 32, 0, FAKE, FAKE, FAKE, None, None, None) == 5
    assert b"65536" in L.nvfp4_last_error()
    assert f(FAKE, 4, 64, 64, 0, FAKE, FAKE, None, None, None, None) == ERR_NULL
    assert f(FAKE_MIS, 4, 64, 64, 0, FAKE, FAKE, FAKE, None, None, None) == ERR_ALIGN


def test_qdq_weights_validation():
    L = F.lib()
    q = lambda w, E, N, K, pc=None, ps=None, sc=FAKE, ws=1 << 20: L.nvfp4_qdq_weights(
        w, E, N, K, FAKE, sc, FAKE, None, pc, ps, FAKE, ws, None)
    assert q(FAKE, 0, 16, 64) == ERR_SHAPE
    # the packed copy is tiled per 16 rows x 64 columns: N % 16 and K % 64
    assert q(FAKE, 2, 24, 64) == ERR_SHAPE
    assert q(FAKE, 2, 16, 96) == ERR_SHAPE
    assert q(None, 2, 16, 64) == ERR_NULL
    assert q(FAKE, 2, 16, 64, pc=FAKE) == ERR_NULL          # both packed outputs or neither
    assert q(FAKE, 2, 16, 64, pc=FAKE_MIS, ps=FAKE) == ERR_ALIGN
    assert q(FAKE, 2, 16, 64, sc=FAKE_MIS) == ERR_ALIGN
    assert q(FAKE, 2, 16, 64, ws=4) == ERR_WS


def test_pack_weights_validation():
    L = F.lib()
    assert L.nvfp4_pack_weights(FAKE, FAKE, 2, 24, 64, FAKE, FAKE, None) == ERR_SHAPE
    assert L.nvfp4_pack_weights(FAKE, FAKE, 2, 16, 96, FAKE, FAKE, None) == ERR_SHAPE
    assert L.nvfp4_pack_weights(FAKE, None, 2, 16, 64, FAKE, FAKE, None) == ERR_NULL
    assert L.nvfp4_pack_weights(FAKE_MIS, FAKE, 2, 16, 64, FAKE, FAKE, None) == ERR_ALIGN


def test_e2m1_encode_validation():
    L = F.lib()
    assert L.nvfp4_e2m1_encode_f32(None, 0, None, None) == OK          # nothing to do
    assert L.nvfp4_e2m1_encode_f32(FAKE, -1, FAKE, None) == ERR_SHAPE
    assert L.nvfp4_e2m1_encode_f32(None, 4, FAKE, None) == ERR_NULL
    assert L.nvfp4_e2m1_encode_f32(FAKE_MIS, 4, FAKE, None) == ERR_ALIGN


def test_select_validation():
    L = F.lib()
    assert L.select_residual_channels(FAKE, 64, FAKE, FAKE, FAKE, FAKE, 4, 64, 65, FAKE, FAKE,
                                      None, 0, None) == ERR_SHAPE
    assert L.select_residual_channels(FAKE, 32768, FAKE, FAKE, FAKE, FAKE, 4, 32768, 8, FAKE,
                                      FAKE, None, 0, None) == ERR_SHAPE
    # k == 0 is a no-op and needs no pointers at all
    assert L.select_residual_channels(None, 64, None, None, None, None, 4, 64, 0, None, None,
                                      None, 0, None) == OK
    assert L.select_residual_channels(FAKE, 64, FAKE, FAKE, FAKE, None, 4, 64, 3, FAKE, FAKE,
                                      None, 0, None) == ERR_NULL


def test_permute_validation():
    L = F.lib()
    ws = L.moe_permute_workspace_size(10, 8)
    assert ws > 0
    assert L.moe_permute(FAKE, None, 10, 8, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == ERR_SHAPE
    assert L.moe_permute(FAKE, None, 10, 2048, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == ERR_SHAPE
    assert L.moe_permute(FAKE, None, 10, 8, 2, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == ERR_NULL
    assert L.moe_permute(FAKE, None, 10, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == ERR_WS


def test_gemm_validation():
    L = F.lib()
    ws = L.grouped_w4a4_gemm_rac_workspace_size(4, 64, 64, 128, 256, 0)
    args = lambda **kw: [kw.get("ac", FAKE), FAKE, FAKE, kw.get("rows", None), kw.get("msrc", 64),
                         kw.get("R", None), kw.get("S", None), kw.get("k", 0), FAKE, FAKE, FAKE,
                         FAKE, kw.get("E", 4), 64, kw.get("N", 128), kw.get("K", 256), FAKE, FAKE,
                         kw.get("ws", ws), None]
    assert L.grouped_w4a4_gemm_rac(*args(K=192)) == ERR_SHAPE           # K % 128
    assert L.grouped_w4a4_gemm_rac(*args(N=120)) == ERR_SHAPE           # N % 16
    assert L.grouped_w4a4_gemm_rac(*args(k=300)) == ERR_SHAPE           # k > K
    assert L.grouped_w4a4_gemm_rac(*args(msrc=10)) == ERR_SHAPE         # no gather, M_src < M_total
    assert L.grouped_w4a4_gemm_rac(*args(k=4)) == ERR_NULL              # k > 0 needs R_S and S
    assert L.grouped_w4a4_gemm_rac(*args(ac=FAKE_MIS)) == ERR_ALIGN
    # y and R_S take 16-byte vector accesses
    y_mis = args()
    y_mis[16] = ctypes.c_void_p(0x10008)
    assert L.grouped_w4a4_gemm_rac(*y_mis) == ERR_ALIGN
    assert L.grouped_w4a4_gemm_rac(*args(k=4, R=ctypes.c_void_p(0x10008), S=FAKE)) == ERR_ALIGN
    assert L.grouped_w4a4_gemm_rac(*args(ws=0)) == ERR_WS
    assert L.grouped_w4a4_gemm_rac(*args(ws=ws - 256)) == ERR_WS        # below the query


def test_gemm_workspace_covers_the_k_split(monkeypatch):
    # the prefix, the f16 image and, for a problem too small to fill the
    # chip, float32 partials for up to 4 slices of K; a large problem none.
    # The correction's weight columns need no workspace (each tile decodes
    # them from the packed weights).
    L = F.lib()
    monkeypatch.delenv("NVFP4RAC_SPLIT", raising=False)
    E, M_src, M_total, N, K, k = 8, 1024, 2048, 1024, 2048, 32
    base = 256 + ((M_src * K * 2 + 255) // 256) * 256
    small = L.grouped_w4a4_gemm_rac_workspace_size(E, M_src, M_total, N, K, k)
    assert small == base + 4 * M_total * N * 4
    big = 768 + ((16384 * 4096 * 2 + 255) // 256) * 256
    for kk in (0, 37, 128):
        assert L.grouped_w4a4_gemm_rac_workspace_size(128, 16384, 131072, 3072, 4096, kk) == big
    monkeypatch.setenv("NVFP4RAC_SPLIT", "1")
    assert L.grouped_w4a4_gemm_rac_workspace_size(E, M_src, M_total, N, K, k) == base
    monkeypatch.setenv("NVFP4RAC_SPLIT", "2")
    assert L.grouped_w4a4_gemm_rac_workspace_size(E, M_src, M_total, N, K, k) == base + 2 * M_total * N * 4


def test_fp8_validation():
    L = F.lib()
    ws = L.fp8_quantize_workspace_size(2)
    assert L.fp8_quantize(FAKE, 0, 16, 64, FAKE, FAKE, FAKE, ws, None) == ERR_SHAPE     # E >= 1
    assert L.fp8_quantize(FAKE, 2, 16, 60, FAKE, FAKE, FAKE, ws, None) == ERR_SHAPE     # K % 8
    assert L.fp8_quantize(None, 2, 16, 64, FAKE, FAKE, FAKE, ws, None) == ERR_NULL
    assert L.fp8_quantize(FAKE_MIS, 2, 16, 64, FAKE, FAKE, FAKE, ws, None) == ERR_ALIGN
    assert L.fp8_quantize(FAKE, 2, 16, 64, FAKE, FAKE, FAKE, 0, None) == ERR_WS
    gws = L.grouped_fp8_gemm_workspace_size(4)
    args = lambda **kw: [kw.get("a", FAKE), FAKE, kw.get("rows", None), kw.get("msrc", 64), FAKE,
                         FAKE, FAKE, kw.get("E", 4), 64, kw.get("N", 128), kw.get("K", 256), FAKE,
                         FAKE, kw.get("ws", gws), None]
    assert L.grouped_fp8_gemm(*args(K=192)) == ERR_SHAPE      # K % 128
    assert L.grouped_fp8_gemm(*args(N=120)) == ERR_SHAPE      # N % 16
    assert L.grouped_fp8_gemm(*args(E=0)) == ERR_SHAPE
    assert L.grouped_fp8_gemm(*args(msrc=10)) == ERR_SHAPE    # no gather, M_src < M_total
    assert L.grouped_fp8_gemm(*args(a=None)) == ERR_NULL
    assert L.grouped_fp8_gemm(*args(a=FAKE_MIS)) == ERR_ALIGN
    assert L.grouped_fp8_gemm(*args(ws=0)) == ERR_WS


def test_combine_validation():
    L = F.lib()
    assert L.moe_unpermute_combine(FAKE, FAKE, FAKE, 4, 2, 12, FAKE, None) == ERR_SHAPE
    assert L.moe_unpermute_combine(None, FAKE, FAKE, 4, 2, 16, FAKE, None) == ERR_NULL
    assert L.moe_unpermute_combine(None, None, None, 0, 2, 16, None, None) == OK


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(F.NvfpError):
        F.nvfp4_quantize_act(torch.zeros(4, 64, dtype=torch.bfloat16))


def test_qdq_residual_validation():
    L = F.lib()
    ws = L.nvfp4_qdq_residual_workspace_size(8, 32)
    assert ws > 0
    assert L.nvfp4_qdq_residual(FAKE, 8, 24, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == ERR_SHAPE
    assert L.nvfp4_qdq_residual(FAKE, 8, 0, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == ERR_SHAPE
    assert L.nvfp4_qdq_residual(FAKE, 8, 32, FAKE, FAKE, None, FAKE, FAKE, ws, None) == ERR_NULL
    assert L.nvfp4_qdq_residual(FAKE, 8, 32, FAKE, FAKE, FAKE, None, FAKE, ws, None) == ERR_NULL
    assert L.nvfp4_qdq_residual(FAKE_MIS, 8, 32, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == ERR_ALIGN
    assert L.nvfp4_qdq_residual(FAKE, 8, 32, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == ERR_WS


def test_w4a16_gemm_validation():
    L = F.lib()
    ws = L.grouped_w4a16_gemm_workspace_size(4)
    args = lambda **kw: [kw.get("x", FAKE), kw.get("rows", None), kw.get("msrc", 64), FAKE, FAKE,
                         FAKE, FAKE, kw.get("E", 4), 64, kw.get("N", 128), kw.get("K", 256),
                         FAKE, FAKE, kw.get("ws", ws), None]
    assert L.grouped_w4a16_gemm(*args(K=192)) == ERR_SHAPE              # K % 128
    assert L.grouped_w4a16_gemm(*args(K=32768)) == ERR_SHAPE            # K > 16384
    assert L.grouped_w4a16_gemm(*args(N=120)) == ERR_SHAPE              # N % 16
    assert L.grouped_w4a16_gemm(*args(msrc=10)) == ERR_SHAPE            # no gather, M_src < M_total
    assert L.grouped_w4a16_gemm(*args(x=None)) == ERR_NULL
    assert L.grouped_w4a16_gemm(*args(x=FAKE_MIS)) == ERR_ALIGN
    assert L.grouped_w4a16_gemm(*args(ws=0)) == ERR_WS


def test_per_expert_validation():
    L = F.lib()
    ws = L.select_residual_channels_per_expert_workspace_size(4, 64)
    assert ws >= 4 * 64 * 8
    sel = lambda **kw: [FAKE, kw.get("ldx", 64), FAKE, FAKE, FAKE, kw.get("rows", FAKE), FAKE,
                        kw.get("E", 4), 32, 32, kw.get("K", 64), kw.get("k", 8), kw.get("S", FAKE),
                        FAKE, FAKE, kw.get("ws", ws), None]
    assert L.select_residual_channels_per_expert(*sel(k=65)) == ERR_SHAPE
    assert L.select_residual_channels_per_expert(*sel(E=0)) == ERR_SHAPE
    assert L.select_residual_channels_per_expert(*sel(K=32768, ldx=32768)) == ERR_SHAPE
    assert L.select_residual_channels_per_expert(*sel(S=None)) == ERR_NULL
    assert L.select_residual_channels_per_expert(*sel(ws=8)) == ERR_WS
    assert L.select_residual_channels_per_expert(*sel(k=0, S=None, ws=0)) == OK   # no-op
    g = L.grouped_w4a4_gemm_rac_workspace_size(4, 64, 64, 128, 256, 8)
    args = lambda **kw: [FAKE, FAKE, FAKE, None, 64, kw.get("R", FAKE), kw.get("S", FAKE),
                         kw.get("k", 8), FAKE, FAKE, FAKE, FAKE, 4, 64, 128, kw.get("K", 256),
                         FAKE, FAKE, g, None]
    assert L.grouped_w4a4_gemm_rac_per_expert(*args(K=192)) == ERR_SHAPE
    assert L.grouped_w4a4_gemm_rac_per_expert(*args(R=None)) == ERR_NULL


def test_swiglu_gemm_validation():
    L = F.lib()
    ws = L.grouped_w4a4_gemm_rac_swiglu_workspace_size(4, 64, 64, 128, 256, 0)
    assert ws >= L.grouped_w4a4_gemm_rac_workspace_size(4, 64, 64, 128, 256, 0) + 64 * 128 * 2
    args = lambda **kw: [FAKE, FAKE, FAKE, None, 64, None, None, 0, FAKE, FAKE, FAKE, FAKE, 4, 64,
                         kw.get("N", 128), 256, kw.get("h", FAKE), kw.get("amax", None), FAKE,
                         kw.get("ws", ws), None]
    assert L.grouped_w4a4_gemm_rac_swiglu(*args(N=144)) == ERR_SHAPE    # N = 2I, N % 32
    assert L.grouped_w4a4_gemm_rac_swiglu(*args(h=FAKE_MIS)) == ERR_ALIGN
    assert L.grouped_w4a4_gemm_rac_swiglu(*args(amax=FAKE_MIS)) == ERR_ALIGN
    assert L.grouped_w4a4_gemm_rac_swiglu(*args(ws=16)) == ERR_WS
    q = lambda **kw: [FAKE, 4, kw.get("K", 64), kw.get("ldx", 64), kw.get("amax", FAKE), FAKE,
                      FAKE, FAKE, None, FAKE, 1 << 20, None]
    assert L.nvfp4_quantize_act_amax(*q(K=48, ldx=48)) == ERR_SHAPE
    assert L.nvfp4_quantize_act_amax(*q(amax=None)) == ERR_NULL
    assert L.nvfp4_quantize_act_amax(*q(ldx=32)) == ERR_SHAPE
