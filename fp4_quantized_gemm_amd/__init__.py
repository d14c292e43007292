"""NVFP4 W4A4 MoE expert GEMM with Residual Activation Compensation for
AMD MI355X (gfx950): Python binding of libnvfp4rac.so.

The binding only marshals arguments: it allocates outputs and workspaces as
torch tensors on the current device, passes raw device pointers and the
current HIP stream to the C ABI declared in include/nvfp4rac.h, and raises on
a non-OK status.  Every step of the path runs in the library's HIP kernels;
there is no fallback: importing the library fails loudly if it is missing.

Calls (same names as the C ABI):
    nvfp4_qdq_weights, nvfp4_quantize_act, select_residual_channels,
    moe_permute, grouped_w4a4_gemm_rac, moe_unpermute_combine
the GEMMs' weight pre-pack for row-major codes quantized elsewhere,
    nvfp4_pack_weights
and, for the variants of the correction, the fused SwiGLU and the
trainer-side W4A16 product,
    nvfp4_qdq_residual, select_residual_channels_per_expert,
    grouped_w4a4_gemm_rac_per_expert, grouped_w4a4_gemm_rac_swiglu,
    grouped_w4a16_gemm
and the FP8 (E4M3) W8A8 baseline the method is compared with,
    fp8_quantize, grouped_fp8_gemm
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

from .build import LIB as LIB_PATH

__all__ = ["lib", "nvfp4_qdq_weights", "nvfp4_pack_weights", "QdqWeights",
           "nvfp4_e2m1_encode_f32", "nvfp4_quantize_act", "nvfp4_quantize_act_noalloc", "select_residual_channels",
           "moe_permute", "grouped_w4a4_gemm_rac", "moe_unpermute_combine", "nvfp4_qdq_residual",
           "grouped_w4a16_gemm", "select_residual_channels_per_expert",
           "grouped_w4a4_gemm_rac_per_expert", "grouped_w4a4_gemm_rac_swiglu",
           "nvfp4_quantize_act_amax", "fp8_quantize", "grouped_fp8_gemm", "NvfpError",
           "EXPORTED_SYMBOLS"]

EXPORTED_SYMBOLS = [
    "nvfp4_version", "nvfp4_status_str", "nvfp4_last_error",
    "nvfp4_qdq_weights_workspace_size", "nvfp4_qdq_weights", "nvfp4_pack_weights",
    "nvfp4_e2m1_encode_f32",
    "nvfp4_quantize_act_workspace_size", "nvfp4_quantize_act", "nvfp4_quantize_act_noalloc",
    "select_residual_channels_workspace_size", "select_residual_channels",
    "moe_permute_workspace_size", "moe_permute",
    "grouped_w4a4_gemm_rac_workspace_size", "grouped_w4a4_gemm_rac",
    "moe_unpermute_combine",
    "nvfp4_qdq_residual_workspace_size", "nvfp4_qdq_residual",
    "grouped_w4a16_gemm_workspace_size", "grouped_w4a16_gemm",
    "select_residual_channels_per_expert_workspace_size", "select_residual_channels_per_expert",
    "grouped_w4a4_gemm_rac_per_expert",
    "grouped_w4a4_gemm_rac_swiglu_workspace_size", "grouped_w4a4_gemm_rac_swiglu",
    "nvfp4_quantize_act_amax",
    "fp8_quantize_workspace_size", "fp8_quantize",
    "grouped_fp8_gemm_workspace_size", "grouped_fp8_gemm",
]


# measurement-only exports (include/nvfp4rac_bench.h)
BENCH_SYMBOLS = ["nvfp4_ceiling_mfma_flops", "nvfp4_ceiling_mfma", "nvfp4_ceiling_mfma_operands",
                 "nvfp4_ceiling_read"]


class NvfpError(RuntimeError):
    pass


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NvfpError(f"{LIB_PATH} is not built; run python -m fp4_quantized_gemm_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    L.nvfp4_version.restype = ctypes.c_int
    L.nvfp4_status_str.restype = ctypes.c_char_p
    L.nvfp4_status_str.argtypes = [ctypes.c_int]
    L.nvfp4_last_error.restype = ctypes.c_char_p
    for name, args in {
        "nvfp4_qdq_weights_workspace_size": [_I64],
        "nvfp4_quantize_act_workspace_size": [_I64, _I64],
        "select_residual_channels_workspace_size": [_I64, _I64, _I64],
        "moe_permute_workspace_size": [_I64, _I64],
        "grouped_w4a4_gemm_rac_workspace_size": [_I64, _I64, _I64, _I64, _I64, _I64],
        "nvfp4_qdq_residual_workspace_size": [_I64, _I64],
        "grouped_w4a16_gemm_workspace_size": [_I64],
        "select_residual_channels_per_expert_workspace_size": [_I64, _I64],
        "grouped_w4a4_gemm_rac_swiglu_workspace_size": [_I64, _I64, _I64, _I64, _I64, _I64],
        "fp8_quantize_workspace_size": [_I64],
        "grouped_fp8_gemm_workspace_size": [_I64],
    }.items():
        f = getattr(L, name)
        f.restype = _SZ
        f.argtypes = args
    sigs = {
        "nvfp4_qdq_weights": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
        "nvfp4_pack_weights": [_P, _P, _I64, _I64, _I64, _P, _P, _P],
        "nvfp4_e2m1_encode_f32": [_P, _I64, _P, _P],
        "nvfp4_quantize_act": [_P, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P, _P, _P, _SZ, _P],
        "nvfp4_quantize_act_noalloc": [_P, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P, _P, _P, _P],
        "select_residual_channels": [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _SZ, _P],
        "moe_permute": [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P],
        "grouped_w4a4_gemm_rac": [_P, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _P, _I64, _I64,
                                  _I64, _I64, _P, _P, _SZ, _P],
        "moe_unpermute_combine": [_P, _P, _P, _I64, _I64, _I64, _P, _P],
        "nvfp4_qdq_residual": [_P, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P],
        "grouped_w4a16_gemm": [_P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _SZ,
                               _P],
        "select_residual_channels_per_expert": [_P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                                _I64, _I64, _P, _P, _P, _SZ, _P],
        "grouped_w4a4_gemm_rac_per_expert": [_P, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _P,
                                             _I64, _I64, _I64, _I64, _P, _P, _SZ, _P],
        "grouped_w4a4_gemm_rac_swiglu": [_P, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P, _P, _I64,
                                         _I64, _I64, _I64, _P, _P, _P, _SZ, _P],
        "nvfp4_quantize_act_amax": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P],
        "fp8_quantize": [_P, _I64, _I64, _I64, _P, _P, _P, _SZ, _P],
        "grouped_fp8_gemm": [_P, _P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    L.nvfp4_ceiling_mfma_flops.restype = ctypes.c_double
    L.nvfp4_ceiling_mfma_flops.argtypes = [ctypes.c_int]
    L.nvfp4_ceiling_mfma.restype = ctypes.c_int
    L.nvfp4_ceiling_mfma.argtypes = [ctypes.c_int, _I64, _I64, _P, _P]
    L.nvfp4_ceiling_mfma_operands.restype = ctypes.c_int
    L.nvfp4_ceiling_mfma_operands.argtypes = [ctypes.c_int, _P, _I64, _I64, _P, _P]
    L.nvfp4_ceiling_read.restype = ctypes.c_int
    L.nvfp4_ceiling_read.argtypes = [_P, _I64, _P, _P]
    _lib = L
    return L


def lib():
    return _load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev=None):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(status, name):
    if status != 0:
        L = _load()
        raise NvfpError(f"{name}: {L.nvfp4_status_str(status).decode()}: "
                        f"{L.nvfp4_last_error().decode()}")


def _wshape(w_codes):
    """(E, N) of packed weight codes [E][2][N/16][K/64][16][32] (the shape the
    packed outputs of nvfp4_qdq_weights and nvfp4_pack_weights carry: per
    expert the code tiles, then the same bytes' worth of channel-major
    codes)."""
    if w_codes.dim() != 6 or w_codes.shape[1] != 2 or tuple(w_codes.shape[4:]) != (16, 32):
        raise NvfpError("weight codes must be the packed copy [E][2][N/16][K/64][16][32] "
                        "(nvfp4_qdq_weights' packed outputs or nvfp4_pack_weights)")
    return int(w_codes.shape[0]), int(w_codes.shape[2]) * 16


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _need(t, dtype, name):
    if not t.is_cuda:
        raise NvfpError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise NvfpError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise NvfpError(f"{name} must be contiguous")


class QdqWeights(NamedTuple):
    """Outputs of nvfp4_qdq_weights."""
    codes: torch.Tensor                    # [E][N][K/2] u8, row-major E2M1 pairs
    scales: torch.Tensor                   # [E][N][K/16] u8, row-major E4M3 block scales
    g: torch.Tensor                        # [E] f32 tensor scales
    qdq: Optional[torch.Tensor]            # [E][N][K] bf16 fake-quantized weight, or None
    # the GEMMs' packed copy: per expert [0] the 512-byte code tiles [N/16][K/64]
    # (bytes ordered [2 column halves][16 rows][16]; viewed as [16][32])
    # (codes) and [..][16][4] (scales), [1] the same sizes holding the
    # channel-major codes [K][N/2] and scales [K/16][N]
    packed_codes: Optional[torch.Tensor]   # [E][2][N/16][K/64][16][32]
    packed_scales: Optional[torch.Tensor]  # [E][2][N/16][K/64][16][4]


def _packed_like(E, N, K, dev):
    return (torch.empty((E, 2, N // 16, K // 64, 16, 32), dtype=torch.uint8, device=dev),
            torch.empty((E, 2, N // 16, K // 64, 16, 4), dtype=torch.uint8, device=dev))


def nvfp4_qdq_weights(w, want_qdq=True, want_packed=True) -> QdqWeights:
    """w [E][N][K] bf16 -> QdqWeights: row-major codes [E][N][K/2] and block
    scales [E][N][K/16], g [E], the bf16 fake-quantized weight (want_qdq),
    and the packed copy the grouped GEMMs take (want_packed)."""
    L = _load()
    _need(w, torch.bfloat16, "w")
    E, N, K = w.shape
    dev = w.device
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((E, N, K // 16), dtype=torch.uint8, device=dev)
    g_w = torch.empty(E, dtype=torch.float32, device=dev)
    w_qdq = torch.empty_like(w) if want_qdq else None
    pc, ps = _packed_like(E, N, K, dev) if want_packed else (None, None)
    ws = _ws(L.nvfp4_qdq_weights_workspace_size(E), dev)
    _check(L.nvfp4_qdq_weights(_ptr(w), E, N, K, _ptr(codes), _ptr(scales), _ptr(g_w),
                               _ptr(w_qdq), _ptr(pc), _ptr(ps), _ptr(ws), ws.numel(),
                               _stream(dev)),
           "nvfp4_qdq_weights")
    return QdqWeights(codes, scales, g_w, w_qdq, pc, ps)


def nvfp4_e2m1_encode_f32(v):
    """E2M1 codes (one per byte) of float32 values v with unit scale: the
    element conversion of every quantizer in the library."""
    L = _load()
    _need(v, torch.float32, "v")
    codes = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(L.nvfp4_e2m1_encode_f32(_ptr(v), v.numel(), _ptr(codes), _stream(v.device)),
           "nvfp4_e2m1_encode_f32")
    return codes


def nvfp4_pack_weights(codes, scales):
    """Row-major codes [E][N][K/2] and scales [E][N][K/16] (u8) -> the
    grouped GEMMs' packed copy (packed_codes, packed_scales)."""
    L = _load()
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    E, N, Kh = codes.shape
    K = 2 * Kh
    if tuple(scales.shape) != (E, N, K // 16):
        raise NvfpError("scales must be [E][N][K/16]")
    pc, ps = _packed_like(E, N, K, codes.device)
    _check(L.nvfp4_pack_weights(_ptr(codes), _ptr(scales), E, N, K, _ptr(pc), _ptr(ps),
                                _stream(codes.device)), "nvfp4_pack_weights")
    return pc, ps


def nvfp4_quantize_act(x, glu=False, want_score=True):
    """x [M][K] bf16 (glu: [M][2K] = [gate | up]) -> dict(codes, scales, g,
    score, x_used).  x_used is x itself for glu=False, else h."""
    L = _load()
    _need(x, torch.bfloat16, "x")
    M, C = x.shape
    K = C // 2 if glu else C
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    score = torch.empty(K, dtype=torch.uint64, device=dev) if want_score else None
    h = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if glu else None
    ws = _ws(L.nvfp4_quantize_act_workspace_size(M, K), dev)
    _check(L.nvfp4_quantize_act(_ptr(x), M, K, C, int(bool(glu)), _ptr(codes), _ptr(scales),
                                _ptr(g), _ptr(score), _ptr(h), _ptr(ws), ws.numel(), _stream(dev)),
           "nvfp4_quantize_act")
    return dict(codes=codes, scales=scales, g=g, score=score, x_used=h if glu else x)


def nvfp4_quantize_act_noalloc(x, glu=False, want_score=True, out=None):
    """nvfp4_quantize_act on the library's fixed device scratch (no
    workspace).  out: optional dict of preallocated codes, scales, g, score
    (and h for glu) tensors to write into, so the call allocates nothing."""
    L = _load()
    _need(x, torch.bfloat16, "x")
    M, C = x.shape
    K = C // 2 if glu else C
    dev = x.device
    o = out or {}
    codes = o.get("codes", None)
    codes = codes if codes is not None else torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = o.get("scales", None)
    scales = scales if scales is not None else torch.empty((M, K // 16), dtype=torch.uint8,
                                                           device=dev)
    g = o.get("g", None)
    g = g if g is not None else torch.empty(1, dtype=torch.float32, device=dev)
    score = o.get("score", None)
    if score is None and want_score:
        score = torch.empty(K, dtype=torch.uint64, device=dev)
    h = o.get("x_used", None) if glu else None
    if glu and h is None:
        h = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    _check(L.nvfp4_quantize_act_noalloc(_ptr(x), M, K, C, int(bool(glu)), _ptr(codes),
                                        _ptr(scales), _ptr(g), _ptr(score), _ptr(h),
                                        _stream(dev)),
           "nvfp4_quantize_act_noalloc")
    return dict(codes=codes, scales=scales, g=g, score=score, x_used=h if glu else x)


def select_residual_channels(x_used, codes, scales, g, score, k):
    """-> (S [k] int32 ascending, R_S [M][k] bf16)."""
    L = _load()
    M, K = x_used.shape
    dev = x_used.device
    S = torch.empty(k, dtype=torch.int32, device=dev)
    R = torch.empty((M, k), dtype=torch.bfloat16, device=dev)
    ws = _ws(L.select_residual_channels_workspace_size(M, K, k), dev)
    _check(L.select_residual_channels(_ptr(x_used), x_used.stride(0), _ptr(codes), _ptr(scales),
                                      _ptr(g), _ptr(score), M, K, k, _ptr(S), _ptr(R), _ptr(ws),
                                      ws.numel(), _stream(dev)),
           "select_residual_channels")
    return S, R


def nvfp4_qdq_residual(R_S):
    """Second-pass NVFP4 quantization of the selected residual R_S [M][k]
    bf16 -> (codes [M][k/2] u8, scales [M][k/16] u8, g_r [1] f32, r_qdq
    [M][k] bf16).  Pass r_qdq as R_S to grouped_w4a4_gemm_rac."""
    L = _load()
    _need(R_S, torch.bfloat16, "R_S")
    M, k = R_S.shape
    dev = R_S.device
    codes = torch.empty((M, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, k // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    r_qdq = torch.empty_like(R_S)
    ws = _ws(L.nvfp4_qdq_residual_workspace_size(M, k), dev)
    _check(L.nvfp4_qdq_residual(_ptr(R_S), M, k, _ptr(codes), _ptr(scales), _ptr(g), _ptr(r_qdq),
                                _ptr(ws), ws.numel(), _stream(dev)),
           "nvfp4_qdq_residual")
    return codes, scales, g, r_qdq


def moe_permute(logits, topk, bias=None):
    """logits [T][E] f32 -> (topk_ids [T][tk] i32, topk_w [T][tk] f32,
    expert_offsets [E+1] i32, perm_token [T*tk] i32, inv_perm [T][tk] i32)."""
    L = _load()
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * topk, dtype=torch.int32, device=dev)
    inv = torch.empty((T, topk), dtype=torch.int32, device=dev)
    ws = _ws(L.moe_permute_workspace_size(T, E), dev)
    _check(L.moe_permute(_ptr(logits), _ptr(bias), T, E, topk, _ptr(ids), _ptr(w), _ptr(offs),
                         _ptr(perm), _ptr(inv), _ptr(ws), ws.numel(), _stream(dev)),
           "moe_permute")
    return ids, w, offs, perm, inv


def select_residual_channels_per_expert(x_used, codes, scales, g, score_unused, k, a_rows,
                                        expert_offsets, M_total=None):
    """Per-expert selection -> (S [E][k] int32, R [M_total][k] bf16 by
    permuted row).  score_unused is accepted for symmetry with
    select_residual_channels and ignored (the per-expert scores are formed
    from the activation itself)."""
    L = _load()
    M_src, K = x_used.shape
    E = int(expert_offsets.numel()) - 1
    if M_total is None:
        M_total = int(a_rows.numel()) if a_rows is not None else M_src
    dev = x_used.device
    S = torch.empty((E, k), dtype=torch.int32, device=dev)
    R = torch.empty((M_total, k), dtype=torch.bfloat16, device=dev)
    ws = _ws(L.select_residual_channels_per_expert_workspace_size(E, K), dev)
    _check(L.select_residual_channels_per_expert(
        _ptr(x_used), x_used.stride(0), _ptr(codes), _ptr(scales), _ptr(g), _ptr(a_rows),
        _ptr(expert_offsets), E, M_src, M_total, K, k, _ptr(S), _ptr(R), _ptr(ws), ws.numel(),
        _stream(dev)), "select_residual_channels_per_expert")
    return S, R


def _gemm_rac(fn_name, a_codes, a_scales, g_x, a_rows, R, S, w_codes, w_scales, g_w,
              expert_offsets, M_total, out, glu=False, h_amax=None):
    L = _load()
    M_src, Kh = a_codes.shape
    K = Kh * 2
    E, N = _wshape(w_codes)
    k = 0 if S is None else int(S.shape[-1])
    if M_total is None:
        M_total = int(a_rows.numel()) if a_rows is not None else M_src
    dev = a_codes.device
    cols = N // 2 if glu else N
    y = out if out is not None else torch.empty((M_total, cols), dtype=torch.bfloat16, device=dev)
    wsq = (L.grouped_w4a4_gemm_rac_swiglu_workspace_size if glu
           else L.grouped_w4a4_gemm_rac_workspace_size)
    ws = _ws(wsq(E, M_src, M_total, N, K, k), dev)
    tail = [_ptr(y), _ptr(h_amax)] if glu else [_ptr(y)]
    _check(getattr(L, fn_name)(_ptr(a_codes), _ptr(a_scales), _ptr(g_x), _ptr(a_rows), M_src,
                               _ptr(R) if k else None, _ptr(S) if k else None, k,
                               _ptr(w_codes), _ptr(w_scales), _ptr(g_w), _ptr(expert_offsets),
                               E, M_total, N, K, *tail, _ptr(ws), ws.numel(), _stream(dev)),
           fn_name)
    return y


def grouped_w4a4_gemm_rac_swiglu(a_codes, a_scales, g_x, a_rows, R_S, S, w_codes, w_scales, g_w,
                                 expert_offsets, M_total=None, out=None, with_amax=False):
    """h [M_total][N/2] bf16 = SwiGLU of the grouped W4A4 GEMM plus correction,
    whose weights' N rows are [gate | up].  with_amax=True returns (h, amax)
    with amax [1] int32 holding max |h| as bf16 bits."""
    amax = torch.empty(1, dtype=torch.int32, device=a_codes.device) if with_amax else None
    h = _gemm_rac("grouped_w4a4_gemm_rac_swiglu", a_codes, a_scales, g_x, a_rows, R_S, S,
                  w_codes, w_scales, g_w, expert_offsets, M_total, out, glu=True, h_amax=amax)
    return (h, amax) if with_amax else h


def nvfp4_quantize_act_amax(x, amax, want_score=True):
    """nvfp4_quantize_act (glu=False) with the tensor amax given as bf16 bits
    in a [1] int32 device tensor (from grouped_w4a4_gemm_rac_swiglu)."""
    L = _load()
    _need(x, torch.bfloat16, "x")
    M, K = x.shape
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    score = torch.empty(K, dtype=torch.uint64, device=dev) if want_score else None
    ws = _ws(L.nvfp4_quantize_act_workspace_size(M, K), dev)
    _check(L.nvfp4_quantize_act_amax(_ptr(x), M, K, x.stride(0), _ptr(amax), _ptr(codes),
                                     _ptr(scales), _ptr(g), _ptr(score), _ptr(ws), ws.numel(),
                                     _stream(dev)),
           "nvfp4_quantize_act_amax")
    return dict(codes=codes, scales=scales, g=g, score=score, x_used=x)


def grouped_w4a4_gemm_rac_per_expert(a_codes, a_scales, g_x, a_rows, R_P, S_E, w_codes,
                                     w_scales, g_w, expert_offsets, M_total=None, out=None):
    """grouped_w4a4_gemm_rac with S_E [E][k] and R_P [M_total][k] by permuted row."""
    return _gemm_rac("grouped_w4a4_gemm_rac_per_expert", a_codes, a_scales, g_x, a_rows, R_P,
                     S_E, w_codes, w_scales, g_w, expert_offsets, M_total, out)


def grouped_w4a4_gemm_rac(a_codes, a_scales, g_x, a_rows, R_S, S, w_codes, w_scales, g_w,
                          expert_offsets, M_total=None, out=None):
    """Y [M_total][N] bf16 for the expert-grouped W4A4 GEMM plus the residual
    correction on the channels S (k = len(S), 0 disables it)."""
    return _gemm_rac("grouped_w4a4_gemm_rac", a_codes, a_scales, g_x, a_rows, R_S, S, w_codes,
                     w_scales, g_w, expert_offsets, M_total, out)


def grouped_w4a16_gemm(x, a_rows, w_codes, w_scales, g_w, expert_offsets, M_total=None,
                       out=None):
    """Y [M_total][N] bf16 = x (bf16, gathered by a_rows) times the
    dequantized NVFP4 weights of each row's expert: the trainer-side W4A16
    product."""
    L = _load()
    _need(x, torch.bfloat16, "x")
    M_src, K = x.shape
    E, N = _wshape(w_codes)
    if M_total is None:
        M_total = int(a_rows.numel()) if a_rows is not None else M_src
    dev = x.device
    y = out if out is not None else torch.empty((M_total, N), dtype=torch.bfloat16, device=dev)
    ws = _ws(L.grouped_w4a16_gemm_workspace_size(E), dev)
    _check(L.grouped_w4a16_gemm(_ptr(x), _ptr(a_rows), M_src, _ptr(w_codes), _ptr(w_scales),
                                _ptr(g_w), _ptr(expert_offsets), E, M_total, N, K, _ptr(y),
                                _ptr(ws), ws.numel(), _stream(dev)),
           "grouped_w4a16_gemm")
    return y


def fp8_quantize(x, stacked=False):
    """FP8 (E4M3) codes of x with one float32 scale per tensor.
    x bf16 [M][K], or with stacked=True [E][N][K] with one scale per x[e]
    (the weights of one expert).  Returns (codes uint8 of x's shape,
    g float32 [1] or [E])."""
    L = _load()
    _need(x, torch.bfloat16, "x")
    if not x.is_contiguous():
        raise NvfpError("x must be contiguous")
    if stacked:
        E, M, K = x.shape
    else:
        (M, K), E = x.shape, 1
    dev = x.device
    codes = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    g = torch.empty(E, dtype=torch.float32, device=dev)
    ws = _ws(L.fp8_quantize_workspace_size(E), dev)
    _check(L.fp8_quantize(_ptr(x), E, M, K, _ptr(codes), _ptr(g), _ptr(ws), ws.numel(),
                          _stream(dev)), "fp8_quantize")
    return codes, g


def grouped_fp8_gemm(a, g_x, a_rows, w, g_w, expert_offsets, M_total=None, out=None):
    """Y [M_total][N] bf16 = g_x g_w[e] (a gathered by a_rows) times the
    E4M3 weights w [E][N][K] of each row's expert: the FP8 W8A8 baseline."""
    L = _load()
    _need(a, torch.uint8, "a")
    _need(w, torch.uint8, "w")
    M_src, K = a.shape
    E, N, _ = w.shape
    if M_total is None:
        M_total = int(a_rows.numel()) if a_rows is not None else M_src
    dev = a.device
    y = out if out is not None else torch.empty((M_total, N), dtype=torch.bfloat16, device=dev)
    ws = _ws(L.grouped_fp8_gemm_workspace_size(E), dev)
    _check(L.grouped_fp8_gemm(_ptr(a), _ptr(g_x), _ptr(a_rows), M_src, _ptr(w), _ptr(g_w),
                              _ptr(expert_offsets), E, M_total, N, K, _ptr(y), _ptr(ws),
                              ws.numel(), _stream(dev)),
           "grouped_fp8_gemm")
    return y


def moe_unpermute_combine(y, inv_perm, topk_w, out=None):
    L = _load()
    T, tk = inv_perm.shape
    N = y.shape[1]
    o = out if out is not None else torch.empty((T, N), dtype=torch.bfloat16, device=y.device)
    _check(L.moe_unpermute_combine(_ptr(y), _ptr(inv_perm), _ptr(topk_w), T, tk, N, _ptr(o),
                                   _stream(y.device)),
           "moe_unpermute_combine")
    return o
