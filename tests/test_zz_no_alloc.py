"""The allocation-free activation quantizer (nvfp4_quantize_act_noalloc,
fixed device scratch) against nvfp4_quantize_act with a workspace, through
the C ABI: codes, scales, g, channel scores and the SwiGLU tensor h must be
the same bits.  Two calls in a row on the shared scratch, the second with a
smaller input, so that nothing left by the first call reaches the second."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import fp4_quantized_gemm_amd as F
from oracle import formats as OF
from tests.gpu_util import heavy_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc_call(x, glu):
    """The entry point through the C ABI with preallocated outputs."""
    L = F.lib()
    M, C = x.shape
    K = C // 2 if glu else C
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(1, dtype=torch.float32, device=x.device)
    score = torch.empty(K, dtype=torch.uint64, device=x.device)
    h = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if glu else None
    st = L.nvfp4_quantize_act_noalloc(_ptr(x), M, K, C, int(glu), _ptr(codes), _ptr(scales),
                                      _ptr(g), _ptr(score), _ptr(h),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.nvfp4_last_error()
    return dict(codes=codes, scales=scales, g=g, score=score, x_used=h)


def same(a, b):
    return torch.equal(a.view(torch.uint8).reshape(-1), b.view(torch.uint8).reshape(-1))


@pytest.mark.parametrize("glu", [0, 1])
def test_noalloc_matches_workspace_call(dev, glu):
    # the second call is smaller: fewer rows and columns, fewer row groups
    # and column tiles, so stale tickets or partial sums would show
    rng = np.random.default_rng(17 + glu)
    for M, K in [(2048, 4096), (37, 768)]:
        say(f"noalloc glu={glu} M={M} K={K}")
        cols = 2 * K if glu else K
        x = to_dev_bf16(OF.f64_to_bf16_bits(heavy_bf16(rng, (M, cols))))
        got = noalloc_call(x, glu)
        ref = F.nvfp4_quantize_act(x, glu=bool(glu))
        torch.cuda.synchronize()
        for key in ("codes", "scales", "g", "score"):
            assert same(got[key], ref[key]), key
        if glu:
            assert same(got["x_used"], ref["x_used"])


def test_noalloc_scratch_cap_and_wide_rows(dev):
    # a shape whose partial sums the fixed scratch holds only with fewer row
    # groups (K = 65536, the largest taken), then one of the bench's shapes
    rng = np.random.default_rng(23)
    for M, K in [(300, 65536), (256, 4096)]:
        say(f"noalloc M={M} K={K}")
        x = to_dev_bf16(OF.f64_to_bf16_bits(heavy_bf16(rng, (M, K))))
        got = noalloc_call(x, 0)
        ref = F.nvfp4_quantize_act(x)
        torch.cuda.synchronize()
        for key in ("codes", "scales", "g", "score"):
            assert same(got[key], ref[key]), key
