"""The whole MoE forward captured once as a HIP graph and replayed.

The library allocates nothing, never synchronizes, fills with kernels rather
than memsets and sizes every grid from shapes, so the forward can be
captured (torch.cuda.CUDAGraph is hipGraph on ROCm).  Each replay, with eager
work and synchronizations between the replays, must give the eager result
bit for bit: on the decode-sized kernel path and on the large-tile path with
the SwiGLU fused into the gate+up GEMM."""
import sys

import numpy as np
import pytest
import torch

import fp4_quantized_gemm_amd as F
from fp4_quantized_gemm_amd import pipeline
from oracle import formats as OF
from tests.gpu_util import heavy_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("T,H,E,tk,I,k,fuse", [
    (64, 512, 8, 2, 256, 16, False),          # decode-sized: few rows per expert
    (1024, 512, 4, 2, 256, 32, True),         # large tiles, SwiGLU fused
])
def test_forward_graph_replays_match_eager(dev, T, H, E, tk, I, k, fuse):
    say(f"graph T={T} H={H} E={E} tk={tk} I={I} k={k} fuse={fuse}")
    rng = np.random.default_rng(T + E + k)
    x = to_dev_bf16(OF.f64_to_bf16_bits(heavy_bf16(rng, (T, H))))
    w1 = pipeline.prepare_weights(to_dev_bf16(OF.f64_to_bf16_bits(
        OF.round_to_bf16(rng.standard_normal((E, 2 * I, H)) * 0.02))))
    w2 = pipeline.prepare_weights(to_dev_bf16(OF.f64_to_bf16_bits(
        OF.round_to_bf16(rng.standard_normal((E, H, I)) * 0.02))))
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()

    def fwd():
        return pipeline.moe_forward(x, logits, tk, w1, w2, k, k, fuse_swiglu=fuse)[0]

    ref = fwd().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fwd()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        # eager work between replays, on other inputs
        other = fwd()
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))
