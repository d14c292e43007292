"""The library's whole path against the oracle's whole path, computed
independently: every stage of the oracle runs on the oracle's own outputs, the
library's on its own, and only the final outputs are compared.

Stage by stage the library is held to the oracle bit for bit or within the
GEMM tolerance, with each stage fed the GPU's own input (the other parity
tests).  Chained independently, a GEMM output one bf16 step away from the
oracle's can move a code of the next quantizer, so this comparison is
informational: it prints the errors and applies a loose gate of 5e-2 on the
row-normwise error of the final output (a moved E2M1 code changes one of K
products by up to a grid step, a few percent of a row at K = 768).

The two smaller workloads run the oracle chain here; the 4096-token
128-expert block's oracle chain takes minutes, so its output rows for a
seeded sample of tokens are read from tests/golden (written by
tests/golden/make_independent_chain.py from oracle/ only).
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import synth
from fp4_quantized_gemm_amd import pipeline
from oracle import formats as OF
from oracle import layer
from tests.gpu_util import host_vals, rownorm_err, to_dev_bf16

pytestmark = pytest.mark.gpu

LOOSE = 5e-2
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "independent_chain_moe_glu_t4096_h2048_e128.txt")
_T0 = time.time()


def say(msg):
    print(f"[{time.time() - _T0:7.1f}s] {msg}", flush=True)
    sys.stdout.flush()


def gpu_block(cfg, wl):
    """The block through the library, in the launch configuration the
    benchmark uses (SwiGLU fused where the large-tile kernel forms it)."""
    x = to_dev_bf16(wl.x)
    w1 = pipeline.prepare_weights(to_dev_bf16(wl.w_first))
    if cfg.kind == "dense":
        y, _ = pipeline.quantized_linear_rac(x, w1, cfg.k_first)
        torch.cuda.synchronize()
        return host_vals(y)
    w2 = pipeline.prepare_weights(to_dev_bf16(wl.w_down)) if wl.w_down is not None else None
    logits = torch.from_numpy(wl.logits).cuda()
    bias = torch.from_numpy(wl.bias).cuda() if wl.bias is not None else None
    fuse = w2 is not None and cfg.rows > 48 * cfg.E
    out, _ = pipeline.moe_forward(x, logits, cfg.topk, w1, w2, cfg.k_first, cfg.k_down,
                                  bias=bias, fuse_swiglu=fuse)
    torch.cuda.synchronize()
    return host_vals(out)


def report(name, got, ref):
    e = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    say(f"  {name}: independent-chain row-normwise error max {e.max():.3e} "
        f"median {np.median(e):.3e}; bit-identical elements {np.mean(got == ref):.4f}")
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= LOOSE


@pytest.mark.parametrize("idx", [1, 2])
def test_independent_chain(dev, idx):
    cfg = synth.get(idx)
    say(f"workload {cfg.name}")
    wl = synth.make(cfg)
    got = gpu_block(cfg, wl)
    x = OF.bf16_bits_to_f64(wl.x)
    if cfg.kind == "dense":
        ref = layer.dense_forward(x, OF.bf16_bits_to_f64(wl.w_first[0]), cfg.k_first)["y"]
    else:
        res = layer.moe_forward(x, wl.logits, wl.bias, cfg.topk,
                                OF.bf16_bits_to_f64(wl.w_first), None, cfg.k_first, 0)
        ref = res["y1"]                 # the up-projection block's output (permuted rows)
    report(cfg.name, got, ref)


def test_independent_chain_glu_block_sampled(dev):
    cfg = synth.get("moe_glu_t4096_h2048_e128")
    say(f"workload {cfg.name} (oracle rows from {os.path.basename(GOLDEN)})")
    toks, rows = [], []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            toks.append(int(parts[0]))
            rows.append([int(h, 16) for h in parts[1:]])
    ref = OF.bf16_bits_to_f64(np.array(rows, dtype=np.uint16))
    wl = synth.make(cfg)
    got = gpu_block(cfg, wl)
    assert ref.shape == (len(toks), cfg.H)
    report(cfg.name, got[np.array(toks)], ref)
