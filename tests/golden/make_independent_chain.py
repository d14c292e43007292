"""Writes tests/golden/independent_chain_moe_glu_t4096_h2048_e128.txt: the
oracle's whole-block output (oracle.layer.moe_forward, every stage computed by
the oracle from the seeded synthetic inputs, nothing from the GPU) for a
seeded sample of tokens of the 4096-token, 128-expert gate+up -> SwiGLU ->
down block.  The oracle chain takes minutes on that block, so the GPU test
that reports the library's independent-chain error reads the sample from
here.

    python tests/golden/make_independent_chain.py

Format: comment lines (#), then one line per sampled token: the token index,
then its output row as bf16 bit patterns in hex.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import formats as OF  # noqa: E402
from oracle import layer  # noqa: E402

WORKLOAD = "moe_glu_t4096_h2048_e128"
N_TOKENS = 8
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                   f"independent_chain_{WORKLOAD}.txt")


def sample_tokens(T):
    return np.sort(np.random.default_rng(2024).choice(T, N_TOKENS, replace=False))


def main():
    cfg = synth.get(WORKLOAD)
    wl = synth.make(cfg)
    x = OF.bf16_bits_to_f64(wl.x)
    w1 = OF.bf16_bits_to_f64(wl.w_first)
    w2 = OF.bf16_bits_to_f64(wl.w_down)
    res = layer.moe_forward(x, wl.logits, wl.bias, cfg.topk, w1, w2, cfg.k_first, cfg.k_down)
    toks = sample_tokens(cfg.T)
    bits = OF.f64_to_bf16_bits(res["out"][toks])
    with open(OUT, "w") as f:
        f.write(f"# oracle.layer.moe_forward output rows, workload {WORKLOAD}\n")
        f.write("# (the MoE expert block of the QUADS pages, gist.science technical summary "
                "sections 2.1-2.2 and 4, on the seeded synthetic inputs of synth/)\n")
        f.write("# written by tests/golden/make_independent_chain.py from oracle/ only\n")
        for t, row in zip(toks, bits):
            f.write(f"{int(t)} " + " ".join(f"{int(b):04x}" for b in row) + "\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
