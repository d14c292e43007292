"""Seeded generation of a workload's inputs on the host.

Recipe (one numpy PCG64 stream per input, spawned from SeedSequence(seed) in
the fixed order [X, channel pattern, first weight, down weight, logits,
bias]; each weight stream spawns one child per expert so experts can be
drawn in parallel threads):

  * normal_outlier_ch: X ~ N(0, 1); chosen channels multiplied by a factor
    (a listed set, or round(frac * H) channels from a seeded permutation).
  * t_lognormal: X = StudentT(df) * c_j with c_j ~ lognormal(0, sigma) per
    channel j.
  * W[e] ~ N(0, w_sigma), stored [N][K] (K contiguous).
  * logits ~ N(0, 1) float32 [T][E]; bias ~ N(0, 1) float32 [E] if enabled.

Draws are float32 (float64 for X), then rounded to nearest-even bfloat16 by
torch's CPU cast.  Arrays come back as uint16 bf16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

from .configs import Config


def to_bf16_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _weights(seq: np.random.SeedSequence, E: int, N: int, K: int, sigma: float) -> np.ndarray:
    out = np.empty((E, N, K), dtype=np.uint16)
    kids = seq.spawn(E)

    def one(e):
        rng = np.random.Generator(np.random.PCG64(kids[e]))
        w = rng.standard_normal((N, K), dtype=np.float32)
        w *= np.float32(sigma)
        out[e] = to_bf16_bits(w)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(E)))
    return out


@dataclass
class Workload:
    cfg: Config
    x: np.ndarray            # uint16 bf16 [T][H]
    w_first: np.ndarray      # uint16 bf16 [E][N1][H]
    w_down: np.ndarray       # uint16 bf16 [E][H][I] or None
    logits: np.ndarray       # float32 [T][E] or None (dense)
    bias: np.ndarray         # float32 [E] or None


def make_x(cfg: Config, seq_x, seq_ch, T=None) -> np.ndarray:
    T = cfg.T if T is None else T
    rx = np.random.Generator(np.random.PCG64(seq_x))
    rc = np.random.Generator(np.random.PCG64(seq_ch))
    H = cfg.H
    if cfg.x_dist == "normal_outlier_ch":
        x = rx.standard_normal((T, H))
        if cfg.outlier_channels:
            ch = np.array(cfg.outlier_channels)
        else:
            ch = rc.permutation(H)[: int(round(cfg.outlier_frac * H))]
        x[:, ch] *= cfg.outlier_mult
    elif cfg.x_dist == "t_lognormal":
        c = rc.lognormal(0.0, cfg.x_ch_sigma, size=H)
        x = rx.standard_t(cfg.x_df, size=(T, H)) * c[None, :]
    else:
        raise ValueError(cfg.x_dist)
    return to_bf16_bits(x)


def make(cfg: Config, with_weights: bool = True) -> Workload:
    seqs = np.random.SeedSequence(cfg.seed).spawn(6)
    x = make_x(cfg, seqs[0], seqs[1])
    w1 = w2 = None
    if with_weights:
        w1 = _weights(seqs[2], cfg.E, cfg.n_first, cfg.H, cfg.w_sigma)
        if cfg.kind == "glu":
            w2 = _weights(seqs[3], cfg.E, cfg.H, cfg.inter, cfg.w_sigma)
    logits = bias = None
    if cfg.kind != "dense":
        rl = np.random.Generator(np.random.PCG64(seqs[4]))
        logits = rl.standard_normal((cfg.T, cfg.E), dtype=np.float32)
        if cfg.logit_bias:
            rb = np.random.Generator(np.random.PCG64(seqs[5]))
            bias = rb.standard_normal(cfg.E, dtype=np.float32)
    return Workload(cfg, x, w1, w2, logits, bias)
