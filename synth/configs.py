"""The five synthetic workloads.

The QUADS pages run a 25B-total / 2.8B-active MoE on reasoning benchmarks
(gist.science technical summary §4) and give no layer shapes; these workloads
stand in for that model's expert blocks: one dense GEMM, an up-projection
MoE block, two gate+up -> SwiGLU -> down MoE blocks (a mid-size and a large
prefill) and a decode-sized step.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    kind: str              # "dense" | "up" | "glu"
    T: int                 # tokens (rows of X)
    H: int                 # hidden (K of the first GEMM)
    E: int                 # experts (1 for dense)
    topk: int
    inter: int             # expert intermediate size I (N of the dense/up GEMM)
    k_first: int           # residual channels for the first GEMM
    k_down: int            # residual channels for the down GEMM (glu only)
    x_dist: str            # "normal_outlier_ch" | "t_lognormal"
    x_df: float = 0.0      # Student-t degrees of freedom
    x_ch_sigma: float = 0.0  # per-channel lognormal(0, sigma) scale
    outlier_channels: tuple = ()
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    w_sigma: float = 0.02
    logit_bias: bool = False
    seed: int = 0

    @property
    def n_first(self) -> int:
        """Output width of the first GEMM: 2I for gate+up, I otherwise."""
        return 2 * self.inter if self.kind == "glu" else self.inter

    @property
    def rows(self) -> int:
        return self.T * self.topk

    def gemm_shapes(self):
        """[(name, M_rows, N, K, k)] for the GEMMs of one forward."""
        out = [("first", self.rows, self.n_first, self.H, self.k_first)]
        if self.kind == "glu":
            out.append(("down", self.rows, self.H, self.inter, self.k_down))
        return out

    def gemm_flops(self):
        """Algorithmic flops of one forward: 2*rows*N*(K + k) per GEMM."""
        return sum(2 * m * n * (k + kk) for _, m, n, k, kk in self.gemm_shapes())


CONFIGS = [
    # 1: single dense GEMM, X 64x512 N(0,1), channels {3,77,200,411} x20,
    #    W 512x512 N(0,0.02), k = 16, seed 0
    Config("dense_64x512x512", "dense", T=64, H=512, E=1, topk=1, inter=512,
           k_first=16, k_down=0, x_dist="normal_outlier_ch",
           outlier_channels=(3, 77, 200, 411), outlier_mult=20.0, w_sigma=0.02),
    # 2: MoE up-projection, 1024 tokens, hidden 2048, 8 experts top-2, I 1024
    Config("moe_up_t1024_h2048_e8", "up", T=1024, H=2048, E=8, topk=2, inter=1024,
           k_first=32, k_down=0, x_dist="t_lognormal", x_df=5.0, x_ch_sigma=0.5,
           w_sigma=0.02),
    # 3: gate+up / SwiGLU / down, 4096 tokens, 128 experts top-8, I 768, biased router
    Config("moe_glu_t4096_h2048_e128", "glu", T=4096, H=2048, E=128, topk=8, inter=768,
           k_first=64, k_down=64, x_dist="t_lognormal", x_df=5.0, x_ch_sigma=0.5,
           w_sigma=0.02, logit_bias=True),
    # 4: decode-sized step, 256 tokens, hidden 4096, 128 experts top-8, I 1536,
    #    1% of channels x30
    Config("moe_decode_t256_h4096_e128", "glu", T=256, H=4096, E=128, topk=8, inter=1536,
           k_first=64, k_down=64, x_dist="normal_outlier_ch", outlier_frac=0.01,
           outlier_mult=30.0, w_sigma=0.02),
    # 5: large prefill, 16384 tokens, hidden 4096, 128 experts top-8, I 1536
    Config("moe_prefill_t16384_h4096_e128", "glu", T=16384, H=4096, E=128, topk=8,
           inter=1536, k_first=128, k_down=128, x_dist="t_lognormal", x_df=3.0,
           x_ch_sigma=1.0, w_sigma=0.015),
]


def get(i_or_name) -> Config:
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name - 1]
    for c in CONFIGS:
        if c.name == i_or_name:
            return c
    raise KeyError(i_or_name)
