"""The rollout-side MoE expert block chained from the oracle's pieces.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Order of the steps (gist.science technical summary §2.1-§2.2 and the arXiv
abstract): weights go through the shared QDQ path once; every forward
quantizes its activation online, picks the high-residual channels, and runs
the W4A4 GEMM with the residual added back.  The expert block around it
(route, permute, gate+up, SwiGLU, down, combine) is the ordinary MoE layer.
"""
from __future__ import annotations

from . import gemm, moe, nvfp4


def dense_forward(x, w, k):
    """One dense GEMM Y = X W^T through NVFP4 + residual compensation
    (E = 1, every row belongs to the single expert)."""
    wc, ws, gw, w_qdq = nvfp4.qdq_weights(w[None])
    qa = nvfp4.quantize_activation(x, k)
    M = x.shape[0]
    y = gemm.grouped_gemm_rac(qa["codes"], qa["scales"], qa["g"], None, qa["R_S"], qa["S"],
                              wc, ws, gw, [0, M])
    return dict(act=qa, w=(wc, ws, gw, w_qdq), y=y)


def moe_forward(x, logits, bias, topk, w_first, w_down, k_first, k_down):
    """x [T][H] bf16 values; logits [T][E]; w_first [E][N1][H] (N1 = 2I for
    gate+up, or I for an up-only block); w_down [E][H][I] or None.

    Returns every intermediate so a test can compare stage by stage."""
    E = w_first.shape[0]
    ids, tw = moe.route(logits, topk, bias)
    offs, perm_token, inv_perm = moe.permute(ids, E)
    w1 = nvfp4.qdq_weights(w_first)
    q1 = nvfp4.quantize_activation(x, k_first)
    y1 = gemm.grouped_gemm_rac(q1["codes"], q1["scales"], q1["g"], perm_token, q1["R_S"],
                               q1["S"], w1[0], w1[1], w1[2], offs)
    out = dict(topk_ids=ids, topk_w=tw, offsets=offs, perm_token=perm_token,
               inv_perm=inv_perm, w1=w1, act1=q1, y1=y1)
    if w_down is None:
        return out
    inter = w_down.shape[2]
    h = moe.swiglu(y1, inter)
    w2 = nvfp4.qdq_weights(w_down)
    q2 = nvfp4.quantize_activation(h, k_down)
    y2 = gemm.grouped_gemm_rac(q2["codes"], q2["scales"], q2["g"], None, q2["R_S"], q2["S"],
                               w2[0], w2[1], w2[2], offs)
    out.update(h=h, w2=w2, act2=q2, y2=y2, out=moe.combine(y2, inv_perm, tw))
    return out
