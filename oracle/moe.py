"""MoE routing, expert-major permutation, SwiGLU and the weighted combine.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The QUADS pages name the model family (a Mixture-of-Experts LLM, 25B total
with 2.8B active, gist.science technical summary §1 and §4) but describe no
router.  The readings here are the plainest ones: top-k experts of
(logit + bias) per token, ties to the lower expert index, softmax over the k
chosen values; rows grouped expert by expert with tokens ascending inside an
expert; gate and up concatenated along the output dimension.
"""
from __future__ import annotations

import numpy as np

from .formats import round_to_bf16


def route(logits, topk: int, bias=None):
    """logits float32 [T][E] (+ bias float32 [E]) -> topk_ids int32 [T][topk],
    topk_w float32 [T][topk].

    l' = float32(logit + bias).  Experts are taken in order of (l'
    descending, index ascending).  Weights are the softmax over the chosen
    l' values, evaluated in float64 and rounded once to float32."""
    lp = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        lp = (lp + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    T, E = lp.shape
    if not 1 <= topk <= E:
        raise ValueError("topk out of range")
    # a stable sort on the negated key keeps the lower index first among equals
    order = np.argsort(-lp, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(lp, order, axis=1).astype(np.float64)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def permute(topk_ids, E: int):
    """Expert-major row order.  Returns expert_offsets int32 [E+1],
    perm_token int32 [T*topk] (row p came from token perm_token[p]) and
    inv_perm int32 [T][topk] (slot j of token t went to row inv_perm[t][j])."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, tk = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in ids.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_token = np.zeros(T * tk, dtype=np.int64)
    inv_perm = np.zeros((T, tk), dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):                                   # tokens ascending ...
        for j in range(tk):
            e = ids[t, j]
            p = fill[e]                                  # ... within each expert
            fill[e] += 1
            perm_token[p] = t
            inv_perm[t, j] = p
    return offsets.astype(np.int32), perm_token.astype(np.int32), inv_perm.astype(np.int32)


def swiglu(y_gu, inter: int):
    """h = bf16(silu(gate) * up), gate = y[:, :I], up = y[:, I:], evaluated in
    float64 from the bf16 inputs and rounded once."""
    y = np.asarray(y_gu, dtype=np.float64)
    gate, up = y[:, :inter], y[:, inter:2 * inter]
    return round_to_bf16(gate / (1.0 + np.exp(-gate)) * up)


def combine(y, inv_perm, topk_w):
    """out[t] = bf16(sum_j topk_w[t][j] * y[inv_perm[t][j]]), float64 sum."""
    y = np.asarray(y, dtype=np.float64)
    inv = np.asarray(inv_perm, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    out = np.zeros((inv.shape[0], y.shape[1]), dtype=np.float64)
    for j in range(inv.shape[1]):
        out += w[:, j:j + 1] * y[inv[:, j]]
    return round_to_bf16(out)
