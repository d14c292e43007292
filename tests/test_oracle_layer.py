"""Pins for the oracle's whole MoE block, oracle/layer.py (CPU only).

layer.moe_forward chains routing, expert-major permutation, the first
grouped GEMM with the residual correction, SwiGLU, the second quantizer, the
down GEMM and the combine.  These tests restate the block token by token, in
token-major order and without the permutation arrays, from the definitions
of its steps (route -> per (token, slot) product with the routed expert's
dequantized weights -> silu(gate) * up with gate the first I columns ->
product with the second expert weight -> weighted sum over the slots), and
check that the permuted chain gives the same bits.  A mistake in how the
chain wires its pieces (a wrong a_rows for the down GEMM, inv_perm used in
place of perm_token, the expert of a row, the combine's slot weights) makes
the two disagree.  The per-step functions themselves are pinned in the
other oracle tests.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import layer
from oracle import moe as MOE
from oracle import nvfp4 as Q


def _bf16(a):
    return F.round_to_bf16(np.asarray(a, dtype=np.float64))


def _inputs(rng, T, H, E, I, glu=True):
    x = _bf16(rng.standard_t(4, size=(T, H)) * rng.lognormal(0, 0.7, size=H)[None, :])
    w1 = _bf16(rng.standard_normal((E, 2 * I if glu else I, H)) * 0.05)
    w2 = _bf16(rng.standard_normal((E, H, I)) * 0.05) if glu else None
    return x, w1, w2


def _row_product(xhat_row, r_row, S, what):
    """bf16 of one output row: xhat_row . W^T + r_row . W[:, S]^T (float64)."""
    y = what @ xhat_row
    if len(S):
        y = y + what[:, S] @ r_row
    return _bf16(y)


def _token_major_block(x, logits, bias, topk, w1, w2, k1, k2):
    """The block restated in token-major order, one (token, slot) at a time."""
    T = x.shape[0]
    E = w1.shape[0]
    ids, tw = MOE.route(logits, topk, bias)
    c1, s1, g1, _ = Q.qdq_weights(w1)
    w1hat = [Q.dequantize(c1[e], s1[e], g1[e]) for e in range(E)]
    q1 = Q.quantize_activation(x, k1)
    x1hat = Q.dequantize(q1["codes"], q1["scales"], q1["g"])
    y1 = np.zeros((T, topk, w1.shape[1]))
    for t in range(T):
        for j in range(topk):
            y1[t, j] = _row_product(x1hat[t], q1["R_S"][t], q1["S"], w1hat[ids[t, j]])
    if w2 is None:
        return dict(ids=ids, tw=tw, y1=y1)
    I = w2.shape[2]
    gate, up = y1[..., :I], y1[..., I:2 * I]
    h = _bf16(gate / (1.0 + np.exp(-gate)) * up)                     # [T][topk][I]
    # the second quantizer sees every routed row (its amax and channel
    # scores are sums and maxima over rows, so row order does not matter)
    q2 = Q.quantize_activation(h.reshape(T * topk, I), k2)
    h2hat = Q.dequantize(q2["codes"], q2["scales"], q2["g"]).reshape(T, topk, I)
    R2 = q2["R_S"].reshape(T, topk, -1)
    c2, s2, g2, _ = Q.qdq_weights(w2)
    w2hat = [Q.dequantize(c2[e], s2[e], g2[e]) for e in range(E)]
    out = np.zeros((T, w2.shape[1]))
    y2 = np.zeros((T, topk, w2.shape[1]))
    for t in range(T):
        acc = np.zeros(w2.shape[1])
        for j in range(topk):
            y2[t, j] = _row_product(h2hat[t, j], R2[t, j], q2["S"], w2hat[ids[t, j]])
            acc += np.float64(tw[t, j]) * y2[t, j]
        out[t] = _bf16(acc)
    return dict(ids=ids, tw=tw, y1=y1, h=h, y2=y2, out=out, S1=q1["S"], S2=q2["S"])


@pytest.mark.parametrize("T,H,E,topk,I,k1,k2,bias", [
    (12, 64, 3, 2, 32, 8, 8, False),
    (9, 128, 5, 3, 48, 16, 0, True),
    (16, 64, 4, 1, 32, 0, 16, False),
])
def test_moe_forward_equals_the_token_major_block(T, H, E, topk, I, k1, k2, bias):
    rng = np.random.default_rng(T * 1000 + H + E)
    x, w1, w2 = _inputs(rng, T, H, E, I)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    got = layer.moe_forward(x, logits, b, topk, w1, w2, k1, k2)
    want = _token_major_block(x, logits, b, topk, w1, w2, k1, k2)
    perm, inv = got["perm_token"], got["inv_perm"]
    # every permuted row holds the product of its token with its expert
    for t in range(T):
        for j in range(topk):
            p = inv[t, j]
            assert perm[p] == t
            assert np.array_equal(got["y1"][p], want["y1"][t, j])
            assert np.array_equal(got["h"][p], want["h"][t, j])
            assert np.array_equal(got["y2"][p], want["y2"][t, j])
    assert np.array_equal(got["act1"]["S"], want["S1"])
    assert np.array_equal(got["act2"]["S"], want["S2"])
    assert np.array_equal(got["out"], want["out"])
    assert np.any(got["out"] != 0)


def test_up_only_block_equals_the_token_major_product():
    rng = np.random.default_rng(7)
    T, H, E, topk, I, k = 10, 64, 4, 2, 48, 8
    x, w1, _ = _inputs(rng, T, H, E, I, glu=False)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    got = layer.moe_forward(x, logits, None, topk, w1, None, k, 0)
    want = _token_major_block(x, logits, None, topk, w1, None, k, 0)
    assert "out" not in got
    for t in range(T):
        for j in range(topk):
            assert np.array_equal(got["y1"][got["inv_perm"][t, j]], want["y1"][t, j])


def test_single_expert_top1_is_the_dense_chain():
    # E = 1, top-1: every token goes to the one expert with weight 1, the
    # permutation is the identity, the first GEMM is dense_forward's GEMM
    # and the combine copies the down GEMM's rows
    rng = np.random.default_rng(11)
    T, H, I, k = 8, 64, 32, 8
    x, w1, w2 = _inputs(rng, T, H, 1, I)
    logits = rng.standard_normal((T, 1)).astype(np.float32)
    got = layer.moe_forward(x, logits, None, 1, w1, w2, k, k)
    assert np.array_equal(got["perm_token"], np.arange(T))
    assert np.array_equal(got["offsets"], [0, T])
    assert np.all(got["topk_w"] == 1.0)
    dense = layer.dense_forward(x, w1[0], k)
    assert np.array_equal(dense["y"], got["y1"])
    assert np.array_equal(dense["act"]["codes"], got["act1"]["codes"])
    assert np.array_equal(got["out"], got["y2"])
    # dense_forward is the plain definition, row by row
    xhat = Q.dequantize(dense["act"]["codes"], dense["act"]["scales"], dense["act"]["g"])
    wc, ws, gw, _ = dense["w"]
    what = Q.dequantize(wc[0], ws[0], gw[0])
    for m in range(T):
        assert np.array_equal(dense["y"][m], _row_product(xhat[m], dense["act"]["R_S"][m],
                                                          dense["act"]["S"], what))


def test_two_experts_with_hand_routing():
    # tokens 0 and 2 to expert 1, tokens 1 and 3 to expert 0 (top-1, weight
    # 1); then top-2 over the same logits, whose weights are the softmax of
    # the two logits
    rng = np.random.default_rng(5)
    T, H, E, I, k = 4, 64, 2, 32, 8
    x, w1, w2 = _inputs(rng, T, H, E, I)
    logits = np.array([[0.0, 3.0], [2.0, -1.0], [-0.5, 0.25], [1.0, 0.5]], dtype=np.float32)
    got = layer.moe_forward(x, logits, None, 1, w1, w2, k, k)
    assert np.array_equal(got["topk_ids"][:, 0], [1, 0, 1, 0])
    assert np.array_equal(got["offsets"], [0, 2, 4])
    assert np.array_equal(got["perm_token"], [1, 3, 0, 2])
    assert np.array_equal(got["inv_perm"][:, 0], [2, 0, 3, 1])
    # the expert of a token matters: the same block with the experts' weights
    # exchanged and the routing mirrored gives the same output
    mirrored = layer.moe_forward(x, logits[:, ::-1].copy(), None, 1, w1[::-1].copy(),
                                 w2[::-1].copy(), k, k)
    assert np.array_equal(mirrored["out"], got["out"])
    swapped = layer.moe_forward(x, logits, None, 1, w1[::-1].copy(), w2[::-1].copy(), k, k)
    assert not np.array_equal(swapped["out"], got["out"])
    # top-2: both experts per token, softmax weights over the two logits
    got2 = layer.moe_forward(x, logits, None, 2, w1, w2, k, k)
    z = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    w_ref = np.sort(z / z.sum(axis=1, keepdims=True), axis=1)[:, ::-1]
    assert np.array_equal(got2["topk_w"], w_ref.astype(np.float32))
    want = _token_major_block(x, logits, None, 2, w1, w2, k, k)
    assert np.array_equal(got2["out"], want["out"])


def test_block_output_tracks_the_unquantized_block():
    # a sanity bound, not a pin of bits: the block's output stays close to
    # the same block computed in float64 without any quantization (relative
    # Frobenius error of a few percent for 4-bit operands), and compensating
    # every channel of both GEMMs brings it closer
    rng = np.random.default_rng(13)
    T, H, E, topk, I = 16, 128, 4, 2, 64
    x, w1, w2 = _inputs(rng, T, H, E, I)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, tw = MOE.route(logits, topk)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(topk):
            y = w1[ids[t, j]] @ x[t]
            g = y[:I]
            h = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * y[I:]
            ref[t] += tw[t, j] * (w2[ids[t, j]] @ h)
    e0 = np.linalg.norm(layer.moe_forward(x, logits, None, topk, w1, w2, 0, 0)["out"] - ref)
    eK = np.linalg.norm(layer.moe_forward(x, logits, None, topk, w1, w2, H, I)["out"] - ref)
    assert e0 / np.linalg.norm(ref) < 0.25
    assert eK < e0
