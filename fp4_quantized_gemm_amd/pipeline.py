"""The rollout-side MoE expert block as a chain of library calls.

Weights go through the shared QDQ path once (per weight sync); each forward
routes and permutes tokens, quantizes the activation online, selects the
high-residual channels, runs the grouped W4A4 GEMM with the residual added
back, forms and quantizes the SwiGLU activation for the down projection the
same way, and combines the expert outputs (QUADS: arXiv abstract;
gist.science technical summary §2.1-§2.2).  Nothing here computes: every
step is one call into libnvfp4rac.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (grouped_w4a4_gemm_rac, grouped_w4a4_gemm_rac_per_expert,
               grouped_w4a4_gemm_rac_swiglu, moe_permute, nvfp4_quantize_act_amax,
               moe_unpermute_combine, nvfp4_qdq_residual, nvfp4_qdq_weights, nvfp4_quantize_act,
               select_residual_channels, select_residual_channels_per_expert)


@dataclass
class QuantWeights:
    codes: torch.Tensor      # [E][N][K/2] u8, row-major E2M1 pairs
    scales: torch.Tensor     # [E][N][K/16] u8, row-major E4M3 block scales
    g: torch.Tensor          # [E] f32
    qdq: torch.Tensor        # [E][N][K] bf16 or None
    packed_codes: torch.Tensor    # the grouped GEMMs' packed copy of codes ...
    packed_scales: torch.Tensor   # ... and block scales


def prepare_weights(w, want_qdq=False) -> QuantWeights:
    return QuantWeights(*nvfp4_qdq_weights(w, want_qdq=want_qdq, want_packed=True))


def quantized_linear_rac(x, wq: QuantWeights, k, a_rows=None, offsets=None, M_total=None,
                         glu=False, rac="bf16", select="shared", swiglu_out=False, amax=None):
    """Quantize x (or SwiGLU of x), select k channels, grouped GEMM.
    rac="bf16" adds the bf16 residual of the selected channels back;
    rac="nvfp4" quantizes that residual a second time to NVFP4 first and adds
    its fake-quantized value back.  select="shared" picks one channel set
    for the whole call; select="per_expert" one per expert, from the rows
    routed to it.  swiglu_out=True returns h = SwiGLU of the [gate | up]
    product instead of the product (fused into the GEMM; shared selection
    only).  amax: x's tensor amax as bf16 bits (from the fused SwiGLU), so the
    quantizer reads x once.  Returns (y or h, stage dict)."""
    if rac not in ("bf16", "nvfp4"):
        raise ValueError(f"rac must be 'bf16' or 'nvfp4', not {rac!r}")
    if select not in ("shared", "per_expert"):
        raise ValueError(f"select must be 'shared' or 'per_expert', not {select!r}")
    per_expert = select == "per_expert"
    if amax is not None:
        q = nvfp4_quantize_act_amax(x, amax, want_score=k > 0 and not per_expert)
    else:
        q = nvfp4_quantize_act(x, glu=glu, want_score=k > 0 and not per_expert)
    if offsets is None:
        offsets = torch.tensor([0, x.shape[0]], dtype=torch.int32, device=x.device)
    S = R = None
    if k > 0:
        if per_expert:
            S, R = select_residual_channels_per_expert(q["x_used"], q["codes"], q["scales"],
                                                       q["g"], None, k, a_rows, offsets,
                                                       M_total=M_total)
        else:
            S, R = select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"],
                                            q["score"], k)
        if rac == "nvfp4":
            R = nvfp4_qdq_residual(R)[3]
    if swiglu_out and per_expert:
        raise ValueError("the fused SwiGLU output takes the shared channel selection")
    args = (q["codes"], q["scales"], q["g"], a_rows, R, S, wq.packed_codes, wq.packed_scales, wq.g,
            offsets)
    if swiglu_out:
        y, amax = grouped_w4a4_gemm_rac_swiglu(*args, M_total=M_total, with_amax=True)
        return y, dict(q=q, S=S, R=R, h_amax=amax)
    gemm = grouped_w4a4_gemm_rac_per_expert if per_expert else grouped_w4a4_gemm_rac
    y = gemm(*args, M_total=M_total)
    return y, dict(q=q, S=S, R=R)


def moe_forward(x, logits, topk, w_first: QuantWeights, w_down: QuantWeights, k_first, k_down,
                bias=None, keep=False, rac="bf16", select="shared", fuse_swiglu=False):
    """x [T][H] bf16, logits [T][E] f32.  w_first [E][N1][H] (N1 = 2I for
    gate+up, I for an up-only block); w_down [E][H][I] or None.  Returns the
    combined output [T][H] (or the first GEMM's permuted output when there is
    no down projection) and, with keep=True, every intermediate.
    fuse_swiglu=True forms h inside the gate+up GEMM (y1 is then h)."""
    ids, tw, offs, perm, inv = moe_permute(logits, topk, bias)
    rows = perm.numel()
    fuse = fuse_swiglu and w_down is not None
    y1, st1 = quantized_linear_rac(x, w_first, k_first, a_rows=perm, offsets=offs, M_total=rows,
                                   rac=rac, select=select, swiglu_out=fuse)
    out = dict(topk_ids=ids, topk_w=tw, offsets=offs, perm_token=perm, inv_perm=inv, y1=y1,
               st1=st1) if keep else {}
    if w_down is None:
        return y1, out
    y2, st2 = quantized_linear_rac(y1, w_down, k_down, a_rows=None, offsets=offs, M_total=rows,
                                   glu=not fuse, rac=rac, select=select,
                                   amax=st1.get("h_amax") if fuse else None)
    o = moe_unpermute_combine(y2, inv, tw)
    if keep:
        out.update(y2=y2, st2=st2, out=o)
    return o, out
