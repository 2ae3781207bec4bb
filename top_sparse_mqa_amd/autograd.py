"""Differentiable top-k sparse MQA: one torch.autograd.Function whose forward is
sparse_mqa_fwd_interface and whose backward is sparse_mqa_bwd_interface (NeMo AutoModel
DeepSeek-V4 pages "...kernels.tilelang_sparse_mla_fwd" and "...kernels.tilelang_sparse_mla_bwd":
the backward takes the forward's O and LSE together with dO).

Gradients flow to q, kv and attn_sink. LSE is returned for inspection but is not differentiable
(the pages' backward takes no LSE gradient). topk_idxs and sm_scale get no gradient.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from .binding import sparse_mqa_bwd_interface, sparse_mqa_fwd_interface


class SparseMQAFunction(torch.autograd.Function):
    """(q, kv, attn_sink, topk_idxs, sm_scale) -> (O, LSE), with O differentiable."""

    @staticmethod
    def forward(ctx, q: torch.Tensor, kv: torch.Tensor, attn_sink: torch.Tensor, topk_idxs: torch.Tensor,
                sm_scale: Optional[float] = None):
        o, lse = sparse_mqa_fwd_interface(q, kv, attn_sink, topk_idxs, sm_scale=sm_scale)
        ctx.save_for_backward(q, kv, attn_sink, topk_idxs, o, lse)
        ctx.sm_scale = sm_scale
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do: torch.Tensor, _dlse: Optional[torch.Tensor]):
        q, kv, attn_sink, topk_idxs, o, lse = ctx.saved_tensors
        if do is None:
            return None, None, None, None, None
        do = do.to(torch.bfloat16).contiguous()
        want_sink = ctx.needs_input_grad[2]
        out = sparse_mqa_bwd_interface(q, kv, attn_sink, o, do, topk_idxs, lse, sm_scale=ctx.sm_scale,
                                       return_d_sink=want_sink)
        dq, dkv = out[0], out[1]
        d_sink = out[2] if want_sink else None
        return (dq if ctx.needs_input_grad[0] else None, dkv if ctx.needs_input_grad[1] else None, d_sink, None,
                None)


def sparse_mqa(q: torch.Tensor, kv: torch.Tensor, attn_sink: torch.Tensor, topk_idxs: torch.Tensor,
               sm_scale: Optional[float] = None, return_lse: bool = False):
    """Differentiable sparse MQA attention. Returns O [B,S,H,D] bf16 (and LSE [B,S,H] fp32, log2
    units, when return_lse). Shapes, dtypes and index rules are those of
    sparse_mqa_fwd_interface."""
    o, lse = SparseMQAFunction.apply(q, kv, attn_sink, topk_idxs, sm_scale)
    return (o, lse) if return_lse else o
