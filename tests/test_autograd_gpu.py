"""The differentiable wrapper (sparse_mqa / SparseMQAFunction) on the GPU: its gradients for q,
kv and attn_sink against the oracle's backward, and against the interface it chains."""
import math

import pytest
import torch

import oracle
import top_sparse_mqa_amd as smqa
from top_sparse_mqa_amd import synthetic as syn
from parity_utils import check_bf16, check_dsink, check_lse, say

pytestmark = pytest.mark.gpu


def leaf(t):
    return t.cuda().requires_grad_(True)


@pytest.mark.parametrize("name", ["tiny_h16_d64", "mid_h64_d512_k300"])
def test_autograd_grads_match_oracle(gpu_lib, name):
    w = syn.WORKLOADS[name]
    say("case", w.describe())
    x = syn.workload_inputs(w)
    x["attn_sink"][1] = -math.inf  # a head without a sink: zero gradient
    q, kv, sink = leaf(x["q"]), leaf(x["kv"]), leaf(x["attn_sink"])
    idx = x["topk_idxs"].to(torch.int64).cuda()  # int64 indices, as the pages allow
    o, lse = smqa.sparse_mqa(q, kv, sink, idx, return_lse=True)
    assert o.requires_grad and not lse.requires_grad
    # loss = sum(O * dO) so that dL/dO = dO
    (o.float() * x["do"].cuda().float()).sum().backward()
    torch.cuda.synchronize()
    assert q.grad.dtype == torch.bfloat16 and kv.grad.dtype == torch.bfloat16 and sink.grad.dtype == torch.float32
    H, D = w.H, w.D
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    check_bf16("O", o.detach().view(-1, H, D), o_ref)
    check_lse("LSE", lse.view(-1, H), lse_ref)
    # The backward autograd ran received the GPU forward's O (bf16) and LSE; the oracle's backward
    # is evaluated on exactly those. (Fed the oracle's own forward instead, the two backwards differ
    # through Delta = <O, dO>: where attention is peaked, |O| reaches 2-4 and one bf16 ulp of O
    # there moves Delta, and the dKV of the rows those tokens pick, by up to ~0.1 -- a difference
    # of inputs, not of the kernels.)
    ob = o.detach().cpu()
    lb = lse.detach().cpu()
    dq_ref, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    check_bf16("dQ", q.grad.view(-1, H, D), dq_ref)
    check_bf16("dKV", kv.grad.view(-1, D), dkv_ref)
    check_dsink("d_sink", sink.grad, oracle.dsink(ob, x["do"], lb, x["attn_sink"]), ob, x["do"], lb,
                x["attn_sink"])
    # the wrapper routes the interface's results: dQ, dKV and d_sink bit for bit on the same O and
    # LSE (the staged backward sums in an order fixed by the indices)
    dq2, dkv2, ds2 = smqa.sparse_mqa_bwd_interface(q.detach(), kv.detach(), sink.detach(), o.detach(),
                                                   x["do"].cuda(), idx, lse, return_d_sink=True)
    torch.cuda.synchronize()
    assert torch.equal(dq2, q.grad) and torch.equal(ds2, sink.grad) and torch.equal(dkv2, kv.grad)


def test_autograd_partial_requires_grad(gpu_lib):
    """Only kv needs a gradient: q and attn_sink get none, kv's equals the full run's."""
    w = syn.WORKLOADS["tiny_h16_d64"]
    x = syn.workload_inputs(w)
    kv = leaf(x["kv"])
    q, sink, idx, do = x["q"].cuda(), x["attn_sink"].cuda(), x["topk_idxs"].cuda(), x["do"].cuda()
    o = smqa.sparse_mqa(q, kv, sink, idx)
    o.backward(do)
    torch.cuda.synchronize()
    assert q.grad is None and sink.grad is None
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    ob = o_ref.view(w.B, w.S, w.H, w.D).to(torch.bfloat16)
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lse_ref.view(w.B, w.S, w.H))
    check_bf16("dKV", kv.grad.view(-1, w.D), dkv_ref)
