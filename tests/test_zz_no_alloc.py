"""The allocation-free backward entry point, sparse_mqa_bwd_noalloc, called through the C ABI and
checked against sparse_mqa_bwd (the same computation on a caller-allocated workspace).

Two calls in a row, the second on a smaller input, must each match: the scratch array keeps the
first call's contents, so anything the kernels fail to clear would show in the second. Where both
entry points run one pass over all tokens the results are bit for bit equal; a size whose one-pass
workspace exceeds the scratch runs in token chunks and is held to the floating-point bar. (Sizes
beyond the scratch are refused by validation, tested on the host.)"""
import ctypes

import pytest
import torch

import oracle
import top_sparse_mqa_amd as smqa
from top_sparse_mqa_amd import synthetic as syn
from parity_utils import check_bf16, say

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20  # SMQA_BWD_SCRATCH_BYTES


def inputs(w):
    x = syn.workload_inputs(w)
    o, lse = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    x["o"] = o.view(w.B, w.S, w.H, w.D).to(torch.bfloat16)
    x["lse"] = lse.view(w.B, w.S, w.H)
    return {k: v.cuda() for k, v in x.items()}


def noalloc(lib, w, xg, fp32):
    dq = torch.empty_like(xg["q"])
    dkv = torch.empty((w.B, w.S_kv, w.D), dtype=torch.float32 if fp32 else torch.bfloat16, device="cuda")
    p = lambda t: t.data_ptr()  # noqa: E731
    st = lib.sparse_mqa_bwd_noalloc(p(xg["q"]), p(xg["kv"]), p(xg["attn_sink"]), p(xg["o"]), p(xg["do"]),
                                    p(xg["topk_idxs"]), p(xg["lse"]), p(dq), p(dkv), 1 if fp32 else 0, w.B, w.S,
                                    w.S_kv, w.H, w.D, w.topk, float("nan"),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, lib.sparse_mqa_status_string(st)
    return dq, dkv


def with_workspace(w, xg, fp32):
    dq, dkv = smqa.sparse_mqa_bwd_interface(xg["q"], xg["kv"], xg["attn_sink"], xg["o"], xg["do"], xg["topk_idxs"],
                                            xg["lse"], return_dkv_accum_dtype=fp32)
    torch.cuda.synchronize()
    return dq, dkv


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    lib = gpu_lib
    chunked = syn.Workload("chunked_h64_d512_k512", 1, 1024, 1024, 64, 512, 512, "causal_distinct", 21, 121)
    # the mid workload, then the smaller tiny one; then one that needs token chunks in the scratch
    for name, w in (("mid", syn.WORKLOADS["mid_h64_d512_k300"]), ("tiny", syn.WORKLOADS["tiny_h16_d64"]),
                    ("chunked", chunked)):
        one_pass = lib.sparse_mqa_bwd_workspace_bytes(w.B, w.S, w.S_kv, w.H, w.D, w.topk) <= SCRATCH
        say("case", name, w.describe(), "one pass in the scratch" if one_pass else "token chunks in the scratch")
        xg = inputs(w)
        for fp32 in (False, True):
            dq0, dkv0 = with_workspace(w, xg, fp32)
            dq1, dkv1 = noalloc(lib, w, xg, fp32)
            assert torch.equal(dq1, dq0), "dQ must not depend on where the workspace lives"
            check_bf16(f"{name} dKV fp32={fp32} vs sparse_mqa_bwd", dkv1.view(-1, w.D), dkv0.view(-1, w.D))
            if one_pass:
                assert torch.equal(dkv1, dkv0), "one pass over all tokens in both: bit for bit equal"
