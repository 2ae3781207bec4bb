"""The forward and backward interfaces captured into a HIP graph and replayed: every kernel
launch goes to the caller's stream, the C library neither allocates nor synchronises, and the
dKV accumulator is cleared by a kernel, so a replay must give the eager results. Each replay is
followed by unrelated eager work and a synchronisation, and checked on its own."""
import pytest
import torch

import top_sparse_mqa_amd as smqa
from top_sparse_mqa_amd import synthetic as syn

pytestmark = pytest.mark.gpu


def run(x):
    o, lse = smqa.sparse_mqa_fwd_interface(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    dq, dkv = smqa.sparse_mqa_bwd_interface(x["q"], x["kv"], x["attn_sink"], o, x["do"], x["topk_idxs"], lse,
                                            return_dkv_accum_dtype=True)
    return o, lse, dq, dkv


def test_graph_capture_replay(gpu_lib):
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    x = {k: v.cuda() for k, v in syn.workload_inputs(w).items()}
    o0, lse0, dq0, dkv0 = run(x)
    torch.cuda.synchronize()
    # warm up on a side stream, as graph capture expects
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run(x)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))  # a replay must rewrite every output element
        g.replay()
        torch.cuda.synchronize()
        o, lse, dq, dkv = outs
        assert torch.equal(o, o0) and torch.equal(lse, lse0), f"replay {rep}: forward differs"
        assert torch.equal(dq, dq0) and torch.equal(dkv, dkv0), f"replay {rep}: backward differs"
        junk.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
