"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small cases are compared element by element over every output. At the full sizes the headline
workload is compared over every token and every kv row, the batched gather-bound workload over
every token and 1024 kv rows, and the long-context workload (the largest) on sampled tokens and
rows that the oracle computes one by one, among them rows referenced from every token chunk of
its chunked dKV pass. Masking and index handling are
checked bit-exactly (zero outputs, untouched rows, NaN-poisoned unreferenced kv rows).
"""
import math
import zlib

import pytest
import torch

import oracle
import top_sparse_mqa_amd as smqa
from top_sparse_mqa_amd import synthetic as syn
from parity_utils import (LSE_ATOL, check_bf16, check_dsink, check_lse, conservation_rhs, referenced_rows,
                          sample_tokens, say, valid_mask)

pytestmark = pytest.mark.gpu

I32MIN, I32MAX = -(2 ** 31), 2 ** 31 - 1


def gpu(x):
    return {k: v.cuda() for k, v in x.items()}


def fwd_gpu(xg, scale=None):
    o, lse = smqa.sparse_mqa_fwd_interface(xg["q"], xg["kv"], xg["attn_sink"], xg["topk_idxs"], sm_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def bwd_gpu(xg, o, lse, scale=None, fp32=False):
    dq, dkv = smqa.sparse_mqa_bwd_interface(xg["q"], xg["kv"], xg["attn_sink"], o, xg["do"], xg["topk_idxs"], lse,
                                            sm_scale=scale, return_dkv_accum_dtype=fp32)
    torch.cuda.synchronize()
    return dq, dkv


def full_parity(x, scale=None, tag=""):
    """Forward and backward over every output element against the fp32 oracle."""
    B, S, H, D = x["q"].shape
    S_kv = x["kv"].shape[1]
    xg = gpu(x)
    o, lse = fwd_gpu(xg, scale)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], sm_scale=scale)
    check_bf16(f"{tag} O", o.view(-1, H, D), o_ref)
    check_lse(f"{tag} LSE", lse.view(-1, H), lse_ref)
    # backward on the oracle's forward outputs (O rounded to bf16, as the interface takes it)
    ob = o_ref.view(B, S, H, D).to(torch.bfloat16)
    lb = lse_ref.view(B, S, H)
    dq, dkv = bwd_gpu(xg, ob.cuda(), lb.cuda(), scale)
    dq_ref, delta_ref = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, sm_scale=scale)
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, sm_scale=scale)
    check_bf16(f"{tag} dQ", dq.view(-1, H, D), dq_ref)
    check_bf16(f"{tag} dKV", dkv.view(-1, D), dkv_ref)
    ref_rows = referenced_rows(x["topk_idxs"], S_kv).view(-1)
    assert torch.count_nonzero(dkv.view(-1, D).cpu()[~ref_rows]) == 0, "unreferenced dKV rows must be exactly 0"
    # fp32 accumulator output
    dq2, dkv32 = bwd_gpu(xg, ob.cuda(), lb.cuda(), scale, fp32=True)
    assert dkv32.dtype == torch.float32
    check_bf16(f"{tag} dKV fp32", dkv32.view(-1, D), dkv_ref)
    assert torch.equal(dq2, dq), "dQ must be deterministic"
    # preprocess stage alone
    delta = smqa.bwd_preprocess(ob.cuda(), xg["do"])
    torch.cuda.synchronize()
    torch.testing.assert_close(delta.view(-1, H).cpu().double(), delta_ref.double(), rtol=1e-4, atol=1e-4)
    # attention-sink gradient, through the interface and as a stage on the same Delta
    dsink_ref = oracle.dsink(ob, x["do"], lb, x["attn_sink"])
    dq3, dkv3, dsink = smqa.sparse_mqa_bwd_interface(xg["q"], xg["kv"], xg["attn_sink"], ob.cuda(), xg["do"],
                                                     xg["topk_idxs"], lb.cuda(), sm_scale=scale, return_d_sink=True)
    torch.cuda.synchronize()
    assert torch.equal(dq3, dq), "dQ must not depend on return_d_sink"
    check_dsink(f"{tag} d_sink", dsink, dsink_ref, ob, x["do"], lb, x["attn_sink"])
    dsink2 = smqa.bwd_dsink(lb.cuda(), delta, xg["attn_sink"])
    torch.cuda.synchronize()
    assert torch.equal(dsink2, dsink), "d_sink must be deterministic"
    return o, lse


def test_tiny_full(gpu_lib):
    w = syn.WORKLOADS["tiny_h16_d64"]
    say("case", w.describe())
    x = syn.workload_inputs(w)
    o, lse = full_parity(x, tag=w.name)
    # forward is deterministic bit for bit
    o2, lse2 = fwd_gpu(gpu(x))
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_mid_full(gpu_lib):
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    say("case", w.describe())
    full_parity(syn.workload_inputs(w), tag=w.name)


EDGE = [
    # name, B, S, S_kv, H, D, topk
    ("h32_d512_k65", 2, 9, 70, 32, 512, 65),
    ("h128_d512_k130", 1, 6, 300, 128, 512, 130),
    ("h16_d512_k1", 1, 7, 40, 16, 512, 1),
    ("h32_d64_k200_dups", 1, 11, 100, 32, 64, 200),
    ("h64_d512_k33", 1, 5, 33, 64, 512, 33),
    ("h64_d512_k5", 1, 3, 20, 64, 512, 5),     # one partial block through the specialised kernels
    ("h64_d512_k1", 2, 3, 10, 64, 512, 1),
    ("h192_d512_k70", 1, 4, 90, 192, 512, 70),
    ("h256_d512_k40", 2, 3, 50, 256, 512, 40),
    ("h64_d256_k50", 1, 6, 80, 64, 256, 50),
    ("h16_d256_k70", 2, 3, 90, 16, 256, 70),
    ("h32_d128_k40", 1, 7, 60, 32, 128, 40),
    ("h128_d128_k33", 1, 4, 40, 128, 128, 33),
    ("h64_d512_k2200", 1, 3, 2500, 64, 512, 2200),  # more than 64 blocks: the forward's index ring refills
    ("h64_d512_k3300", 1, 2, 4000, 64, 512, 3300),  # 104 blocks: two refills of the ring
]


def edge_inputs(name, B, S, S_kv, H, D, topk, seed):
    g = torch.Generator().manual_seed(seed)
    x = {
        "q": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
        "kv": torch.randn(B, S_kv, D, generator=g).to(torch.bfloat16),
        "attn_sink": torch.randn(H, generator=g),
        "do": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
    }
    idx = torch.randint(-2, S_kv + 2, (B, S, topk), generator=g)
    pick = torch.rand(B, S, topk, generator=g)
    idx = torch.where(pick < 0.04, torch.full_like(idx, I32MIN), idx)
    idx = torch.where((pick > 0.96), torch.full_like(idx, I32MAX), idx)
    idx[0, 0] = -1  # a fully masked token
    x["topk_idxs"] = idx.to(torch.int32)
    x["attn_sink"][0] = -math.inf  # one head without a sink
    return x


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_shapes_full(gpu_lib, case):
    name, B, S, S_kv, H, D, topk = case
    say("case", name, dict(B=B, S=S, S_kv=S_kv, H=H, D=D, topk=topk))
    x = edge_inputs(*case, seed=zlib.crc32(name.encode()) % 1000)
    # NaN-poison every kv row that no valid slot references: such rows must never be read
    ref_rows = referenced_rows(x["topk_idxs"], S_kv)
    kv = x["kv"].clone()
    kv[~ref_rows] = float("nan")
    x["kv"] = kv
    o, lse = full_parity(x, tag=name)
    # the fully masked token: O exactly +0, LSE = sink*log2(e) (or -inf for the sinkless head)
    o0 = o[0, 0].cpu()
    assert torch.count_nonzero(o0) == 0 and not torch.signbit(o0.float()).any()
    l0 = lse[0, 0].cpu()
    assert l0[0] == -math.inf
    torch.testing.assert_close(l0[1:].double(), x["attn_sink"][1:].double() / math.log(2), rtol=0, atol=1e-5)


def test_trailing_masked_slots_64_head_kernels(gpu_lib):
    """Selections shorter than topk, padded with masked slots at the end (as causal top-k picks of
    early tokens are): the 64-head D = 512 kernels stop after the last block holding a valid slot.
    topk = 1100 spans 35 blocks; the tokens keep 1100, 1025 (one slot into block 32), 700, 33, 32
    and 0 valid slots, and the padding mixes -1 with out-of-range values."""
    B, S, S_kv, H, D, topk = 1, 6, 1500, 64, 512, 1100
    keep = [1100, 1025, 700, 33, 32, 0]
    say("case", "trailing masked slots", dict(topk=topk, keep=keep))
    g = torch.Generator().manual_seed(77)
    x = {
        "q": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
        "kv": torch.randn(B, S_kv, D, generator=g).to(torch.bfloat16),
        "attn_sink": torch.randn(H, generator=g),
        "do": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
    }
    idx = torch.full((B, S, topk), -1, dtype=torch.int64)
    for s_, n in enumerate(keep):
        idx[0, s_, :n] = torch.randperm(S_kv, generator=g)[:n]
        pad = torch.rand(topk - n, generator=g)
        tail = torch.where(pad < 0.5, torch.full_like(pad, -1), torch.full_like(pad, S_kv + 7)).long()
        idx[0, s_, n:] = tail
    x["topk_idxs"] = idx.to(torch.int32)
    full_parity(x, tag="trailing masked")


@pytest.mark.parametrize("H", [64, 128])
def test_empty_blocks_64_head_kernels(gpu_lib, H):
    """The 64-head D = 512 kernels skip 32-slot blocks with no valid slot in both of their wave
    roles; here whole blocks are masked for every token (at the start, in the middle, between
    valid blocks), one token keeps only its last block, one token has none, and the last block is
    ragged (topk = 200)."""
    B, S, S_kv, D, topk = 1, 6, 400, 512, 200
    say("case", "empty blocks", dict(H=H))
    g = torch.Generator().manual_seed(31 + H)
    x = {
        "q": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
        "kv": torch.randn(B, S_kv, D, generator=g).to(torch.bfloat16),
        "attn_sink": torch.randn(H, generator=g),
        "do": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
    }
    idx = torch.stack([torch.randperm(S_kv, generator=g)[:topk] for _ in range(B * S)]).view(B, S, topk)
    idx[:, :, 0:32] = -1      # first block
    idx[:, :, 96:160] = -1    # two middle blocks
    idx[0, 2, :192] = -1      # only the ragged last block left
    idx[0, 4, :] = -1         # nothing left
    x["topk_idxs"] = idx.to(torch.int32)
    full_parity(x, tag=f"empty blocks H={H}")


def test_operand_scales_and_row_norms(gpu_lib):
    """Magnitudes away from 1 for the fp16 operands of the dKV product: q scaled by 1/128, one
    referenced kv row 8x the others (it sets the dS bound of the tokens that reference it) and one
    unreferenced row 1e5x (it must not change anything). Then dO scaled by 2^10: every gradient
    is linear in dO and the kernels' scale exponents absorb a power of two, so dQ, Delta, d_sink and
    dKV must scale by exactly 2^10 (bit for bit; dKV through its fp32 output)."""
    g = torch.Generator().manual_seed(77)
    B, S, S_kv, H, D, topk = 1, 8, 64, 64, 512, 32
    kv = torch.randn(B, S_kv, D, generator=g)
    kv[0, 5] *= 8.0
    kv[0, S_kv - 1] *= 1e5
    idx = torch.stack([torch.randperm(S_kv - 1, generator=g)[:topk] for _ in range(S)]).view(B, S, topk)
    idx[0, :4, 0] = 5  # tokens 0..3 reference the large row (5 may then repeat, as allowed)
    x = {
        "q": (torch.randn(B, S, H, D, generator=g) / 128).to(torch.bfloat16),
        "kv": kv.to(torch.bfloat16),
        "attn_sink": torch.randn(H, generator=g),
        "do": torch.randn(B, S, H, D, generator=g).to(torch.bfloat16),
        "topk_idxs": idx.to(torch.int32),
    }
    say("case operand scales", dict(B=B, S=S, S_kv=S_kv, H=H, D=D, topk=topk))
    o, lse = full_parity(x, tag="scales")
    xg = gpu(x)
    outs = []
    for f in (1.0, 1024.0):
        do = (xg["do"].float() * f).to(torch.bfloat16)
        dq, dkv, ds = smqa.sparse_mqa_bwd_interface(xg["q"], xg["kv"], xg["attn_sink"], o, do, xg["topk_idxs"], lse,
                                                    return_dkv_accum_dtype=True, return_d_sink=True)
        torch.cuda.synchronize()
        outs.append((dq.float(), dkv, ds))
    (dq1, dkv1, ds1), (dq2, dkv2, ds2) = outs
    assert torch.equal(dq2, dq1 * 1024) and torch.equal(ds2, ds1 * 1024)
    # dKV sums staged rows in an order that may differ between calls: compare to fp32 rounding
    torch.testing.assert_close(dkv2, dkv1 * 1024, rtol=1e-5, atol=1e-3)


@pytest.mark.parametrize("scale", [-0.125, 0.0], ids=["negative", "zero"])
def test_negative_and_zero_scale(gpu_lib, scale):
    """sm_scale is any finite value: a negative one (the forward takes it as a positive scale of
    -Q) and zero (every valid slot gets the same weight)."""
    w = syn.WORKLOADS["tiny_h16_d64"]
    say("case", w.describe(), "sm_scale", scale)
    x = syn.workload_inputs(w)
    o, lse = full_parity(x, scale=scale, tag=f"scale={scale}")
    if scale == 0.0:
        # P is uniform over the valid slots and the sink: LSE = log2(n_valid + e^sink)
        n = valid_mask(x["topk_idxs"], w.S_kv).sum(-1).double().view(-1, 1)
        expect = torch.log2(n + torch.exp(x["attn_sink"].double()).view(1, -1))
        torch.testing.assert_close(lse.view(-1, w.H).double().cpu(), expect, rtol=0, atol=1e-5)


def test_negative_scale_large_do_64_head_kernels(gpu_lib):
    """A negative sm_scale through the 64-head D = 512 kernels with q x 4 (peaked rows) and dO x 2^16,
    so that dS = P (dP - Delta) sm_scale reaches ~10^5: the dKV kernel's fp16 dS operand scale must
    take |sm_scale| into its bound, or dS saturates at the fp16 maximum. The gradients are linear in
    dO, so they are compared after dividing both sides by 2^16 (the elementwise bar of the unscaled
    problem)."""
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    scale = -1.0 / math.sqrt(w.D)
    say("case", w.describe(), "q x 4, dO x 2^16, sm_scale", scale)
    x = syn.workload_inputs(w)
    x["q"] = (x["q"].float() * 4).to(torch.bfloat16)
    x["do"] = (x["do"].float() * 65536.0).to(torch.bfloat16)
    B, S, H, D = x["q"].shape
    xg = gpu(x)
    o, lse = fwd_gpu(xg, scale)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], sm_scale=scale)
    check_bf16("neg O", o.view(-1, H, D), o_ref)
    check_lse("neg LSE", lse.view(-1, H), lse_ref)
    ob = o_ref.view(B, S, H, D).to(torch.bfloat16)
    lb = lse_ref.view(B, S, H)
    dq_ref, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, sm_scale=scale)
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, sm_scale=scale)
    for fp32 in (False, True):
        dq, dkv = bwd_gpu(xg, ob.cuda(), lb.cuda(), scale, fp32=fp32)
        check_bf16(f"neg dQ / 2^16 (fp32 dkv {fp32})", dq.view(-1, H, D).float() / 65536.0, dq_ref / 65536.0)
        check_bf16(f"neg dKV / 2^16 (fp32 dkv {fp32})", dkv.view(-1, D).float() / 65536.0, dkv_ref / 65536.0)


def test_sharp_scores_mid(gpu_lib):
    """q x 8: peaked softmax rows (scores spread over ~60 log2 units), so that errors in the max
    tracking and rescaling of the online softmax show, and dKV rows sum large contributions that
    cancel (typical |dKV| ~ 16, up to ~170). Every output meets the elementwise bar: O, LSE, dQ,
    dKV through the staged path (bf16 and fp32 outputs) and through the atomic stage."""
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    say("case", w.describe(), "q x 8")
    x = syn.workload_inputs(w)
    x["q"] = (x["q"].float() * 8).to(torch.bfloat16)
    B, S, H, D = x["q"].shape
    xg = gpu(x)
    o, lse = fwd_gpu(xg)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    check_bf16("sharp O", o.view(-1, H, D), o_ref)
    check_lse("sharp LSE", lse.view(-1, H), lse_ref)
    ob = o_ref.view(B, S, H, D).to(torch.bfloat16)
    lb = lse_ref.view(B, S, H)
    dq, dkv32 = bwd_gpu(xg, ob.cuda(), lb.cuda(), fp32=True)
    dq_ref, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    check_bf16("sharp dQ", dq.view(-1, H, D), dq_ref)
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    check_bf16("sharp dKV fp32", dkv32.view(-1, D), dkv_ref)
    _, dkv16 = bwd_gpu(xg, ob.cuda(), lb.cuda())
    check_bf16("sharp dKV bf16", dkv16.view(-1, D), dkv_ref)
    delta = smqa.bwd_preprocess(ob.cuda(), xg["do"])
    acc = torch.zeros(B, w.S_kv, D, dtype=torch.float32, device="cuda")
    smqa.bwd_main(xg["q"], xg["kv"], xg["do"], xg["topk_idxs"], lb.cuda(), delta, acc)
    torch.cuda.synchronize()
    check_bf16("sharp dKV atomic", acc.view(-1, D), dkv_ref)


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16)


def test_postprocess_round_to_nearest_even(gpu_lib):
    """sparse_mqa_bwd_postprocess alone (bwd page, postprocess factory): the fp32 accumulator to
    bf16, bit for bit equal to the CPU's round-to-nearest-even conversion, on values spread over
    60 binades, exact ties (half an ulp: the even neighbour wins), values just beside ties, signed
    zeros, infinities, the largest floats (which round to infinity), subnormals, and NaN (stays
    NaN). Shape [2, 37, 512] (a ragged last workgroup)."""
    g = torch.Generator().manual_seed(5)
    B, S_kv, D = 2, 37, 512
    mant = torch.randn(B * S_kv * D, generator=g)
    expo = torch.randint(-30, 31, (B * S_kv * D,), generator=g).double()
    flat = (mant.double() * torch.pow(2.0, expo)).float()
    bits = flat.view(torch.int32)
    n = 8192
    # ties and their neighbours: low 16 bits 0x8000, 0x7fff and 0x8001 under random high bits
    hi = torch.randint(0, 2 ** 15, (n,), generator=g, dtype=torch.int32) << 16
    sign = (torch.randint(0, 2, (n,), generator=g, dtype=torch.int32) << 31)
    bits[:n] = hi | sign | 0x8000
    bits[n:2 * n] = hi | sign | 0x7FFF
    bits[2 * n:3 * n] = hi | sign | 0x8001
    flat[3 * n:3 * n + 8] = torch.tensor([0.0, -0.0, float("inf"), -float("inf"), 3.4028235e38, -3.4028235e38,
                                          1.0e-40, -2.5e-42])
    flat[3 * n + 8] = float("nan")
    acc = flat.view(B, S_kv, D)
    got = smqa.bwd_postprocess(acc.cuda())
    torch.cuda.synchronize()
    got = got.cpu()
    ref = acc.to(torch.bfloat16)
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    differ = (_bf16_bits(got) != _bf16_bits(ref)) & ~nan
    say(f"  postprocess: {int(differ.sum())} of {ref.numel()} elements differ from the CPU conversion")
    assert not differ.any(), f"first differing input: {float(acc.view(-1)[differ.view(-1)][0])!r}"


def test_power_of_two_rescaling_is_exact(gpu_lib):
    """O(2q, scale/2) == O(q, scale) and LSE alike, bit for bit: a power of two moves through
    the bf16 operands, the fp32 sums and the scale without rounding."""
    w = syn.WORKLOADS["tiny_h16_d64"]
    x = syn.workload_inputs(w)
    xg = gpu(x)
    scale = 0.3
    o1, l1 = fwd_gpu(xg, scale)
    xg2 = dict(xg, q=(xg["q"].float() * 2).to(torch.bfloat16))
    o2, l2 = fwd_gpu(xg2, scale / 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_explicit_scale_and_int64_indices(gpu_lib):
    w = syn.WORKLOADS["tiny_h16_d64"]
    x = syn.workload_inputs(w)
    xg = gpu(x)
    o, lse = fwd_gpu(xg, scale=0.2)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], sm_scale=0.2)
    check_bf16("O scale=0.2", o.view(-1, w.H, w.D), o_ref)
    check_lse("LSE scale=0.2", lse.view(-1, w.H), lse_ref)
    # int64 indices, including values that int32 narrowing alone would wrap into range
    idx64 = x["topk_idxs"].long()
    idx64[:, :, -1] = 2 ** 32 + 3
    xg["topk_idxs"] = idx64.cuda()
    o64, _ = fwd_gpu(xg)
    x32 = dict(x)
    x32["topk_idxs"] = torch.where(idx64 >= w.S_kv, -1, idx64).to(torch.int32)
    o32, _ = fwd_gpu(gpu(x32))
    assert torch.equal(o64, o32)


def test_dkv_paths_agree(gpu_lib):
    """Staged dKV in one pass, in forced token chunks (bf16 and fp32 outputs), and the atomic
    stage all match the oracle; the separately enqueued steps reproduce the one-call dKV, and their
    dQ step (from the stored dS) the recompute dQ kernel."""
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    say("case", w.name, "dKV paths")
    x = syn.workload_inputs(w)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    ob = o_ref.view(w.B, w.S, w.H, w.D).to(torch.bfloat16)
    lb = lse_ref.view(w.B, w.S, w.H)
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    xg = gpu(x)
    og, lg = ob.cuda(), lb.cuda()
    delta = smqa.bwd_preprocess(og, xg["do"])
    args = (xg["q"], xg["kv"], xg["do"], xg["topk_idxs"], lg, delta)
    one = smqa.bwd_dkv(*args)
    lib = smqa.load_library()
    low = lib.sparse_mqa_bwd_workspace_min_bytes(w.B, w.S, w.S_kv, w.H, w.D, w.topk)
    # positions, staging rows (fp16 + one exponent per 128 values) and the spare row
    per_tok = w.topk * 4 + (w.topk + 1) * (w.D * 2 + max(1, w.D // 128))
    for fp32 in (False, True):
        # about 38 tokens per chunk (the selection bitmap grows by a word per row every 32 tokens)
        ws = torch.empty(low + 37 * per_tok, dtype=torch.uint8, device="cuda")
        chunked = smqa.bwd_dkv(*args, dkv_fp32=fp32, workspace=ws)
        torch.cuda.synchronize()
        check_bf16(f"dKV chunked fp32={fp32}", chunked.view(-1, w.D), dkv_ref)
    acc = torch.zeros(w.B, w.S_kv, w.D, dtype=torch.float32, device="cuda")
    smqa.bwd_main(xg["q"], xg["kv"], xg["do"], xg["topk_idxs"], lg, delta, acc)
    torch.cuda.synchronize()
    check_bf16("dKV one pass", one.view(-1, w.D), dkv_ref)
    check_bf16("dKV atomic", acc.view(-1, w.D), dkv_ref)
    # the three separately enqueued steps run the same kernels on the same staging plan (positions
    # depend on the indices only), so they reproduce the one-call result bit for bit
    steps = smqa.DkvSteps(*args)
    steps.prepare()
    steps.partials()
    dq_steps = steps.dq()
    split = steps.reduce()
    torch.cuda.synchronize()
    check_bf16("dKV steps", split.view(-1, w.D), dkv_ref)
    assert torch.equal(split, one)
    # dQ from the dS the partials step stored equals the recompute kernel's bit for bit (same bf16 dS,
    # same order of the dQ products)
    dq_recompute = smqa.bwd_dq(*args)
    torch.cuda.synchronize()
    assert torch.equal(dq_steps, dq_recompute), "dQ from stored dS differs from the recompute kernel"


def test_backward_is_deterministic(gpu_lib):
    """No atomics decide anything in the staged backward (staging positions come from the indices,
    every sum runs in a fixed order), so repeated calls agree bit for bit."""
    for name in ("mid_h64_d512_k300", "tiny_h16_d64"):
        w = syn.WORKLOADS[name]
        say("case", w.name, "determinism")
        xg = gpu(syn.workload_inputs(w))
        o, lse = fwd_gpu(xg)
        dq0, dkv0 = bwd_gpu(xg, o, lse, fp32=True)
        for _ in range(3):
            dq, dkv = bwd_gpu(xg, o, lse, fp32=True)
            assert torch.equal(dq, dq0) and torch.equal(dkv, dkv0), name


def test_non_default_stream(gpu_lib):
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    x = syn.workload_inputs(w)
    xg = gpu(x)
    o_ref, lse_ref = fwd_gpu(xg)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = smqa.sparse_mqa_fwd_interface(xg["q"], xg["kv"], xg["attn_sink"], xg["topk_idxs"])
    s.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_reference_rounding_mid(gpu_lib):
    """reference_rounding on an ordinary workload: within the bar of the fp32 oracle (whose
    arithmetic rounds the scaled logit the same way), and close to the default mode."""
    w = syn.WORKLOADS["mid_h64_d512_k300"]
    say("case", w.describe(), "reference_rounding")
    x = syn.workload_inputs(w)
    xg = gpu(x)
    o, lse = smqa.sparse_mqa_fwd_interface(xg["q"], xg["kv"], xg["attn_sink"], xg["topk_idxs"],
                                           reference_rounding=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    check_bf16("O rr", o.view(-1, w.H, w.D), o_ref)
    check_lse("LSE rr", lse.view(-1, w.H), lse_ref)
    o2, lse2 = fwd_gpu(xg)
    check_bf16("O rr vs default", o.view(-1, w.H, w.D), o2.view(-1, w.H, w.D))
    check_lse("LSE rr vs default", lse, lse2)


def large_logit_inputs(B=1, S=16, S_kv=128, H=16, D=64, topk=64, seed=3):
    """Logits near 2^21 from integer-valued bf16 inputs: every dot product is an integer below
    2^24 (exact in fp32 in any order), so the only rounding before the softmax is that of the
    scaled logit, and it moves the weights by up to e^(1/8)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-2, 3, (B, S, H, D), generator=g).float()
    q[..., 0] = 2048.0
    kv = torch.randint(-3, 4, (B, S_kv, D), generator=g).float()
    kv[..., 0] = 7936.0
    idx = torch.stack([torch.randperm(S_kv, generator=g)[:topk] for _ in range(B * S)]).view(B, S, topk)
    return {"q": q.to(torch.bfloat16), "kv": kv.to(torch.bfloat16), "attn_sink": torch.zeros(H),
            "topk_idxs": idx.to(torch.int32)}


@pytest.mark.parametrize("H,D", [(16, 64), (64, 512)])
def test_reference_rounding_large_logits(gpu_lib, H, D):
    x = large_logit_inputs(H=H, D=D)
    say("case reference_rounding large logits", dict(H=H, D=D))
    dots = x["q"].double().view(-1, D) @ x["kv"].double().view(-1, D).T
    assert float(dots.abs().max()) < 2 ** 24
    sm = 0.13
    xg = gpu(x)
    o, lse = smqa.sparse_mqa_fwd_interface(xg["q"], xg["kv"], xg["attn_sink"], xg["topk_idxs"], sm_scale=sm,
                                           reference_rounding=True)
    od, _ = fwd_gpu(xg, sm)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], sm_scale=sm)
    check_bf16("O rr", o.view(-1, H, D), o_ref)
    # LSE near 3e6 (log2 units): fp32 spacing there is 0.25, so the bar is a few spacings
    g, r = lse.view(-1, H).double().cpu(), lse_ref.double()
    spacing = torch.tensor(2.0).pow(torch.floor(torch.log2(r.abs())) - 23)
    err = (g - r).abs()
    say(f"  LSE rr: max|err| {float(err.max()):.3e} (spacing {float(spacing.max()):.3e})")
    assert torch.all(err <= 4 * spacing + LSE_ATOL)
    # the default mode scales into base 2 before rounding: its weights differ here
    dd = (od.view(-1, H, D).double().cpu() - o_ref.double()).abs()
    say(f"  O default mode vs fp32 oracle: max|err| {float(dd.max()):.3e}")
    assert not torch.equal(od, o)


# ------------------------------------------------------------------------------------------------
# full-size workloads
HEADLINE = syn.WORKLOADS["causal_h64_d512_k2048"]


@pytest.fixture(scope="module")
def headline():
    say("generating", HEADLINE.describe())
    return syn.workload_inputs(HEADLINE)


@pytest.mark.timeout(600)
def test_headline_forward_full(gpu_lib, headline):
    """O and LSE of every token at the headline shapes against the oracle."""
    w, x = HEADLINE, headline
    say("case", w.name, "forward, every token")
    o, lse = fwd_gpu(gpu(x))
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    check_bf16("O", o.view(-1, w.H, w.D), o_ref)
    check_lse("LSE", lse.view(-1, w.H), lse_ref)
    o2, lse2 = fwd_gpu(gpu(x))
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "forward must be deterministic"


@pytest.mark.timeout(900)
def test_headline_backward_full(gpu_lib, headline):
    """Backward at the headline shapes on the oracle's forward outputs (O as bf16, LSE fp32): dQ of
    every token and dKV of every kv row (fp32 and bf16 outputs), the conservation identity and the
    sink gradient."""
    w, x = HEADLINE, headline
    say("case", w.name, "backward: oracle forward over all tokens")
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    ob = o_ref.view(w.B, w.S, w.H, w.D).to(torch.bfloat16)
    lb = lse_ref.view(w.B, w.S, w.H)
    xg = gpu(x)
    dq, dkv32 = bwd_gpu(xg, ob.cuda(), lb.cuda(), fp32=True)
    say("  oracle dQ, every token")
    dq_ref, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    check_bf16("dQ", dq.view(-1, w.H, w.D), dq_ref)
    del dq_ref
    say("  oracle dKV, every row")
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    check_bf16("dKV fp32", dkv32.view(-1, w.D), dkv_ref)
    # conservation over every row (holds up to the bf16 rounding of O)
    rhs = conservation_rhs(x["q"], ob, x["do"], lb, x["attn_sink"], 1.0 / math.sqrt(w.D))
    lhs = dkv32.double().sum(1).cpu()
    rel = float((lhs - rhs).norm() / rhs.norm())
    say(f"  conservation rel-L2 {rel:.3e}")
    assert rel < 1e-2
    _, dkv16 = bwd_gpu(xg, ob.cuda(), lb.cuda())
    check_bf16("dKV bf16", dkv16.view(-1, w.D), dkv_ref)
    # attention-sink gradient over every token
    dsink = smqa.bwd_dsink(lb.cuda(), smqa.bwd_preprocess(ob.cuda(), xg["do"]), xg["attn_sink"])
    torch.cuda.synchronize()
    check_dsink("d_sink", dsink, oracle.dsink(ob, x["do"], lb, x["attn_sink"]), ob, x["do"], lb, x["attn_sink"])


def end_to_end_sampled(w, x, toks, rows, bf16_dkv=False):
    """GPU forward against the oracle's forward on sampled tokens; then the GPU backward and the
    oracle's backward, both evaluated on the GPU forward's outputs (O bf16, LSE fp32), on sampled
    tokens (dQ) and kv rows (dKV). Fed the oracle's own forward instead, the two backwards would
    differ through Delta = <O, dO> wherever attention is peaked (early tokens: |O| up to 2-4, where
    one bf16 ulp of O moves the dKV of the rows they pick by up to ~0.1): a difference of inputs,
    not of the kernels."""
    xg = gpu(x)
    o, lse = fwd_gpu(xg)
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], tokens=toks)
    check_bf16("O", o.view(-1, w.H, w.D)[toks], o_ref)
    check_lse("LSE", lse.view(-1, w.H)[toks], lse_ref)
    dq, dkv32 = bwd_gpu(xg, o, lse, fp32=True)
    dkv16 = bwd_gpu(xg, o, lse)[1] if bf16_dkv else None
    del xg
    O, L = o.cpu(), lse.cpu()
    dq_ref, _ = oracle.dq(x["q"], x["kv"], O, x["do"], x["topk_idxs"], L, tokens=toks)
    check_bf16("dQ", dq.view(-1, w.H, w.D)[toks], dq_ref)
    dkv_ref = oracle.dkv(x["q"], x["kv"], O, x["do"], x["topk_idxs"], L, rows=rows)
    check_bf16("dKV fp32", dkv32.view(-1, w.D)[rows], dkv_ref)
    if bf16_dkv:
        check_bf16("dKV bf16", dkv16.view(-1, w.D)[rows], dkv_ref)
    return o, lse, dkv32


@pytest.mark.timeout(900)
def test_long_context_h128_sampled(gpu_lib):
    w = syn.WORKLOADS["long_h128_s16k"]
    say("case", w.describe())
    x = syn.workload_inputs(w)
    toks = sample_tokens(w.S, 12, seed=10, fixed=[0, 1, 2047, 2048, 2049, 16383])
    # The bf16 dKV output at this size runs in token chunks with an fp32 running sum between them.
    # Rows 0 and 1 (every early token and the random picks of later ones) and a middle row (its
    # recent window and later random picks) are referenced by tokens of every chunk; the tail rows
    # only by the last tokens.
    rows = [0, 1, w.S_kv // 2, w.S_kv - 1, w.S_kv - 2, w.S_kv - 17, w.S_kv - 40]
    end_to_end_sampled(w, x, toks, rows, bf16_dkv=True)


@pytest.mark.timeout(900)
def test_gather_b4_masked_full(gpu_lib):
    """The batched gather-bound workload: O, LSE of every token; the backward on the oracle's
    forward outputs with dQ of every token and dKV of 1024 kv rows (the 256 most referenced, the
    first and last rows of every batch, and a random sample), fp32 and bf16 outputs; unreferenced
    rows exactly 0."""
    w = syn.WORKLOADS["gather_b4_skv64k"]
    say("case", w.describe())
    x = syn.workload_inputs(w)
    xg = gpu(x)
    o, lse = fwd_gpu(xg)
    say("  oracle forward, every token")
    o_ref, lse_ref = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    check_bf16("O", o.view(-1, w.H, w.D), o_ref)
    check_lse("LSE", lse.view(-1, w.H), lse_ref)
    del o, lse
    ob = o_ref.view(w.B, w.S, w.H, w.D).to(torch.bfloat16)
    lb = lse_ref.view(w.B, w.S, w.H)
    del o_ref
    dq, dkv32 = bwd_gpu(xg, ob.cuda(), lb.cuda(), fp32=True)
    _, dkv16 = bwd_gpu(xg, ob.cuda(), lb.cuda())
    del xg
    say("  oracle dQ, every token")
    dq_ref, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    check_bf16("dQ", dq.view(-1, w.H, w.D), dq_ref)
    del dq_ref, dq
    idx = x["topk_idxs"].reshape(w.B, -1).long()
    ok = (idx >= 0) & (idx < w.S_kv)
    flat = (idx + torch.arange(w.B).view(-1, 1) * w.S_kv)[ok]
    counts = torch.bincount(flat, minlength=w.B * w.S_kv)
    heavy = torch.topk(counts, 256).indices.tolist()
    edges = [b * w.S_kv + j for b in range(w.B) for j in (0, 1, w.S_kv - 2, w.S_kv - 1)]
    rows = sorted(set(heavy) | set(edges) | set(sample_tokens(w.B * w.S_kv, 1024 - 256 - 16, seed=12)))
    say(f"  oracle dKV, {len(rows)} rows (most referenced: {int(counts.max())} references)")
    dkv_ref = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, rows=rows)
    check_bf16("dKV fp32", dkv32.view(-1, w.D)[rows], dkv_ref)
    check_bf16("dKV bf16", dkv16.view(-1, w.D)[rows], dkv_ref)
    ref_rows = referenced_rows(x["topk_idxs"], w.S_kv).view(-1)
    assert torch.count_nonzero(dkv32.view(-1, w.D).cpu()[~ref_rows]) == 0
    assert torch.count_nonzero(dkv16.view(-1, w.D).cpu()[~ref_rows]) == 0


def _plan_arrays(steps, w):
    """pos [tokens, topk] and offset [words + 1] read back from a one-pass dKV workspace, at the
    byte offsets of the documented layout (kv row norms, plan words, offsets, scan tiles, pos)."""
    r256 = lambda n: (n + 255) // 256 * 256
    n_rows, tokens = w.B * w.S_kv, w.B * w.S
    nw = (min(tokens, w.S) + 31) // 32  # a kv row's words cover the tokens of its own batch
    words = n_rows * nw
    o_off = r256(n_rows * 4) + r256((3 * words + 4) * 4)
    o_pos = o_off + r256((words + 1) * 4) + r256(((words + 4095) // 4096) * 4)
    ws = steps.workspace.cpu()
    offset = ws[o_off:o_off + (words + 1) * 4].view(torch.int32).clone()
    pos = ws[o_pos:o_pos + tokens * w.topk * 4].view(torch.int32).view(tokens, w.topk).clone()
    return pos, offset, nw


@pytest.mark.parametrize("case", ["distinct", "duplicates", "sparse_distinct", "sparse_duplicates"])
def test_staging_plan_structure(gpu_lib, case):
    """The dKV staging plan as the prepare step leaves it in the workspace: every valid (token,
    slot) pair owns n_hblk consecutive staging rows, the pairs of a kv row fill that row's segment
    [offset[r nw], offset[(r + 1) nw]) exactly, masked slots get -1, and (distinct indices) the
    order inside a segment is (k mod nw, k div nw) for k the token's place in its batch,
    independent of timing. The sparse cases have fewer slots than plan words (most words empty),
    as on long kv sequences."""
    g = torch.Generator().manual_seed(77)

    def random_inputs(w, idx):
        return {"q": torch.randn(w.B, w.S, w.H, w.D, generator=g).to(torch.bfloat16),
                "kv": torch.randn(w.B, w.S_kv, w.D, generator=g).to(torch.bfloat16),
                "do": torch.randn(w.B, w.S, w.H, w.D, generator=g).to(torch.bfloat16),
                "topk_idxs": idx.to(torch.int32)}
    if case == "distinct":
        w = syn.WORKLOADS["mid_h64_d512_k300"]
        x = syn.workload_inputs(w)
        n_hblk = 1
    elif case == "duplicates":  # random indices with repeats and out-of-range values, two 64-head blocks
        w = syn.Workload("plan_dups", 2, 40, 70, 128, 512, 90, "causal_distinct", 0, 0)
        x = random_inputs(w, torch.randint(-3, w.S_kv + 3, (w.B, w.S, w.topk), generator=g))
        n_hblk = 2
    elif case == "sparse_distinct":  # distinct rows per token out of 4096, a few masked slots
        w = syn.Workload("plan_sparse", 2, 64, 4096, 64, 512, 64, "causal_distinct", 0, 0)
        idx = torch.stack([torch.randperm(w.S_kv, generator=g)[:w.topk] for _ in range(w.B * w.S)])
        idx[torch.rand(idx.shape, generator=g) < 0.05] = -1
        x = random_inputs(w, idx.view(w.B, w.S, w.topk))
        n_hblk = 1
    else:  # sparse, with repeats and out-of-range values, two 64-head blocks
        w = syn.Workload("plan_sparse_dups", 2, 64, 4096, 128, 512, 64, "causal_distinct", 0, 0)
        idx = torch.randint(-3, w.S_kv + 3, (w.B, w.S, w.topk), generator=g)
        idx[:, :, 1::7] = idx[:, :, 0::7][:, :, :idx[:, :, 1::7].shape[2]]  # repeats inside each token
        x = random_inputs(w, idx)
        n_hblk = 2
    say("case", "staging plan", case)
    xg = gpu({k: x[k] for k in ("q", "kv", "do", "topk_idxs")})
    lse = torch.zeros(w.B, w.S, w.H, device="cuda")
    delta = torch.zeros(w.B, w.S, w.H, device="cuda")
    steps = smqa.DkvSteps(xg["q"], xg["kv"], xg["do"], xg["topk_idxs"], lse, delta)
    steps.prepare()
    torch.cuda.synchronize()
    pos, offset, nw = _plan_arrays(steps, w)
    idx = x["topk_idxs"].view(w.B * w.S, w.topk).long()
    valid = (idx >= 0) & (idx < w.S_kv)
    assert torch.equal(pos[~valid], torch.full_like(pos[~valid], -1))
    p = pos[valid].long()
    n_pairs = int(valid.sum())
    assert int(offset[-1]) == n_hblk * n_pairs
    assert torch.equal(torch.sort(p).values, n_hblk * torch.arange(n_pairs))  # each pair n_hblk rows, no overlap
    ct = torch.arange(w.B * w.S).view(-1, 1).expand_as(idx)
    row = (ct // w.S) * w.S_kv + idx.clamp(0, w.S_kv - 1)
    r, t = row[valid], ct[valid]
    assert bool((p >= offset[r * nw].long()).all()) and bool((p < offset[(r + 1) * nw].long()).all())
    if case.endswith("distinct"):
        # inside a row's segment the pairs follow (token mod nw, token div nw)
        k = t % w.S
        key = r * (32 * nw) + (k % nw) * 32 + k // nw
        order = torch.argsort(p)
        assert bool((key[order][1:] > key[order][:-1]).all())
