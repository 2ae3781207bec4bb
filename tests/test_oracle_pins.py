"""Pins of the CPU oracle to references independent of it (no GPU needed).

The pages print no worked values, so each pin is an independent route to the same numbers:
  - dense masked softmax attention in float64 with torch.autograd gradients (a different
    formulation: all kv rows, a log-multiplicity mask and an appended sink column);
  - torch's scaled_dot_product_attention when the sink is -inf (library routine);
  - closed forms (zero query, one slot, two slots, identical rows, fully masked tokens);
  - exact invariants (slot permutation, power-of-two rescaling, masked values of every kind);
  - central finite differences of L = sum(O * dO);
  - the dKV conservation identity sum_j dKV[j] = sum_{s,h} (sm_scale Delta P_sink q + (1-P_sink) dO).
A plausible slip in the oracle (a dropped sink, the scale applied twice, natural instead of base-2
LSE, a transposed operand, a wrong sign in dS, a dKV row off by one) fails at least one of these.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from top_sparse_mqa_amd import synthetic as syn

LN2 = math.log(2.0)
I32MIN, I32MAX = -(2 ** 31), 2 ** 31 - 1


def dense_reference(q, kv, sink, idx, scale):
    """O and base-2 LSE from dense softmax over all kv rows, masked by slot multiplicity."""
    B, S, H, D = q.shape
    S_kv = kv.shape[1]
    valid = (idx >= 0) & (idx < S_kv)
    cnt = torch.zeros(B, S, S_kv, dtype=torch.float64)
    cnt.scatter_add_(2, torch.where(valid, idx, torch.zeros_like(idx)).long(), valid.double())
    logits = torch.einsum("bshd,bjd->bshj", q, kv) * scale + torch.log(cnt)[:, :, None, :]
    allz = torch.cat([logits, sink.view(1, 1, H, 1).expand(B, S, H, 1)], dim=-1)
    lse = torch.logsumexp(allz, dim=-1)
    p = torch.exp(allz - lse[..., None])[..., :S_kv]
    return torch.einsum("bshj,bjd->bshd", p, kv), lse / LN2


def dense_grads(q, kv, sink, idx, scale, do):
    qq = q.clone().requires_grad_(True)
    kk = kv.clone().requires_grad_(True)
    o, _ = dense_reference(qq, kk, sink, idx, scale)
    (o * do).sum().backward()
    return qq.grad, kk.grad


def rand_case(seed, B, S, S_kv, H, D, topk, lo=-3, hi_extra=3, extremes=True, sink_inf=False):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    kv = torch.randn(B, S_kv, D, generator=g, dtype=torch.float64)
    sink = torch.randn(H, generator=g, dtype=torch.float64)
    if sink_inf:
        sink[:] = -math.inf
    idx = torch.randint(lo, S_kv + hi_extra, (B, S, topk), generator=g, dtype=torch.int64)
    if extremes:
        pick = torch.rand(B, S, topk, generator=g)
        idx = torch.where(pick < 0.05, torch.full_like(idx, I32MIN), idx)
        idx = torch.where((pick >= 0.05) & (pick < 0.1), torch.full_like(idx, I32MAX), idx)
    do = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    return q, kv, sink, idx.to(torch.int32), do


def tokens_with_valid(idx, S_kv):
    return ((idx >= 0) & (idx < S_kv)).any(-1)


CASES = [
    # seed, B, S, S_kv, H, D, topk
    (0, 1, 4, 7, 1, 4, 1),
    (1, 2, 3, 9, 3, 8, 5),
    (2, 1, 5, 6, 2, 8, 12),   # topk > S_kv: duplicates certain
    (3, 2, 2, 16, 4, 16, 9),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_matches_dense_f64(case):
    seed, B, S, S_kv, H, D, topk = case
    q, kv, sink, idx, _ = rand_case(seed, B, S, S_kv, H, D, topk)
    scale = 0.37
    o_ref, lse_ref = dense_reference(q, kv, sink, idx, scale)
    o, lse = oracle.fwd(q, kv, sink.float(), idx, sm_scale=scale, precision="f64")
    # the sink is compared in fp32 by the oracle's interface; use the same rounded sink in the reference
    o_ref, lse_ref = dense_reference(q, kv, sink.float().double(), idx, scale)
    torch.testing.assert_close(o.view(B, S, H, D), o_ref, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(lse.view(B, S, H), lse_ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_dense_autograd_f64(case):
    seed, B, S, S_kv, H, D, topk = case
    q, kv, sink, idx, do = rand_case(seed, B, S, S_kv, H, D, topk)
    sink = sink.float().double()
    scale = 0.29
    o, lse = oracle.fwd(q, kv, sink.float(), idx, sm_scale=scale, precision="f64")
    o, lse = o.view(B, S, H, D), lse.view(B, S, H)
    dq, delta = oracle.dq(q, kv, o, do, idx, lse, sm_scale=scale, precision="f64")
    dkv = oracle.dkv(q, kv, o, do, idx, lse, sm_scale=scale, precision="f64")
    gq, gkv = dense_grads(q, kv, sink, idx, scale, do)
    torch.testing.assert_close(dq.view(B, S, H, D), gq, rtol=1e-9, atol=1e-11)
    torch.testing.assert_close(dkv.view(B, S_kv, D), gkv, rtol=1e-9, atol=1e-11)
    torch.testing.assert_close(delta.view(B, S, H), (o * do).sum(-1), rtol=1e-12, atol=1e-12)


def test_f32_instance_close_to_dense():
    q, kv, sink, idx, do = rand_case(7, 1, 6, 20, 4, 32, 10)
    q, kv, do = q.float().double(), kv.float().double(), do.float().double()
    sink = sink.float().double()
    o_ref, lse_ref = dense_reference(q, kv, sink, idx, 0.2)
    o, lse = oracle.fwd(q.float(), kv.float(), sink.float(), idx, sm_scale=0.2, precision="f32")
    torch.testing.assert_close(o.double().view_as(o_ref), o_ref, rtol=2e-5, atol=2e-6)
    torch.testing.assert_close(lse.double().view_as(lse_ref), lse_ref, rtol=2e-5, atol=2e-5)
    gq, gkv = dense_grads(q, kv, sink, idx, 0.2, do)
    o64, lse64 = oracle.fwd(q, kv, sink.float(), idx, sm_scale=0.2, precision="f64")
    dq, _ = oracle.dq(q.float(), kv.float(), o64.float().view(q.shape), do.float(), idx, lse64.float().view(1, 6, 4),
                      sm_scale=0.2, precision="f32")
    dkv = oracle.dkv(q.float(), kv.float(), o64.float().view(q.shape), do.float(), idx,
                     lse64.float().view(1, 6, 4), sm_scale=0.2, precision="f32")
    torch.testing.assert_close(dq.double().view_as(gq), gq, rtol=1e-4, atol=1e-5)
    torch.testing.assert_close(dkv.double().view_as(gkv), gkv, rtol=1e-4, atol=1e-5)


def test_sdpa_when_sink_is_minus_inf():
    """sink = -inf turns the method into ordinary masked softmax attention (library routine)."""
    g = torch.Generator().manual_seed(11)
    B, S, S_kv, H, D, topk = 2, 5, 12, 3, 16, 6
    q = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    kv = torch.randn(B, S_kv, D, generator=g, dtype=torch.float64)
    idx = torch.stack([torch.stack([torch.randperm(S_kv, generator=g)[:topk] for _ in range(S)]) for _ in range(B)])
    idx[:, :, -1] = -1  # one masked slot per token; no duplicates
    idx = idx.to(torch.int32)
    sink = torch.full((H,), -math.inf)
    scale = 0.3
    o, lse = oracle.fwd(q, kv, sink, idx, sm_scale=scale, precision="f64")
    hits = torch.zeros(B, S, S_kv, dtype=torch.int64)
    hits.scatter_add_(2, torch.where(idx >= 0, idx, torch.zeros_like(idx)).long(), (idx >= 0).long())
    mask = hits > 0
    qh = q.permute(0, 2, 1, 3)                                  # [B,H,S,D]
    kh = kv[:, None].expand(B, H, S_kv, D)
    ref = F.scaled_dot_product_attention(qh, kh, kh, attn_mask=mask[:, None], scale=scale)
    torch.testing.assert_close(o.view(B, S, H, D), ref.permute(0, 2, 1, 3), rtol=1e-11, atol=1e-12)
    logits = torch.einsum("bshd,bjd->bshj", q, kv) * scale
    lse_ref = torch.logsumexp(logits.masked_fill(~mask[:, :, None], -math.inf), -1) / LN2
    torch.testing.assert_close(lse.view(B, S, H), lse_ref, rtol=1e-11, atol=1e-12)


def test_zero_query_closed_form():
    """q = 0: every score is 0, so O = sum_valid kv / (n + e^sink) and LSE = log2(n + e^sink)."""
    g = torch.Generator().manual_seed(3)
    B, S, S_kv, H, D, topk = 1, 3, 10, 2, 8, 6
    q = torch.zeros(B, S, H, D, dtype=torch.float64)
    kv = torch.randn(B, S_kv, D, generator=g, dtype=torch.float64)
    sink = torch.tensor([0.5, -1.25], dtype=torch.float32)
    idx = torch.tensor([[[0, 1, 2, -1, 5, 12], [3, 3, 9, -7, -1, -1], [4, -1, -1, -1, -1, -1]]], dtype=torch.int32)
    o, lse = oracle.fwd(q, kv, sink, idx, precision="f64")
    o = o.view(S, H, D)
    for s in range(S):
        rows = [int(i) for i in idx[0, s] if 0 <= i < S_kv]
        n = len(rows)
        for h in range(H):
            z = n + math.exp(float(sink[h]))
            torch.testing.assert_close(o[s, h], kv[0, rows].sum(0) / z, rtol=1e-13, atol=1e-14)
            assert abs(float(lse[s, h]) - math.log2(z)) < 1e-13


def test_single_valid_slot_closed_form():
    """One valid slot and a -inf sink: O = kv_i exactly, LSE = z log2(e), dQ = 0 exactly,
    dKV[i] = sum_h dO_h, every other dKV row exactly 0."""
    g = torch.Generator().manual_seed(5)
    B, S, S_kv, H, D = 1, 2, 6, 3, 8
    q = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    kv = torch.randn(B, S_kv, D, generator=g, dtype=torch.float64)
    do = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    sink = torch.full((H,), -math.inf)
    idx = torch.tensor([[[-1, 4, -1], [2, 7, -5]]], dtype=torch.int32)
    o, lse = oracle.fwd(q, kv, sink, idx, sm_scale=0.5, precision="f64")
    o, lse = o.view(B, S, H, D), lse.view(B, S, H)
    assert torch.equal(o[0, 0], kv[0, 4].expand(H, D))
    assert torch.equal(o[0, 1], kv[0, 2].expand(H, D))
    z = 0.5 * torch.einsum("hd,d->h", q[0, 0], kv[0, 4])
    torch.testing.assert_close(lse[0, 0], z / LN2, rtol=1e-14, atol=1e-14)
    dq, _ = oracle.dq(q, kv, o, do, idx, lse, sm_scale=0.5, precision="f64")
    assert torch.count_nonzero(dq) == 0
    dkv = oracle.dkv(q, kv, o, do, idx, lse, sm_scale=0.5, precision="f64").view(S_kv, D)
    torch.testing.assert_close(dkv[4], do[0, 0].sum(0), rtol=1e-13, atol=1e-14)
    torch.testing.assert_close(dkv[2], do[0, 1].sum(0), rtol=1e-13, atol=1e-14)
    for j in (0, 1, 3, 5):
        assert torch.count_nonzero(dkv[j]) == 0


def test_two_slots_logistic():
    g = torch.Generator().manual_seed(8)
    q = torch.randn(1, 1, 2, 8, generator=g, dtype=torch.float64)
    kv = torch.randn(1, 4, 8, generator=g, dtype=torch.float64)
    idx = torch.tensor([[[1, 3]]], dtype=torch.int32)
    o, _ = oracle.fwd(q, kv, torch.full((2,), -math.inf), idx, sm_scale=0.7, precision="f64")
    for h in range(2):
        z1 = 0.7 * float(q[0, 0, h] @ kv[0, 1])
        z3 = 0.7 * float(q[0, 0, h] @ kv[0, 3])
        w = 1.0 / (1.0 + math.exp(z3 - z1))
        torch.testing.assert_close(o[0, h], w * kv[0, 1] + (1 - w) * kv[0, 3], rtol=1e-13, atol=1e-14)


def test_identical_rows_show_the_sink_weight():
    """All kv rows equal c: O = (1 - P_sink) c with P_sink = e^sink / (n e^z + e^sink)."""
    c = torch.linspace(-1, 1, 16, dtype=torch.float64)
    kv = c.expand(1, 9, 16).clone()
    g = torch.Generator().manual_seed(2)
    q = torch.randn(1, 2, 3, 16, generator=g, dtype=torch.float64)
    sink = torch.tensor([1.5, 0.0, -2.0], dtype=torch.float32)
    idx = torch.tensor([[[0, 3, 5, 8], [1, -1, 2, 20]]], dtype=torch.int32)
    o, lse = oracle.fwd(q, kv, sink, idx, sm_scale=0.25, precision="f64")
    o, lse = o.view(2, 3, 16), lse.view(2, 3)
    for s, n in ((0, 4), (1, 2)):
        for h in range(3):
            z = 0.25 * float(q[0, s, h] @ c)
            tot = n * math.exp(z) + math.exp(float(sink[h]))
            torch.testing.assert_close(o[s, h], (n * math.exp(z) / tot) * c, rtol=1e-13, atol=1e-14)
            assert abs(float(lse[s, h]) - math.log2(tot)) < 1e-12


@pytest.mark.parametrize("sink_value", [0.75, -math.inf])
def test_fully_masked_token(sink_value):
    g = torch.Generator().manual_seed(9)
    B, S, S_kv, H, D = 1, 2, 5, 2, 8
    q = torch.randn(B, S, H, D, generator=g)
    kv = torch.randn(B, S_kv, D, generator=g)
    do = torch.randn(B, S, H, D, generator=g)
    sink = torch.full((H,), sink_value)
    idx = torch.tensor([[[-1, 5, I32MIN, I32MAX], [-2, 99, -1, 5]]], dtype=torch.int32)
    for prec in ("f32", "f64"):
        o, lse = oracle.fwd(q, kv, sink, idx, precision=prec)
        assert torch.count_nonzero(o) == 0 and not torch.isnan(o).any()
        assert torch.all(torch.signbit(o) == 0)  # +0, not -0
        expect = sink_value / LN2 if math.isfinite(sink_value) else -math.inf
        assert torch.all(lse == torch.tensor(expect, dtype=lse.dtype)) or torch.allclose(
            lse, torch.full_like(lse, expect), rtol=1e-6)
        lse_in = lse.view(B, S, H)
        dq, _ = oracle.dq(q, kv, o.view(B, S, H, D), do, idx, lse_in, precision=prec)
        assert torch.count_nonzero(dq) == 0 and not torch.isnan(dq).any()
        dkv = oracle.dkv(q, kv, o.view(B, S, H, D), do, idx, lse_in, precision=prec)
        assert torch.count_nonzero(dkv) == 0


def test_out_of_range_values_equal_dropping_them():
    g = torch.Generator().manual_seed(4)
    B, S, S_kv, H, D = 1, 3, 8, 2, 16
    q = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    kv = torch.randn(B, S_kv, D, generator=g, dtype=torch.float64)
    do = torch.randn(B, S, H, D, generator=g, dtype=torch.float64)
    sink = torch.tensor([0.1, -0.4])
    clean = torch.tensor([[[0, 5, 7, -1, -1, -1, -1]] * 3], dtype=torch.int32).view(1, 3, 7)
    dirty = torch.tensor([[[0, 5, 7, 8, I32MIN, I32MAX, -123456]] * 3], dtype=torch.int32).view(1, 3, 7)
    oc, lc = oracle.fwd(q, kv, sink, clean, precision="f64")
    od, ld = oracle.fwd(q, kv, sink, dirty, precision="f64")
    assert torch.equal(oc, od) and torch.equal(lc, ld)
    o, lse = oc.view(B, S, H, D), lc.view(B, S, H)
    assert torch.equal(oracle.dq(q, kv, o, do, clean, lse, precision="f64")[0],
                       oracle.dq(q, kv, o, do, dirty, lse, precision="f64")[0])
    assert torch.equal(oracle.dkv(q, kv, o, do, clean, lse, precision="f64"),
                       oracle.dkv(q, kv, o, do, dirty, lse, precision="f64"))


def test_slot_permutation_invariance():
    q, kv, sink, idx, do = rand_case(21, 2, 4, 11, 3, 8, 9)
    sink = sink.float()
    perm = torch.randperm(9, generator=torch.Generator().manual_seed(1))
    o1, l1 = oracle.fwd(q, kv, sink, idx, precision="f64")
    o2, l2 = oracle.fwd(q, kv, sink, idx[:, :, perm].contiguous(), precision="f64")
    torch.testing.assert_close(o1, o2, rtol=1e-13, atol=1e-14)
    torch.testing.assert_close(l1, l2, rtol=1e-13, atol=1e-14)
    o, lse = o1.view(2, 4, 3, 8), l1.view(2, 4, 3)
    d1 = oracle.dq(q, kv, o, do, idx, lse, precision="f64")[0]
    d2 = oracle.dq(q, kv, o, do, idx[:, :, perm].contiguous(), lse, precision="f64")[0]
    torch.testing.assert_close(d1, d2, rtol=1e-12, atol=1e-13)
    k1 = oracle.dkv(q, kv, o, do, idx, lse, precision="f64")
    k2 = oracle.dkv(q, kv, o, do, idx[:, :, perm].contiguous(), lse, precision="f64")
    torch.testing.assert_close(k1, k2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_power_of_two_rescaling_is_exact(precision):
    """Doubling q while halving sm_scale leaves every score bit-identical; doubling dO doubles
    dQ and dKV exactly."""
    q, kv, sink, idx, do = rand_case(13, 1, 5, 10, 2, 16, 7, extremes=False)
    sink = sink.float()
    o1, l1 = oracle.fwd(q, kv, sink, idx, sm_scale=0.25, precision=precision)
    o2, l2 = oracle.fwd(2 * q, kv, sink, idx, sm_scale=0.125, precision=precision)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o, lse = o1.view(1, 5, 2, 16), l1.view(1, 5, 2)
    a = oracle.dq(q, kv, o, do, idx, lse, sm_scale=0.25, precision=precision)[0]
    b = oracle.dq(q, kv, o, 2 * do, idx, lse, sm_scale=0.25, precision=precision)[0]
    # Delta doubles too, so dS doubles exactly
    assert torch.equal(2 * a, b)
    ka = oracle.dkv(q, kv, o, do, idx, lse, sm_scale=0.25, precision=precision)
    kb = oracle.dkv(q, kv, o, 2 * do, idx, lse, sm_scale=0.25, precision=precision)
    assert torch.equal(2 * ka, kb)


def test_finite_differences():
    """Central differences of L = sum(O*dO) against dQ and dKV of the float64 oracle."""
    q, kv, sink, idx, do = rand_case(17, 1, 3, 7, 2, 8, 6, extremes=False)
    sink = sink.float()
    scale = 0.4
    o, lse = oracle.fwd(q, kv, sink, idx, sm_scale=scale, precision="f64")
    o, lse = o.view(q.shape), lse.view(1, 3, 2)
    dq = oracle.dq(q, kv, o, do, idx, lse, sm_scale=scale, precision="f64")[0].view(q.shape)
    dkv = oracle.dkv(q, kv, o, do, idx, lse, sm_scale=scale, precision="f64").view(kv.shape)

    def loss(qq, kk):
        oo, _ = oracle.fwd(qq, kk, sink, idx, sm_scale=scale, precision="f64")
        return float((oo.view(q.shape) * do).sum())

    g = torch.Generator().manual_seed(0)
    eps = 1e-6
    for _ in range(24):
        i = tuple(int(torch.randint(0, n, (1,), generator=g)) for n in q.shape)
        qp, qm = q.clone(), q.clone()
        qp[i] += eps
        qm[i] -= eps
        fd = (loss(qp, kv) - loss(qm, kv)) / (2 * eps)
        assert abs(fd - float(dq[i])) <= 1e-6 * max(1.0, abs(fd)), (i, fd, float(dq[i]))
    for _ in range(24):
        i = tuple(int(torch.randint(0, n, (1,), generator=g)) for n in kv.shape)
        kp, km = kv.clone(), kv.clone()
        kp[i] += eps
        km[i] -= eps
        fd = (loss(q, kp) - loss(q, km)) / (2 * eps)
        assert abs(fd - float(dkv[i])) <= 1e-6 * max(1.0, abs(fd)), (i, fd, float(dkv[i]))


def test_dkv_conservation_identity():
    """sum_t dS_t = Delta * P_sink (when O is the exact forward output), hence
    sum_j dKV[j] = sum_{s,h} (sm_scale * Delta * P_sink * q + (1 - P_sink) * dO)."""
    q, kv, sink, idx, do = rand_case(31, 2, 6, 13, 4, 16, 8)
    sink = sink.float()
    scale = 0.3
    o, lse = oracle.fwd(q, kv, sink, idx, sm_scale=scale, precision="f64")
    o, lse = o.view(q.shape), lse.view(2, 6, 4)
    dkv = oracle.dkv(q, kv, o, do, idx, lse, sm_scale=scale, precision="f64").view(kv.shape)
    delta = (o * do).sum(-1)
    p_sink = torch.exp2(sink.double() / LN2 - lse)
    expect = (scale * (delta * p_sink)[..., None] * q + (1 - p_sink)[..., None] * do).sum((1, 2))
    torch.testing.assert_close(dkv.sum(1), expect, rtol=1e-10, atol=1e-11)


def test_token_and_row_subsets_match_full_outputs():
    w = syn.WORKLOADS["tiny_h16_d64"]
    x = syn.workload_inputs(w)
    o, lse = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"])
    toks = [0, 5, 127, 64]
    os_, ls_ = oracle.fwd(x["q"], x["kv"], x["attn_sink"], x["topk_idxs"], tokens=toks)
    assert torch.equal(os_, o[toks]) and torch.equal(ls_, lse[toks])
    ob, lb = o.view(1, w.S, w.H, w.D).bfloat16(), lse.view(1, w.S, w.H)
    dq, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    dqs, _ = oracle.dq(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, tokens=toks)
    assert torch.equal(dqs, dq[toks])
    dk = oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb)
    rows = [0, 17, 255, 127]
    assert torch.equal(oracle.dkv(x["q"], x["kv"], ob, x["do"], x["topk_idxs"], lb, rows=rows), dk[rows])
    # rows no token references are exactly zero (tokens only see positions <= s < 128)
    assert torch.count_nonzero(dk[128:]) == 0


def dense_sink_grad(q, kv, sink, idx, scale, do):
    """d_sink from torch.autograd through the dense reference (the sink as a leaf)."""
    ss = sink.clone().requires_grad_(True)
    o, _ = dense_reference(q, kv, ss, idx, scale)
    (o * do).sum().backward()
    return ss.grad


@pytest.mark.parametrize("case", CASES)
def test_dsink_matches_dense_autograd_f64(case):
    seed, B, S, S_kv, H, D, topk = case
    q, kv, sink, idx, do = rand_case(seed, B, S, S_kv, H, D, topk)
    sink = sink.float().double()
    scale = 0.31
    o, lse = oracle.fwd(q, kv, sink.float(), idx, sm_scale=scale, precision="f64")
    ds = oracle.dsink(o.view(B, S, H, D), do, lse.view(B, S, H), sink.float())
    torch.testing.assert_close(ds, dense_sink_grad(q, kv, sink, idx, scale, do), rtol=1e-9, atol=1e-11)


def test_dsink_finite_differences():
    """Central differences of L(sink) = sum(O(sink) * dO) through the oracle's own forward."""
    B, S, S_kv, H, D, topk = 1, 6, 11, 3, 8, 7
    q, kv, sink, idx, do = rand_case(5, B, S, S_kv, H, D, topk)
    sink = sink.float().double()
    scale = 0.4
    o, lse = oracle.fwd(q, kv, sink.float(), idx, sm_scale=scale, precision="f64")
    ds = oracle.dsink(o.view(B, S, H, D), do, lse.view(B, S, H), sink.float())
    eps = 2.0 ** -12  # exact in fp32, the precision the oracle takes the sink in
    for h in range(H):
        e = torch.zeros(H, dtype=torch.float64)
        e[h] = eps
        op, _ = oracle.fwd(q, kv, (sink + e).float(), idx, sm_scale=scale, precision="f64")
        om, _ = oracle.fwd(q, kv, (sink - e).float(), idx, sm_scale=scale, precision="f64")
        fd = ((op - om).view(B, S, H, D) * do).sum() / (2 * eps)
        assert abs(float(ds[h]) - float(fd)) <= 1e-6 * (1 + abs(float(fd))), (h, float(ds[h]), float(fd))


def test_dsink_single_slot_closed_form():
    """One head, one token, one valid slot: Z = e^z + e^sink, O = p v, d_sink = -(e^sink / Z) p (v . dO)."""
    g = torch.Generator().manual_seed(11)
    D = 8
    q = torch.randn(1, 1, 1, D, generator=g, dtype=torch.float64)
    kv = torch.randn(1, 3, D, generator=g, dtype=torch.float64)
    do = torch.randn(1, 1, 1, D, generator=g, dtype=torch.float64)
    idx = torch.tensor([[[2, -1]]], dtype=torch.int32)
    sink = torch.tensor([0.25], dtype=torch.float32)
    scale = 0.5
    o, lse = oracle.fwd(q, kv, sink, idx, sm_scale=scale, precision="f64")
    z = scale * float((q[0, 0, 0] * kv[0, 2]).sum())
    zs = math.exp(z) + math.exp(0.25)
    p = math.exp(z) / zs
    expect = -(math.exp(0.25) / zs) * p * float((kv[0, 2] * do[0, 0, 0]).sum())
    ds = oracle.dsink(o.view(1, 1, 1, D), do, lse.view(1, 1, 1), sink)
    assert abs(float(ds[0]) - expect) <= 1e-12 * (1 + abs(expect))


def test_dsink_minus_inf_sink_and_masked_tokens():
    """A -inf sink has zero gradient (no NaN from its -inf LSE); a fully masked token adds nothing."""
    B, S, S_kv, H, D, topk = 1, 4, 6, 2, 8, 3
    q, kv, sink, idx, do = rand_case(9, B, S, S_kv, H, D, topk, extremes=False)
    idx[0, 1] = -1  # token 1 fully masked
    sink = torch.tensor([-math.inf, 0.5], dtype=torch.float32)
    o, lse = oracle.fwd(q, kv, sink, idx, precision="f64")
    ds = oracle.dsink(o.view(B, S, H, D), do, lse.view(B, S, H), sink)
    assert float(ds[0]) == 0.0
    keep = torch.ones(S, dtype=torch.bool)
    keep[1] = False
    ds_wo = oracle.dsink(o.view(B, S, H, D)[:, keep], do[:, keep], lse.view(B, S, H)[:, keep], sink)
    assert torch.equal(ds, ds_wo) or abs(float(ds[1] - ds_wo[1])) < 1e-15


def large_logit_case(H=1, D=8, seed=0):
    """Scores near 2^21 (fp32 spacing 0.25) whose exact dot products are integers < 2^24, so a
    dot product is exact in fp32 and only the product with sm_scale rounds. Slots differ by
    O(1) in the logit, so that rounding moves the softmax weights visibly."""
    g = torch.Generator().manual_seed(seed)
    K = 6
    q = torch.zeros(1, 1, H, D)
    q[..., 0] = 2048.0
    q[..., 1] = 1.0
    kv = torch.zeros(1, K, D)
    kv[0, :, 0] = 7936.0
    kv[0, :, 1] = torch.tensor([0.0, 1.0, 2.0, 3.0, 5.0, 8.0])
    kv[0, :, 2:] = torch.randint(-3, 4, (K, D - 2), generator=g).float()
    idx = torch.arange(K, dtype=torch.int32).view(1, 1, K)
    return q.to(torch.bfloat16), kv.to(torch.bfloat16), torch.zeros(H), idx


def test_f32_oracle_rounds_the_scaled_logit_to_fp32():
    """fwd page, reference_rounding option: the fp32 arithmetic rounds the scaled logit
    dot * sm_scale to fp32 before the softmax. Computed here by hand (numpy float32 for the one
    rounding, float64 for the rest) and compared with the fp32 oracle; the float64 oracle, which
    keeps the exact logits, lands visibly elsewhere on this case."""
    q, kv, sink, idx = large_logit_case()
    sm = 0.13
    o32, lse32 = oracle.fwd(q, kv, sink, idx, sm_scale=sm, precision="f32")
    dots = (q[0, 0, 0].double() @ kv[0].double().T).numpy()
    assert np.all(dots == np.round(dots)) and dots.max() < 2 ** 24
    z = (dots.astype(np.float32) * np.float32(sm)).astype(np.float32).astype(np.float64)
    w = np.exp(z - z.max())
    expect = (w @ kv[0].double().numpy()) / w.sum()
    np.testing.assert_allclose(o32[0, 0].double().numpy(), expect, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(float(lse32[0, 0]), (z.max() + math.log(w.sum())) / math.log(2), rtol=1e-7)
    o64, _ = oracle.fwd(q, kv, sink, idx, sm_scale=sm, precision="f64")
    assert float((o64[0, 0, 2:] - o32[0, 0, 2:]).abs().max()) > 0.05
