"""Helpers for the GPU parity tests: tolerance checks against the oracle and sample choice."""
from __future__ import annotations

import math
import sys
from typing import Iterable, List

import torch

# Floating-point bar: |err| <= 2e-2 + 2e-2 |ref| for bf16 O, dQ and dKV; 1e-3 absolute for the
# fp32 (base-2) LSE. A relative-L2 gate of 1e-2 is applied as well so that an error hidden by the
# absolute term on small-magnitude outputs still fails.
BF16_ATOL = 2e-2
BF16_RTOL = 2e-2
LSE_ATOL = 1e-3
REL_L2_MAX = 1e-2


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def check_bf16(name: str, got: torch.Tensor, ref: torch.Tensor, rel_l2_max: float = REL_L2_MAX) -> float:
    g = got.detach().double().cpu()
    r = ref.detach().double().cpu()
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert not torch.isnan(g).any(), f"{name}: NaN in GPU output"
    err = (g - r).abs()
    bad = err > BF16_ATOL + BF16_RTOL * r.abs()
    nbad = int(bad.sum())
    rel = float((g - r).norm() / max(float(r.norm()), 1e-30))
    say(f"  {name}: max|err| {float(err.max()):.3e}  rel-L2 {rel:.3e}  n={r.numel()}")
    assert nbad == 0, f"{name}: {nbad} of {r.numel()} elements outside |err| <= {BF16_ATOL} + {BF16_RTOL}|ref|"
    assert rel <= rel_l2_max, f"{name}: relative L2 error {rel:.3e} > {rel_l2_max}"
    return rel


def check_lse(name: str, got: torch.Tensor, ref: torch.Tensor) -> None:
    g = got.detach().double().cpu()
    r = ref.detach().double().cpu()
    assert g.shape == r.shape
    inf_r = torch.isinf(r)
    assert torch.equal(torch.isinf(g), inf_r) and torch.equal(g[inf_r], r[inf_r]), f"{name}: infinite entries differ"
    fin = ~inf_r
    err = (g[fin] - r[fin]).abs()
    m = float(err.max()) if err.numel() else 0.0
    say(f"  {name}: max|err| {m:.3e}")
    assert not torch.isnan(g).any()
    assert m <= LSE_ATOL, f"{name}: max |err| {m} > {LSE_ATOL}"


def check_dsink(name: str, got: torch.Tensor, ref: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
                lse: torch.Tensor, sink: torch.Tensor, rel: float = 1e-4) -> None:
    """d_sink against the oracle, per head: |err| <= rel * sum_t p_sink(t) sum_d |O dO| + 1e-30.
    The scale bounds every term before cancellation. On the same O and LSE the GPU forms Delta as
    an fp32 dot of D products (error <= D * 2^-24 of that scale) and sums B*S fp32 terms in a
    tree, so rel = 1e-4 leaves room while a dropped term, a wrong sign or a wrong head index is
    off by O(scale). When the GPU's O is its own bf16 forward output rather than the oracle's,
    each element may differ by one bf16 ulp (2^-7 relative), so rel = 1e-2 bounds that case."""
    g = got.detach().double().cpu()
    r = ref.detach().double().cpu()
    H = r.shape[0]
    assert g.shape == r.shape
    assert not torch.isnan(g).any(), f"{name}: NaN in GPU output"
    absdot = (o.double() * do.double()).abs().sum(-1).reshape(-1, H)
    p = torch.exp2(sink.double().view(1, H) / math.log(2) - lse.double().reshape(-1, H))
    p = torch.where(torch.isfinite(sink.double()).view(1, H), p, torch.zeros_like(p))
    scale = (p * absdot).sum(0)
    err = (g - r).abs()
    say(f"  {name}: max|err| {float(err.max()):.3e}  max err/scale {float((err / (scale + 1e-30)).max()):.3e}")
    bad = err > rel * scale + 1e-30
    assert not bad.any(), f"{name}: heads {torch.nonzero(bad).view(-1).tolist()} outside the bound"
    inf_heads = ~torch.isfinite(sink)
    assert torch.all(g[inf_heads] == 0), f"{name}: heads with a -inf sink must get exactly 0"


def sample_tokens(n_tokens: int, extra: int, seed: int, fixed: Iterable[int] = ()) -> List[int]:
    g = torch.Generator().manual_seed(seed)
    base = [t for t in fixed if 0 <= t < n_tokens]
    rnd = torch.randperm(n_tokens, generator=g)[:extra].tolist()
    return sorted(set(base + rnd))


def bf16_round(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def valid_mask(idx: torch.Tensor, s_kv: int) -> torch.Tensor:
    return (idx >= 0) & (idx < s_kv)


def referenced_rows(idx: torch.Tensor, s_kv: int) -> torch.Tensor:
    """Boolean [B, S_kv]: rows that at least one valid slot references."""
    B = idx.shape[0]
    v = valid_mask(idx, s_kv)
    hit = torch.zeros(B, s_kv, dtype=torch.int64)
    hit.scatter_add_(1, torch.where(v, idx, torch.zeros_like(idx)).long().view(B, -1), v.long().view(B, -1))
    return hit > 0


def conservation_rhs(q, o, do, lse, sink, sm_scale):
    """sum_{s,h} (sm_scale * Delta * P_sink * q + (1 - P_sink) * dO) per batch, in float64."""
    qd, od, dod = q.double(), o.double(), do.double()
    delta = (od * dod).sum(-1)
    p_sink = torch.exp2(sink.double() / math.log(2.0) - lse.double())
    p_sink = torch.where(torch.isinf(lse), torch.zeros_like(p_sink), p_sink)
    return (sm_scale * (delta * p_sink)[..., None] * qd + (1 - p_sink)[..., None] * dod).sum((1, 2))
