"""Seeded synthetic inputs for top-k sparse MQA workloads.

Only random draws and index structure live here; nothing of the attention arithmetic. Both the
HIP path and the CPU oracle consume exactly these bytes (generated on the CPU, copied to the GPU).

Every tensor comes from torch.Generator(seed) on the CPU in the fixed order q, kv, attn_sink,
topk_idxs; dO comes from its own generator (do_seed). Values: q, kv, dO ~ N(0,1) drawn in fp32 and
rounded to bf16; attn_sink ~ N(0,1) fp32.

Index recipes (per token s of batch b; unused slots are -1 at the tail):
  causal_distinct    min(s+1, topk) distinct positions drawn uniformly from [0, s], in draw order.
  recent_plus_random s+1 <= topk: all of [0, s]. Otherwise the topk/2 most recent positions
                     [s - topk/2 + 1, s] plus topk/2 distinct positions drawn uniformly from the
                     older range [0, s - topk/2]; all sorted ascending.
  uniform_masked     topk distinct positions drawn uniformly from [0, S_kv), in draw order; then
                     each slot independently (p = 0.05) replaced by an out-of-range value chosen
                     uniformly from {-1, INT32_MIN, S_kv, S_kv + r, INT32_MAX}, r in [1, 2^20).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

INT32_MIN = -(2 ** 31)
INT32_MAX = 2 ** 31 - 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    S_kv: int
    H: int
    D: int
    topk: int
    index_recipe: str
    seed: int
    do_seed: int

    @property
    def shapes(self) -> Dict[str, tuple]:
        return {"q": (self.B, self.S, self.H, self.D), "kv": (self.B, self.S_kv, self.D),
                "attn_sink": (self.H,), "topk_idxs": (self.B, self.S, self.topk)}

    def describe(self) -> Dict[str, object]:
        return {"workload": self.name, "B": self.B, "S": self.S, "S_kv": self.S_kv, "H": self.H, "D": self.D,
                "topk": self.topk, "indices": self.index_recipe, "seed": self.seed, "do_seed": self.do_seed}


WORKLOADS: Dict[str, Workload] = {
    # tiny fwd+bwd parity case
    "tiny_h16_d64": Workload("tiny_h16_d64", 1, 128, 256, 16, 64, 64, "causal_distinct", 0, 100),
    # mid-size parity case: several 64-slot blocks and a ragged tail (300 = 4*64 + 44)
    "mid_h64_d512_k300": Workload("mid_h64_d512_k300", 1, 384, 512, 64, 512, 300, "causal_distinct", 5, 105),
    # the headline shapes: S = S_kv = 4096, H = 64, D = 512, topk = 2048, causal sampling
    "causal_h64_d512_k2048": Workload("causal_h64_d512_k2048", 1, 4096, 4096, 64, 512, 2048,
                                      "causal_distinct", 1, 2),
    # long context, H = 128, sorted recent + random older indices
    "long_h128_s16k": Workload("long_h128_s16k", 1, 16384, 16384, 128, 512, 2048, "recent_plus_random", 3, 103),
    # batched gather stress: S_kv = 65536, uniform indices, 5% masked slots
    "gather_b4_skv64k": Workload("gather_b4_skv64k", 4, 2048, 65536, 64, 512, 2048, "uniform_masked", 4, 104),
}


def _causal_distinct(B: int, S: int, S_kv: int, topk: int, g: torch.Generator) -> torch.Tensor:
    if S_kv < S:
        raise ValueError("causal_distinct needs S_kv >= S")
    idx = torch.full((B, S, topk), -1, dtype=torch.int32)
    for b in range(B):
        for s in range(S):
            n = min(s + 1, topk)
            idx[b, s, :n] = torch.randperm(s + 1, generator=g)[:n].to(torch.int32)
    return idx


def _recent_plus_random(B: int, S: int, S_kv: int, topk: int, g: torch.Generator) -> torch.Tensor:
    if S_kv < S or topk % 2:
        raise ValueError("recent_plus_random needs S_kv >= S and an even topk")
    half = topk // 2
    idx = torch.full((B, S, topk), -1, dtype=torch.int32)
    for b in range(B):
        for s in range(S):
            if s + 1 <= topk:
                idx[b, s, : s + 1] = torch.arange(s + 1, dtype=torch.int32)
                continue
            recent = torch.arange(s - half + 1, s + 1)
            older = torch.randperm(s - half + 1, generator=g)[:half]
            idx[b, s] = torch.sort(torch.cat([older, recent])).values.to(torch.int32)
    return idx


def _uniform_masked(B: int, S: int, S_kv: int, topk: int, g: torch.Generator) -> torch.Tensor:
    if topk > S_kv:
        raise ValueError("uniform_masked needs topk <= S_kv")
    idx = torch.empty((B, S, topk), dtype=torch.int32)
    for b in range(B):
        for s in range(S):
            idx[b, s] = torch.randperm(S_kv, generator=g)[:topk].to(torch.int32)
    masked = torch.rand((B, S, topk), generator=g) < 0.05
    kind = torch.randint(0, 5, (B, S, topk), generator=g)
    r = torch.randint(1, 2 ** 20, (B, S, topk), generator=g)
    bad = torch.stack([torch.full_like(r, -1), torch.full_like(r, INT32_MIN), torch.full_like(r, S_kv),
                       S_kv + r, torch.full_like(r, INT32_MAX)], dim=-1)
    bad = torch.gather(bad, -1, kind.unsqueeze(-1)).squeeze(-1).to(torch.int32)
    return torch.where(masked, bad, idx)


_RECIPES = {"causal_distinct": _causal_distinct, "recent_plus_random": _recent_plus_random,
            "uniform_masked": _uniform_masked}


def generate_inputs(B: int, S: int, S_kv: int, H: int, D: int, topk: int, index_recipe: str, seed: int,
                    do_seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """CPU tensors q, kv (bf16), attn_sink (fp32), topk_idxs (int32) and, if do_seed is given, do."""
    g = torch.Generator().manual_seed(seed)
    out = {
        "q": torch.randn((B, S, H, D), generator=g, dtype=torch.float32).to(torch.bfloat16),
        "kv": torch.randn((B, S_kv, D), generator=g, dtype=torch.float32).to(torch.bfloat16),
        "attn_sink": torch.randn((H,), generator=g, dtype=torch.float32),
        "topk_idxs": _RECIPES[index_recipe](B, S, S_kv, topk, g),
    }
    if do_seed is not None:
        gd = torch.Generator().manual_seed(do_seed)
        out["do"] = torch.randn((B, S, H, D), generator=gd, dtype=torch.float32).to(torch.bfloat16)
    return out


def workload_inputs(w: Workload, with_do: bool = True) -> Dict[str, torch.Tensor]:
    return generate_inputs(w.B, w.S, w.S_kv, w.H, w.D, w.topk, w.index_recipe, w.seed,
                           w.do_seed if with_do else None)


def valid_pairs(topk_idxs: torch.Tensor, S_kv: int) -> int:
    """Number of (token, slot) pairs whose index lies in [0, S_kv)."""
    return int(((topk_idxs >= 0) & (topk_idxs < S_kv)).sum().item())
