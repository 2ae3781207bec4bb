"""CPU oracle for top-k sparse MQA (ctypes wrapper around liboracle_sparse_mqa.so).

TEST INFRASTRUCTURE ONLY. This is the correctness reference the HIP kernels are checked against.
Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import it; the
product package (top_sparse_mqa_amd) never does, and the two share no code.

The arithmetic lives in sparse_mqa_oracle.cpp (plain loops; its header states the definitions
and the pages they follow). This wrapper only converts tensors: bf16 inputs are widened exactly
to the working precision ("f32", the pages' fp32 accumulation, or "f64").
"""
from __future__ import annotations

import ctypes
import math
import subprocess
from pathlib import Path
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

DIR = Path(__file__).resolve().parent
SRC = DIR / "sparse_mqa_oracle.cpp"
LIB = DIR / "liboracle_sparse_mqa.so"

_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I = ctypes.c_int64
_D = ctypes.c_double


def build() -> Path:
    """Compile the oracle with g++: OpenMP, AVX2 (every x86-64-v3 host has it), and no FMA
    contraction, so every multiply and add rounds separately, exactly as the loops are written."""
    tmp = LIB.with_suffix(".so.tmp")
    subprocess.run(["g++", "-O3", "-fopenmp", "-mavx2", "-mfma", "-ffp-contract=off", "-shared", "-fPIC", str(SRC), "-o", str(tmp)],
                   check=True)
    tmp.replace(LIB)
    return LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB.exists():
            build()
        lib = ctypes.CDLL(str(LIB))
        fwd_args = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _D, _P, _I, _P, _P]
        bwd_args = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _D, _P, _I, _P, _P]
        dkv_args = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _D, _P, _I, _P]
        for suf in ("f32", "f64"):
            getattr(lib, f"oracle_fwd_{suf}").argtypes = fwd_args
            getattr(lib, f"oracle_dq_{suf}").argtypes = bwd_args
            getattr(lib, f"oracle_dkv_{suf}").argtypes = dkv_args
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def _dtype(precision: str) -> torch.dtype:
    if precision not in ("f32", "f64"):
        raise ValueError("precision must be 'f32' or 'f64'")
    return torch.float32 if precision == "f32" else torch.float64


def _real(t: torch.Tensor, dt: torch.dtype) -> torch.Tensor:
    return t.detach().to("cpu").to(dt).contiguous()


def _ids(ids: Optional[Sequence[int]]) -> Tuple[Optional[np.ndarray], int]:
    if ids is None:
        return None, 0
    arr = np.ascontiguousarray(np.asarray(ids, dtype=np.int64))
    return arr, int(arr.size)


def _scale(sm_scale: Optional[float], D: int) -> float:
    return 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)


def fwd(q, kv, attn_sink, topk_idxs, sm_scale: Optional[float] = None, tokens: Optional[Sequence[int]] = None,
        precision: str = "f32") -> Tuple[torch.Tensor, torch.Tensor]:
    """O [n,H,D] and LSE [n,H] (log2) for the listed flat tokens b*S+s (all if None)."""
    dt = _dtype(precision)
    B, S, H, D = q.shape
    S_kv, topk = kv.shape[1], topk_idxs.shape[2]
    qr, kvr = _real(q, dt), _real(kv, dt)
    sink = attn_sink.detach().cpu().to(torch.float32).contiguous()
    idx = topk_idxs.detach().cpu().to(torch.int32).contiguous()
    tok, n = _ids(tokens)
    n = n if tok is not None else B * S
    o = torch.empty((n, H, D), dtype=dt)
    lse = torch.empty((n, H), dtype=dt)
    getattr(_load(), f"oracle_fwd_{precision}")(
        qr.data_ptr(), kvr.data_ptr(), sink.data_ptr(), idx.data_ptr(), B, S, S_kv, H, D, topk,
        _scale(sm_scale, D), None if tok is None else tok.ctypes.data, n if tok is not None else 0,
        o.data_ptr(), lse.data_ptr())
    return o, lse


def dq(q, kv, o, do, topk_idxs, lse, sm_scale: Optional[float] = None, tokens: Optional[Sequence[int]] = None,
       precision: str = "f32") -> Tuple[torch.Tensor, torch.Tensor]:
    """dQ [n,H,D] and Delta [n,H] for the listed flat tokens (all if None)."""
    dt = _dtype(precision)
    B, S, H, D = q.shape
    S_kv, topk = kv.shape[1], topk_idxs.shape[2]
    qr, kvr, orr, dor, lser = _real(q, dt), _real(kv, dt), _real(o, dt), _real(do, dt), _real(lse, dt)
    idx = topk_idxs.detach().cpu().to(torch.int32).contiguous()
    tok, n = _ids(tokens)
    n = n if tok is not None else B * S
    dqo = torch.empty((n, H, D), dtype=dt)
    delta = torch.empty((n, H), dtype=dt)
    getattr(_load(), f"oracle_dq_{precision}")(
        qr.data_ptr(), kvr.data_ptr(), orr.data_ptr(), dor.data_ptr(), idx.data_ptr(), lser.data_ptr(),
        B, S, S_kv, H, D, topk, _scale(sm_scale, D), None if tok is None else tok.ctypes.data,
        n if tok is not None else 0, dqo.data_ptr(), delta.data_ptr())
    return dqo, delta


def dkv(q, kv, o, do, topk_idxs, lse, sm_scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
        precision: str = "f32") -> torch.Tensor:
    """dKV [n,D] for the listed flat kv rows b*S_kv+j (all if None)."""
    dt = _dtype(precision)
    B, S, H, D = q.shape
    S_kv, topk = kv.shape[1], topk_idxs.shape[2]
    qr, kvr, orr, dor, lser = _real(q, dt), _real(kv, dt), _real(o, dt), _real(do, dt), _real(lse, dt)
    idx = topk_idxs.detach().cpu().to(torch.int32).contiguous()
    rw, n = _ids(rows)
    n = n if rw is not None else B * S_kv
    out = torch.empty((n, D), dtype=dt)
    getattr(_load(), f"oracle_dkv_{precision}")(
        qr.data_ptr(), kvr.data_ptr(), orr.data_ptr(), dor.data_ptr(), idx.data_ptr(), lser.data_ptr(),
        B, S, S_kv, H, D, topk, _scale(sm_scale, D), None if rw is None else rw.ctypes.data,
        n if rw is not None else 0, out.data_ptr())
    return out


def dsink(o, do, lse, attn_sink, precision: str = "f64") -> torch.Tensor:
    """Gradient of L = sum(O * dO) with respect to attn_sink, d_sink [H].

    The sink adds exp(sink_h) to the softmax denominator and carries no value vector (fwd page,
    attn_sink note), so O = sum_t p_t v_t with p_t = exp(z_t) / Z and dZ/dsink_h = exp(sink_h).
    Then dO . dO/dsink_h = -p_sink * sum_t p_t (dO . v_t) = -p_sink * Delta, with
    p_sink = exp(sink_h) / Z = 2^(sink_h log2 e - LSE) (LSE in log2 units) and Delta = <O, dO>
    from the O that is passed (as for dQ and dKV). Summed over all tokens:
        d_sink[h] = -sum_{b,s} 2^(sink_h log2 e - LSE[b,s,h]) * Delta[b,s,h].
    A sink of -inf has p_sink = 0 (its gradient is 0); plain torch ops in the working precision.
    """
    dt = _dtype(precision)
    orr, dor = _real(o, dt), _real(do, dt)
    B, S, H, D = orr.shape
    lser = _real(lse, dt).view(B, S, H)
    sink = attn_sink.detach().cpu().to(torch.float32).to(dt)
    delta = (orr * dor).sum(-1)
    log2e = 1.0 / math.log(2.0)
    finite = torch.isfinite(sink)
    expo = torch.where(finite.view(1, 1, H), sink.view(1, 1, H) * log2e - lser, torch.full_like(lser, -math.inf))
    p_sink = torch.exp2(expo)
    return -(p_sink * delta).sum(dim=(0, 1))
