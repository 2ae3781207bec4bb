"""Python binding of libsparse_mqa (ctypes). Argument marshalling only: every step of the
computation runs in the HIP kernels behind the C ABI (include/sparse_mqa.h). PyTorch supplies
device memory and the current stream.

The interface functions mirror the NeMo AutoModel DeepSeek-V4 pages
"...kernels.tilelang_sparse_mla_fwd" (sparse_mqa_fwd_interface) and
"...kernels.tilelang_sparse_mla_bwd" (sparse_mqa_bwd_interface).
"""
from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path
from typing import Optional, Tuple

import torch

LIB_PATH = Path(__file__).resolve().parent / "libsparse_mqa.so"

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64

_SIGS = {
    "sparse_mqa_fwd": [_c_void_p] * 6 + [_i64] * 6 + [ctypes.c_float, ctypes.c_int, _c_void_p],
    "sparse_mqa_bwd_workspace_bytes": [_i64] * 6,
    "sparse_mqa_bwd_workspace_min_bytes": [_i64] * 6,
    "sparse_mqa_bwd": [_c_void_p] * 9 + [ctypes.c_int, _c_void_p, ctypes.c_size_t] + [_i64] * 6
    + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_noalloc": [_c_void_p] * 9 + [ctypes.c_int] + [_i64] * 6 + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_preprocess": [_c_void_p] * 3 + [_i64] * 4 + [_c_void_p],
    "sparse_mqa_bwd_dsink": [_c_void_p] * 4 + [_i64] * 3 + [_c_void_p],
    "sparse_mqa_bwd_main": [_c_void_p] * 8 + [_i64] * 6 + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_dq": [_c_void_p] * 7 + [_i64] * 6 + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_dkv": [_c_void_p] * 7 + [ctypes.c_int, _c_void_p, ctypes.c_size_t] + [_i64] * 6
    + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_dkv_prepare": [_c_void_p] * 2 + [ctypes.c_size_t] + [_i64] * 6 + [_c_void_p],
    "sparse_mqa_bwd_dkv_partials": [_c_void_p] * 7 + [ctypes.c_size_t] + [_i64] * 6 + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_dkv_dq": [_c_void_p] * 4 + [ctypes.c_size_t] + [_i64] * 6 + [ctypes.c_float, _c_void_p],
    "sparse_mqa_bwd_dkv_reduce": [_c_void_p, ctypes.c_int, _c_void_p, ctypes.c_size_t] + [_i64] * 6 + [_c_void_p],
    "sparse_mqa_bwd_postprocess": [_c_void_p] * 2 + [_i64] * 3 + [_c_void_p],
    "sparse_mqa_status_string": [ctypes.c_int],
}
EXPORTED = tuple(_SIGS)

_lib: Optional[ctypes.CDLL] = None


class SparseMQAError(RuntimeError):
    """A non-zero status returned by libsparse_mqa."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load the in-tree libsparse_mqa.so. There is no fallback: a missing library is an error."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m top_sparse_mqa_amd.build` "
                "(the HIP library is required; there is no CPU fallback)")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.sparse_mqa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.sparse_mqa_bwd_workspace_min_bytes.restype = ctypes.c_size_t
        lib.sparse_mqa_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = load_library().sparse_mqa_status_string(status).decode()
        raise SparseMQAError(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# Largest backward workspace the binding allocates on its own; above it the library processes the
# tokens in chunks (set SMQA_BWD_WORKSPACE_CAP_GIB to change).
WORKSPACE_CAP = int(float(os.environ.get("SMQA_BWD_WORKSPACE_CAP_GIB", "32")) * 2 ** 30)


def bwd_workspace_bytes(B: int, S: int, S_kv: int, H: int, D: int, topk: int, cap: Optional[int] = None) -> int:
    """Workspace the binding uses: one pass over all tokens if that fits under the cap, else the
    cap (at least the library's minimum), which the library turns into token chunks."""
    lib = load_library()
    full = lib.sparse_mqa_bwd_workspace_bytes(B, S, S_kv, H, D, topk)
    low = lib.sparse_mqa_bwd_workspace_min_bytes(B, S, S_kv, H, D, topk)
    if full == 0 or low == 0:
        raise ValueError("invalid sizes for the backward workspace")
    cap = WORKSPACE_CAP if cap is None else cap
    return full if full <= cap else max(low, cap)


def _scale_arg(sm_scale: Optional[float]) -> float:
    return float("nan") if sm_scale is None else float(sm_scale)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_shapes(q: torch.Tensor, kv: Optional[torch.Tensor] = None, topk_idxs: Optional[torch.Tensor] = None, *,
                 o: Optional[torch.Tensor] = None, do: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, delta: Optional[torch.Tensor] = None,
                 attn_sink: Optional[torch.Tensor] = None, dkv_accum: Optional[torch.Tensor] = None) -> None:
    """Raises ValueError unless the given tensors have the pages' shapes for one (B, S, S_kv, H, D,
    topk): q, o, do [B,S,H,D]; kv, dkv_accum [B,S_kv,D]; topk_idxs [B,S,topk]; lse, delta [B,S,H];
    attn_sink [H]; all on q's device. The library trusts the sizes it is given, so every entry point
    of this binding runs this check before it calls the library."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B,S,H,D], got shape {tuple(q.shape)}")
    B, S, H, D = q.shape
    given = {"kv": kv, "topk_idxs": topk_idxs, "o": o, "do": do, "lse": lse, "delta": delta,
             "attn_sink": attn_sink, "dkv_accum": dkv_accum}
    for name, t in given.items():
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    S_kv = None
    if kv is not None:
        if kv.dim() != 3 or kv.shape[0] != B or kv.shape[2] != D:
            raise ValueError(f"kv shape {tuple(kv.shape)} does not match q {tuple(q.shape)} ([B,S_kv,D])")
        S_kv = kv.shape[1]
    if topk_idxs is not None and (topk_idxs.dim() != 3 or topk_idxs.shape[0] != B or topk_idxs.shape[1] != S):
        raise ValueError(f"topk_idxs must be [B,S,topk] = [{B},{S},topk], got {tuple(topk_idxs.shape)}")
    for name in ("o", "do"):
        t = given[name]
        if t is not None and tuple(t.shape) != (B, S, H, D):
            raise ValueError(f"{name} must have the shape of q {tuple(q.shape)}, got {tuple(t.shape)}")
    for name in ("lse", "delta"):
        t = given[name]
        if t is not None and tuple(t.shape) != (B, S, H):
            raise ValueError(f"{name} must be [B,S,H] = [{B},{S},{H}], got {tuple(t.shape)}")
    if attn_sink is not None and tuple(attn_sink.shape) != (H,):
        raise ValueError(f"attn_sink must be [H] = [{H}], got {tuple(attn_sink.shape)}")
    if dkv_accum is not None:
        want = (B, S_kv if S_kv is not None else dkv_accum.shape[1], D)
        if tuple(dkv_accum.shape) != want:
            raise ValueError(f"dkv_accum must be [B,S_kv,D] = {list(want)}, got {tuple(dkv_accum.shape)}")


def _indices_int32(topk_idxs: torch.Tensor, s_kv: int) -> torch.Tensor:
    """int32 indices for the ABI. int64 input is narrowed after every value outside
    [0, S_kv) is replaced by -1, so narrowing cannot turn a masked index into a valid one."""
    if topk_idxs.device.type != "cuda":
        raise ValueError("topk_idxs must be a GPU tensor")
    if topk_idxs.dtype == torch.int32:
        if not topk_idxs.is_contiguous():
            raise ValueError("topk_idxs must be contiguous")
        return topk_idxs
    if topk_idxs.dtype != torch.int64:
        raise TypeError(f"topk_idxs must be int32 or int64, got {topk_idxs.dtype}")
    bad = (topk_idxs < 0) | (topk_idxs >= s_kv)
    return torch.where(bad, torch.full_like(topk_idxs, -1), topk_idxs).to(torch.int32).contiguous()


def sparse_mqa_fwd_interface(q: torch.Tensor, kv: torch.Tensor, attn_sink: torch.Tensor,
                             topk_idxs: torch.Tensor, sm_scale: Optional[float] = None,
                             block_I: int = 64, num_stages: int = 2, threads: int = 256,
                             reference_rounding: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward: returns (O [B,S,H,D] bf16, LSE [B,S,H] fp32 in log2 units).

    reference_rounding rounds each scaled logit dot * sm_scale to fp32 in natural units and
    subtracts the running max there before the exponential (the default scales straight into
    base 2); LSE is in log2 units either way, so the backward is the same.
    block_I, num_stages and threads are tuning knobs of the pages' kernel generator; they are
    accepted and ignored (the gfx950 kernels pick their own tiling)."""
    del block_I, num_stages, threads
    _need(q, "q", torch.bfloat16, 4)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(attn_sink, "attn_sink", torch.float32, 1)
    check_shapes(q, kv, topk_idxs, attn_sink=attn_sink)
    B, S, H, D = q.shape
    S_kv = kv.shape[1]
    idx = _indices_int32(topk_idxs, S_kv)
    topk = idx.shape[2]
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, S, H), dtype=torch.float32, device=q.device)
    lib = load_library()
    _check("sparse_mqa_fwd", lib.sparse_mqa_fwd(
        _ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(idx), _ptr(o), _ptr(lse),
        B, S, S_kv, H, D, topk, _scale_arg(sm_scale), 1 if reference_rounding else 0, _stream()))
    return o, lse


def sparse_mqa_bwd_interface(q: torch.Tensor, kv: torch.Tensor, attn_sink: torch.Tensor, o: torch.Tensor,
                             do: torch.Tensor, topk_idxs: torch.Tensor, lse: torch.Tensor,
                             sm_scale: Optional[float] = None,
                             return_dkv_accum_dtype: bool = False,
                             return_d_sink: bool = False) -> Tuple[torch.Tensor, ...]:
    """Backward: returns (dQ [B,S,H,D] bf16, dKV [B,S_kv,D] bf16, or fp32 when
    return_dkv_accum_dtype), and with return_d_sink also d_sink [H] fp32, the gradient of
    attn_sink."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(attn_sink, "attn_sink", torch.float32, 1)
    _need(o, "o", torch.bfloat16, 4)
    _need(do, "do", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    check_shapes(q, kv, topk_idxs, o=o, do=do, lse=lse, attn_sink=attn_sink)
    B, S, H, D = q.shape
    S_kv = kv.shape[1]
    idx = _indices_int32(topk_idxs, S_kv)
    topk = idx.shape[2]
    lib = load_library()
    dq = torch.empty_like(q)
    dkv = torch.empty((B, S_kv, D), dtype=torch.float32 if return_dkv_accum_dtype else torch.bfloat16,
                      device=q.device)
    ws_bytes = bwd_workspace_bytes(B, S, S_kv, H, D, topk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check("sparse_mqa_bwd", lib.sparse_mqa_bwd(
        _ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(o), _ptr(do), _ptr(idx), _ptr(lse), _ptr(dq), _ptr(dkv),
        1 if return_dkv_accum_dtype else 0, _ptr(ws), ws_bytes, B, S, S_kv, H, D, topk,
        _scale_arg(sm_scale), _stream()))
    if return_d_sink:
        return dq, dkv, bwd_dsink(lse, bwd_preprocess(o, do), attn_sink)
    return dq, dkv


def bwd_dsink(lse: torch.Tensor, delta: torch.Tensor, attn_sink: torch.Tensor) -> torch.Tensor:
    """d_sink[h] = -sum_{b,s} exp(attn_sink[h] - LSE[b,s,h]) * Delta[b,s,h] (fp32 [H]); delta is
    bwd_preprocess(o, do)."""
    _need(lse, "lse", torch.float32, 3)
    _need(delta, "delta", torch.float32, 3)
    _need(attn_sink, "attn_sink", torch.float32, 1)
    B, S, H = lse.shape
    if tuple(delta.shape) != (B, S, H) or tuple(attn_sink.shape) != (H,):
        raise ValueError("delta must be [B,S,H] like lse and attn_sink [H]")
    if delta.device != lse.device or attn_sink.device != lse.device:
        raise ValueError("lse, delta and attn_sink must be on one device")
    d_sink = torch.empty(H, dtype=torch.float32, device=lse.device)
    _check("sparse_mqa_bwd_dsink", load_library().sparse_mqa_bwd_dsink(
        _ptr(lse), _ptr(delta), _ptr(attn_sink), _ptr(d_sink), B, S, H, _stream()))
    return d_sink


def bwd_preprocess(o: torch.Tensor, do: torch.Tensor) -> torch.Tensor:
    """Delta[b,s,h] = sum_d O*dO (fp32)."""
    _need(o, "o", torch.bfloat16, 4)
    _need(do, "do", torch.bfloat16, 4)
    check_shapes(o, do=do)
    B, S, H, D = o.shape
    delta = torch.empty((B, S, H), dtype=torch.float32, device=o.device)
    _check("sparse_mqa_bwd_preprocess", load_library().sparse_mqa_bwd_preprocess(
        _ptr(o), _ptr(do), _ptr(delta), B, S, H, D, _stream()))
    return delta


def bwd_main(q: torch.Tensor, kv: torch.Tensor, do: torch.Tensor, topk_idxs: torch.Tensor, lse: torch.Tensor,
             delta: torch.Tensor, dkv_accum: torch.Tensor, sm_scale: Optional[float] = None) -> torch.Tensor:
    """Main backward stage: returns dQ and adds the dKV contributions into dkv_accum (fp32,
    which the caller zeroes beforehand)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(do, "do", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(delta, "delta", torch.float32, 3)
    _need(dkv_accum, "dkv_accum", torch.float32, 3)
    check_shapes(q, kv, topk_idxs, do=do, lse=lse, delta=delta, dkv_accum=dkv_accum)
    B, S, H, D = q.shape
    S_kv = kv.shape[1]
    idx = _indices_int32(topk_idxs, S_kv)
    dq = torch.empty_like(q)
    _check("sparse_mqa_bwd_main", load_library().sparse_mqa_bwd_main(
        _ptr(q), _ptr(kv), _ptr(do), _ptr(idx), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dkv_accum),
        B, S, S_kv, H, D, idx.shape[2], _scale_arg(sm_scale), _stream()))
    return dq


def _main_stage_args(q, kv, do, topk_idxs, lse, delta):
    _need(q, "q", torch.bfloat16, 4)
    _need(kv, "kv", torch.bfloat16, 3)
    _need(do, "do", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(delta, "delta", torch.float32, 3)
    check_shapes(q, kv, topk_idxs, do=do, lse=lse, delta=delta)
    return _indices_int32(topk_idxs, kv.shape[1])


def bwd_dq(q: torch.Tensor, kv: torch.Tensor, do: torch.Tensor, topk_idxs: torch.Tensor, lse: torch.Tensor,
           delta: torch.Tensor, sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dQ kernel of the main backward stage alone."""
    idx = _main_stage_args(q, kv, do, topk_idxs, lse, delta)
    B, S, H, D = q.shape
    if out is not None:
        _need(out, "out", torch.bfloat16, 4)
        check_shapes(q, o=out)
    dq = torch.empty_like(q) if out is None else out
    _check("sparse_mqa_bwd_dq", load_library().sparse_mqa_bwd_dq(
        _ptr(q), _ptr(kv), _ptr(do), _ptr(idx), _ptr(lse), _ptr(delta), _ptr(dq),
        B, S, kv.shape[1], H, D, idx.shape[2], _scale_arg(sm_scale), _stream()))
    return dq


def bwd_dkv(q: torch.Tensor, kv: torch.Tensor, do: torch.Tensor, topk_idxs: torch.Tensor, lse: torch.Tensor,
            delta: torch.Tensor, sm_scale: Optional[float] = None, dkv_fp32: bool = False,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dKV stage alone (segmented scatter-add and per-row reduction): returns dKV."""
    idx = _main_stage_args(q, kv, do, topk_idxs, lse, delta)
    B, S, H, D = q.shape
    S_kv, topk = kv.shape[1], idx.shape[2]
    dkv = torch.empty((B, S_kv, D), dtype=torch.float32 if dkv_fp32 else torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = torch.empty(bwd_workspace_bytes(B, S, S_kv, H, D, topk), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    _check("sparse_mqa_bwd_dkv", load_library().sparse_mqa_bwd_dkv(
        _ptr(q), _ptr(kv), _ptr(do), _ptr(idx), _ptr(lse), _ptr(delta), _ptr(dkv), 1 if dkv_fp32 else 0,
        _ptr(workspace), workspace.numel(), B, S, S_kv, H, D, topk, _scale_arg(sm_scale), _stream()))
    return dkv


class DkvSteps:
    """The steps of a single-pass staged backward (prepare, partials, dq, reduce) over one workspace,
    for callers that time or schedule them separately; prepare, partials and reduce together equal
    bwd_dkv, and dq (D = 512 with H a multiple of 64) equals bwd_dq."""

    def __init__(self, q: torch.Tensor, kv: torch.Tensor, do: torch.Tensor, topk_idxs: torch.Tensor,
                 lse: torch.Tensor, delta: torch.Tensor, sm_scale: Optional[float] = None, dkv_fp32: bool = False):
        self.idx = _main_stage_args(q, kv, do, topk_idxs, lse, delta)
        self.q, self.kv, self.do, self.lse, self.delta = q, kv, do, lse, delta
        self.B, self.S, self.H, self.D = q.shape
        self.S_kv, self.topk = kv.shape[1], self.idx.shape[2]
        lib = load_library()
        full = lib.sparse_mqa_bwd_workspace_bytes(self.B, self.S, self.S_kv, self.H, self.D, self.topk)
        if full == 0:
            raise ValueError("invalid sizes for the backward workspace")
        # sparse_mqa_bwd_workspace_bytes includes Delta's part, which these steps do not use
        self.workspace = torch.empty(full, dtype=torch.uint8, device=q.device)
        self.scale = _scale_arg(sm_scale)
        self.dkv_fp32 = dkv_fp32
        self.dkv = torch.empty((self.B, self.S_kv, self.D), dtype=torch.float32 if dkv_fp32 else torch.bfloat16,
                               device=q.device)

    def _dims(self):
        return (self.B, self.S, self.S_kv, self.H, self.D, self.topk)

    def prepare(self) -> None:
        _check("sparse_mqa_bwd_dkv_prepare", load_library().sparse_mqa_bwd_dkv_prepare(
            _ptr(self.idx), _ptr(self.workspace), self.workspace.numel(), *self._dims(), _stream()))

    def partials(self) -> None:
        _check("sparse_mqa_bwd_dkv_partials", load_library().sparse_mqa_bwd_dkv_partials(
            _ptr(self.q), _ptr(self.kv), _ptr(self.do), _ptr(self.idx), _ptr(self.lse), _ptr(self.delta),
            _ptr(self.workspace), self.workspace.numel(), *self._dims(), self.scale, _stream()))

    def dq(self) -> torch.Tensor:
        """dQ from the dS that partials stored (D = 512 with H a multiple of 64)."""
        out = torch.empty((self.B, self.S, self.H, self.D), dtype=torch.bfloat16, device=self.q.device)
        _check("sparse_mqa_bwd_dkv_dq", load_library().sparse_mqa_bwd_dkv_dq(
            _ptr(self.kv), _ptr(self.idx), _ptr(out), _ptr(self.workspace), self.workspace.numel(), *self._dims(),
            self.scale, _stream()))
        return out

    def reduce(self) -> torch.Tensor:
        _check("sparse_mqa_bwd_dkv_reduce", load_library().sparse_mqa_bwd_dkv_reduce(
            _ptr(self.dkv), 1 if self.dkv_fp32 else 0, _ptr(self.workspace), self.workspace.numel(), *self._dims(),
            _stream()))
        return self.dkv


def bwd_postprocess(dkv_accum: torch.Tensor) -> torch.Tensor:
    """bf16 (round to nearest even) copy of the fp32 dKV accumulator."""
    _need(dkv_accum, "dkv_accum", torch.float32, 3)
    B, S_kv, D = dkv_accum.shape
    out = torch.empty((B, S_kv, D), dtype=torch.bfloat16, device=dkv_accum.device)
    _check("sparse_mqa_bwd_postprocess", load_library().sparse_mqa_bwd_postprocess(
        _ptr(dkv_accum), _ptr(out), B, S_kv, D, _stream()))
    return out


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
