"""Host-side checks of libsparse_mqa that need no GPU: the library loads, exports every entry
point include/sparse_mqa.h declares, and rejects invalid arguments with the documented status
before any HIP call (every call below is invalid in at least one checked way)."""
import ctypes
import math
import re
from pathlib import Path

import pytest
import torch

import top_sparse_mqa_amd as smqa

HEADER = Path(__file__).resolve().parents[1] / "include" / "sparse_mqa.h"
OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WORKSPACE, HIP, ARG = range(9)

# fake, never dereferenced device addresses (validation fails before any use)
A = 0x10000000
Bp = 0x20000000
C = 0x30000000
Dp = 0x40000000
E = 0x50000000
F_ = 0x60000000
G = 0x70000000
NAN = float("nan")


# entry points that take only sizes (no device pointers, nothing enqueued)
QUERIES = {"sparse_mqa_bwd_workspace_bytes", "sparse_mqa_bwd_workspace_min_bytes", "sparse_mqa_status_string"}


class ValidationOnly:
    """The library as these tests may use it: every call that takes device pointers must be
    rejected by validation. A status of OK or SMQA_ERR_HIP would mean kernels were (or were tried
    to be) enqueued on the fake addresses above, which on a GPU host could fault the device."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        fn = getattr(self._lib, name)
        if name in QUERIES or not name.startswith("sparse_mqa_"):
            return fn

        def checked(*args):
            st = fn(*args)
            assert st not in (OK, HIP), f"{name} passed validation in a host test (status {st})"
            return st
        return checked


@pytest.fixture(scope="module")
def lib():
    if not smqa.LIB_PATH.exists():
        pytest.fail("libsparse_mqa.so is not built (python -m top_sparse_mqa_amd.build)")
    return ValidationOnly(smqa.load_library())


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(sparse_mqa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(smqa.EXPORTED) == names


def test_status_strings(lib):
    for st in range(9):
        assert lib.sparse_mqa_status_string(st)
    assert lib.sparse_mqa_status_string(99) == b"unknown status"


def fwd(lib, q=A, kv=Bp, sink=C, idx=Dp, o=E, lse=F_, B=1, S=8, S_kv=16, H=64, D=512, topk=4, scale=NAN, rr=0):
    return lib.sparse_mqa_fwd(q, kv, sink, idx, o, lse, B, S, S_kv, H, D, topk, scale, rr, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, rr=2) == ARG
    assert fwd(lib, rr=-1) == ARG
    assert fwd(lib, lse=None) == NULL
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, topk=-1) == SHAPE
    assert fwd(lib, S_kv=2 ** 31) == SHAPE
    assert fwd(lib, H=48) == UNSUP
    assert fwd(lib, H=96) == UNSUP
    assert fwd(lib, H=1088) == UNSUP
    assert fwd(lib, H=256, o=A) == ALIAS  # a supported head count: validation reaches the alias check
    assert fwd(lib, H=1024, S=2 ** 19) == SHAPE  # 2^19 tokens x 16 head blocks = 2^23 workgroups
    assert fwd(lib, H=1024, S=2 ** 19 - 1, o=A) == ALIAS  # one token fewer: below the limit
    assert fwd(lib, H=64, S=2 ** 23) == SHAPE  # 2^23 workgroups of 512 threads = 2^32 threads
    assert fwd(lib, D=96) == UNSUP
    # one batch's kv rows are gathered through a 32-bit byte range: 4 GiB and above are refused
    # just below the limit: validation reaches the alias check (kv's 4 GiB then covers o)
    assert fwd(lib, S_kv=(1 << 22) - 1) == ALIAS
    assert fwd(lib, S_kv=1 << 22) == UNSUP
    assert fwd(lib, S_kv=1 << 25, D=64, H=16) == UNSUP
    assert fwd(lib, D=1024) == UNSUP
    assert fwd(lib, H=64, D=128, o=A) == ALIAS  # D = 128 and 256 are supported
    assert fwd(lib, H=64, D=64) == UNSUP
    assert fwd(lib, q=A + 8) == ALIGN
    assert fwd(lib, idx=Dp + 2) == ALIGN
    assert fwd(lib, scale=math.inf) == ARG
    # o overlaps q; lse overlaps kv; o overlaps lse
    assert fwd(lib, o=A + 1024) == ALIAS
    assert fwd(lib, lse=Bp + 64) == ALIAS
    assert fwd(lib, lse=E + 4096) == ALIAS


def r256(n):
    return (n + 255) // 256 * 256


def dkv_layout_bytes(B, S_kv, H, D, K, chunk, acc, ds=None, S=None):
    """The dKV workspace layout restated: kv row norms, the selection bitmap (one bit per kv row and
    chunk token of the row's batch, in 32-bit words: ceil(min(chunk, S) / 32) per row) with a pair
    count and a cursor per word (cleared together as whole 16-byte pieces), the scanned offsets (+ total),
    the scan's tile sums, the fp32 accumulator when chunked with bf16 output, the slots' positions,
    the staging rows (one per slot and 64-head block plus one spare per token and head block; a
    row is D int16 values and one int8 exponent per segment of min(128, D / (heads per workgroup /
    16)) values), and, for the full backward at D = 512 with H a multiple of 64 (ds=None picks it by
    shape), the stored dS: [chunk][H / 64][ceil(K / 32)][64][32] bf16."""
    if ds is None:
        ds = D == 512 and H % 64 == 0
    n_rows = B * S_kv
    words = n_rows * ((min(chunk, S if S is not None else chunk) + 31) // 32)
    hb = max(1, H // 64)
    seg = min(128, D // (min(H, 64) // 16))
    rows = chunk * (K + 1) * hb
    return (r256(n_rows * 4) + r256((3 * words + 4) * 4) + r256((words + 1) * 4) + r256(((words + 4095) // 4096) * 4)
            + (r256(n_rows * D * 4) if acc else 0) + r256(chunk * K * 4) + r256(rows * D * 2)
            + r256(rows * (D // seg)) + (r256(chunk * (H // 64) * ((K + 31) // 32) * 64 * 32 * 2) if ds else 0))


def test_workspace_bytes(lib):
    B, S, S_kv, H, D, K = 1, 4096, 4096, 64, 512, 2048
    full = lib.sparse_mqa_bwd_workspace_bytes(B, S, S_kv, H, D, K)
    assert full == r256(B * S * H * 4) + dkv_layout_bytes(B, S_kv, H, D, K, B * S, False)
    # at the headline shape the bitmap and offsets are 2 MiB each; the staging rows dominate
    assert dkv_layout_bytes(B, S_kv, H, D, K, B * S, False) > 6.4e9
    # batched: a kv row's bitmap words cover its own batch's tokens (S of them), not the whole pass
    bb, sb, skvb = 4, 2048, 65536
    assert lib.sparse_mqa_bwd_workspace_bytes(bb, sb, skvb, H, D, K) == r256(bb * sb * H * 4) + dkv_layout_bytes(
        bb, skvb, H, D, K, bb * sb, False, S=sb)
    low = lib.sparse_mqa_bwd_workspace_min_bytes(B, S, S_kv, H, D, K)
    assert low == r256(B * S * H * 4) + dkv_layout_bytes(B, S_kv, H, D, K, 1, True)
    # few tokens over many rows: a single pass (no fp32 running sum) is the smaller layout
    b, s_, skv, h, d, k = 1, 8, 1 << 20, 64, 512, 4
    assert lib.sparse_mqa_bwd_workspace_min_bytes(b, s_, skv, h, d, k) == r256(b * s_ * h * 4) + min(
        dkv_layout_bytes(b, skv, h, d, k, 1, True), dkv_layout_bytes(b, skv, h, d, k, b * s_, False))
    assert dkv_layout_bytes(b, skv, h, d, k, b * s_, False) < dkv_layout_bytes(b, skv, h, d, k, 1, True)
    # H = 128 runs two 64-head workgroups per token: two staging rows per slot (and two spare rows)
    for (b, s_, skv, h, d, k) in ((1, 8, 16, 128, 512, 4), (2, 40, 33, 16, 64, 7), (1, 100, 70, 192, 256, 9)):
        assert lib.sparse_mqa_bwd_workspace_bytes(b, s_, skv, h, d, k) == (
            r256(b * s_ * h * 4) + dkv_layout_bytes(b, skv, h, d, k, b * s_, False, S=s_))
    assert lib.sparse_mqa_bwd_workspace_bytes(0, 1, 1, 16, 64, 1) == 0
    assert lib.sparse_mqa_bwd_workspace_min_bytes(1, 1, 1, 48, 512, 1) == 0


def bwd(lib, dkv_fp32=0, ws=G, wsb=1 << 30, dq=0x71000000, dkv=0x72000000, o=E, B=1, S=8, S_kv=16, H=64, D=512,
        topk=4, scale=NAN):
    return lib.sparse_mqa_bwd(A, Bp, C, o, 0x11000000, Dp, F_, dq, dkv, dkv_fp32, ws, wsb, B, S, S_kv, H, D, topk,
                              scale, None)


def test_bwd_validation(lib):
    assert bwd(lib, dq=None) == NULL
    assert bwd(lib, S=0) == SHAPE
    assert bwd(lib, H=8) == UNSUP
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, wsb=100) == WORKSPACE
    low = lib.sparse_mqa_bwd_workspace_min_bytes(1, 8, 16, 64, 512, 4)
    # The minimum passes the workspace check; one token's staging (positions + 5 rows of 512 int16
    # values and 4 exponents) less does not. The alias check runs after the workspace check, so
    # an output overlap stops both calls before anything is enqueued (no call here reaches a launch,
    # with or without a GPU).
    overlapping_dkv = 0x71000000 + 64
    assert bwd(lib, wsb=low, ws=0x7A000000, dkv=overlapping_dkv) == ALIAS
    assert bwd(lib, wsb=low - (4 * 4 + 5 * (1024 + 4)), ws=0x7A000000, dkv=overlapping_dkv) == WORKSPACE
    assert bwd(lib, ws=G + 4) == ALIGN
    assert bwd(lib, dq=A) == ALIAS
    assert bwd(lib, dkv=0x71000000 + 64) == ALIAS
    assert bwd(lib, ws=0x72000000) == ALIAS
    assert bwd(lib, scale=-math.inf) == ARG


def bwd_noalloc(lib, dkv_fp32=0, dq=0x71000000, dkv=0x72000000, o=E, B=1, S=8, S_kv=16, H=64, D=512, topk=4,
                scale=NAN):
    return lib.sparse_mqa_bwd_noalloc(A, Bp, C, o, 0x11000000, Dp, F_, dq, dkv, dkv_fp32, B, S, S_kv, H, D, topk,
                                      scale, None)


def test_bwd_noalloc_validation(lib):
    """Every argument check of the allocation-free backward runs before its scratch lookup, with
    the statuses of sparse_mqa_bwd; sizes whose smallest workspace exceeds the static scratch are
    refused with SMQA_ERR_WORKSPACE."""
    assert bwd_noalloc(lib, dq=None) == NULL
    assert bwd_noalloc(lib, S=0) == SHAPE
    assert bwd_noalloc(lib, H=8) == UNSUP
    assert bwd_noalloc(lib, dq=0x71000000 + 8) == ALIGN
    assert bwd_noalloc(lib, scale=math.inf) == ARG
    assert bwd_noalloc(lib, dq=A) == ALIAS
    assert bwd_noalloc(lib, dkv=0x71000000 + 64) == ALIAS
    # 2^20 kv rows, 4096 tokens, bf16 output: one pass needs 8 GiB of staging rows and token chunks
    # the fp32 running sum (2 GiB), both beyond the scratch
    scratch = 128 << 20
    assert lib.sparse_mqa_bwd_workspace_min_bytes(1, 4096, 1 << 20, 64, 512, 2048) > scratch
    assert bwd_noalloc(lib, S=4096, S_kv=1 << 20, topk=2048) == WORKSPACE
    # with 8 tokens one pass (no running sum) takes ~24 MiB: that is the minimum, and it fits
    assert lib.sparse_mqa_bwd_workspace_min_bytes(1, 8, 1 << 20, 64, 512, 4) <= scratch
    assert bwd_noalloc(lib, S_kv=1 << 20, dq=A) == ALIAS
    # the headline shape fits in token chunks (its one-pass workspace does not)
    assert lib.sparse_mqa_bwd_workspace_min_bytes(1, 4096, 4096, 64, 512, 2048) <= scratch
    assert lib.sparse_mqa_bwd_workspace_bytes(1, 4096, 4096, 64, 512, 2048) > scratch
    assert bwd_noalloc(lib, S=4096, S_kv=4096, topk=2048, dq=A) == ALIAS
    header = HEADER.read_text()
    assert "#define SMQA_BWD_SCRATCH_BYTES ((size_t)128 << 20)" in header


def test_stage_validation(lib):
    assert lib.sparse_mqa_bwd_preprocess(None, A, Bp, 1, 8, 64, 512, None) == NULL
    assert lib.sparse_mqa_bwd_preprocess(A, Bp, C, 1, 8, 64, 100, None) == UNSUP
    assert lib.sparse_mqa_bwd_preprocess(A, Bp, A + 64, 1, 8, 64, 512, None) == ALIAS
    assert lib.sparse_mqa_bwd_main(A, Bp, C, Dp, E, F_, G, None, 1, 8, 16, 64, 512, 4, NAN, None) == NULL
    assert lib.sparse_mqa_bwd_main(A, Bp, C, Dp, E, F_, G, A, 1, 8, 16, 64, 512, 4, NAN, None) == ALIAS
    assert lib.sparse_mqa_bwd_dq(A, Bp, C, Dp, E, F_, None, 1, 8, 16, 64, 512, 4, NAN, None) == NULL
    assert lib.sparse_mqa_bwd_dq(A, Bp, C, Dp, E, F_, G + 2, 1, 8, 16, 64, 512, 4, NAN, None) == ALIGN
    assert lib.sparse_mqa_bwd_dkv(A, Bp, C, Dp, E, F_, None, 0, G, 1 << 30, 1, 8, 16, 64, 512, 4, NAN, None) == NULL
    assert lib.sparse_mqa_bwd_dkv(A, Bp, C, Dp, E, F_, G, 0, G, 1 << 30, 1, 8, 16, 64, 512, 0, NAN, None) == SHAPE
    assert lib.sparse_mqa_bwd_dkv(A, Bp, C, Dp, E, F_, G, 0, None, 1 << 30, 1, 8, 16, 64, 512, 4, NAN, None) == WORKSPACE
    assert lib.sparse_mqa_bwd_dkv(A, Bp, C, Dp, E, F_, G, 0, 0x7C000000, 64, 1, 8, 16, 64, 512, 4, NAN, None) == WORKSPACE
    assert lib.sparse_mqa_bwd_dkv(A, Bp, C, Dp, E, F_, G, 0, A, 1 << 30, 1, 8, 16, 64, 512, 4, NAN, None) == ALIAS
    assert lib.sparse_mqa_bwd_postprocess(None, A, 1, 16, 512, None) == NULL
    assert lib.sparse_mqa_bwd_postprocess(A, Bp, 1, 16, 12, None) == SHAPE
    assert lib.sparse_mqa_bwd_postprocess(A, A + 16, 1, 16, 512, None) == ALIAS


def test_dsink_validation(lib):
    assert lib.sparse_mqa_bwd_dsink(None, Bp, C, Dp, 1, 8, 64, None) == NULL
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, None, 1, 8, 64, None) == NULL
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, Dp, 0, 8, 64, None) == SHAPE
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, Dp, 1, 8, -1, None) == SHAPE
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, Dp + 2, 1, 8, 64, None) == ALIGN
    # d_sink over the last head of lse / delta, or over attn_sink itself
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, A + 4 * (8 * 64 - 1), 1, 8, 64, None) == ALIAS
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, Bp, 1, 8, 64, None) == ALIAS
    assert lib.sparse_mqa_bwd_dsink(A, Bp, C, C + 4, 1, 8, 64, None) == ALIAS


def test_dkv_step_validation(lib):
    """The separately enqueued dKV steps need a one-pass workspace and valid arguments."""
    B, S, S_kv, H, D, K = 1, 8, 16, 64, 512, 4
    full = lib.sparse_mqa_bwd_workspace_bytes(B, S, S_kv, H, D, K)
    dims = (B, S, S_kv, H, D, K)
    assert lib.sparse_mqa_bwd_dkv_prepare(None, G, full, *dims, None) == NULL
    assert lib.sparse_mqa_bwd_dkv_prepare(Dp, None, full, *dims, None) == WORKSPACE
    assert lib.sparse_mqa_bwd_dkv_prepare(Dp, G + 8, full, *dims, None) == ALIGN
    # a workspace that only allows token chunks is refused (the steps are one pass)
    low = lib.sparse_mqa_bwd_workspace_min_bytes(*dims)
    assert lib.sparse_mqa_bwd_dkv_prepare(Dp, G, low, *dims, None) == WORKSPACE
    assert lib.sparse_mqa_bwd_dkv_prepare(Dp, Dp, full, *dims, None) == ALIAS
    assert lib.sparse_mqa_bwd_dkv_prepare(Dp, G, full, 1, 8, 16, 48, 512, 4, None) == UNSUP
    assert lib.sparse_mqa_bwd_dkv_partials(A, Bp, C, Dp, E, None, G, full, *dims, NAN, None) == NULL
    assert lib.sparse_mqa_bwd_dkv_partials(A, Bp, C, Dp, E, F_ + 2, G, full, *dims, NAN, None) == ALIGN
    assert lib.sparse_mqa_bwd_dkv_partials(A, Bp, C, Dp, E, F_, G, low, *dims, NAN, None) == WORKSPACE
    assert lib.sparse_mqa_bwd_dkv_partials(A, Bp, C, Dp, E, F_, A, full, *dims, NAN, None) == ALIAS
    assert lib.sparse_mqa_bwd_dkv_partials(A, Bp, C, Dp, E, F_, G, full, *dims, -math.inf, None) == ARG
    assert lib.sparse_mqa_bwd_dkv_reduce(None, 0, G, full, *dims, None) == NULL
    assert lib.sparse_mqa_bwd_dkv_reduce(A + 8, 0, G, full, *dims, None) == ALIGN
    assert lib.sparse_mqa_bwd_dkv_reduce(A, 0, G, 100, *dims, None) == WORKSPACE
    assert lib.sparse_mqa_bwd_dkv_reduce(G + 256, 1, G, full, *dims, None) == ALIAS


def test_autograd_refuses_cpu_tensors():
    """The differentiable wrapper has no CPU path: CPU tensors are an error, not a fallback."""
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, requires_grad=True)
    kv = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        smqa.sparse_mqa(q, kv, torch.zeros(16), torch.zeros(1, 2, 4, dtype=torch.int32))
