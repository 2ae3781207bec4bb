"""Host-side checks of the Python binding: the shape validator that every entry point runs before
it calls the library rejects each inconsistent argument with ValueError. The library trusts the
sizes it is given, so a mismatch that slipped through would become out-of-bounds device reads."""
import pytest
import torch

from top_sparse_mqa_amd.binding import check_shapes

B, S, S_kv, H, D, K = 2, 5, 7, 64, 128, 3


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def good():
    return dict(q=t(B, S, H, D), kv=t(B, S_kv, D), topk_idxs=t(B, S, K, dtype=torch.int32), o=t(B, S, H, D),
                do=t(B, S, H, D), lse=t(B, S, H, dtype=torch.float32), delta=t(B, S, H, dtype=torch.float32),
                attn_sink=t(H, dtype=torch.float32), dkv_accum=t(B, S_kv, D, dtype=torch.float32))


def call(args):
    q, kv, idx = args.pop("q"), args.pop("kv"), args.pop("topk_idxs")
    check_shapes(q, kv, idx, **args)


def test_consistent_shapes_pass():
    call(good())
    check_shapes(t(B, S, H, D))  # q alone
    check_shapes(t(B, S, H, D), do=t(B, S, H, D))  # the preprocess pair


BAD = {
    "q_3d": ("q", (B, S, H * D)),
    "kv_batch": ("kv", (B + 1, S_kv, D)),
    "kv_dim": ("kv", (B, S_kv, D // 2)),
    "kv_2d": ("kv", (S_kv, D)),
    "idx_batch": ("topk_idxs", (B + 1, S, K)),
    "idx_tokens": ("topk_idxs", (B, S + 1, K)),
    "idx_2d": ("topk_idxs", (B * S, K)),
    "o_heads": ("o", (B, S, H // 2, D)),
    "do_tokens": ("do", (B, S - 1, H, D)),
    "lse_heads": ("lse", (B, S, H + 1)),
    "lse_4d": ("lse", (B, S, H, 1)),
    "delta_tokens": ("delta", (B, S + 2, H)),
    "sink_heads": ("attn_sink", (H - 1,)),
    "accum_rows": ("dkv_accum", (B, S_kv + 1, D)),
    "accum_dim": ("dkv_accum", (B, S_kv, D + 8)),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_each_mismatch_raises(case):
    name, shape = BAD[case]
    args = good()
    args[name] = torch.zeros(shape, dtype=args[name].dtype)
    with pytest.raises(ValueError):
        call(args)


def test_device_mismatch_raises():
    args = good()
    args["lse"] = torch.zeros((B, S, H), dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match="lse"):
        call(args)
