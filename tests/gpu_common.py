"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, move results to NumPy, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

SENT = 0xFFFFFFFF


def gpu_available() -> bool:
    return torch.cuda.is_available()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def i32(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def bf16_from_bits(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between finite patterns (+0 == -0)."""
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


def run_path(mod, ids: np.ndarray, real_count: int, n_experts: int, x: torch.Tensor, y: torch.Tensor,
             w: np.ndarray, variants=("bf16", "mxfp4"), tp_rank: int = 0, device="cuda"):
    """mask -> indices -> dispatch (each variant) -> combine on the GPU.  Returns a dict of
    device tensors."""
    n, k = ids.shape
    h = x.shape[1]
    s = n * k
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(device)
    d_cnt = torch.tensor([real_count], dtype=torch.int32, device=device)
    d_w = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(device)
    mod.moe_mask_padding(d_ids, d_cnt, tp_rank)
    idx = mod.alloc_indices(s, n_experts, device)
    mod.moe_create_indices(d_ids, n_experts, idx["token_expert_order"], idx["expert_start_indices"],
                           idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                           idx["workspace"])
    res = dict(ids=d_ids, count=d_cnt, weights=d_w, **idx)
    if "bf16" in variants:
        out = mod.alloc_dispatch(s, h, device)
        mod.moe_dispatch(x, k, idx["restore_token_order"], out)
        res["dispatch"] = out
    if "mxfp4" in variants:
        q, sc = mod.alloc_dispatch_mxfp4(s, h, device)
        mod.moe_dispatch_mxfp4(x, k, idx["restore_token_order"], q, sc)
        res["q"], res["scales"] = q, sc
    if y is not None:
        o = torch.empty((n, h), dtype=torch.bfloat16, device=device)
        mod.moe_combine(y, d_w, idx["restore_token_order"], k, o)
        res["combine"] = o
    torch.cuda.synchronize()
    return res


INDEX_KEYS = ("token_expert_order", "expert_start_indices", "restore_token_order", "expert_ids",
              "expert_usage_stats")


def check_indices(res: dict, ref: dict) -> None:
    for key in INDEX_KEYS:
        got = res[key]
        got = i32(got).astype(np.int64) if got.dtype == torch.int32 else u32(got).astype(np.int64)
        np.testing.assert_array_equal(got, ref[key].astype(np.int64), err_msg=key)
